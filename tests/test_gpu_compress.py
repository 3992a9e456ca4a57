"""GPU parity of cskv_compress against the oracle (compression of
overlapping 2m-token windows with a per-dimension softmax)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import TOL, dev, host_f64, rowwise_err

pytestmark = pytest.mark.gpu
D = 512


def _cskv():
    import compressed_sparse_kv_overlapping_amd as cskv
    return cskv


def _inputs(T, m, dt, seed, bias_std=0.1, cfg=90):
    x = wl.normal(cfg, seed, 1, (T, D))
    z = wl.normal(cfg, seed, 2, (T, D))
    b = wl.normal(cfg, seed, 3, (2 * m, D), bias_std)
    return wl.encode(x, dt), wl.encode(z, dt), b


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
@pytest.mark.parametrize("m,T", [(4, 4096), (128, 4096), (4, 4099), (1, 37), (2, 64), (3, 50),
                                 (8, 200), (16, 1000), (128, 1300), (256, 2048)])
def test_compress_matches_oracle(dt, m, T):
    cskv = _cskv()
    x, z, b = _inputs(T, m, dt, seed=m * 7919 + T)
    got = cskv.compress(dev(x), dev(z), dev(b), m)
    torch.cuda.synchronize()
    ref = oracle.compress(x.raw, z.raw, dt, b, m)
    assert got.shape == (T // m, D)
    assert rowwise_err(host_f64(got), ref) <= TOL[dt]


def test_compress_tiny_workload_both_scales():
    """The fp32 4096-token workload: m=4 -> 1024 entries, m'=128 -> 32."""
    cskv = _cskv()
    inp = wl.make_inputs("tiny", seed=0)
    for m, bname in ((4, "b4"), (128, "b128")):
        got = cskv.compress(dev(inp["x"]), dev(inp["z"]), dev(inp[bname]), m)
        torch.cuda.synchronize()
        ref = oracle.compress(inp["x"].raw, inp["z"].raw, wl.DT_F32, inp[bname].raw, m)
        assert got.shape[0] == 4096 // m
        assert rowwise_err(host_f64(got), ref) <= 1e-4


def test_compress_into_entry_buffer_and_append():
    """ld_out = 576: only content columns written; entry ranges append."""
    cskv = _cskv()
    T, m = 1024, 4
    x, z, b = _inputs(T, m, wl.DT_BF16, seed=5)
    N = T // m
    ent = torch.full((N, 576), 7.0, dtype=torch.bfloat16, device="cuda")
    X, Z, Bb = dev(x), dev(z), dev(b)
    cskv.compress(X, Z, Bb, m, out=ent, entry_begin=0, entry_end=N - 1)
    cskv.compress(X, Z, Bb, m, out=ent, entry_begin=N - 1, entry_end=N)   # streaming append
    torch.cuda.synchronize()
    ref = oracle.compress(x.raw, z.raw, wl.DT_BF16, b, m)
    e = host_f64(ent)
    assert (e[:, 512:] == 7.0).all()
    assert rowwise_err(e[:, :512], ref) <= 2e-2


def test_compress_special_inputs():
    """Constant rows compress to that row; zero logits and bias give the mean."""
    cskv = _cskv()
    T, m = 512, 4
    rng = np.random.default_rng(3)
    row = rng.standard_normal(D).astype(np.float32)
    x = np.tile(row, (T, 1))
    z = (5 * rng.standard_normal((T, D))).astype(np.float32)
    b = rng.standard_normal((2 * m, D)).astype(np.float32)
    got = host_f64(cskv.compress(dev(x), dev(z), dev(b), m))
    np.testing.assert_allclose(got, np.tile(row, (T // m, 1)), rtol=2e-6, atol=1e-6)
    x2 = rng.standard_normal((T, D)).astype(np.float32)
    zero = np.zeros((T, D), np.float32)
    got = host_f64(cskv.compress(dev(x2), dev(zero), dev(np.zeros((2 * m, D), np.float32)), m))
    ref = oracle.compress(x2, zero, wl.DT_F32, np.zeros((2 * m, D), np.float32), m)
    assert rowwise_err(got, ref) <= 1e-5


def test_compress_large_logits_and_bias():
    """Logits up to +-80 and a bias spread of +-20 stay finite and accurate."""
    cskv = _cskv()
    T, m = 2048, 128
    rng = np.random.default_rng(4)
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = (30 * rng.standard_normal((T, D))).clip(-80, 80).astype(np.float32)
    b = (10 * rng.standard_normal((2 * m, D))).clip(-20, 20).astype(np.float32)
    got = host_f64(cskv.compress(dev(x), dev(z), dev(b), m))
    ref = oracle.compress(x, z, wl.DT_F32, b, m)
    assert np.isfinite(got).all()
    assert rowwise_err(got, ref) <= 1e-4


def test_compress_degenerate_sizes():
    cskv = _cskv()
    x = torch.zeros((3, D), device="cuda")
    out = cskv.compress(x, x, torch.zeros((8, D), device="cuda"), 4)   # T < m: no entries
    assert out.shape == (0, D)


def test_compress_1m_tokens_sampled():
    """The 1M-token bf16 layer: both scales at full size, sampled entries."""
    cskv = _cskv()
    inp = wl.make_inputs("layer_1m", seed=0)
    X, Z = dev(inp["x"]), dev(inp["z"])
    rng = np.random.default_rng(0)
    for m, bname in ((4, "b4"), (128, "b128")):
        N = (1 << 20) // m
        ent = torch.empty((N, 576), dtype=torch.bfloat16, device="cuda")
        cskv.compress(X, Z, dev(inp[bname]), m, out=ent)
        torch.cuda.synchronize()
        ids = np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 400)]))
        ref = oracle.compress(inp["x"].raw, inp["z"].raw, wl.DT_BF16, inp[bname].raw, m, entry_ids=ids)
        got = host_f64(ent[torch.from_numpy(ids).cuda(), :512])
        assert rowwise_err(got, ref) <= 2e-2


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
@pytest.mark.parametrize("ms,ml,T", [(4, 128, 4096), (4, 128, 4099), (4, 128, 4196), (2, 16, 1000),
                                     (1, 8, 517), (3, 12, 600), (4, 8, 333), (4, 128, 100),
                                     (4, 64, 64 * 61 + 7), (4, 128, 128 * 40), (4, 256, 256 * 9 + 5),
                                     (2, 6, 300)])
def test_compress2_matches_oracle(dt, ms, ml, T):
    """Both scales in one pass equal the oracle at each scale (ragged T,
    a whole number of blocks of waves or not; m' > 128 and an odd m'/m take
    the two single-scale kernels)."""
    cskv = _cskv()
    x, z, _ = _inputs(T, ms, dt, seed=ms * 31 + ml * 7 + T)
    bs = wl.normal(90, T, 5, (2 * ms, D), 0.1)
    bl = wl.normal(90, T, 6, (2 * ml, D), 0.1)
    os_, ol = cskv.compress2(dev(x), dev(z), dev(bs), ms, dev(bl), ml)
    torch.cuda.synchronize()
    assert os_.shape == (T // ms, D) and ol.shape == (T // ml, D)
    assert rowwise_err(host_f64(os_), oracle.compress(x.raw, z.raw, dt, bs, ms)) <= TOL[dt]
    if T // ml:
        assert rowwise_err(host_f64(ol), oracle.compress(x.raw, z.raw, dt, bl, ml)) <= TOL[dt]


def test_compress2_large_logits():
    cskv = _cskv()
    T, ms, ml = 4096 + 64, 4, 128
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = (30 * rng.standard_normal((T, D))).clip(-80, 80).astype(np.float32)
    bs = (3 * rng.standard_normal((2 * ms, D))).astype(np.float32)
    bl = (10 * rng.standard_normal((2 * ml, D))).clip(-20, 20).astype(np.float32)
    os_, ol = cskv.compress2(dev(x), dev(z), dev(bs), ms, dev(bl), ml)
    torch.cuda.synchronize()
    got_s, got_l = host_f64(os_), host_f64(ol)
    assert np.isfinite(got_s).all() and np.isfinite(got_l).all()
    assert rowwise_err(got_s, oracle.compress(x, z, wl.DT_F32, bs, ms)) <= 1e-4
    assert rowwise_err(got_l, oracle.compress(x, z, wl.DT_F32, bl, ml)) <= 1e-4


def test_compress2_1m_tokens_sampled():
    """The 1M-token bf16 layer: both scales from one pass, sampled entries,
    and equal (to bf16 rounding) to the single-scale kernels."""
    cskv = _cskv()
    inp = wl.make_inputs("layer_1m", seed=0)
    X, Z = dev(inp["x"]), dev(inp["z"])
    e4 = torch.empty(((1 << 20) // 4, 576), dtype=torch.bfloat16, device="cuda")
    e128 = torch.empty(((1 << 20) // 128, 576), dtype=torch.bfloat16, device="cuda")
    cskv.compress2(X, Z, dev(inp["b4"]), 4, dev(inp["b128"]), 128, out_small=e4, out_large=e128)
    s4 = cskv.compress(X, Z, dev(inp["b4"]), 4)
    s128 = cskv.compress(X, Z, dev(inp["b128"]), 128)
    torch.cuda.synchronize()
    assert rowwise_err(host_f64(e4[:, :512]), host_f64(s4)) <= 1e-2
    assert rowwise_err(host_f64(e128[:, :512]), host_f64(s128)) <= 1e-2
    rng = np.random.default_rng(1)
    for m, ent, bname in ((4, e4, "b4"), (128, e128, "b128")):
        N = (1 << 20) // m
        ids = np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 300)]))
        ref = oracle.compress(inp["x"].raw, inp["z"].raw, wl.DT_BF16, inp[bname].raw, m, entry_ids=ids)
        assert rowwise_err(host_f64(ent[torch.from_numpy(ids).cuda(), :512]), ref) <= 2e-2
