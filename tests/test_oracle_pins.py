"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: counts the
pages print, small cases worked by hand (tests/golden), closed forms,
invariants, library routines and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from oracle import numpy_ref
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32, BF16, E4M3 = 0, 1, 2


def _num(v):
    if isinstance(v, str):
        return math.log(float(v[2:])) if v.startswith("ln") else float(v)
    return float(v)


def _arr(a):
    return np.array([[_num(v) for v in row] for row in a], dtype=np.float32)


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- page counts

def test_entry_counts_printed_by_pages():
    g = _gold("page_counts.json")
    for it in g["entries"]:
        n = oracle.num_entries(it["T"], it["m"])
        if it["approx"]:
            assert abs(n - it["entries"]) <= it["rel_tol"] * it["entries"], it["cite"]
        else:
            assert n == it["entries"], it["cite"]
    # the workloads: 4096 -> 1024 / 32 and 2^20 -> 262,144 / 8,192
    assert oracle.num_entries(4096, 4) == 1024 and oracle.num_entries(4096, 128) == 32
    assert oracle.num_entries(1 << 20, 4) == 262144 and oracle.num_entries(1 << 20, 128) == 8192
    # the compress output really has floor(T/m) rows, including ragged T
    rng = np.random.default_rng(0)
    for T, m in [(13, 4), (16, 4), (3, 4), (300, 128)]:
        x = rng.standard_normal((T, 3)).astype(np.float32)
        b = np.zeros((2 * m, 3), np.float32)
        assert oracle.compress(x, x, F32, b, m).shape == (T // m, 3)


def test_attended_positions_printed_by_pages():
    g = _gold("page_counts.json")["csa_positions"]
    # count the rows the oracle attends: with q = 0 every row gets the same
    # weight, so lse = ln(number of rows)
    rng = np.random.default_rng(1)
    N, k, W, Ee, Dv = 2048, g["k"], g["window"], 8, 4
    ent = rng.standard_normal((N, Ee)).astype(np.float32)
    win = rng.standard_normal((W, Ee)).astype(np.float32)
    q = np.zeros((1, 1, Ee), np.float32)
    idx = np.arange(k, dtype=np.int32)[None]
    _, lse = oracle.csa_attend(q, ent, win, F32, idx, Dv=Dv)
    n_rows = math.exp(lse[0, 0])
    assert round(n_rows) == k + W
    assert abs(n_rows - g["approx_positions"]) <= g["positions_rel_tol"] * g["approx_positions"]
    red = g["context"] / n_rows
    assert abs(red - g["approx_reduction"]) <= g["reduction_rel_tol"] * g["approx_reduction"]


# ------------------------------------------------------------ decoders (OCP)

def test_e4m3_decode_matches_ocp_table():
    g = _gold("worked_examples.json")["e4m3"]
    for code, val in g["codes"].items():
        v = oracle.e4m3_value(int(code, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_value(int(code, 16)))
    # monotone over the positive finite codes, max 448
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:])) and vals[-1] == 448.0


def test_e4m3_roundtrip_of_the_input_encoder():
    # encoding then decoding lands on the nearest representable value
    rng = np.random.default_rng(2)
    a = rng.standard_normal(5000).astype(np.float32) * 3
    s = wl.e4m3_scale(a)
    codes = wl.e4m3_encode(a, s)
    dec = oracle.decode(codes, E4M3) * s
    table = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    near = table[np.abs(np.abs(a[:, None] / s) - table[None]).argmin(1)] * np.sign(a) * s
    assert np.allclose(dec, near, rtol=0, atol=1e-12 * s)
    assert np.abs(dec).max() == pytest.approx(np.abs(a).max(), rel=1e-6)


def test_mxfp4_decode_matches_ocp_tables():
    g = _gold("worked_examples.json")["mxfp4"]
    for code, val in g["e2m1"].items():
        v = oracle.e2m1_value(int(code, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for x, val in g["e8m0"].items():
        assert oracle.e8m0_value(int(x)) == val, x
    for x in g["e8m0_nan"]:
        assert math.isnan(oracle.e8m0_value(x))


def _one_hot_mxfp4(i, code, s0, s1):
    codes = np.zeros((1, 32), np.uint8)
    codes[0, i // 2] = code << (4 * (i % 2))
    return codes, np.array([[s0, s1]], np.uint8)


def test_mxfp4_element_placement():
    """Element i sits in nibble i % 2 of byte i // 2 and takes the scale of
    block i // 32: a single non-zero code lands at i with that block's
    power of two, nowhere else."""
    for i in range(64):
        for code, val in ((0x2, 1.0), (0xF, -6.0), (0x1, 0.5)):
            c, sc = _one_hot_mxfp4(i, code, 120, 131)
            row = oracle.mxfp4_decode(c, sc)[0]
            want = np.zeros(64)
            want[i] = val * 2.0 ** ((120 if i < 32 else 131) - 127)
            assert np.array_equal(row, want), (i, code)


def test_mxfp4_element_placement_in_entry_rows():
    """576-element entry rows (18 blocks): element i sits in nibble i % 2 of
    byte i // 2 with the scale of block i // 32, each block its own power."""
    rng = np.random.default_rng(9)
    xs = rng.integers(100, 150, 18).astype(np.uint8)
    for i in list(range(0, 576, 7)) + [31, 32, 63, 64, 543, 544, 575]:
        codes = np.zeros((1, 288), np.uint8)
        codes[0, i // 2] = 0x5 << (4 * (i % 2))                 # 3.0
        row = oracle.mxfp4_decode(codes, xs[None])[0]
        want = np.zeros(576)
        want[i] = 3.0 * 2.0 ** (int(xs[i // 32]) - 127)
        assert np.array_equal(row, want), i


def test_decoded_inputs_attend_like_stored_ones():
    """The fp64 input path (used for MXFP4 entries, decoded first) gives the
    bf16 path's results exactly on the decoded values, and MXFP4 entries
    holding bf16-exact values attend like those bf16 rows."""
    rng = np.random.default_rng(12)
    B, H, N, W, k = 2, 3, 40, 5, 7
    q = wl.bf16_bits(rng.standard_normal((B, H, 576)).astype(np.float32) / 24)
    vals = rng.integers(-6, 7, (N, 576)).astype(np.float64) * 0.5     # on the E2M1 grid
    vals[np.abs(vals) == 2.5] = 2.0
    ent = wl.bf16_bits(vals.astype(np.float32))
    win = wl.bf16_bits(rng.standard_normal((W, 576)).astype(np.float32))
    idx = np.sort(rng.choice(N, (B, k)), axis=1).astype(np.int32)
    o1, l1 = oracle.csa_attend(q, ent, win, BF16, idx)
    o2, l2 = oracle.csa_attend(oracle.decode(q, BF16), oracle.decode(ent, BF16),
                               oracle.decode(win, BF16), oracle.F64, idx)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    codes, scales = wl.mxfp4_encode(vals)
    assert np.array_equal(oracle.mxfp4_decode(codes, scales), vals)
    o3, l3 = oracle.csa_attend_mxfp4(q, codes, scales, win, idx)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    h1, hl1 = oracle.hca_attend(q, ent, BF16)
    h3, hl3 = oracle.hca_attend_mxfp4(q, codes, scales)
    assert np.array_equal(h1, h3) and np.array_equal(hl1, hl3)


def _unpack_codes(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (64,))


def test_mxfp4_scores_reduce_to_the_f32_path():
    """With unit scales (X = 127) MXFP4 scores equal the fp32 scores of the
    E2M1 table values; other scales multiply each block's share of the dot
    product by 2^(Xq + Xk - 254)."""
    table = np.array([_gold("worked_examples.json")["mxfp4"]["e2m1"]["0x%x" % c] for c in range(16)])
    rng = np.random.default_rng(41)
    B, N = 3, 50
    qc = rng.integers(0, 256, (B, 32), dtype=np.uint8)
    kc = rng.integers(0, 256, (N, 32), dtype=np.uint8)
    ones_q, ones_k = np.full((B, 2), 127, np.uint8), np.full((N, 2), 127, np.uint8)
    s, v = oracle.index_scores_mxfp4(qc, ones_q, kc, ones_k, 0.75)
    qf = table[_unpack_codes(qc)].astype(np.float32)
    kf = table[_unpack_codes(kc)].astype(np.float32)
    s32, v32 = oracle.index_scores(qf, kf, F32, 0.75)
    assert np.array_equal(s, s32) and np.array_equal(v, v32)
    # per-block scale: blocks scored on their own with unit scales
    xq = rng.integers(120, 135, (B, 2)).astype(np.uint8)
    xk = rng.integers(120, 135, (N, 2)).astype(np.uint8)
    sx, _ = oracle.index_scores_mxfp4(qc, xq, kc, xk, 1.0)
    part = []
    for blk in range(2):
        keep = np.zeros(64, bool)
        keep[32 * blk:32 * blk + 32] = True
        sb, _ = oracle.index_scores((qf * keep).astype(np.float32), kf, F32, 1.0)
        f = 2.0 ** (xq[:, blk, None].astype(float) + xk[None, :, blk].astype(float) - 254)
        part.append(sb * f)
    assert np.array_equal(sx, part[0] + part[1])


def test_mxfp4_encoder_roundtrip():
    """The input encoder keeps values that MXFP4 holds exactly, and rounds
    others to the nearest value on their block's grid."""
    rng = np.random.default_rng(5)
    table = np.array([oracle.e2m1_value(c) for c in range(16)])
    # exact: table values times a block power of two, each block reaching 4 or 6
    c = rng.integers(0, 16, (20, 64))
    c[:, 0], c[:, 32] = 6, 15
    e = rng.integers(-10, 10, (20, 2))
    a = table[c] * np.repeat(2.0 ** e, 32, axis=1)
    codes, scales = wl.mxfp4_encode(a)
    assert np.array_equal(oracle.mxfp4_decode(codes, scales), a)
    # general values: nearest grid point of the chosen block scale
    a = rng.standard_normal((200, 64)) * 3
    codes, scales = wl.mxfp4_encode(a)
    dec = oracle.mxfp4_decode(codes, scales)
    unit = np.repeat(np.array([[oracle.e8m0_value(x) for x in r] for r in scales]), 32, axis=1)
    grid = table[None, None, :] * unit[..., None]
    best = np.abs(a[..., None] - grid).min(axis=-1)
    assert np.allclose(np.abs(a - dec), best, rtol=0, atol=1e-12)
    assert (np.abs(dec) <= 6 * unit).all()


def test_bf16_decode():
    g = _gold("worked_examples.json")["bf16"]
    for code, val in g["codes"].items():
        assert oracle.bf16_value(int(code, 16)) == pytest.approx(val, rel=1e-12)


# -------------------------------------------------------------- compression

def test_compress_worked_examples():
    for c in _gold("worked_examples.json")["compress"]:
        x, z, b = _arr(c["x"]), _arr(c["z"]), _arr(c["bias"])
        got = oracle.compress(x, z, F32, b, c["m"])
        np.testing.assert_allclose(got, np.array(c["expect"], float), rtol=1e-6, err_msg=c["name"])


@pytest.mark.parametrize("m,T", [(4, 64), (4, 67), (128, 640), (1, 9), (3, 20)])
def test_compress_constant_rows(m, T):
    """A window whose rows are all equal compresses to that row, whatever z, b."""
    rng = np.random.default_rng(m * 1000 + T)
    D = 16
    row = rng.standard_normal(D).astype(np.float32)
    x = np.tile(row, (T, 1))
    z = (3 * rng.standard_normal((T, D))).astype(np.float32)
    b = rng.standard_normal((2 * m, D)).astype(np.float32)
    got = oracle.compress(x, z, F32, b, m)
    np.testing.assert_allclose(got, np.tile(row, (T // m, 1)), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("m,T", [(4, 64), (4, 70), (128, 1024), (2, 7)])
def test_compress_zero_logits_is_window_mean(m, T):
    """z = 0 and b = 0: the plain mean of the present window rows."""
    rng = np.random.default_rng(T)
    D = 8
    x = rng.standard_normal((T, D)).astype(np.float32)
    zero = np.zeros_like(x)
    got = oracle.compress(x, zero, F32, np.zeros((2 * m, D), np.float32), m)
    xd = x.astype(np.float64)
    for i in range(T // m):
        lo = max(0, (i - 1) * m)
        np.testing.assert_allclose(got[i], xd[lo:(i + 1) * m].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_compress_bias_only_closed_form():
    """z = 0, b != 0: weights are softmax over window positions of b (scipy)."""
    rng = np.random.default_rng(5)
    m, T, D = 4, 40, 6
    x = rng.standard_normal((T, D)).astype(np.float32)
    b = rng.standard_normal((2 * m, D)).astype(np.float32)
    got = oracle.compress(x, np.zeros_like(x), F32, b, m)
    xd, bd = x.astype(np.float64), b.astype(np.float64)
    for i in range(1, T // m):
        w = sp_softmax(bd, axis=0)                        # [2m, D]
        np.testing.assert_allclose(got[i], (w * xd[(i - 1) * m:(i + 1) * m]).sum(0), rtol=1e-12)
    w0 = sp_softmax(bd[m:], axis=0)                       # entry 0: positions m..2m-1 only
    np.testing.assert_allclose(got[0], (w0 * xd[:m]).sum(0), rtol=1e-12)


def test_compress_one_hot_logit_picks_that_token():
    rng = np.random.default_rng(6)
    m, T, D = 4, 32, 5
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = np.zeros_like(x)
    i, p = 3, 5                                            # token (i-1)m + p
    z[(i - 1) * m + p] = 60.0
    got = oracle.compress(x, z, F32, np.zeros((2 * m, D), np.float32), m, entry_ids=[i])
    np.testing.assert_allclose(got[0], x[(i - 1) * m + p], rtol=1e-12, atol=1e-20)


def test_compress_shift_linear_bounded():
    rng = np.random.default_rng(7)
    m, T, D = 4, 48, 7
    x = rng.standard_normal((T, D)).astype(np.float32)
    x2 = rng.standard_normal((T, D)).astype(np.float32)
    # logits on a 2^-10 grid so that z + shift stays exact in fp32
    z = (np.round(rng.standard_normal((T, D)) * 1024) / 1024).astype(np.float32)
    b = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    base = oracle.compress(x, z, F32, b, m)
    # a per-column constant added to every logit changes nothing
    shift = np.arange(D, dtype=np.float32)[None] * 3
    np.testing.assert_allclose(oracle.compress(x, z + shift, F32, b, m), base, rtol=1e-12, atol=1e-13)
    # linear in x for fixed z
    both = oracle.compress((x + 2 * x2).astype(np.float32), z, F32, b, m)
    np.testing.assert_allclose(both, base + 2 * oracle.compress(x2, z, F32, b, m), rtol=1e-6, atol=1e-6)
    # each output lies within its window's column range
    xd = x.astype(np.float64)
    for i in range(T // m):
        win = xd[max(0, (i - 1) * m):(i + 1) * m]
        assert np.all(base[i] <= win.max(0) + 1e-12) and np.all(base[i] >= win.min(0) - 1e-12)


def test_compress_bf16_storage_decoded_exactly():
    rng = np.random.default_rng(8)
    m, T, D = 4, 40, 8
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal((T, D)).astype(np.float32)
    b = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    xb, zb = wl.bf16_bits(x), wl.bf16_bits(z)
    got = oracle.compress(xb, zb, BF16, b, m)
    ref = oracle.compress(wl.bf16_bits_to_f32(xb), wl.bf16_bits_to_f32(zb), F32, b, m)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("m,T", [(4, 256), (4, 257), (128, 1024), (128, 1100)])
def test_compress_matches_numpy_formulation(m, T):
    rng = np.random.default_rng(m + T)
    D = 32
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = (2 * rng.standard_normal((T, D))).astype(np.float32)
    b = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    got = oracle.compress(x, z, F32, b, m)
    ref = numpy_ref.compress(x.astype(np.float64), z.astype(np.float64), b, m)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_compress_entry_subset_equals_full():
    rng = np.random.default_rng(9)
    m, T, D = 4, 64, 4
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal((T, D)).astype(np.float32)
    b = rng.standard_normal((2 * m, D)).astype(np.float32)
    full = oracle.compress(x, z, F32, b, m)
    ids = np.array([15, 0, 7])
    np.testing.assert_array_equal(oracle.compress(x, z, F32, b, m, entry_ids=ids), full[ids])


def test_compress_rejects_out_of_range_entries():
    x = np.zeros((8, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.compress(x, x, F32, np.zeros((8, 2), np.float32), 4, entry_ids=[2])


# ------------------------------------------------------------------ indexer

def test_index_scores_worked_example():
    c = _gold("worked_examples.json")["index_scores"][0]
    s, v = oracle.index_scores(_arr(c["qI"]), _arr(c["kI"]), F32, c["scale"])
    np.testing.assert_array_equal(s, np.array(c["expect"], float))
    assert v.all()


def test_index_scores_small_integers_exact_in_all_dtypes():
    rng = np.random.default_rng(10)
    q = rng.integers(-4, 5, size=(3, 64)).astype(np.float32)
    k = rng.integers(-4, 5, size=(50, 64)).astype(np.float32)
    want = q.astype(np.int64) @ k.astype(np.int64).T
    for dt in (F32, BF16):
        qs, ks = wl.encode(q, dt).raw, wl.encode(k, dt).raw
        s, _ = oracle.index_scores(qs, ks, dt)
        np.testing.assert_array_equal(s, want)
    # e4m3 with scale 1 represents the integers -4..4 exactly
    s, _ = oracle.index_scores(wl.e4m3_encode(q, 1.0), wl.e4m3_encode(k, 1.0), E4M3, 1.0)
    np.testing.assert_array_equal(s, want)
    # per-tensor scales multiply in
    s2, _ = oracle.index_scores(wl.e4m3_encode(q, 1.0), wl.e4m3_encode(k, 1.0), E4M3, 0.25)
    np.testing.assert_array_equal(s2, 0.25 * want)


def test_index_scores_match_matmul():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((300, 64)).astype(np.float32)
    s, _ = oracle.index_scores(q, k, F32, 0.5)
    np.testing.assert_allclose(s, numpy_ref.index_scores(q.astype(float), k.astype(float), 0.5), rtol=1e-12, atol=1e-12)


def test_causal_visibility():
    for c in _gold("worked_examples.json")["visibility"]:
        q = np.ones((1, 4), np.float32)
        k = np.ones((c["N"], 4), np.float32)
        _, v = oracle.index_scores(q, k, F32, 1.0, q_pos=np.array([c["pos"]]), m=c["m"])
        assert int(v.sum()) == c["visible"], c["why"]
        assert v[0, :c["visible"]].all()
    # prefill positions of the 1M workload: the last query sees all 262,144 entries
    q = np.ones((2, 1), np.float32)
    k = np.ones((262144, 1), np.float32)
    _, v = oracle.index_scores(q, k, F32, 1.0, q_pos=np.array([1044480, 1048575]), m=4)
    assert v[1].sum() == 262144 and v[0].sum() == 261120   # (i+1)*4 <= 1044481


# -------------------------------------------------------------------- top-k

def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(12)
    s = np.round(rng.standard_normal((5, 400)), 1)        # many exact ties
    v = (rng.random((5, 400)) < 0.8).astype(np.uint8)
    got = oracle.topk(s, v, 37)
    np.testing.assert_array_equal(got, numpy_ref.topk(s, v, 37))


def test_topk_permutation_and_ties_and_padding():
    N, k = 100, 10
    perm = np.random.default_rng(13).permutation(N).astype(np.float64)
    got = oracle.topk(perm[None], np.ones((1, N), np.uint8), k)
    assert set(got[0]) == set(np.nonzero(perm >= N - k)[0])
    assert list(perm[got[0]]) == sorted(perm[got[0]], reverse=True)
    # all scores equal -> the lowest indices, in order
    eq = oracle.topk(np.zeros((1, N)), np.ones((1, N), np.uint8), k)
    assert list(eq[0]) == list(range(k))
    # fewer visible than k -> -1 padding
    vis = np.zeros((1, N), np.uint8)
    vis[0, [5, 50, 7]] = 1
    got = oracle.topk(perm[None], vis, k)
    assert set(got[0, :3]) == {5, 50, 7} and (got[0, 3:] == -1).all()


# ---------------------------------------------------------------- attention

def test_attention_worked_example():
    c = _gold("worked_examples.json")["attention"][0]
    q = _arr(c["q"])[None]
    rows = _arr(c["rows"])
    out, lse = oracle.hca_attend(q, rows, F32, Dv=c["Dv"])
    np.testing.assert_allclose(out[0], np.array(c["expect_out"]), rtol=1e-7)
    np.testing.assert_allclose(lse[0], [_num(v) for v in c["expect_lse"]], rtol=1e-7)


def _rand_attn(seed, B=2, H=3, N=40, W=6, Ee=12):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, H, Ee)) / 2).astype(np.float32)
    ent = rng.standard_normal((N, Ee)).astype(np.float32)
    win = rng.standard_normal((W, Ee)).astype(np.float32)
    return q, ent, win


def test_csa_all_entries_equals_dense_attention():
    """k >= number of entries: CSA is dense softmax attention over entries + window."""
    q, ent, win = _rand_attn(14)
    N, Dv = ent.shape[0], 8
    idx = np.tile(np.arange(N + 5, dtype=np.int32), (2, 1))       # k = N + 5 > N
    idx[idx >= N] = -1
    out, lse = oracle.csa_attend(q, ent, win, F32, idx, Dv=Dv)
    rows = np.concatenate([ent, win]).astype(np.float64)
    for b in range(2):
        ro, rl = numpy_ref.attend(q[b].astype(np.float64), rows, Dv)
        np.testing.assert_allclose(out[b], ro, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-12)


def test_tiny_end_to_end_brute_force():
    """Tiny T: compress at m=4, select all, attend -> brute-force dense attention
    (scipy softmax of a matrix product) over the same rows."""
    rng = np.random.default_rng(15)
    T, m, D, Rr, W, H = 64, 4, 8, 4, 8, 2
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal((T, D)).astype(np.float32)
    b = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    N = T // m
    ent = np.empty((N, D + Rr), np.float32)
    ent[:, :D] = oracle.compress(x, z, F32, b, m)
    ent[:, D:] = rng.standard_normal((N, Rr))
    win = np.concatenate([x[T - W:], rng.standard_normal((W, Rr)).astype(np.float32)], axis=1)
    q = (rng.standard_normal((1, H, D + Rr)) / 3).astype(np.float32)
    qI = rng.standard_normal((1, 4)).astype(np.float32)
    kI = rng.standard_normal((N, 4)).astype(np.float32)
    s, v = oracle.index_scores(qI, kI, F32)
    idx = oracle.topk(s, v, N)                             # k = N selects everything
    out, lse = oracle.csa_attend(q, ent, win, F32, idx, Dv=D)
    rows = np.concatenate([ent, win]).astype(np.float64)
    logits = q[0].astype(np.float64) @ rows.T
    p = sp_softmax(logits, axis=1)
    np.testing.assert_allclose(out[0], p @ rows[:, :D], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], np.log(np.exp(logits).sum(1)), rtol=1e-12)


def test_attention_special_cases():
    q, ent, win = _rand_attn(16)
    N, Dv = ent.shape[0], 8
    idx = np.array([[3, 9, -1, 20], [0, 1, 2, 3]], dtype=np.int32)
    # q = 0: uniform mean of the V rows, lse = ln(rows)
    zq = np.zeros_like(q)
    out, lse = oracle.csa_attend(zq, ent, win, F32, idx, Dv=Dv)
    rows0 = np.concatenate([ent[[3, 9, 20]], win]).astype(np.float64)
    np.testing.assert_allclose(out[0, 0], rows0[:, :Dv].mean(0), rtol=1e-12)
    np.testing.assert_allclose(lse[0], np.log(len(rows0)), rtol=1e-12)
    # one dominant logit: the output is that row's value
    q2 = np.zeros_like(q)
    q2[0, 0] = 80.0 * ent[9] / np.linalg.norm(ent[9]) ** 2
    out, _ = oracle.csa_attend(q2, ent, win, F32, idx, Dv=Dv)
    l = (q2[0, 0].astype(np.float64) @ rows0.T)
    assert l.argmax() == 1 and np.sort(l)[-1] - np.sort(l)[-2] > 40
    np.testing.assert_allclose(out[0, 0], ent[9, :Dv], rtol=1e-9, atol=1e-9)
    # permuting the selected rows changes nothing
    outA, lseA = oracle.csa_attend(q, ent, win, F32, idx, Dv=Dv)
    outB, lseB = oracle.csa_attend(q, ent, win, F32, idx[:, ::-1].copy(), Dv=Dv)
    np.testing.assert_allclose(outA, outB, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lseA, lseB, rtol=1e-13)


def test_hca_equals_csa_with_all_entries_and_no_window():
    q, ent, _ = _rand_attn(17)
    N = ent.shape[0]
    o1, l1 = oracle.hca_attend(q, ent, F32, Dv=8)
    idx = np.tile(np.arange(N, dtype=np.int32), (2, 1))
    o2, l2 = oracle.csa_attend(q, ent, None, F32, idx, W=0, Dv=8)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    for b in range(2):
        ro, rl = numpy_ref.attend(q[b].astype(float), ent.astype(float), 8)
        np.testing.assert_allclose(o1[b], ro, rtol=1e-12, atol=1e-14)


def test_hca_prefill_causal_visibility():
    """HCA at a prefill chunk: the query at position pos sees entries i with
    (i+1)m <= pos+1.  Pins: no visible entry gives a zero output and lse
    -inf; otherwise the result equals the NumPy formulation over the first
    min(N, (pos+1)//m) entries; with every entry visible it is the decode
    result itself; one more block of m positions adds exactly one entry."""
    m, N, Dv = 4, 40, 8
    pos = np.array([2, 3, 57, 60, 61, N * m - 1, 10**6], dtype=np.int64)
    q, ent, _ = _rand_attn(19, B=len(pos), N=N)
    out, lse = oracle.hca_attend(q, ent, F32, Dv=Dv, q_pos=pos, m=m)
    full, lfull = oracle.hca_attend(q, ent, F32, Dv=Dv)
    nvis = [min(N, (int(p) + 1) // m) for p in pos]
    assert nvis == [0, 1, 14, 15, 15, N, N]
    for b, n in enumerate(nvis):
        if n == 0:
            assert (out[b] == 0).all() and np.isneginf(lse[b]).all()
            continue
        ro, rl = numpy_ref.attend(q[b].astype(float), ent[:n].astype(float), Dv)
        np.testing.assert_allclose(out[b], ro, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-13)
        if n == N:
            np.testing.assert_array_equal(out[b], full[b])
            np.testing.assert_array_equal(lse[b], lfull[b])
    # the same query at positions 57 and 61 (one block later): exactly
    # entry 14 more
    oa, _ = oracle.hca_attend(q[2:3], ent, F32, Dv=Dv, q_pos=np.array([57]), m=m)
    ob, _ = oracle.hca_attend(q[2:3], ent, F32, Dv=Dv, q_pos=np.array([61]), m=m)
    o15, _ = oracle.hca_attend(q[2:3], ent[:15], F32, Dv=Dv)
    np.testing.assert_array_equal(oa, out[2:3])
    np.testing.assert_array_equal(ob, o15)
    assert not np.allclose(oa, ob)


def test_attention_sink():
    """Attention-sink logits: one more softmax term per head with a zero
    value.  Pins: a sink of -inf is no sink; with all logits 0 (q = 0) the
    output is the rows' mean times n / (n + e^s) and lse = ln(n + e^s); a
    sink far above every logit takes all the mass (output -> 0, lse -> s);
    both HCA and CSA equal the NumPy formulation with a virtual zero row;
    the lse-weighted merge of sink-free partials plus the sink term in the
    denominator equals the unsplit result with the sink."""
    q, ent, win = _rand_attn(20, H=3)
    N, Dv = ent.shape[0], 8
    sink = np.array([0.3, -1.5, 2.0])
    o0, l0 = oracle.hca_attend(q, ent, F32, Dv=Dv)
    oi, li = oracle.hca_attend(q, ent, F32, Dv=Dv, sink=np.full(3, -np.inf))
    np.testing.assert_array_equal(o0, oi)
    np.testing.assert_array_equal(l0, li)
    zq = np.zeros_like(q)
    oz, lz = oracle.hca_attend(zq, ent, F32, Dv=Dv, sink=sink)
    mean = ent[:, :Dv].astype(np.float64).mean(0)
    for h in range(3):
        np.testing.assert_allclose(oz[0, h], mean * N / (N + np.exp(sink[h])), rtol=1e-12)
        np.testing.assert_allclose(lz[0, h], np.log(N + np.exp(sink[h])), rtol=1e-13)
    big = np.full(3, 300.0)
    ob, lb = oracle.hca_attend(q, ent, F32, Dv=Dv, sink=big)
    assert np.abs(ob).max() < 1e-90
    np.testing.assert_allclose(lb, 300.0, rtol=1e-15)
    os_, ls = oracle.hca_attend(q, ent, F32, Dv=Dv, sink=sink)
    idx = np.array([[3, 9, -1, 20], [0, 1, 2, 3]], dtype=np.int32)
    oc, lc = oracle.csa_attend(q, ent, win, F32, idx, Dv=Dv, sink=sink)
    for b in range(2):
        ro, rl = numpy_ref.attend(q[b].astype(float), ent.astype(float), Dv, sink=sink)
        np.testing.assert_allclose(os_[b], ro, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ls[b], rl, rtol=1e-13)
        sel = [i for i in idx[b] if i >= 0]
        rows = np.concatenate([ent[sel], win]).astype(float)
        ro, rl = numpy_ref.attend(q[b].astype(float), rows, Dv, sink=sink)
        np.testing.assert_allclose(oc[b], ro, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lc[b], rl, rtol=1e-13)
    parts = np.array_split(np.arange(N), 5)
    po, pl = zip(*[oracle.hca_attend(q, ent[p], F32, Dv=Dv) for p in parts])
    pl = np.stack(pl)                                                 # [S, B, H]
    L = np.log(np.exp(pl).sum(0) + np.exp(sink))
    mo = sum(np.exp(pl[s] - L)[..., None] * po[s] for s in range(5))
    np.testing.assert_allclose(L, ls, rtol=1e-12)
    np.testing.assert_allclose(mo, os_, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 7, 40])
def test_split_merge_formula_recovers_unsplit(splits):
    """lse-weighted merge of partial attentions over a partition of the rows
    equals attention over all rows (pins the oracle's lse)."""
    q, ent, _ = _rand_attn(18, N=40)
    o, l = oracle.hca_attend(q, ent, F32, Dv=8)
    parts = np.array_split(np.arange(40), splits)
    po, pl = zip(*[oracle.hca_attend(q, ent[p], F32, Dv=8) for p in parts])
    pl = np.stack(pl)                                      # [S, B, H]
    L = np.log(np.exp(pl).sum(0))
    mo = sum(np.exp(pl[s] - L)[..., None] * po[s] for s in range(splits))
    np.testing.assert_allclose(L, l, rtol=1e-12)
    np.testing.assert_allclose(mo, o, rtol=1e-11, atol=1e-13)


def test_prefill_window_positions():
    """Prefill: the window of a query at pos is raw positions max(0,pos-W+1)..pos."""
    rng = np.random.default_rng(19)
    W, Ee, Dv = 4, 6, 3
    src = rng.standard_normal((10, Ee)).astype(np.float32)     # positions 100..109
    ent = rng.standard_normal((5, Ee)).astype(np.float32)
    q = np.zeros((2, 1, Ee), np.float32)                       # uniform weights
    idx = np.full((2, 2), -1, np.int32)                        # no entries selected
    out, lse = oracle.csa_attend(q, ent, src, F32, idx, q_pos=np.array([103, 109]),
                                 win_pos0=100, W=W, Dv=Dv)
    sd = src.astype(np.float64)
    np.testing.assert_allclose(out[0, 0], sd[0:4, :Dv].mean(0), rtol=1e-12)
    np.testing.assert_allclose(out[1, 0], sd[6:10, :Dv].mean(0), rtol=1e-12)
    np.testing.assert_allclose(lse, np.log(4), rtol=1e-12)
    with pytest.raises(ValueError):                           # window outside the buffer
        oracle.csa_attend(q, ent, src, F32, idx, q_pos=np.array([102, 109]), win_pos0=100, W=W, Dv=Dv)


# ------------------------------------------- query / entry normalisation
# ("DeepSeek V4 comprimeix el context", section "CSA: buscar primer i atendre
# despres": queries and compressed entries are normalised to stabilise the
# logits.  Reading: unit root-mean-square over the 576 dims, x / sqrt(mean(x^2)
# + eps), no learned gain; the normalised entry is key and value; raw window
# rows stay as they are.)

def _norm_inputs(seed, B=2, H=3, N=40, W=6, k=9, dt=wl.DT_BF16):
    rng = np.random.default_rng(seed)
    q = wl.encode(rng.standard_normal((B, H, 576)) * rng.uniform(0.01, 0.2, (B, H, 1)), dt).raw
    ent = wl.encode(rng.standard_normal((N, 576)) * rng.uniform(0.2, 5.0, (N, 1)), dt).raw
    win = wl.encode(rng.standard_normal((W, 576)) * 0.7, dt).raw
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[0, 2] = -1
    return q, ent, win, idx


def test_norm_single_row_is_that_row_over_its_rms():
    """One selected entry and no window: every weight is 1, so the output is
    the normalised entry's value part, whatever the query."""
    eps = 1e-6
    q, ent, win, idx = _norm_inputs(11)
    idx1 = idx[:, :1]
    out, lse = oracle.csa_attend(q, ent, None, wl.DT_BF16, idx1, W=0, norm_eps=eps)
    dec = oracle.decode(ent, wl.DT_BF16)
    for b in range(q.shape[0]):
        row = dec[idx1[b, 0]]
        want = row[:512] / math.sqrt(float(np.mean(row * row)) + eps)
        np.testing.assert_allclose(out[b], np.tile(want, (q.shape[1], 1)), rtol=1e-13, atol=1e-15)


def test_norm_equals_attention_over_prenormalised_rows():
    """The oracle's folded factors equal a NumPy attention over rows that were
    normalised first (entries only; window rows as given), with and without a
    sink, for CSA and HCA."""
    eps = 1e-5
    q, ent, win, idx = _norm_inputs(12)
    qv = oracle.decode(q, wl.DT_BF16)
    ev = oracle.decode(ent, wl.DT_BF16)
    wv = oracle.decode(win, wl.DT_BF16)
    sink = np.array([0.3, -1.0, 2.0])
    for s in (None, sink):
        out, lse = oracle.csa_attend(q, ent, win, wl.DT_BF16, idx, scale=0.05, norm_eps=eps, sink=s)
        for b in range(q.shape[0]):
            sel = idx[b][idx[b] >= 0]
            rows = np.concatenate([numpy_ref.rms_normalize(ev[sel], eps), wv])
            ro, rl = numpy_ref.attend(numpy_ref.rms_normalize(qv[b], eps), rows, scale=0.05, sink=s)
            np.testing.assert_allclose(out[b], ro, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse[b], rl, rtol=1e-12)
        out, lse = oracle.hca_attend(q, ent, wl.DT_BF16, scale=0.05, norm_eps=eps, sink=s)
        for b in range(q.shape[0]):
            ro, rl = numpy_ref.attend(numpy_ref.rms_normalize(qv[b], eps),
                                      numpy_ref.rms_normalize(ev, eps), scale=0.05, sink=s)
            np.testing.assert_allclose(out[b], ro, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse[b], rl, rtol=1e-12)


def test_norm_of_unit_rms_inputs_is_the_plain_path():
    """Elements of +-1 have a root-mean-square of exactly 1: with eps = 0 the
    normalised attention is the plain one."""
    rng = np.random.default_rng(13)
    B, H, N, W, k = 2, 4, 30, 5, 7
    q = rng.choice([-1.0, 1.0], (B, H, 576)).astype(np.float32)
    ent = rng.choice([-1.0, 1.0], (N, 576)).astype(np.float32)
    win = rng.standard_normal((W, 576)).astype(np.float32)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B)]).astype(np.int32)
    a = oracle.csa_attend(q, ent, win, wl.DT_F32, idx, scale=1 / 24, norm_eps=0.0)
    b = oracle.csa_attend(q, ent, win, wl.DT_F32, idx, scale=1 / 24)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14)


def test_norm_scale_invariance():
    """With eps = 0 the result does not change when a query head or an entry
    row is multiplied by a positive factor (powers of two keep the bf16
    inputs exact); scaling a window row does change it, since raw window
    rows are not normalised."""
    q, ent, win, idx = _norm_inputs(14)
    rng = np.random.default_rng(15)
    qf = oracle.decode(q, wl.DT_BF16) * 2.0 ** rng.integers(-3, 4, (q.shape[0], q.shape[1], 1))
    ef = oracle.decode(ent, wl.DT_BF16) * 2.0 ** rng.integers(-3, 4, (ent.shape[0], 1))
    q2, e2 = wl.bf16_bits(qf.astype(np.float32)), wl.bf16_bits(ef.astype(np.float32))
    a = oracle.csa_attend(q, ent, win, wl.DT_BF16, idx, scale=0.04, norm_eps=0.0)
    b = oracle.csa_attend(q2, e2, win, wl.DT_BF16, idx, scale=0.04, norm_eps=0.0)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    w2 = wl.bf16_bits((oracle.decode(win, wl.DT_BF16) * 2.0).astype(np.float32))
    c = oracle.csa_attend(q, ent, w2, wl.DT_BF16, idx, scale=0.04, norm_eps=0.0)
    assert np.abs(c[0] - a[0]).max() > 1e-3
    h1 = oracle.hca_attend(q, ent, wl.DT_BF16, scale=0.04, norm_eps=0.0)
    h2 = oracle.hca_attend(q2, e2, wl.DT_BF16, scale=0.04, norm_eps=0.0)
    np.testing.assert_allclose(h1[0], h2[0], rtol=1e-12, atol=1e-14)


# ------------------------------------------------ MXFP8 (E4M3) entry rows
# (FP8 storage of the compressed entries with block scales, "Compressed
# attention - CSA / HCA", section 3; read as OCP MXFP8: 32 E4M3 elements per
# E8M0 scale, one byte an element.)

def test_mxfp8_element_placement_in_entry_rows():
    """Element i of a 576-element row is code byte i and takes the scale of
    block i // 32: one non-zero code lands at i with that block's power of
    two times its E4M3 value (from the OCP table pinned above), nowhere else."""
    rng = np.random.default_rng(21)
    xs = rng.integers(100, 150, 18).astype(np.uint8)
    for i in list(range(0, 576, 11)) + [31, 32, 63, 64, 543, 544, 575]:
        for code in (0x38, 0xC5, 0x01, 0x7E):                  # 1.0, -3.25, 2^-9, 448
            codes = np.zeros((1, 576), np.uint8)
            codes[0, i] = code
            row = oracle.mxfp8_decode(codes, xs[None])[0]
            want = np.zeros(576)
            want[i] = oracle.e4m3_value(code) * 2.0 ** (int(xs[i // 32]) - 127)
            assert np.array_equal(row, want), (i, code)
    assert oracle.e4m3_value(0x38) == 1.0 and oracle.e4m3_value(0x7E) == 448.0


def test_mxfp8_encoder_roundtrip_and_nearest():
    """Values on a block's grid (an E4M3 value times the block's power of two)
    decode back exactly; other values decode to the nearest grid point."""
    rng = np.random.default_rng(22)
    grid = np.array([oracle.e4m3_value(c) for c in range(127)])
    ex = rng.integers(-20, 20, (6, 18))
    vals = rng.choice(grid, (6, 18, 32)) * rng.choice([-1, 1], (6, 18, 32))
    vals[:, :, 0] = 448.0                                    # fixes each block's exponent at 8
    vals = (vals * np.ldexp(1.0, ex)[..., None]).reshape(6, 576)
    codes, scales = wl.mxfp8_encode(vals)
    assert np.array_equal(oracle.mxfp8_decode(codes, scales), vals)
    v = rng.standard_normal((4, 576)) * 3
    codes, scales = wl.mxfp8_encode(v)
    dec = oracle.mxfp8_decode(codes, scales)
    s = np.ldexp(1.0, scales.astype(int) - 127).repeat(32, axis=1)
    allv = np.concatenate([-grid[::-1], grid])
    nearest = np.abs((v / s)[..., None] - allv).min(axis=-1) * s
    np.testing.assert_allclose(np.abs(dec - v), nearest, rtol=0, atol=1e-12)


def test_mxfp8_entries_attend_like_bf16_rows():
    """MXFP8 entries holding bf16-exact values attend exactly like those
    values stored as bf16 (CSA over a selection with the window, and HCA)."""
    rng = np.random.default_rng(23)
    B, H, N, W, k = 2, 3, 40, 5, 7
    q = wl.bf16_bits(rng.standard_normal((B, H, 576)).astype(np.float32) / 24)
    grid = np.array([oracle.e4m3_value(c) for c in range(0, 127, 3)])
    vals = rng.choice(grid, (N, 576)) * rng.choice([-1, 1], (N, 576))
    vals[:, ::32] = 448.0                 # each block's maximum: its scale is 2^0 (then x 2^-6)
    vals *= 2.0 ** -6
    ent = wl.bf16_bits(vals.astype(np.float32))
    assert np.array_equal(oracle.decode(ent, BF16), vals)
    codes, scales = wl.mxfp8_encode(vals)
    assert np.array_equal(oracle.mxfp8_decode(codes, scales), vals)
    win = wl.bf16_bits(rng.standard_normal((W, 576)).astype(np.float32))
    idx = np.sort(rng.choice(N, (B, k)), axis=1).astype(np.int32)
    o1, l1 = oracle.csa_attend(q, ent, win, BF16, idx)
    o2, l2 = oracle.csa_attend_mxfp8(q, codes, scales, win, idx)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    h1, hl1 = oracle.hca_attend(q, ent, BF16)
    h2, hl2 = oracle.hca_attend_mxfp8(q, codes, scales)
    assert np.array_equal(h1, h2) and np.array_equal(hl1, hl2)
