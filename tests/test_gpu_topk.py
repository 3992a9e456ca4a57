"""GPU parity of cskv_index_topk: indexer scores and top-k selection."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import dev
from tests.selection import check_selection

pytestmark = pytest.mark.gpu


def _cskv():
    import compressed_sparse_kv_overlapping_amd as cskv
    return cskv


def _run(qI, kI, dt, k, scale=1.0, q_pos=None, m=4, per_seq=False):
    cskv = _cskv()
    qp = None if q_pos is None else torch.from_numpy(np.asarray(q_pos, np.int64)).cuda()
    idx = cskv.index_topk(dev(qI), dev(kI), k, q_pos=qp, m=m, idx_scale=scale, per_seq=per_seq)
    torch.cuda.synchronize()
    s, v = oracle.index_scores(qI, kI, dt, scale, q_pos=q_pos, m=m, per_seq=per_seq)
    return idx.cpu().numpy(), s, v


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
@pytest.mark.parametrize("B,N,k", [(1, 1024, 64), (8, 16384, 1024), (3, 5000, 100), (40, 3001, 17),
                                   (2, 70000, 7), (5, 777, 1), (1, 4096, 4096)])
def test_topk_matches_oracle(dt, B, N, k):
    rng_cfg = 91
    qI = wl.encode(wl.normal(rng_cfg, N, 1, (B, 64)), dt).raw
    kI = wl.encode(wl.normal(rng_cfg, N, 2, (N, 64)), dt).raw
    idx, s, v = _run(qI, kI, dt, k)
    exact = check_selection(idx, s, v, k)
    assert exact >= B - 1          # near-ties inside the band are rare for random scores


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16, wl.DT_E4M3])
def test_topk_many_queries(dt):
    """1,536 queries: the score passes give each wave its own query set and
    share the entry tiles; a causal mask leaves some tiles partly visible."""
    rng_cfg = 94
    B, N, k, m = 1536, 6000, 256, 4
    q = wl.normal(rng_cfg, 0, 1, (B, 64))
    kk = wl.normal(rng_cfg, 0, 2, (N, 64))
    pos = np.random.default_rng(3).integers(0, N * m, B)
    pos[:4] = [0, 3, 4, N * m - 1]
    if dt == wl.DT_E4M3:
        sq, sk = wl.e4m3_scale(q), wl.e4m3_scale(kk)
        qI, kI, scale = wl.e4m3_encode(q, sq), wl.e4m3_encode(kk, sk), sq * sk
    else:
        qI, kI, scale = wl.encode(q, dt).raw, wl.encode(kk, dt).raw, 0.37
    idx, s, v = _run(qI, kI, dt, k, scale=scale, q_pos=pos, m=m)
    check_selection(idx, s, v, k)
    idx, s, v = _run(qI, kI, dt, k, scale=scale)
    check_selection(idx, s, v, k)


def test_topk_workload_sizes():
    """The decode selections of the workloads: top-64 of 1,024 (fp32),
    top-1024 of 16,384 (bf16, 8 queries) and of 262,144 (bf16, 32 queries)."""
    for name in ("tiny", "csa_decode"):
        inp = wl.make_inputs(name, seed=0)
        cfg = wl.CONFIGS[name]
        idx, s, v = _run(inp["qI"].raw, inp["kI"].raw, cfg.idx_dt, cfg.k)
        check_selection(idx, s, v, cfg.k)
    cfg = wl.CONFIGS["layer_1m"]
    inp = wl.make_inputs(cfg, seed=0, with_compress_source=False)
    idx, s, v = _run(inp["qI"].raw, inp["kI"].raw, wl.DT_BF16, cfg.k)
    check_selection(idx, s, v, cfg.k)


def test_topk_exact_ties_resolve_by_index():
    """Small-integer inputs: exact scores with many ties; the order (score
    descending, index ascending) makes the set unique."""
    rng = np.random.default_rng(5)
    B, N, k = 4, 20000, 300
    qI = rng.integers(-2, 3, (B, 64)).astype(np.float32)
    kI = rng.integers(-2, 3, (N, 64)).astype(np.float32)
    for dt in (wl.DT_F32, wl.DT_BF16):
        idx, s, v = _run(wl.encode(qI, dt).raw, wl.encode(kI, dt).raw, dt, k)
        ref = oracle.topk(s, v, k)
        np.testing.assert_array_equal(idx, np.sort(ref, axis=1))


def test_topk_crowded_bin_in_list():
    """Three score values only: every entry of the top score is a candidate
    (about 6k, within the list's capacity), and the k-th one sits in a bin far
    too crowded to rank member by member, so the select narrows it by further
    passes and the index word."""
    rng = np.random.default_rng(8)
    B, N, k = 2, 20000, 1000
    qI = np.zeros((B, 64), np.float32)
    qI[:, 0] = 1.0
    kI = np.zeros((N, 64), np.float32)
    kI[:, 0] = rng.choice([0.0, 1.0, 2.0], size=N, p=[0.4, 0.3, 0.3])
    for dt in (wl.DT_F32, wl.DT_BF16):
        idx, s, v = _run(wl.encode(qI, dt).raw, wl.encode(kI, dt).raw, dt, k)
        ref = oracle.topk(s, v, k)
        np.testing.assert_array_equal(idx, np.sort(ref, axis=1))


def test_topk_all_equal_scores_takes_lowest_indices():
    """Every score equal: the candidate list overflows and the streaming path
    must return entries 0..k-1."""
    B, N, k = 3, 30000, 50
    qI = np.zeros((B, 64), np.float32)
    kI = np.random.default_rng(6).standard_normal((N, 64)).astype(np.float32)
    idx, _, _ = _run(wl.bf16_bits(qI), wl.bf16_bits(kI), wl.DT_BF16, k)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (B, 1)))


def test_topk_fewer_entries_than_k():
    qI = np.ones((2, 64), np.float32)
    kI = np.random.default_rng(7).standard_normal((10, 64)).astype(np.float32)
    idx, _, _ = _run(qI, kI, wl.DT_F32, 16)
    np.testing.assert_array_equal(idx[:, :10], np.tile(np.arange(10), (2, 1)))
    assert (idx[:, 10:] == -1).all()


def test_topk_per_sequence_keys():
    rng_cfg = 92
    B, N, k = 6, 9000, 256
    qI = wl.bf16_bits(wl.normal(rng_cfg, 0, 1, (B, 64)))
    kI = wl.bf16_bits(wl.normal(rng_cfg, 0, 2, (B, N, 64)))
    idx, s, v = _run(qI, kI, wl.DT_BF16, k, per_seq=True)
    check_selection(idx, s, v, k)


def test_topk_prefill_fp8_causal():
    """fp8 e4m3 indexer with per-tensor scales and a causal mask: queries at
    the end of a context whose visible entry count varies per query."""
    rng_cfg = 93
    B, N, k, m = 64, 40000, 1024, 4
    q = wl.normal(rng_cfg, 0, 1, (B, 64))
    kk = wl.normal(rng_cfg, 0, 2, (N, 64))
    sq, sk = wl.e4m3_scale(q), wl.e4m3_scale(kk)
    qI, kI = wl.e4m3_encode(q, sq), wl.e4m3_encode(kk, sk)
    pos = np.concatenate([[0, 3, 4, 100, 4099], np.arange(N * m - B + 5, N * m)])[:B]
    idx, s, v = _run(qI, kI, wl.DT_E4M3, k, scale=sq * sk, q_pos=pos, m=m)
    check_selection(idx, s, v, k)


def test_topk_prefill_workload_sampled():
    """The 4,096-query fp8 prefill chunk over 262,144 entries, checked on a
    sample of queries (first, last and evenly spaced positions)."""
    cfg = wl.CONFIGS["csa_prefill"]
    inp = wl.make_inputs(cfg, seed=0)
    qI, kI = inp["qI"], inp["kI"]
    scale = qI.scale * kI.scale
    cskv = _cskv()
    qp = torch.from_numpy(inp["q_pos"]).cuda()
    idx = cskv.index_topk(dev(qI), dev(kI), cfg.k, q_pos=qp, m=4, idx_scale=scale).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, cfg.B - 1], np.linspace(0, cfg.B - 1, 64).round().astype(int)]))
    s, v = oracle.index_scores(qI.raw[rows], kI.raw, wl.DT_E4M3, scale, q_pos=inp["q_pos"][rows], m=4)
    check_selection(idx[rows], s, v, cfg.k)


# ------------------------------------------------------------------ MXFP4

def _run_mx(qc, qs, kc, ks, k, scale=1.0, q_pos=None, m=4, per_seq=False):
    cskv = _cskv()
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qp = None if q_pos is None else up(np.asarray(q_pos, np.int64))
    idx = cskv.index_topk_mxfp4(up(qc), up(qs), up(kc), up(ks), k, q_pos=qp, m=m, idx_scale=scale,
                                per_seq=per_seq)
    torch.cuda.synchronize()
    s, v = oracle.index_scores_mxfp4(qc, qs, kc, ks, scale, q_pos=q_pos, m=m, per_seq=per_seq)
    return idx.cpu().numpy(), s, v


def _exact(idx, s, v, k):
    """MXFP4 scores are exact in fp32 here (few significant bits, a narrow
    scale range, a power-of-two idx_scale): the selection must be the
    oracle's, ties broken by index."""
    check_selection(idx, s, v, k)
    ref = oracle.topk(s, v, k)
    for b in range(idx.shape[0]):
        want = np.sort(ref[b][ref[b] >= 0])
        np.testing.assert_array_equal(idx[b, :len(want)], want)


@pytest.mark.parametrize("B,N,k", [(1, 1024, 64), (32, 16384, 1024), (3, 5000, 100), (40, 3001, 17),
                                   (5, 777, 1), (2, 100, 128)])
def test_topk_mxfp4_matches_oracle(B, N, k):
    qc, qs = wl.mxfp4_encode(wl.normal(95, N, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(95, N, 2, (N, 64)))
    idx, s, v = _run_mx(qc, qs, kc, ks, k, scale=0.5)
    _exact(idx, s, v, k)


def test_topk_mxfp4_many_queries_causal():
    """1,536 queries (key tiles staged through LDS, shared by four query
    sets) with a causal mask, and a non-power-of-two idx_scale."""
    B, N, k, m = 1536, 6000, 256, 4
    qc, qs = wl.mxfp4_encode(wl.normal(96, 0, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(96, 0, 2, (N, 64)))
    pos = np.random.default_rng(4).integers(0, N * m, B)
    pos[:4] = [0, 3, 4, N * m - 1]
    idx, s, v = _run_mx(qc, qs, kc, ks, k, scale=1.0, q_pos=pos, m=m)
    _exact(idx, s, v, k)
    idx, s, v = _run_mx(qc, qs, kc, ks, k, scale=0.37)
    check_selection(idx, s, v, k)


def test_topk_mxfp4_per_sequence_keys():
    B, N, k = 6, 9000, 256
    qc, qs = wl.mxfp4_encode(wl.normal(97, 0, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(97, 0, 2, (B, N, 64)))
    idx, s, v = _run_mx(qc, qs, kc, ks, k, per_seq=True)
    _exact(idx, s, v, k)


def test_topk_mxfp4_all_equal_scores_take_lowest_indices():
    """Identical keys: every score ties, the candidate list overflows and the
    streaming path (scores recomputed from the codes) must keep 0..k-1."""
    B, N, k = 3, 30000, 50
    qc, qs = wl.mxfp4_encode(wl.normal(98, 0, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(np.tile(wl.normal(98, 0, 2, (1, 64)), (N, 1)))
    idx, s, v = _run_mx(qc, qs, kc, ks, k)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (B, 1)))
    assert (s == s[:, :1]).all()


def test_topk_mxfp4_scale_bytes_across_the_range():
    """Row scales from 2^-125 to 2^73 (one per row, so each score is exact),
    and rows at byte 0 (2^-127) holding elements of magnitude >= 2, which
    decode to fp32 normals; with query scales of 2^103 those rows score
    well inside fp32 and must rank exactly."""
    rng = np.random.default_rng(8)
    B, N, k = 4, 4000, 300
    kc = rng.integers(0, 256, (N, 32), dtype=np.uint8)
    ks = np.repeat(rng.integers(2, 201, (N, 1)), 2, axis=1).astype(np.uint8)
    big = np.array([4, 5, 6, 7, 12, 13, 14, 15], np.uint8)     # |E2M1| >= 2
    c = rng.choice(big, (50, 64))
    kc[:50] = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    ks[:50] = 0
    qc = rng.integers(0, 256, (B, 32), dtype=np.uint8)
    qs = np.full((B, 2), 127, np.uint8)
    idx, s, v = _run_mx(qc, qs, kc, ks, k)
    _exact(idx, s, v, k)
    qs[:] = 230
    idx, s, v = _run_mx(qc, qs, kc[:50].copy(), ks[:50].copy(), 20)
    _exact(idx, s, v, 20)


def test_topk_mxfp4_decode_workload():
    """The 1M-token decode shape: 32 queries over 262,144 entries, top-1024,
    with the bf16 workload's draws quantised to MXFP4; every query checked."""
    cfg = wl.CONFIGS["layer_1m"]
    qc, qs = wl.mxfp4_encode(wl.normal(cfg.config_id, 0, 8, (cfg.B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(cfg.config_id, 0, 9, (cfg.N_csa, 64)))
    idx, s, v = _run_mx(qc, qs, kc, ks, cfg.k)
    _exact(idx, s, v, cfg.k)


def test_topk_maximum_sizes():
    """The largest selection the kernels take: k = 4096 over 1,048,576
    entries (16,384 groups of 64), bf16 and MXFP4 keys."""
    B, N, k = 2, 1 << 20, 4096
    q = wl.normal(102, 0, 1, (B, 64))
    kk = wl.normal(102, 0, 2, (N, 64))
    idx, s, v = _run(wl.bf16_bits(q), wl.bf16_bits(kk), wl.DT_BF16, k)
    check_selection(idx, s, v, k)
    qc, qs = wl.mxfp4_encode(q)
    kc, ks = wl.mxfp4_encode(kk)
    idx, s, v = _run_mx(qc, qs, kc, ks, k)
    _exact(idx, s, v, k)


def test_topk_per_sequence_keys_read_once_or_twice():
    """Per-query keys with and without room to keep the scores between the
    passes (each key read once, or twice): the same selection, the
    oracle's, including causal queries that see part of their keys."""
    cskv = _cskv()
    B, N, k, m = 5, 20000, 300, 4
    q = wl.normal(103, 0, 1, (B, 64))
    kk = wl.normal(103, 0, 2, (B, N, 64))
    qI, kI = dev(wl.bf16_bits(q)), dev(wl.bf16_bits(kk))
    pos = np.array([0, 1500, 40000, 79999, 123456], np.int64)
    qp = torch.from_numpy(pos).cuda()
    small = torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda")
    big = torch.empty(cskv.index_topk_workspace_size(B, N, k, per_seq=True), dtype=torch.uint8,
                      device="cuda")
    assert big.numel() > small.numel()
    a = cskv.index_topk(qI, kI, k, q_pos=qp, m=m, per_seq=True, workspace=small).cpu().numpy()
    b = cskv.index_topk(qI, kI, k, q_pos=qp, m=m, per_seq=True, workspace=big).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    s, v = oracle.index_scores(wl.bf16_bits(q), wl.bf16_bits(kk), wl.DT_BF16, q_pos=pos, m=m,
                               per_seq=True)
    check_selection(b, s, v, k)


# ------------------------------------- many queries on 32x32 tiles (GS >= 32)

def _sample_rows(B, n=96):
    return np.unique(np.concatenate([[0, 1, B - 1], np.linspace(0, B - 1, n).round().astype(int)]))


@pytest.mark.parametrize("dt", [wl.DT_BF16, wl.DT_E4M3])
def test_topk_many_queries_groups_of_32_and_more(dt):
    """1,100 causal queries over 70,000 keys, top-512: the many-query score
    passes on 32x32 MFMA tiles (groups of 32 entries), with queries whose
    visible prefix ends inside a tile, at the first entry and past the end."""
    B, N, k, m = 1100, 70000, 512, 4
    q = wl.normal(105, 0, 1, (B, 64))
    kk = wl.normal(105, 0, 2, (N, 64))
    pos = np.random.default_rng(5).integers(0, N * m, B)
    pos[:6] = [0, 3, 4, 2047, N * m - 1, N * m + 77]
    if dt == wl.DT_E4M3:
        sq, sk = wl.e4m3_scale(q), wl.e4m3_scale(kk)
        qI, kI, scale = wl.e4m3_encode(q, sq), wl.e4m3_encode(kk, sk), sq * sk
    else:
        qI, kI, scale = wl.bf16_bits(q), wl.bf16_bits(kk), 0.37
    rows = _sample_rows(B)
    for qp in (pos, None):
        cskv = _cskv()
        qpt = None if qp is None else torch.from_numpy(qp).cuda()
        idx = cskv.index_topk(dev(qI), dev(kI), k, q_pos=qpt, m=m, idx_scale=scale).cpu().numpy()
        s, v = oracle.index_scores(qI[rows], kI, dt, scale, q_pos=None if qp is None else qp[rows], m=m)
        check_selection(idx[rows], s, v, k)


def test_topk_many_queries_exact_ties():
    """Small-integer keys and queries (exact scores, many ties) for 1,024
    queries over 40,000 keys: the 32x32-tile passes must give the oracle's
    set exactly, ties resolved by index."""
    rng = np.random.default_rng(6)
    B, N, k = 1024, 40000, 300
    qI = rng.integers(-2, 3, (B, 64)).astype(np.float32)
    kI = rng.integers(-2, 3, (N, 64)).astype(np.float32)
    for dt in (wl.DT_BF16, wl.DT_E4M3):
        qe = wl.bf16_bits(qI) if dt == wl.DT_BF16 else wl.e4m3_encode(qI, 1.0)
        ke = wl.bf16_bits(kI) if dt == wl.DT_BF16 else wl.e4m3_encode(kI, 1.0)
        idx = _cskv().index_topk(dev(qe), dev(ke), k).cpu().numpy()
        rows = _sample_rows(B, 64)
        s, v = oracle.index_scores(qe[rows], ke, dt)
        ref = oracle.topk(s, v, k)
        np.testing.assert_array_equal(idx[rows], np.sort(ref, axis=1))


def test_topk_mxfp4_many_queries_groups_of_32():
    """MXFP4 queries and keys (per-block scales) for 1,100 causal queries over
    70,000 keys: the scaled 32x32x64 MFMA path, exact against the oracle."""
    B, N, k, m = 1100, 70000, 512, 4
    qc, qs = wl.mxfp4_encode(wl.normal(106, 0, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(106, 0, 2, (N, 64)))
    pos = np.random.default_rng(7).integers(0, N * m, B)
    pos[:4] = [0, 5, N * m - 1, 2047]
    cskv = _cskv()
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx = cskv.index_topk_mxfp4(up(qc), up(qs), up(kc), up(ks), k, q_pos=up(pos), m=m,
                                idx_scale=0.5).cpu().numpy()
    rows = _sample_rows(B)
    s, v = oracle.index_scores_mxfp4(qc[rows], qs[rows], kc, ks, 0.5, q_pos=pos[rows], m=m)
    _exact(idx[rows], s, v, k)


@pytest.mark.parametrize("dt", [wl.DT_BF16, wl.DT_E4M3, wl.DT_F32])
@pytest.mark.parametrize("B,N,k", [(32, 1 << 18, 1024), (20, 100003, 333), (7, 30000, 64), (7, 300000, 512)])
def test_topk_decode_one_launch_equals_four(dt, B, N, k):
    """Up to 32 queries over shared keys with every entry visible run the
    selection in one launch (its blocks waiting for each other between phases);
    positions that make every entry visible take the four launches instead.
    Both compute the same scores in the same order, so the selections are
    identical, and the one-launch result matches the oracle."""
    rng_cfg = 105
    q = wl.normal(rng_cfg, N, 1, (B, 64))
    kk = wl.normal(rng_cfg, N, 2, (N, 64))
    if dt == wl.DT_E4M3:
        sq, sk = wl.e4m3_scale(q), wl.e4m3_scale(kk)
        qI, kI, scale = wl.e4m3_encode(q, sq), wl.e4m3_encode(kk, sk), sq * sk
    else:
        qI, kI, scale = wl.encode(q, dt).raw, wl.encode(kk, dt).raw, 0.61
    idx1, s, v = _run(qI, kI, dt, k, scale=scale)
    check_selection(idx1, s, v, k)
    idx4, _, _ = _run(qI, kI, dt, k, scale=scale, q_pos=np.full(B, 4 * N - 1), m=4)
    np.testing.assert_array_equal(idx1, idx4)


def test_topk_mxfp4_decode_one_launch_equals_four():
    """The same for MXFP4 keys at the 1M-token decode shape."""
    B, N, k = 32, 1 << 18, 1024
    qc, qs = wl.mxfp4_encode(wl.normal(106, 0, 1, (B, 64)))
    kc, ks = wl.mxfp4_encode(wl.normal(106, 0, 2, (N, 64)))
    idx1, s, v = _run_mx(qc, qs, kc, ks, k)
    _exact(idx1, s, v, k)
    idx4, _, _ = _run_mx(qc, qs, kc, ks, k, q_pos=np.full(B, 4 * N - 1), m=4)
    np.testing.assert_array_equal(idx1, idx4)


def test_topk_decode_in_a_replayed_graph():
    """The one-launch decode selection (a reset kernel, then the selection
    kernel) captured in a HIP graph with the workspace and allocation-free
    entry points: every replay, with new queries copied in and the outputs
    cleared in between and eager calls between the replays, equals the eager
    result."""
    cskv = _cskv()
    B, N, k = 20, 100003, 333
    kk = torch.from_numpy(wl.bf16_bits(wl.normal(107, 0, 2, (N, 64))).view(np.int16)).cuda()
    keys = kk.view(torch.bfloat16)
    q = torch.empty(B, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, k, dtype=torch.int32, device="cuda")
    out_na = torch.empty(B, k, dtype=torch.int32, device="cuda")
    ref = torch.empty(B, k, dtype=torch.int32, device="cuda")
    ws = torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)

    def draw(i):
        return torch.from_numpy(wl.bf16_bits(wl.normal(107, i, 1, (B, 64))).view(np.int16)).cuda().view(torch.bfloat16)

    q.copy_(draw(0))
    cskv.index_topk(q, keys, k, idx_out=out, workspace=ws)          # warm up outside the capture
    cskv.index_topk_noalloc(q, keys, k, idx_out=out_na)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cskv.index_topk(q, keys, k, idx_out=out, workspace=ws)
        cskv.index_topk_noalloc(q, keys, k, idx_out=out_na)
    for i in range(1, 5):
        q.copy_(draw(i))
        out.fill_(-7)
        out_na.fill_(-7)
        g.replay()
        cskv.index_topk(q, keys, k, idx_out=ref, workspace=ws_e)       # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert torch.equal(out_na, ref), f"replay {i} (allocation-free)"


def test_topk_decode_on_two_streams_at_once():
    """Decode selections issued on two streams at once (each with its own
    workspace) equal the same selections run one at a time.  Two one-launch
    selection kernels must never run together (each could hold part of the
    chip while it waits for blocks of its own), so once calls come on a
    second stream every later decode selection takes the multi-launch path."""
    cskv = _cskv()
    B, N, k = 32, 1 << 18, 1024
    keys = torch.from_numpy(wl.bf16_bits(wl.normal(108, 0, 2, (N, 64))).view(np.int16)).cuda().view(torch.bfloat16)
    qs = [torch.from_numpy(wl.bf16_bits(wl.normal(108, i, 1, (B, 64))).view(np.int16)).cuda().view(torch.bfloat16)
          for i in (1, 2)]
    wss = [torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda") for _ in qs]
    refs = [cskv.index_topk(q, keys, k) for q in qs]
    outs = [torch.empty(B, k, dtype=torch.int32, device="cuda") for _ in qs]
    streams = [torch.cuda.Stream() for _ in qs]
    torch.cuda.synchronize()
    for it in range(8):
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        for q, ws, o, st in zip(qs, wss, outs, streams):
            cskv.index_topk(q, keys, k, idx_out=o, workspace=ws, stream=st)
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"iteration {it}"
