"""GPU parity of the attention entry points (HCA, sparse attention over a
given selection, fused CSA, merge) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import TOL, dev, host_f64, rowwise_err
from tests.selection import check_selection

pytestmark = pytest.mark.gpu
E = 576


def _cskv():
    import compressed_sparse_kv_overlapping_amd as cskv
    return cskv


def _rand(cfg_id, seed, tid, shape, dt, std=1.0):
    return wl.encode(wl.normal(cfg_id, seed, tid, shape, std), dt).raw


def _check_attn(out, lse, ref_out, ref_lse, dt):
    assert rowwise_err(host_f64(out), ref_out) <= TOL[dt]
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4 if dt == wl.DT_F32 else 2e-3,
                               atol=1e-4 if dt == wl.DT_F32 else 2e-3)


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
@pytest.mark.parametrize("B,H,N", [(1, 16, 32), (2, 128, 1000), (3, 48, 33), (1, 16, 1), (4, 130, 300)])
def test_hca_matches_oracle(dt, B, H, N):
    q = _rand(94, N, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(94, N, 2, (N, E), dt)
    out, lse = _cskv().hca_attend(dev(q), dev(ent))
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt)
    _check_attn(out, lse, ro, rl, dt)


def test_hca_decode_workload():
    """16 queries x 128 heads over 8,192 bf16 entries (the HCA decode
    workload at its full size and launch configuration); every query checked."""
    cfg = wl.CONFIGS["hca_decode"]
    inp = wl.make_inputs(cfg, seed=0)
    out, lse = _cskv().hca_attend(dev(inp["q_hca"]), dev(inp["entries_hca"]))
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(inp["q_hca"].raw, inp["entries_hca"].raw, wl.DT_BF16)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_hca_per_sequence_caches():
    B, H, N, dt = 3, 64, 700, wl.DT_BF16
    q = _rand(95, 0, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(95, 0, 2, (B, N, E), dt)
    out, lse = _cskv().hca_attend(dev(q), dev(ent), per_seq=True)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, per_seq=True)
    _check_attn(out, lse, ro, rl, dt)


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
def test_hca_prefill_matches_oracle(dt):
    """HCA at a prefill chunk: the query at position pos attends over entries
    i with (i+1)m <= pos+1; positions from none visible through one, part
    and all to past the end."""
    B, H, N, m = 7, 128 if dt == wl.DT_BF16 else 16, 300, 128
    pos = np.array([0, 126, 127, 37 * m + 5, 150 * m - 1, N * m - 1, 10**7], dtype=np.int64)
    q = _rand(99, 0, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(99, 0, 2, (N, E), dt)
    out, lse = _cskv().hca_attend(dev(q), dev(ent), q_pos=torch.from_numpy(pos).cuda(), m=m)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, q_pos=pos, m=m)
    assert np.isneginf(rl[:2]).all() and (host_f64(out)[:2] == 0).all()
    assert np.isneginf(lse[:2].cpu().numpy()).all()
    _check_attn(out[2:], lse[2:], ro[2:], rl[2:], dt)


def test_hca_prefill_chunk_sampled():
    """4,096 queries at positions 1,044,480..1,048,575 over 8,192 m'=128
    entries (8,160..8,192 visible); the first and last query checked."""
    cfg = wl.CONFIGS["hca_prefill"]
    inp = wl.make_inputs(cfg, seed=0)
    qp = torch.from_numpy(inp["q_pos"]).cuda()
    out, lse = _cskv().hca_attend(dev(inp["q_hca"]), dev(inp["entries_hca"]), q_pos=qp, m=cfg.m_hca)
    torch.cuda.synchronize()
    rows = [0, cfg.B - 1]
    ro, rl = oracle.hca_attend(inp["q_hca"].raw[rows], inp["entries_hca"].raw, wl.DT_BF16,
                               q_pos=inp["q_pos"][rows], m=cfg.m_hca)
    _check_attn(out[rows], lse[rows], ro, rl, wl.DT_BF16)


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
def test_sparse_attend_given_selection(dt):
    """Attention over a given index list (with -1 holes, unsorted) plus the window."""
    B, H, N, W, k = 3, 128 if dt == wl.DT_BF16 else 16, 5000, 128, 200
    q = _rand(96, 0, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(96, 0, 2, (N, E), dt)
    win = _rand(96, 0, 3, (W, E), dt)
    rng = np.random.default_rng(0)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[0, 5:40] = -1
    idx[2, :] = -1
    out, lse = _cskv().sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(q, ent, win, dt, idx)
    _check_attn(out, lse, ro, rl, dt)


def test_sparse_attend_special_cases():
    cskv = _cskv()
    dt = wl.DT_BF16
    B, H, N, W, k = 2, 64, 300, 128, 1024
    ent = _rand(97, 0, 2, (N, E), dt)
    win = _rand(97, 0, 3, (W, E), dt)
    idx = np.full((B, k), -1, np.int32)
    idx[:, :N] = np.arange(N)                                   # k >= N: all entries
    q = np.zeros((B, H, E), np.uint16)                          # q = 0: uniform weights
    out, lse = cskv.sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rows = np.concatenate([oracle.decode(ent, dt), oracle.decode(win, dt)])
    assert rowwise_err(host_f64(out)[0], np.tile(rows[:, :512].mean(0), (H, 1))) <= 2e-2
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(N + W), rtol=1e-5)
    # no rows at all: zero output, lse = -inf
    q2 = _rand(97, 0, 1, (B, H, E), dt, 1 / 24)
    none = np.full((B, 4), -1, np.int32)
    out, lse = cskv.sparse_attend(dev(q2), dev(ent), dev(win), torch.from_numpy(none).cuda(), W=0)
    torch.cuda.synchronize()
    assert (host_f64(out) == 0).all() and np.isneginf(lse.cpu().numpy()).all()
    out, lse = cskv.hca_attend(dev(q2), dev(ent), scale=0.0)       # scale 0: uniform weights
    torch.cuda.synchronize()
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(N), rtol=1e-5)


@pytest.mark.parametrize("N", [300, 8192])
def test_logits_past_reference_band(N):
    """Rows of tile 0 have small logits, and one row in every later tile a
    logit about 200 log2-units higher: past the 64-unit band that a split
    accumulates against after its first tile, so the split holding tile 0
    (two or more tiles here) redoes its rows exactly, while later splits set
    their reference from a large logit.  HCA and sparse attention must still
    match the oracle."""
    dt, B, H = wl.DT_BF16, 2, 128
    rng = np.random.default_rng(N)
    qf = 0.5 + 0.01 * rng.standard_normal((B, H, E))
    ef = 0.1 * rng.standard_normal((N, E))
    big = np.arange(32 + 5, N, 32)
    ef[big] = 0.5 + 0.01 * rng.standard_normal((len(big), E))
    q, ent = wl.encode(qf, dt).raw, wl.encode(ef, dt).raw
    out, lse = _cskv().hca_attend(dev(q), dev(ent))
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt)
    _check_attn(out, lse, ro, rl, dt)
    # the same rows as a selection (entries in index order), plus a window
    # of small rows
    W = 128
    win = wl.encode(0.1 * rng.standard_normal((W, E)), dt).raw
    k = min(N, 1024)
    idx = np.tile(np.arange(k, dtype=np.int32), (B, 1))
    out, lse = _cskv().sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(q, ent, win, dt, idx)
    _check_attn(out, lse, ro, rl, dt)


@pytest.mark.parametrize("norm", [False, True])
def test_logits_past_reference_band_in_some_heads(norm):
    """Only the odd heads of each wave have logits past the band a split
    accumulates against (rows of the later tiles along their queries); head
    0 of every wave stays inside it.  The redo must be triggered by any
    head's excess, not by head 0's alone; HCA and sparse attention must match
    the oracle, with and without the query / entry normalisation."""
    dt, B, H, N = wl.DT_BF16, 2, 128, 600
    rng = np.random.default_rng(17)
    qf = 0.05 * rng.standard_normal((B, H, E))
    qf[:, 1::2] = 0.5 + 0.01 * rng.standard_normal((B, H // 2, E))
    ef = 0.1 * rng.standard_normal((N, E))
    big = np.arange(32 + 5, N, 32)
    ef[big] = 0.5 + 0.01 * rng.standard_normal((len(big), E))
    q, ent = wl.encode(qf, dt).raw, wl.encode(ef, dt).raw
    eps = 1e-6 if norm else None
    scale = 0.3 if norm else 1.0
    out, lse = _cskv().hca_attend(dev(q), dev(ent), scale=scale, norm_eps=eps)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, scale=scale, norm_eps=eps)
    _check_attn(out, lse, ro, rl, dt)
    W = 128
    win = wl.encode(0.1 * rng.standard_normal((W, E)), dt).raw
    idx = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    idx[1, 40:100] = -1
    out, lse = _cskv().sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda(),
                                     scale=scale, norm_eps=eps)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(q, ent, win, dt, idx, scale=scale, norm_eps=eps)
    _check_attn(out, lse, ro, rl, dt)


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
def test_attention_sink(dt):
    """Per-head attention-sink logits: split paths (the merge adds the sink)
    and single-split paths (the attention kernel adds it), HCA decode and
    prefill, sparse attention, and a query with no rows (output 0, lse =
    sink)."""
    cskv = _cskv()
    H = 128 if dt == wl.DT_BF16 else 16
    rng = np.random.default_rng(5)
    sink_h = rng.uniform(-2.0, 4.0, H)
    sink = torch.from_numpy(sink_h.astype(np.float32)).cuda()
    # HCA decode, several splits
    B, N = 3, 1000
    q = _rand(101, 0, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(101, 0, 2, (N, E), dt)
    out, lse = cskv.hca_attend(dev(q), dev(ent), sink=sink)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, sink=sink_h)
    _check_attn(out, lse, ro, rl, dt)
    # one split per query (300 queries), at prefill positions
    B2, N2, m = 300, 96, 128
    q2 = _rand(101, 0, 3, (B2, H, E), dt, 1 / 24)
    ent2 = _rand(101, 0, 4, (N2, E), dt)
    pos = (np.arange(B2, dtype=np.int64) * 41) % (N2 * m + 200)
    out, lse = cskv.hca_attend(dev(q2), dev(ent2), q_pos=torch.from_numpy(pos).cuda(), m=m,
                               sink=sink)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q2, ent2, dt, q_pos=pos, m=m, sink=sink_h)
    _check_attn(out, lse, ro, rl, dt)
    none = np.nonzero((pos + 1) // m == 0)[0]
    assert len(none) > 0
    assert (host_f64(out)[none] == 0).all()
    np.testing.assert_allclose(lse.cpu().numpy()[none], np.tile(sink_h, (len(none), 1)), rtol=1e-6)
    # sparse attention over a selection plus the window; query 2 has no rows
    Bs, Ns, W, k = 3, 5000, 128, 200
    qs = _rand(101, 0, 5, (Bs, H, E), dt, 1 / 24)
    ents = _rand(101, 0, 6, (Ns, E), dt)
    win = _rand(101, 0, 7, (W, E), dt)
    idx = np.stack([rng.choice(Ns, k, replace=False) for _ in range(Bs)]).astype(np.int32)
    idx[1, 10:50] = -1
    out, lse = cskv.sparse_attend(dev(qs), dev(ents), dev(win), torch.from_numpy(idx).cuda(),
                                  sink=sink)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(qs, ents, win, dt, idx, sink=sink_h)
    _check_attn(out, lse, ro, rl, dt)
    idx0 = np.full((Bs, 4), -1, np.int32)
    out, lse = cskv.sparse_attend(dev(qs), dev(ents), dev(win), torch.from_numpy(idx0).cuda(), W=0,
                                  sink=sink)
    torch.cuda.synchronize()
    assert (host_f64(out) == 0).all()
    np.testing.assert_allclose(lse.cpu().numpy(), np.tile(sink_h, (Bs, 1)), rtol=1e-6)


@pytest.mark.parametrize("S", [7, 12])
def test_merge_of_split_partials(S):
    """cskv_merge combines oracle partials over a row partition into the
    oracle's unsplit result (up to eight splits load every row with the lse
    values; more take the lse first)."""
    B, H, N = 2, 32, 300
    q = _rand(98, 0, 1, (B, H, E), wl.DT_F32, 1 / 24)
    ent = _rand(98, 0, 2, (N, E), wl.DT_F32)
    parts = np.array_split(np.arange(N), S - 1)
    parts.insert(3, np.arange(0))                               # plus one empty split
    po, pl = [], []
    for p in parts:
        if len(p):
            o, l = oracle.hca_attend(q, ent[p], wl.DT_F32)
        else:
            o, l = np.zeros((B, H, 512)), np.full((B, H), -np.inf)
        po.append(o)
        pl.append(l)
    o_part = torch.from_numpy(np.stack(po, 2).astype(np.float32)).cuda()      # [B, H, S, 512]
    l_part = torch.from_numpy(np.stack(pl, 2).astype(np.float32)).cuda()
    out, lse = _cskv().merge(o_part, l_part, dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, wl.DT_F32)
    assert rowwise_err(host_f64(out), ro) <= 1e-5
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-5)
    # the same partials with a per-head sink in the merge's denominator
    sink_h = np.linspace(-1.0, 3.0, H)
    out, lse = _cskv().merge(o_part, l_part, dtype=torch.float32,
                             sink=torch.from_numpy(sink_h.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, wl.DT_F32, sink=sink_h)
    assert rowwise_err(host_f64(out), ro) <= 1e-5
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-5)


@pytest.mark.parametrize("S", [3, 12])
def test_merge_of_empty_splits(S):
    """Every split empty (lse -inf, zero rows): the output is 0 and the lse
    -inf, or with a sink, the sink's logit."""
    B, H = 2, 8
    o_part = torch.zeros(B, H, S, 512, dtype=torch.float32, device="cuda")
    l_part = torch.full((B, H, S), -np.inf, dtype=torch.float32, device="cuda")
    out, lse = _cskv().merge(o_part, l_part, dtype=torch.float32)
    torch.cuda.synchronize()
    assert (host_f64(out) == 0).all()
    assert np.isneginf(lse.cpu().numpy()).all()
    sink_h = np.linspace(-1.0, 3.0, H)
    out, lse = _cskv().merge(o_part, l_part, dtype=torch.float32,
                             sink=torch.from_numpy(sink_h.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    assert (host_f64(out) == 0).all()
    np.testing.assert_allclose(lse.cpu().numpy(), np.tile(sink_h, (B, 1)), rtol=1e-6)


def prefill_sample(B, n=64):
    """At least n query rows of a prefill chunk: the first, the second, the
    last and evenly spaced ones between."""
    return np.unique(np.concatenate([[0, 1, B - 1], np.linspace(0, B - 1, n).round().astype(int)]))


@pytest.mark.parametrize("name", ["tiny", "csa_decode"])
def test_csa_decode_matches_oracle(name):
    """Fused CSA decode: the selection within the tie band, and for every
    query the attention equal to the oracle's over the GPU's own selection
    plus the window."""
    cfg = wl.CONFIGS[name]
    inp = wl.make_inputs(cfg, seed=0)
    cskv = _cskv()
    if cfg.T:
        ent = np.empty((cfg.N_csa, E), np.float32 if cfg.dt == wl.DT_F32 else np.uint16)
        c = oracle.compress(inp["x"].raw, inp["z"].raw, cfg.dt, inp["b4"].raw, 4)
        ent[:, :512] = c if cfg.dt == wl.DT_F32 else wl.bf16_bits(c.astype(np.float32))
        ent[:, 512:] = inp["rope4"].raw
    else:
        ent = inp["entries"].raw
    out, lse, idx = cskv.csa_attend(dev(inp["q"]), dev(inp["qI"]), dev(ent), dev(inp["kI"]),
                                    dev(inp["window"]), cfg.k)
    torch.cuda.synchronize()
    s, v = oracle.index_scores(inp["qI"].raw, inp["kI"].raw, cfg.idx_dt)
    idx = idx.cpu().numpy()
    check_selection(idx, s, v, cfg.k)
    ro, rl = oracle.csa_attend(inp["q"].raw, ent, inp["window"].raw, cfg.dt, idx)
    _check_attn(out, lse, ro, rl, cfg.dt)


def test_csa_prefill_attention_sampled():
    """Prefill attention with per-query causal windows, on the 1M-context
    chunk shapes, for 65 sampled queries (first, last and evenly spaced),
    using the oracle's own selection."""
    cfg = wl.CONFIGS["csa_prefill"]
    inp = wl.make_inputs(cfg, seed=0)
    rows = prefill_sample(cfg.B)
    qI, kI = inp["qI"], inp["kI"]
    s, v = oracle.index_scores(qI.raw[rows], kI.raw, wl.DT_E4M3, qI.scale * kI.scale,
                               q_pos=inp["q_pos"][rows], m=4)
    idx = np.sort(oracle.topk(s, v, cfg.k), axis=1)
    qp = inp["q_pos"][rows]
    out, lse = _cskv().sparse_attend(dev(inp["q"].raw[rows]), dev(inp["entries"]), dev(inp["window"]),
                                     torch.from_numpy(idx).cuda(), q_pos=torch.from_numpy(qp).cuda(),
                                     win_pos0=inp["win_pos0"], W=cfg.W)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(inp["q"].raw[rows], inp["entries"].raw, inp["window"].raw, wl.DT_BF16,
                               idx, q_pos=qp, win_pos0=inp["win_pos0"], W=cfg.W)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_csa_prefill_fused_call_sampled():
    """The fused CSA call at a prefill chunk (cskv_csa_attend with q_pos):
    4,096 causal queries at positions 1,044,480..1,048,575 over 262,144
    entries, fp8 e4m3 indexer with idx_scale = s_q * s_k, top-1024 plus each
    query's 128-row raw window, in the launch configuration of the whole
    chunk.  65 sampled queries (first, last, evenly spaced): the selection
    within the tie band, and the attention equal to the oracle's over the
    GPU's own selection."""
    cfg = wl.CONFIGS["csa_prefill"]
    inp = wl.make_inputs(cfg, seed=0)
    qI, kI = inp["qI"], inp["kI"]
    scale = qI.scale * kI.scale
    qp = torch.from_numpy(inp["q_pos"]).cuda()
    out, lse, idx = _cskv().csa_attend(dev(inp["q"]), dev(qI), dev(inp["entries"]), dev(kI),
                                       dev(inp["window"]), cfg.k, m=4, q_pos=qp,
                                       win_pos0=inp["win_pos0"], W=cfg.W, idx_scale=scale)
    torch.cuda.synchronize()
    rows = prefill_sample(cfg.B)
    assert len(rows) >= 64
    sel = idx.cpu().numpy()[rows]
    s, v = oracle.index_scores(qI.raw[rows], kI.raw, wl.DT_E4M3, scale, q_pos=inp["q_pos"][rows], m=4)
    check_selection(sel, s, v, cfg.k)
    ro, rl = oracle.csa_attend(inp["q"].raw[rows], inp["entries"].raw, inp["window"].raw, wl.DT_BF16,
                               sel, q_pos=inp["q_pos"][rows], win_pos0=inp["win_pos0"], W=cfg.W)
    t = torch.from_numpy(rows).cuda()
    _check_attn(out[t], lse[t], ro, rl, wl.DT_BF16)


def test_csa_per_sequence_decode():
    """Per-sequence caches: each query has its own entries, keys and window;
    every query's attention checked over the GPU's own selection."""
    B, H, N, W, k, dt = 4, 128, 6000, 128, 512, wl.DT_BF16
    q = _rand(99, 0, 1, (B, H, E), dt, 1 / 24)
    ent = _rand(99, 0, 2, (B, N, E), dt)
    win = _rand(99, 0, 3, (B, W, E), dt)
    qI = _rand(99, 0, 4, (B, 64), dt)
    kI = _rand(99, 0, 5, (B, N, 64), dt)
    out, lse, idx = _cskv().csa_attend(dev(q), dev(qI), dev(ent), dev(kI), dev(win), k, per_seq=True)
    torch.cuda.synchronize()
    s, v = oracle.index_scores(qI, kI, dt, per_seq=True)
    idx = idx.cpu().numpy()
    check_selection(idx, s, v, k)
    ro, rl = oracle.csa_attend(q, ent, win, dt, idx, per_seq=True)
    _check_attn(out, lse, ro, rl, dt)


def test_layer_1m_step_sampled():
    """The benchmarked step at its full size and launch configuration: both
    scales compressed from the 1M raw rows into the entry buffers, then the
    CSA indexer top-1024, CSA attention and HCA attention for 32 queries x
    128 heads; queries 0 and 31 checked, with every entry they read rebuilt
    by the oracle from the raw rows."""
    cfg = wl.CONFIGS["layer_1m"]
    inp = wl.make_inputs(cfg, seed=0)
    cskv = _cskv()
    T, B, H, k, W = cfg.T, cfg.B, cfg.H, cfg.k, cfg.W
    e4 = torch.empty((T // 4, E), dtype=torch.bfloat16, device="cuda")
    e128 = torch.empty((T // 128, E), dtype=torch.bfloat16, device="cuda")
    e4[:, 512:] = dev(inp["rope4"])
    e128[:, 512:] = dev(inp["rope128"])
    cskv.compress2(dev(inp["x"]), dev(inp["z"]), dev(inp["b4"]), 4, dev(inp["b128"]), 128,
                   out_small=e4, out_large=e128)
    idx = cskv.index_topk(dev(inp["qI"]), dev(inp["kI"]), k)
    out_c, lse_c = cskv.sparse_attend(dev(inp["q"]), e4, dev(inp["window"]), idx)
    out_h, lse_h = cskv.hca_attend(dev(inp["q_hca"]), e128)
    torch.cuda.synchronize()
    rows = [0, B - 1]
    # selection
    s, v = oracle.index_scores(inp["qI"].raw[rows], inp["kI"].raw, wl.DT_BF16)
    sel = idx.cpu().numpy()[rows]
    check_selection(sel, s, v, k)

    def entries(m, bias, rope, ids):
        c = oracle.compress(inp["x"].raw, inp["z"].raw, wl.DT_BF16, bias, m, entry_ids=ids)
        ent = np.empty((len(ids), E), np.uint16)
        ent[:, :512] = wl.bf16_bits(c.astype(np.float32))
        ent[:, 512:] = rope[ids]
        return ent

    # CSA over each checked query's own selection (entries rebuilt by the oracle)
    for r, b in enumerate(rows):
        ids = sel[r].astype(np.int64)
        ent = entries(4, inp["b4"].raw, inp["rope4"].raw, ids)
        ro, rl = oracle.csa_attend(inp["q"].raw[[b]], ent, inp["window"].raw, wl.DT_BF16,
                                   np.arange(k, dtype=np.int32)[None, :])
        _check_attn(out_c[[b]], lse_c[[b]], ro, rl, wl.DT_BF16)
    # HCA over all 8,192 large-scale entries
    ent = entries(128, inp["b128"].raw, inp["rope128"].raw, np.arange(T // 128, dtype=np.int64))
    ro, rl = oracle.hca_attend(inp["q_hca"].raw[rows], ent, wl.DT_BF16)
    _check_attn(out_h[rows], lse_h[rows], ro, rl, wl.DT_BF16)


def test_index_reuse_across_layers():
    """A later layer reuses an earlier layer's selection: the indices that
    cskv_csa_attend returns for layer 1 drive cskv_sparse_attend over layer
    2's own queries, entries and window, which must equal the oracle's
    attention over that same selection."""
    cfg = wl.CONFIGS["csa_decode"]
    l1 = wl.make_inputs(cfg, seed=0)
    l2 = wl.make_inputs(cfg, seed=1)
    cskv = _cskv()
    _, _, idx = cskv.csa_attend(dev(l1["q"]), dev(l1["qI"]), dev(l1["entries"]), dev(l1["kI"]),
                                dev(l1["window"]), cfg.k)
    out, lse = cskv.sparse_attend(dev(l2["q"]), dev(l2["entries"]), dev(l2["window"]), idx)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s, v = oracle.index_scores(l1["qI"].raw, l1["kI"].raw, cfg.idx_dt)
    check_selection(idx, s, v, cfg.k)
    ro, rl = oracle.csa_attend(l2["q"].raw, l2["entries"].raw, l2["window"].raw, cfg.dt, idx)
    _check_attn(out, lse, ro, rl, cfg.dt)


# ------------------------------------------------------- MXFP4 entries

def _mx_entries(cfg_id, seed, shape):
    """Entries drawn ~N(0,1) in fp32 and quantised to MXFP4 (codes, scales)."""
    return wl.mxfp4_encode(wl.normal(cfg_id, seed, 2, shape))


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("B,H,N,W,k", [(2, 128, 5000, 128, 1024), (3, 80, 700, 16, 37),
                                       (1, 16, 40, 0, 40), (4, 128, 300, 5, 1)])
def test_sparse_attend_mxfp4_matches_oracle(B, H, N, W, k):
    """CSA over MXFP4 entries plus bf16 window rows; some selections hold -1
    (no row)."""
    rng = np.random.default_rng(B * 1000 + k)
    q = _rand(97, N, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(97, N, (N, E))
    win = _rand(97, N, 3, (max(W, 1), E), wl.DT_BF16)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[0, -1] = -1
    out, lse = _cskv().sparse_attend_mxfp4(dev(q), _up(codes), _up(scales), dev(win), _up(idx), W=W)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp4(q, codes, scales, win, idx, W=W)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_sparse_attend_mxfp4_prefill_and_sink():
    """Prefill queries with per-query causal windows, per-sequence entries,
    and attention-sink logits."""
    rng = np.random.default_rng(3)
    B, H, N, W, k = 3, 128, 900, 128, 64
    q = _rand(98, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(98, 0, (B, N, E))
    pos0, rows = 1000, 300
    win = _rand(98, 0, 3, (B, rows, E), wl.DT_BF16)
    qp = np.array([pos0 + W - 1, pos0 + 200, pos0 + rows - 1], np.int64)   # windows inside the rows
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    sink = rng.standard_normal(H) * 2
    out, lse = _cskv().sparse_attend_mxfp4(dev(q), _up(codes), _up(scales), dev(win), _up(idx),
                                           q_pos=_up(qp), win_pos0=pos0, W=W, per_seq=True,
                                           sink=torch.from_numpy(sink).float().cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp4(q, codes, scales, win, idx, q_pos=qp, win_pos0=pos0, W=W,
                                     per_seq=True, sink=sink.astype(np.float32).astype(np.float64))
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


@pytest.mark.parametrize("B,H,N", [(2, 128, 1000), (3, 48, 33), (1, 16, 1)])
def test_hca_attend_mxfp4_matches_oracle(B, H, N):
    q = _rand(99, N, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(99, N, (N, E))
    out, lse = _cskv().hca_attend_mxfp4(dev(q), _up(codes), _up(scales))
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp4(q, codes, scales)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_hca_attend_mxfp4_prefill():
    B, H, N, m = 4, 128, 600, 128
    q = _rand(100, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(100, 0, (N, E))
    qp = np.array([0, 127, 50000, N * m + 9], np.int64)          # none, one, part, all visible
    out, lse = _cskv().hca_attend_mxfp4(dev(q), _up(codes), _up(scales), q_pos=_up(qp), m=m)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp4(q, codes, scales, q_pos=qp, m=m)
    assert np.isneginf(rl[:1]).all() and (host_f64(out)[:1] == 0).all()
    assert np.isneginf(lse[:1].cpu().numpy()).all()
    _check_attn(out[1:], lse[1:], ro[1:], rl[1:], wl.DT_BF16)


def test_attend_mxfp4_decode_workload_sampled():
    """The 1M-token decode shapes with MXFP4 entries: HCA over 8,192 entries
    and CSA over 1,024 selected of 262,144 plus 128 window rows, 32 queries x
    128 heads, checked on sampled queries."""
    cfg = wl.CONFIGS["layer_1m"]
    B, H, k, W = cfg.B, cfg.H, cfg.k, cfg.W
    rng = np.random.default_rng(11)
    q = _rand(cfg.config_id, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    c128, s128 = _mx_entries(cfg.config_id, 1, (cfg.N_hca, E))
    out, lse = _cskv().hca_attend_mxfp4(dev(q), _up(c128), _up(s128))
    c4, s4 = _mx_entries(cfg.config_id, 2, (cfg.N_csa, E))
    win = _rand(cfg.config_id, 0, 3, (W, E), wl.DT_BF16)
    idx = np.stack([np.sort(rng.choice(cfg.N_csa, k, replace=False)) for _ in range(B)]).astype(np.int32)
    o2, l2 = _cskv().sparse_attend_mxfp4(dev(q), _up(c4), _up(s4), dev(win), _up(idx))
    torch.cuda.synchronize()
    rows = np.array([0, 13, B - 1])
    sel = torch.from_numpy(rows).cuda()
    ro, rl = oracle.hca_attend_mxfp4(q[rows], c128, s128)
    _check_attn(out[sel], lse[sel], ro, rl, wl.DT_BF16)
    ro, rl = oracle.csa_attend_mxfp4(q[rows], c4, s4, win, idx[rows])
    _check_attn(o2[sel], l2[sel], ro, rl, wl.DT_BF16)


def test_attend_mxfp4_per_sequence_hca_and_window_only():
    """HCA over per-sequence MXFP4 entries with sinks, and CSA with an empty
    selection (the window rows alone)."""
    rng = np.random.default_rng(21)
    B, H, N, W = 3, 128, 500, 128
    q = _rand(101, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(101, 0, (B, N, E))
    sink = rng.standard_normal(H)
    out, lse = _cskv().hca_attend_mxfp4(dev(q), _up(codes), _up(scales), per_seq=True,
                                        sink=torch.from_numpy(sink).float().cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp4(q, codes, scales, per_seq=True,
                                     sink=sink.astype(np.float32).astype(np.float64))
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    win = _rand(101, 0, 3, (W, E), wl.DT_BF16)
    idx = np.zeros((B, 0), np.int32)
    out, lse = _cskv().sparse_attend_mxfp4(dev(q), _up(codes[0]), _up(scales[0]), dev(win), _up(idx))
    torch.cuda.synchronize()
    # the oracle takes k >= 1: one empty slot (-1) is the same window-only attention
    ro, rl = oracle.csa_attend_mxfp4(q, codes[0], scales[0], win, np.full((B, 1), -1, np.int32))
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


# ------------------------------------- query / entry normalisation (norm_eps)

def _scaled_rows(cfg_id, seed, tid, shape, dt, lo, hi):
    """~N(0,1) rows times a per-row factor in [lo, hi): the normalisation
    factors then differ widely between rows."""
    v = wl.normal(cfg_id, seed, tid, shape)
    f = np.random.default_rng(seed * 7 + tid).uniform(lo, hi, shape[:-1] + (1,))
    return wl.encode((v * f).astype(np.float32), dt).raw


@pytest.mark.parametrize("dt", [wl.DT_F32, wl.DT_BF16])
def test_normalised_attention(dt):
    """Queries and compressed entries normalised to unit RMS: sparse attention
    over a selection with -1 holes plus raw window rows (not normalised),
    with and without a sink; HCA at decode (several splits), at a prefill
    chunk and over per-sequence entries."""
    cskv = _cskv()
    eps = 1e-6
    H = 128 if dt == wl.DT_BF16 else 16
    B, N, W, k = 3, 3000, 128, 300
    q = _scaled_rows(110, 0, 1, (B, H, E), dt, 0.1, 4.0)
    ent = _scaled_rows(110, 0, 2, (N, E), dt, 0.05, 20.0)
    win = _rand(110, 0, 3, (W, E), dt)
    rng = np.random.default_rng(1)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[1, 7:90] = -1
    sink_h = rng.uniform(-1.0, 3.0, H)
    for sk in (None, sink_h):
        st = None if sk is None else torch.from_numpy(sk.astype(np.float32)).cuda()
        out, lse = cskv.sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda(),
                                      scale=1 / 24, norm_eps=eps, sink=st)
        torch.cuda.synchronize()
        ro, rl = oracle.csa_attend(q, ent, win, dt, idx, scale=1 / 24, norm_eps=eps, sink=sk)
        _check_attn(out, lse, ro, rl, dt)
    out, lse = cskv.hca_attend(dev(q), dev(ent), scale=1 / 24, norm_eps=eps)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, scale=1 / 24, norm_eps=eps)
    _check_attn(out, lse, ro, rl, dt)
    m = 128
    pos = np.array([0, 127, 1000, 40 * m + 3, N * m + 5], np.int64)
    q5 = _scaled_rows(110, 0, 4, (5, H, E), dt, 0.1, 4.0)
    out, lse = cskv.hca_attend(dev(q5), dev(ent[:600]), scale=1 / 24, norm_eps=eps,
                               q_pos=torch.from_numpy(pos).cuda(), m=m)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q5, ent[:600], dt, scale=1 / 24, norm_eps=eps, q_pos=pos, m=m)
    _check_attn(out[1:], lse[1:], ro[1:], rl[1:], dt)
    assert (host_f64(out)[0] == 0).all()
    eps2 = _scaled_rows(110, 0, 5, (B, 500, E), dt, 0.05, 20.0)
    out, lse = cskv.hca_attend(dev(q), dev(eps2), scale=1 / 24, norm_eps=0.0, per_seq=True)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, eps2, dt, scale=1 / 24, norm_eps=0.0, per_seq=True)
    _check_attn(out, lse, ro, rl, dt)


@pytest.mark.parametrize("N", [300, 8192])
def test_normalised_attention_past_reference_band(N):
    """Normalised rows of tile 0 nearly orthogonal to the query, and one row
    in every later tile along it: their logits (scale 0.3 x up to 576) are far
    past the band a split accumulates against, so splits redo their rows
    exactly; HCA and sparse attention must still match the oracle."""
    dt, B, H = wl.DT_BF16, 2, 128
    rng = np.random.default_rng(N + 1)
    qf = 0.5 + 0.01 * rng.standard_normal((B, H, E))
    ef = 0.1 * rng.standard_normal((N, E))
    big = np.arange(32 + 5, N, 32)
    ef[big] = (0.5 + 0.01 * rng.standard_normal((len(big), E))) * rng.uniform(0.1, 10, (len(big), 1))
    q, ent = wl.encode(qf, dt).raw, wl.encode(ef, dt).raw
    out, lse = _cskv().hca_attend(dev(q), dev(ent), scale=0.3, norm_eps=1e-6)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend(q, ent, dt, scale=0.3, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, dt)
    W = 128
    win = wl.encode(0.1 * rng.standard_normal((W, E)), dt).raw
    k = min(N, 1024)
    idx = np.tile(np.arange(k, dtype=np.int32), (B, 1))
    out, lse = _cskv().sparse_attend(dev(q), dev(ent), dev(win), torch.from_numpy(idx).cuda(),
                                     scale=0.3, norm_eps=1e-6)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend(q, ent, win, dt, idx, scale=0.3, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, dt)


def test_normalised_csa_decode_workload():
    """The fused CSA call with normalisation on the 16,384-entry decode
    workload (8 queries x 128 heads, top-1024 + 128 window rows): every
    query's attention over the GPU's own selection."""
    cfg = wl.CONFIGS["csa_decode"]
    inp = wl.make_inputs(cfg, seed=0)
    out, lse, idx = _cskv().csa_attend(dev(inp["q"]), dev(inp["qI"]), dev(inp["entries"]),
                                       dev(inp["kI"]), dev(inp["window"]), cfg.k, scale=1 / 24,
                                       norm_eps=1e-6)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s, v = oracle.index_scores(inp["qI"].raw, inp["kI"].raw, cfg.idx_dt)
    check_selection(idx, s, v, cfg.k)
    ro, rl = oracle.csa_attend(inp["q"].raw, inp["entries"].raw, inp["window"].raw, cfg.dt, idx,
                               scale=1 / 24, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, cfg.dt)


def test_normalised_attention_mxfp4_entries():
    """Normalisation over MXFP4 entries (decoded exactly, then normalised):
    sparse attention with bf16 window rows, and HCA."""
    B, H, N, W, k = 2, 128, 900, 128, 200
    q = _rand(111, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx_entries(111, 0, (N, E))
    win = _rand(111, 0, 3, (W, E), wl.DT_BF16)
    rng = np.random.default_rng(2)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    out, lse = _cskv().sparse_attend_mxfp4(dev(q), _up(codes), _up(scales), dev(win), _up(idx),
                                           scale=1 / 24, norm_eps=1e-6)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp4(q, codes, scales, win, idx, scale=1 / 24, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    out, lse = _cskv().hca_attend_mxfp4(dev(q), _up(codes), _up(scales), scale=1 / 24, norm_eps=1e-6)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp4(q, codes, scales, scale=1 / 24, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def _scales_at(scales, off):
    """The scale rows on the device, starting off bytes past a 16-byte
    boundary (a view into a larger buffer)."""
    flat = np.ascontiguousarray(scales).reshape(-1)
    buf = torch.zeros(flat.size + 32, dtype=torch.uint8, device="cuda")
    buf[off:off + flat.size] = torch.from_numpy(flat).cuda()
    return buf[off:off + flat.size].view(scales.shape)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("off", [1, 2, 3])
def test_attend_mx_scales_at_any_byte_offset(bits, off):
    """Scale rows that start at any byte address: CSA with a selection that
    is not a whole number of tiles (k = 45, some -1) plus window rows, and
    HCA over a ragged entry count, per sequence."""
    B, H, N, W, k = 2, 32, 301, 7, 45
    rng = np.random.default_rng(off * 10 + bits)
    q = _rand(131, N, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    enc = wl.mxfp4_encode if bits == 4 else wl.mxfp8_encode
    codes, scales = enc(wl.normal(131, N + bits, 2, (B, N, E)))
    win = _rand(131, N, 3, (W, E), wl.DT_BF16)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[1, 3] = -1
    sc = _scales_at(scales, off)
    cskv = _cskv()
    sparse = cskv.sparse_attend_mxfp4 if bits == 4 else cskv.sparse_attend_mxfp8
    hca = cskv.hca_attend_mxfp4 if bits == 4 else cskv.hca_attend_mxfp8
    ocsa = oracle.csa_attend_mxfp4 if bits == 4 else oracle.csa_attend_mxfp8
    ohca = oracle.hca_attend_mxfp4 if bits == 4 else oracle.hca_attend_mxfp8
    out, lse = sparse(dev(q), _up(codes[0]), sc[0], dev(win), _up(idx), W=W)
    torch.cuda.synchronize()
    ro, rl = ocsa(q, codes[0], scales[0], win, idx, W=W)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    out, lse = hca(dev(q), _up(codes), sc, per_seq=True)
    torch.cuda.synchronize()
    ro, rl = ohca(q, codes, scales, per_seq=True)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


# ------------------------------------------------------- MXFP8 entries

def _mx8_entries(cfg_id, seed, shape):
    """Entries drawn ~N(0,1) in fp32 and quantised to MXFP8 (E4M3 codes, scales)."""
    return wl.mxfp8_encode(wl.normal(cfg_id, seed, 2, shape))


@pytest.mark.parametrize("B,H,N,W,k", [(2, 128, 5000, 128, 1024), (3, 80, 700, 16, 37),
                                       (1, 16, 40, 0, 40), (4, 128, 300, 5, 1)])
def test_sparse_attend_mxfp8_matches_oracle(B, H, N, W, k):
    """CSA over MXFP8 entries plus bf16 window rows; some selections hold -1."""
    rng = np.random.default_rng(B * 1000 + k + 7)
    q = _rand(112, N, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx8_entries(112, N, (N, E))
    win = _rand(112, N, 3, (max(W, 1), E), wl.DT_BF16)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[0, -1] = -1
    out, lse = _cskv().sparse_attend_mxfp8(dev(q), _up(codes), _up(scales), dev(win), _up(idx), W=W)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp8(q, codes, scales, win, idx, W=W)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_attend_mxfp8_prefill_sink_per_sequence_and_norm():
    """Prefill windows over per-sequence MXFP8 entries with sinks; HCA decode
    (several splits), prefill visibility and per-sequence entries; and the
    query / entry normalisation."""
    cskv = _cskv()
    rng = np.random.default_rng(4)
    B, H, N, W, k = 3, 128, 900, 128, 64
    q = _rand(113, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    codes, scales = _mx8_entries(113, 0, (B, N, E))
    pos0, rows = 1000, 300
    win = _rand(113, 0, 3, (B, rows, E), wl.DT_BF16)
    qp = np.array([pos0 + W - 1, pos0 + 200, pos0 + rows - 1], np.int64)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    sink = rng.standard_normal(H) * 2
    st = torch.from_numpy(sink).float().cuda()
    sk = sink.astype(np.float32).astype(np.float64)
    out, lse = cskv.sparse_attend_mxfp8(dev(q), _up(codes), _up(scales), dev(win), _up(idx),
                                        q_pos=_up(qp), win_pos0=pos0, W=W, per_seq=True, sink=st)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp8(q, codes, scales, win, idx, q_pos=qp, win_pos0=pos0, W=W,
                                     per_seq=True, sink=sk)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    out, lse = cskv.hca_attend_mxfp8(dev(q), _up(codes[0]), _up(scales[0]), sink=st)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp8(q, codes[0], scales[0], sink=sk)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    out, lse = cskv.hca_attend_mxfp8(dev(q), _up(codes), _up(scales), per_seq=True)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp8(q, codes, scales, per_seq=True)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)
    m = 128
    hp = np.array([0, 127, 40000], np.int64)
    out, lse = cskv.hca_attend_mxfp8(dev(q), _up(codes[1]), _up(scales[1]), q_pos=_up(hp), m=m)
    torch.cuda.synchronize()
    ro, rl = oracle.hca_attend_mxfp8(q, codes[1], scales[1], q_pos=hp, m=m)
    assert (host_f64(out)[0] == 0).all()
    _check_attn(out[1:], lse[1:], ro[1:], rl[1:], wl.DT_BF16)
    out, lse = cskv.sparse_attend_mxfp8(dev(q), _up(codes[2]), _up(scales[2]), dev(win[0]),
                                        _up(idx), scale=1 / 24, norm_eps=1e-6)
    torch.cuda.synchronize()
    ro, rl = oracle.csa_attend_mxfp8(q, codes[2], scales[2], win[0], idx, scale=1 / 24, norm_eps=1e-6)
    _check_attn(out, lse, ro, rl, wl.DT_BF16)


def test_attend_mxfp8_decode_workload_sampled():
    """The 1M-token decode shapes with MXFP8 entries: HCA over 8,192 entries
    and CSA over 1,024 selected of 262,144 plus 128 window rows, 32 queries x
    128 heads, checked on sampled queries."""
    cfg = wl.CONFIGS["layer_1m"]
    B, H, k, W = cfg.B, cfg.H, cfg.k, cfg.W
    rng = np.random.default_rng(12)
    q = _rand(cfg.config_id, 0, 1, (B, H, E), wl.DT_BF16, 1 / 24)
    c128, s128 = _mx8_entries(cfg.config_id, 3, (cfg.N_hca, E))
    out, lse = _cskv().hca_attend_mxfp8(dev(q), _up(c128), _up(s128))
    c4, s4 = _mx8_entries(cfg.config_id, 4, (cfg.N_csa, E))
    win = _rand(cfg.config_id, 0, 3, (W, E), wl.DT_BF16)
    idx = np.stack([np.sort(rng.choice(cfg.N_csa, k, replace=False)) for _ in range(B)]).astype(np.int32)
    o2, l2 = _cskv().sparse_attend_mxfp8(dev(q), _up(c4), _up(s4), dev(win), _up(idx))
    torch.cuda.synchronize()
    rows = np.array([0, 17, B - 1])
    sel = torch.from_numpy(rows).cuda()
    ro, rl = oracle.hca_attend_mxfp8(q[rows], c128, s128)
    _check_attn(out[sel], lse[sel], ro, rl, wl.DT_BF16)
    ro, rl = oracle.csa_attend_mxfp8(q[rows], c4, s4, win, idx[rows])
    _check_attn(o2[sel], l2[sel], ro, rl, wl.DT_BF16)
