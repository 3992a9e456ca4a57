"""The five synthetic workloads of the hot path, as seeded input recipes.

Shapes and distributions follow the workload descriptions: a tiny fp32
CSA+HCA case, a bf16 CSA decode at 16,384 entries, a bf16 HCA decode at
8,192 entries, a CSA prefill chunk with an fp8 indexer, and the 1M-token
layer pair (compress at m=4 and m'=128, then CSA and HCA decode).

Layouts (row-major, element counts):
  x, z        [T, 512]        raw shared-KV rows and compressor score logits
  b<m>        [2m, 512] fp32  per-window-position compressor bias
  rope<m>     [N, 64]         RoPE part of each compressed entry
  entries     [N, 576]        512 content dims then 64 RoPE dims (V = dims 0..511)
  kI          [N, 64]         indexer keys;  qI [B, 64] indexer queries
  q           [B, H, 576]     attention queries (~N(0, 1/576): 1/sqrt(576) folded in)
  window      [W, 576]        raw recent rows (512 content + 64 RoPE)
In per-sequence mode entries/kI/window get a leading batch dimension.
"""
from dataclasses import dataclass, field

import numpy as np

from .formats import DT_F32, DT_BF16, DT_E4M3
from .gen import normal, encode

D, R, E, I = 512, 64, 576, 64
TID = dict(x=1, z=2, b4=3, b128=4, rope4=5, rope128=6, q=7, qI=8, kI=9,
           win_rope=10, entries=11, window=12, q_hca=13, entries_hca=14,
           win_src=15)


@dataclass
class Config:
    name: str
    config_id: int
    dt: int                      # dtype of x, z, entries, q, window
    idx_dt: int                  # dtype of the indexer keys / queries
    B: int = 1                   # decode queries (or prefill query tokens)
    H: int = 128
    k: int = 1024
    W: int = 128
    T: int = 0                   # raw tokens to compress (0: entries given)
    N_csa: int = 0               # m=4 entries
    N_hca: int = 0               # m'=128 entries
    m_csa: int = 4
    m_hca: int = 128
    bias_std: float = 0.1
    prefill_pos0: int = -1       # first query position (prefill only)
    notes: str = ""
    parts: tuple = field(default_factory=tuple)


CONFIGS = {
    "tiny": Config("tiny", 0, DT_F32, DT_F32, B=1, H=16, k=64, W=128, T=4096,
                   N_csa=1024, N_hca=32, parts=("compress", "csa", "hca"),
                   notes="T=4096 fp32; m=4 -> 1024 entries, m'=128 -> 32; 1 query, 16 heads, top-64 + 128 window"),
    "csa_decode": Config("csa_decode", 1, DT_BF16, DT_BF16, B=8, H=128, k=1024, W=128,
                         N_csa=16384, parts=("csa",),
                         notes="16,384 m=4 entries (T=65,536), 8 queries x 128 heads, top-1024 + 128 window, bf16"),
    "hca_decode": Config("hca_decode", 2, DT_BF16, DT_BF16, B=16, H=128, N_hca=8192,
                         parts=("hca",),
                         notes="8,192 m'=128 entries (T=2^20), 16 queries x 128 heads, dense, bf16"),
    "csa_prefill": Config("csa_prefill", 3, DT_BF16, DT_E4M3, B=4096, H=128, k=1024, W=128,
                          N_csa=262144, prefill_pos0=1044480, parts=("csa",),
                          notes="4,096 causal queries at positions 1,044,480..1,048,575; 262,144 entries; fp8 e4m3 indexer"),
    "hca_prefill": Config("hca_prefill", 5, DT_BF16, DT_BF16, B=4096, H=128, N_hca=8192,
                          prefill_pos0=1044480, parts=("hca",),
                          notes="4,096 causal queries at positions 1,044,480..1,048,575 over 8,192 m'=128 entries, bf16"),
    "layer_1m": Config("layer_1m", 4, DT_BF16, DT_BF16, B=32, H=128, k=1024, W=128,
                       T=1 << 20, N_csa=262144, N_hca=8192,
                       parts=("compress", "csa", "hca"),
                       notes="1M-token layer pair: compress at m=4 and m'=128, then CSA (top-1024 + 128 window) and HCA decode, 32 queries x 128 heads, bf16"),
}


def _n(cfg, seed, name, shape, std=1.0):
    return normal(cfg.config_id, seed, TID[name], shape, std)


def make_inputs(cfg, seed=0, per_seq=False, with_compress_source=True):
    """Build the stored inputs of a workload.

    Returns a dict of `Tensor`s (plus plain ints for positions).  For the
    workloads that start from raw tokens ("tiny", "layer_1m") the compressed
    entries are NOT included: their content dims are what compress produces.
    The dict then holds x, z, b4, b128, rope4, rope128 and the window.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    dt, out = cfg.dt, {}
    qstd = 1.0 / np.sqrt(E)
    if cfg.T and with_compress_source:
        x = _n(cfg, seed, "x", (cfg.T, D))
        out["x"] = encode(x, dt)
        out["z"] = encode(_n(cfg, seed, "z", (cfg.T, D)), dt)
        out["b4"] = encode(_n(cfg, seed, "b4", (2 * cfg.m_csa, D), cfg.bias_std), DT_F32)
        out["b128"] = encode(_n(cfg, seed, "b128", (2 * cfg.m_hca, D), cfg.bias_std), DT_F32)
        out["rope4"] = encode(_n(cfg, seed, "rope4", (cfg.T // cfg.m_csa, R)), dt)
        out["rope128"] = encode(_n(cfg, seed, "rope128", (cfg.T // cfg.m_hca, R)), dt)
        # the raw window: the last W raw rows plus a RoPE part
        win = np.empty((cfg.W, E), dtype=np.float32)
        win[:, :D] = x[cfg.T - cfg.W:]
        win[:, D:] = _n(cfg, seed, "win_rope", (cfg.W, R))
        out["window"] = encode(win, dt)
        del x
    nb = cfg.B if per_seq else None

    def bshape(*s):
        return ((nb,) + s) if nb else s

    if "csa" in cfg.parts:
        if not cfg.T:
            out["entries"] = encode(_n(cfg, seed, "entries", bshape(cfg.N_csa, E)), dt)
            if cfg.prefill_pos0 < 0:
                out["window"] = encode(_n(cfg, seed, "window", bshape(cfg.W, E)), dt)
        out["q"] = encode(_n(cfg, seed, "q", (cfg.B, cfg.H, E), qstd), dt)
        out["qI"] = encode(_n(cfg, seed, "qI", (cfg.B, I)), cfg.idx_dt)
        out["kI"] = encode(_n(cfg, seed, "kI", bshape(cfg.N_csa, I)), cfg.idx_dt)
        if cfg.prefill_pos0 >= 0:
            nsrc = cfg.B + cfg.W - 1
            out["window"] = encode(_n(cfg, seed, "win_src", (nsrc, E)), dt)
            out["win_pos0"] = cfg.prefill_pos0 - (cfg.W - 1)
            out["q_pos"] = np.arange(cfg.prefill_pos0, cfg.prefill_pos0 + cfg.B, dtype=np.int64)
    if "hca" in cfg.parts:
        if not cfg.T:
            out["entries_hca"] = encode(_n(cfg, seed, "entries_hca", bshape(cfg.N_hca, E)), dt)
        qname = "q_hca" if "csa" in cfg.parts else "q"
        out["q_hca"] = encode(_n(cfg, seed, qname, (cfg.B, cfg.H, E), qstd), dt)
        if cfg.prefill_pos0 >= 0:
            out["q_pos"] = np.arange(cfg.prefill_pos0, cfg.prefill_pos0 + cfg.B, dtype=np.int64)
    return out
