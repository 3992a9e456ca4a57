"""CPU oracle of the compressed sparse KV attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library.  `cskv_oracle.c` is
the definition (plain fp64 loops); this module builds it with gcc, loads it
with ctypes and wraps it for NumPy arrays.  `numpy_ref` is a second,
independent NumPy formulation used only to cross-check the C code.

Inputs are passed as stored bytes plus a dtype code (0 fp32, 1 bf16 as uint16
bits, 2 fp8 e4m3 as uint8 codes); outputs are float64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cskv_oracle.c")
_LIB = os.path.join(_HERE, "libcskv_oracle.so")
_lib = None

F32, BF16, E4M3, F64 = 0, 1, 2, 3
D, R, E, I = 512, 64, 576, 64


def build(force=True):
    """Compile the C oracle with gcc (OpenMP, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.cskv_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.cskv_oracle_e4m3_value.restype = dbl
        L.cskv_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.cskv_oracle_bf16_value.restype = dbl
        L.cskv_oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.cskv_oracle_e2m1_value.restype = dbl
        L.cskv_oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.cskv_oracle_e8m0_value.restype = dbl
        L.cskv_oracle_mxfp4_decode.argtypes = [vp, vp, i64, i32, vp]
        L.cskv_oracle_mxfp8_decode.argtypes = [vp, vp, i64, i32, vp]
        L.cskv_oracle_num_entries.argtypes = [i64, i32]
        L.cskv_oracle_num_entries.restype = i64
        L.cskv_oracle_compress.argtypes = [vp, vp, i32, vp, i64, i64, i32, vp, i64, vp]
        L.cskv_oracle_index_scores.argtypes = [vp, vp, i32, i64, i64, i64, dbl, i64, vp, i32, vp, vp]
        L.cskv_oracle_topk.argtypes = [vp, vp, i64, i64, i32, vp]
        L.cskv_oracle_csa_attend.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, vp,
                                             i64, i64, i64, i64, vp, i64, dbl, vp, dbl, vp, vp]
        L.cskv_oracle_hca_attend.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, vp, i32, dbl,
                                             vp, dbl, vp, vp]
        L.cskv_oracle_max_threads.restype = i32
        L.cskv_oracle_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (code {rc})")


def max_threads():
    return lib().cskv_oracle_max_threads()


def set_threads(n):
    """Thread count of the oracle's OpenMP loops (the results do not depend
    on it)."""
    lib().cskv_oracle_set_threads(int(n))


def e4m3_value(code):
    return lib().cskv_oracle_e4m3_value(int(code))


def bf16_value(bits):
    return lib().cskv_oracle_bf16_value(int(bits))


def num_entries(T, m):
    return lib().cskv_oracle_num_entries(int(T), int(m))


def decode(raw, dt):
    """Exact values of stored bytes, via the oracle's own decoders."""
    raw = np.asarray(raw)
    if dt == F32:
        return raw.astype(np.float64)
    if dt == BF16:
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[raw]


def compress(x, z, dt, bias, m, entry_ids=None):
    """Compressed content dims of the requested entries: float64 [n, D]."""
    x, z = _c(x), _c(z)
    T, Dd = x.shape
    bias = _c(bias, np.float32)
    if entry_ids is None:
        entry_ids = np.arange(T // m, dtype=np.int64)
    ids = _c(entry_ids, np.int64)
    out = np.empty((len(ids), Dd), dtype=np.float64)
    _check(lib().cskv_oracle_compress(_p(x), _p(z), dt, _p(bias), T, Dd, m, _p(ids), len(ids),
                                      _p(out)), "compress")
    return out


def index_scores(qI, kI, dt, scale=1.0, q_pos=None, m=4, per_seq=False):
    """Indexer scores float64 [B, N] and visibility uint8 [B, N]."""
    qI, kI = _c(qI), _c(kI)
    B, Id = qI.shape
    N = kI.shape[-2]
    kstride = N * Id if per_seq else 0
    qp = _c(q_pos, np.int64)
    s = np.empty((B, N), dtype=np.float64)
    v = np.empty((B, N), dtype=np.uint8)
    _check(lib().cskv_oracle_index_scores(_p(qI), _p(kI), dt, B, N, Id, float(scale), kstride,
                                          _p(qp), m, _p(s), _p(v)), "index_scores")
    return s, v


def e2m1_value(code):
    return lib().cskv_oracle_e2m1_value(code)


def e8m0_value(x):
    return lib().cskv_oracle_e8m0_value(x)


def mxfp4_decode(codes, scales):
    """MXFP4 rows of C elements (C a multiple of 32) -> float64 [..., C]
    (codes uint8 [..., C/2], scales uint8 [..., C/32]; leading dimensions
    are kept)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    cols = 2 * codes.shape[-1]
    if cols % 32 or scales.shape != lead + (cols // 32,):
        raise ValueError("mxfp4 rows: codes [..., C/2] and scales [..., C/32], C % 32 == 0")
    out = np.empty(lead + (cols,), dtype=np.float64)
    _check(lib().cskv_oracle_mxfp4_decode(_p(codes), _p(scales), rows, cols, _p(out)),
           "mxfp4_decode")
    return out


def mxfp8_decode(codes, scales):
    """MXFP8 (E4M3) rows of C elements (C a multiple of 32) -> float64
    [..., C] (codes uint8 [..., C], scales uint8 [..., C/32])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    cols = codes.shape[-1]
    if cols % 32 or scales.shape != lead + (cols // 32,):
        raise ValueError("mxfp8 rows: codes [..., C] and scales [..., C/32], C % 32 == 0")
    out = np.empty(lead + (cols,), dtype=np.float64)
    _check(lib().cskv_oracle_mxfp8_decode(_p(codes), _p(scales), rows, cols, _p(out)),
           "mxfp8_decode")
    return out


def index_scores_mxfp4(q_codes, q_scales, k_codes, k_scales, scale=1.0, q_pos=None, m=4,
                       per_seq=False):
    """Indexer scores of MXFP4 queries and keys: the rows are decoded exactly,
    then scored like any other input."""
    return index_scores(mxfp4_decode(q_codes, q_scales), mxfp4_decode(k_codes, k_scales), F64,
                        scale, q_pos=q_pos, m=m, per_seq=per_seq)


def topk(scores, visible, k):
    scores = _c(scores, np.float64)
    visible = _c(visible, np.uint8)
    B, N = scores.shape
    idx = np.empty((B, k), dtype=np.int32)
    _check(lib().cskv_oracle_topk(_p(scores), _p(visible), B, N, k, _p(idx)), "topk")
    return idx


def csa_attend(q, entries, window, dt, idx, scale=1.0, q_pos=None, win_pos0=0, W=None,
               per_seq=False, Dv=D, sink=None, norm_eps=None):
    """CSA attention over selected entries plus the raw window; sink: per-head
    attention-sink logits [H] (None: no sink); norm_eps: normalise the
    queries and the selected entries to unit RMS with this epsilon (None: no
    normalisation; window rows are never normalised).
    Returns (out float64 [B, H, Dv], lse float64 [B, H])."""
    q, entries, window = _c(q), _c(entries), _c(window)
    idx = _c(idx, np.int32)
    B, H, Ee = q.shape
    N = entries.shape[-2]
    k = idx.shape[1]
    if W is None:
        W = 0 if window is None else window.shape[-2]
    win_rows = 0 if window is None else window.shape[-2]
    ent_bs = N * Ee if per_seq else 0
    win_bs = win_rows * Ee if per_seq else 0
    qp = _c(q_pos, np.int64)
    out = np.empty((B, H, Dv), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    _check(lib().cskv_oracle_csa_attend(_p(q), _p(entries), _p(window), dt, B, H, Ee, Dv, N, W,
                                        _p(idx), k, ent_bs, win_bs, win_rows, _p(qp), int(win_pos0),
                                        float(scale), _p(_c(sink, np.float64)),
                                        -1.0 if norm_eps is None else float(norm_eps), _p(out), _p(lse)),
           "csa_attend")
    return out, lse


def csa_attend_mxfp4(q, ent_codes, ent_scales, window, idx, **kw):
    """csa_attend with MXFP4 entries (codes [.., N, 288], scales [.., N, 18])
    and bf16 queries and window rows: every input is decoded exactly, then
    attended in fp64."""
    win = None if window is None else decode(window, BF16)
    return csa_attend(decode(q, BF16), mxfp4_decode(ent_codes, ent_scales), win, F64, idx, **kw)


def csa_attend_mxfp8(q, ent_codes, ent_scales, window, idx, **kw):
    """csa_attend with MXFP8 entries (codes [.., N, 576], scales [.., N, 18])
    and bf16 queries and window rows, every input decoded exactly."""
    win = None if window is None else decode(window, BF16)
    return csa_attend(decode(q, BF16), mxfp8_decode(ent_codes, ent_scales), win, F64, idx, **kw)


def hca_attend_mxfp8(q, ent_codes, ent_scales, **kw):
    """hca_attend with MXFP8 entries and bf16 queries."""
    return hca_attend(decode(q, BF16), mxfp8_decode(ent_codes, ent_scales), F64, **kw)


def hca_attend_mxfp4(q, ent_codes, ent_scales, **kw):
    """hca_attend with MXFP4 entries and bf16 queries."""
    return hca_attend(decode(q, BF16), mxfp4_decode(ent_codes, ent_scales), F64, **kw)


def hca_attend(q, entries, dt, scale=1.0, per_seq=False, Dv=D, q_pos=None, m=None, sink=None,
               norm_eps=None):
    """Dense attention over the entries each query sees: all of them at
    decode (q_pos None); at a prefill chunk, entries i with (i+1)*m <=
    q_pos[b] + 1; norm_eps as in csa_attend.  Returns (out [B, H, Dv],
    lse [B, H])."""
    q, entries = _c(q), _c(entries)
    B, H, Ee = q.shape
    N = entries.shape[-2]
    qp = None if q_pos is None else np.ascontiguousarray(q_pos, dtype=np.int64)
    out = np.empty((B, H, Dv), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    _check(lib().cskv_oracle_hca_attend(_p(q), _p(entries), dt, B, H, Ee, Dv, N,
                                        N * Ee if per_seq else 0, _p(qp),
                                        int(m) if m is not None else 0, float(scale),
                                        _p(_c(sink, np.float64)),
                                        -1.0 if norm_eps is None else float(norm_eps), _p(out),
                                        _p(lse)),
           "hca_attend")
    return out, lse
