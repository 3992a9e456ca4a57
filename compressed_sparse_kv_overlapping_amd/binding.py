"""ctypes binding of libcskv (include/cskv.h).

Argument marshalling only.  Every wrapper first checks the dtype and shape
of each tensor it is given (and that a given workspace is uint8 and large
enough), raising ValueError before anything reaches the library; then that
the tensors are contiguous and in GPU memory.  Device pointers and the
current HIP stream are passed to the C-ABI, and a non-zero status raises
CskvError with the library's message.  Outputs are
allocated here with torch (the library itself never allocates).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcskv.so")
DT_F32, DT_BF16, DT_E4M3 = 0, 1, 2
D, R, E, I = 512, 64, 576, 64

_TORCH_DT = {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float8_e4m3fn: DT_E4M3}
_OUT_DT = {DT_F32: torch.float32, DT_BF16: torch.bfloat16}
_lib = None


class CskvError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_vp, _i64, _i32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                              ctypes.c_size_t)
_SIGS = {
    "cskv_version": ([], ctypes.c_int),
    "cskv_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "cskv_last_error": ([], ctypes.c_char_p),
    "cskv_compress": ([_vp, _vp, _vp, _i64, _i32, _i64, _i64, _vp, _i64, ctypes.c_int, _vp],
                      ctypes.c_int),
    "cskv_compress2_workspace_size": ([_i64, _i32], _sz),
    "cskv_compress2": ([_vp, _vp, _i64, _vp, _i32, _vp, _i64, _vp, _i32, _vp, _i64, ctypes.c_int,
                        _vp, _sz, _vp], ctypes.c_int),
    "cskv_index_topk_workspace_size": ([_i64, _i64, _i32], _sz),
    "cskv_index_topk": ([_vp, _vp, _i64, _i64, _i32, _i64, _vp, _i32, _f32, ctypes.c_int, _vp,
                         _vp, _sz, _vp], ctypes.c_int),
    "cskv_index_topk_mxfp4": ([_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i64, _vp, _i32, _f32, _vp,
                               _vp, _sz, _vp], ctypes.c_int),
    "cskv_index_topk_per_seq_workspace_size": ([_i64, _i64, _i32], _sz),
    "cskv_index_topk_noalloc_max_bytes": ([], _sz),
    "cskv_index_topk_noalloc": ([_vp, _vp, _i64, _i64, _i32, _i64, _vp, _i32, _f32, ctypes.c_int,
                                 _vp, _vp], ctypes.c_int),
    "cskv_attend_workspace_size": ([_i64, _i32, _i64], _sz),
    "cskv_sparse_attend": ([_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i64, _i64, _i64,
                            _vp, _i64, _f32, _vp, _f32, ctypes.c_int, _vp, _vp, _vp, _sz, _vp],
                           ctypes.c_int),
    "cskv_csa_workspace_size": ([_i64, _i32, _i64, _i32, _i32], _sz),
    "cskv_csa_attend": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32, _i64, _i64,
                         _i64, _i64, _vp, _i64, _f32, _vp, _f32, _f32, ctypes.c_int, ctypes.c_int,
                         _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "cskv_hca_workspace_size": ([_i64, _i32, _i64], _sz),
    "cskv_hca_attend": ([_vp, _vp, _i64, _i32, _i64, _i64, _vp, _i32, _f32, _vp, _f32, ctypes.c_int,
                         _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "cskv_sparse_attend_mxfp4_workspace_size": ([_i64, _i32, _i32, _i32], _sz),
    "cskv_hca_attend_mxfp4_workspace_size": ([_i64, _i32, _i64, _i32], _sz),
    "cskv_sparse_attend_mxfp4": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i64, _i64,
                                  _i64, _vp, _i64, _f32, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
                                 ctypes.c_int),
    "cskv_hca_attend_mxfp4": ([_vp, _vp, _vp, _i64, _i32, _i64, _i64, _vp, _i32, _f32, _vp, _f32, _vp,
                               _vp, _vp, _sz, _vp], ctypes.c_int),
    "cskv_sparse_attend_mxfp8": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i64, _i64,
                                  _i64, _vp, _i64, _f32, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
                                 ctypes.c_int),
    "cskv_hca_attend_mxfp8": ([_vp, _vp, _vp, _i64, _i32, _i64, _i64, _vp, _i32, _f32, _vp, _f32, _vp,
                               _vp, _vp, _sz, _vp], ctypes.c_int),
    "cskv_merge": ([_vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, ctypes.c_int, _vp], ctypes.c_int),
}
EXPORTS = tuple(_SIGS)


def library():
    """Load libcskv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_sparse_kv_overlapping_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            if hasattr(lib, name):
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
        _lib = lib
    return _lib


def _call(name, *args):
    st = getattr(library(), name)(*args)
    if st != 0:
        raise CskvError(name, st, library().cskv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, shape):
    """Check one argument before anything reaches the library: dtype in
    `dtypes` (a dtype or a tuple), shape equal to `shape` (None entries
    match any size).  None arguments are skipped."""
    if t is None:
        return
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name}: dtype {str(t.dtype).replace('torch.', '')}, expected {names}")
    if len(t.shape) != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
        raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")


def _need_ws(ws, nbytes, name="workspace"):
    """A caller-supplied workspace: uint8, at least nbytes long."""
    if ws is None:
        return
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError(f"{name}: a 1-D uint8 tensor is expected")
    if ws.numel() < nbytes:
        raise ValueError(f"{name}: {ws.numel()} bytes, at least {nbytes} needed")


_VAL_DT = (torch.float32, torch.bfloat16)               # attention / compressor data
_IDX_DT = (torch.float32, torch.bfloat16, torch.float8_e4m3fn)


def _kv(t, name, per_seq, B, cols, dtype):
    """A cache tensor: [N, cols] shared, or [B, N, cols] per sequence."""
    if t is None:
        return
    _need(t, name, dtype, (B, None, cols) if per_seq else (None, cols))


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("cskv tensors must live in GPU memory")
            if not t.is_contiguous():
                raise ValueError("cskv tensors must be contiguous")


def _sink(sink, H):
    """Per-head attention-sink logits: None, or fp32 [H] on the device."""
    if sink is None:
        return None
    _dev(sink)
    if sink.dtype != torch.float32 or sink.shape != (H,):
        raise ValueError(f"sink must be fp32 [{H}]")
    return _ptr(sink)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t):
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ compress

def compress(x, z, bias, m, out=None, entry_begin=0, entry_end=None, stream=None):
    """Compress raw rows x [T, 512] with logits z [T, 512] and fp32 position
    bias [2m, 512] into entries.  `out` may be a [N, 576] entry buffer (only
    columns 0..511 are written) or is allocated as [N, 512]."""
    _need(x, "x", _VAL_DT, (None, D))
    T = x.shape[0]
    _need(z, "z", x.dtype, (T, D))
    _need(bias, "bias", torch.float32, (2 * m, D))
    N = T // m
    if entry_end is None:
        entry_end = N
    if out is not None:
        _need(out, "out", x.dtype, (None, None))
        if out.stride(1) != 1 or out.shape[1] < D or out.shape[0] < entry_end:
            raise ValueError(f"out: a row-major [>= {entry_end}, >= {D}] tensor is expected")
    _dev(x, z, bias)
    if out is None:
        out = torch.empty((N, D), dtype=x.dtype, device=x.device)
    _call("cskv_compress", _ptr(x), _ptr(z), _ptr(bias), T, m, entry_begin, entry_end, _ptr(out),
          out.stride(0), _dt(x), _stream(stream))
    return out


def compress2_workspace_size(T, m_large):
    return library().cskv_compress2_workspace_size(T, m_large)


def compress2(x, z, bias_small, m_small, bias_large, m_large, out_small=None, out_large=None,
              workspace=None, stream=None):
    """Both scales in one pass: returns (out_small, out_large), each either
    given (e.g. [N, 576] entry buffers; columns 0..511 written) or allocated
    as [N, 512]."""
    _need(x, "x", _VAL_DT, (None, D))
    T = x.shape[0]
    _need(z, "z", x.dtype, (T, D))
    _need(bias_small, "bias_small", torch.float32, (2 * m_small, D))
    _need(bias_large, "bias_large", torch.float32, (2 * m_large, D))
    for o, n, name in ((out_small, T // m_small, "out_small"), (out_large, T // m_large, "out_large")):
        if o is not None:
            _need(o, name, x.dtype, (None, None))
            if o.stride(1) != 1 or o.shape[1] < D or o.shape[0] < n:
                raise ValueError(f"{name}: a row-major [>= {n}, >= {D}] tensor is expected")
    _need_ws(workspace, compress2_workspace_size(T, m_large))
    _dev(x, z, bias_small, bias_large)
    if out_small is None:
        out_small = torch.empty((T // m_small, D), dtype=x.dtype, device=x.device)
    if out_large is None:
        out_large = torch.empty((T // m_large, D), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = _workspace(compress2_workspace_size(T, m_large), x.device)
    _call("cskv_compress2", _ptr(x), _ptr(z), T, _ptr(bias_small), m_small, _ptr(out_small),
          out_small.stride(0), _ptr(bias_large), m_large, _ptr(out_large), out_large.stride(0),
          _dt(x), _ptr(workspace), workspace.numel(), _stream(stream))
    return out_small, out_large


# -------------------------------------------------------------- indexer/top-k

def index_topk_workspace_size(B, N, k, per_seq=False):
    """Workspace bytes of index_topk; with per_seq, the size with which
    per-query keys are read once."""
    if per_seq:
        return library().cskv_index_topk_per_seq_workspace_size(B, N, k)
    return library().cskv_index_topk_workspace_size(B, N, k)


def index_topk(q_idx, idx_keys, k, q_pos=None, m=4, idx_scale=1.0, per_seq=False, idx_out=None,
               workspace=None, stream=None):
    """Top-k entries per query by indexer score: int32 [B, k], ascending
    indices then -1 padding."""
    _need(q_idx, "q_idx", _IDX_DT, (None, I))
    B = q_idx.shape[0]
    _kv(idx_keys, "idx_keys", per_seq, B, I, q_idx.dtype)
    N = idx_keys.shape[-2]
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(idx_out, "idx_out", torch.int32, (B, k))
    # the per-sequence size (keys read once) is optional: the base size is the minimum
    _need_ws(workspace, index_topk_workspace_size(B, N, k))
    ws = index_topk_workspace_size(B, N, k, per_seq)
    _dev(q_idx, idx_keys, q_pos, idx_out)
    if idx_out is None:
        idx_out = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        workspace = _workspace(ws, q_idx.device)
    _call("cskv_index_topk", _ptr(q_idx), _ptr(idx_keys), B, N, k, N * I if per_seq else 0,
          _ptr(q_pos), m, float(idx_scale), _dt(q_idx), _ptr(idx_out), _ptr(workspace),
          workspace.numel(), _stream(stream))
    return idx_out


def index_topk_noalloc(q_idx, idx_keys, k, q_pos=None, m=4, idx_scale=1.0, per_seq=False,
                       idx_out=None, stream=None):
    """index_topk through the allocation-free entry point: the library's own
    fixed scratch array replaces the workspace (calls on one GPU must not
    overlap).  With idx_out given, nothing is allocated here either."""
    _need(q_idx, "q_idx", _IDX_DT, (None, I))
    B = q_idx.shape[0]
    _kv(idx_keys, "idx_keys", per_seq, B, I, q_idx.dtype)
    N = idx_keys.shape[-2]
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(idx_out, "idx_out", torch.int32, (B, k))
    _dev(q_idx, idx_keys, q_pos, idx_out)
    if idx_out is None:
        idx_out = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    _call("cskv_index_topk_noalloc", _ptr(q_idx), _ptr(idx_keys), B, N, k, N * I if per_seq else 0,
          _ptr(q_pos), m, float(idx_scale), _dt(q_idx), _ptr(idx_out), _stream(stream))
    return idx_out


def index_topk_mxfp4(q_codes, q_scales, key_codes, key_scales, k, q_pos=None, m=4, idx_scale=1.0,
                     per_seq=False, idx_out=None, workspace=None, stream=None):
    """index_topk over MXFP4 rows: codes uint8 [B, 32] / [N, 32] (or
    [B, N, 32] per sequence), E8M0 scales uint8 [B, 2] / [N, 2] (or
    [B, N, 2])."""
    _need(q_codes, "q_codes", torch.uint8, (None, I // 2))
    B = q_codes.shape[0]
    _need(q_scales, "q_scales", torch.uint8, (B, I // 32))
    _kv(key_codes, "key_codes", per_seq, B, I // 2, torch.uint8)
    N = key_codes.shape[-2]
    _need(key_scales, "key_scales", torch.uint8, (B, N, I // 32) if per_seq else (N, I // 32))
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(idx_out, "idx_out", torch.int32, (B, k))
    _need_ws(workspace, index_topk_workspace_size(B, N, k))
    ws = index_topk_workspace_size(B, N, k, per_seq)
    _dev(q_codes, q_scales, key_codes, key_scales, q_pos, idx_out)
    if idx_out is None:
        idx_out = torch.empty((B, k), dtype=torch.int32, device=q_codes.device)
    if workspace is None:
        workspace = _workspace(ws, q_codes.device)
    _call("cskv_index_topk_mxfp4", _ptr(q_codes), _ptr(q_scales), _ptr(key_codes), _ptr(key_scales),
          B, N, k, N if per_seq else 0, _ptr(q_pos), m, float(idx_scale), _ptr(idx_out),
          _ptr(workspace), workspace.numel(), _stream(stream))
    return idx_out


# ---------------------------------------------------------------- attention

def attend_workspace_size(B, H, rows_per_query):
    return library().cskv_attend_workspace_size(B, H, rows_per_query)


def _eps(norm_eps):
    """The ABI's norm_eps: the epsilon of the query / entry normalisation, or
    -1 for none."""
    if norm_eps is None:
        return -1.0
    if not norm_eps >= 0.0:
        raise ValueError("norm_eps must be >= 0 (None: no normalisation)")
    return float(norm_eps)


def sparse_attend(q, entries, window, idx, q_pos=None, win_pos0=0, W=None, scale=1.0,
                  per_seq=False, out=None, lse=None, workspace=None, stream=None, sink=None,
                  norm_eps=None):
    """Attention of q [B, H, 576] over entries[idx] plus the raw window;
    sink: per-head attention-sink logits, fp32 [H] (None: no sink);
    norm_eps: normalise the queries and the selected entries to unit RMS
    with this epsilon (None: no normalisation)."""
    _need(q, "q", _VAL_DT, (None, None, E))
    B, H = q.shape[0], q.shape[1]
    _kv(entries, "entries", per_seq, B, E, q.dtype)
    _kv(window, "window", per_seq, B, E, q.dtype)
    _need(idx, "idx", torch.int32, (B, None))
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(out, "out", q.dtype, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    N = entries.shape[-2]
    k = idx.shape[1]
    win_rows = 0 if window is None else window.shape[-2]
    if W is None:
        W = win_rows
    _need_ws(workspace, attend_workspace_size(B, H, k + W))
    _dev(q, entries, window, idx, q_pos, out, lse)
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(attend_workspace_size(B, H, k + W), q.device)
    _call("cskv_sparse_attend", _ptr(q), _ptr(entries), _ptr(window), _ptr(idx), B, H, N, W, k,
          N * E if per_seq else 0, win_rows * E if per_seq else 0, win_rows, _ptr(q_pos),
          int(win_pos0), float(scale), _sink(sink, H), _eps(norm_eps), _dt(q), _ptr(out), _ptr(lse),
          _ptr(workspace), workspace.numel(), _stream(stream))
    return out, lse


def csa_workspace_size(B, H, N, W, k):
    return library().cskv_csa_workspace_size(B, H, N, W, k)


def csa_attend(q, q_idx, entries, idx_keys, window, k, m=4, q_pos=None, win_pos0=0, W=None,
               scale=1.0, idx_scale=1.0, per_seq=False, out=None, lse=None, idx_out=None,
               workspace=None, stream=None, sink=None, norm_eps=None):
    """CSA: indexer top-k then attention over the selection plus the window
    (sink, norm_eps as in sparse_attend).
    Returns (out [B, H, 512], lse [B, H], idx [B, k])."""
    _need(q, "q", _VAL_DT, (None, None, E))
    B, H = q.shape[0], q.shape[1]
    _need(q_idx, "q_idx", _IDX_DT, (B, I))
    _kv(entries, "entries", per_seq, B, E, q.dtype)
    _kv(idx_keys, "idx_keys", per_seq, B, I, q_idx.dtype)
    _kv(window, "window", per_seq, B, E, q.dtype)
    N = entries.shape[-2]
    if idx_keys.shape[-2] != N:
        raise ValueError(f"idx_keys: {idx_keys.shape[-2]} rows for {N} entries")
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(out, "out", q.dtype, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    _need(idx_out, "idx_out", torch.int32, (B, k))
    win_rows = 0 if window is None else window.shape[-2]
    if W is None:
        W = win_rows
    _need_ws(workspace, csa_workspace_size(B, H, N, W, k))
    _dev(q, q_idx, entries, idx_keys, window, q_pos, out, lse, idx_out)
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = _workspace(csa_workspace_size(B, H, N, W, k), q.device)
    _call("cskv_csa_attend", _ptr(q), _ptr(q_idx), _ptr(entries), _ptr(idx_keys), _ptr(window),
          B, H, N, W, k, m, N * E if per_seq else 0, N * I if per_seq else 0,
          win_rows * E if per_seq else 0, win_rows, _ptr(q_pos), int(win_pos0), float(scale),
          _sink(sink, H), _eps(norm_eps), float(idx_scale), _dt(q), _dt(q_idx), _ptr(out), _ptr(lse),
          _ptr(idx_out),
          _ptr(workspace), workspace.numel(), _stream(stream))
    return out, lse, idx_out


def hca_workspace_size(B, H, N):
    return library().cskv_hca_workspace_size(B, H, N)


def hca_attend(q, entries, scale=1.0, per_seq=False, q_pos=None, m=None, out=None, lse=None,
               workspace=None, stream=None, sink=None, norm_eps=None):
    """HCA: dense attention of q [B, H, 576] over the entries [N, 576] each
    query sees: all of them (q_pos None), or at a prefill chunk those with
    (i+1)*m <= q_pos[b] + 1 (q_pos [B] int64 on the device)."""
    if q_pos is not None and m is None:
        raise ValueError("hca_attend: q_pos needs the block size m")
    _need(q, "q", _VAL_DT, (None, None, E))
    B, H = q.shape[0], q.shape[1]
    _kv(entries, "entries", per_seq, B, E, q.dtype)
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(out, "out", q.dtype, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    N = entries.shape[-2]
    _need_ws(workspace, hca_workspace_size(B, H, N))
    _dev(q, entries, q_pos, out, lse)
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(hca_workspace_size(B, H, N), q.device)
    _call("cskv_hca_attend", _ptr(q), _ptr(entries), B, H, N, N * E if per_seq else 0,
          _ptr(q_pos), int(m) if q_pos is not None else 0, float(scale), _sink(sink, H),
          _eps(norm_eps), _dt(q), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
          _stream(stream))
    return out, lse


def _mx_entries(codes, scales, per_seq, B, bits=4):
    """MX entry rows: codes uint8 [N, 288] (MXFP4) or [N, 576] (MXFP8) and
    scales uint8 [N, 18], with a leading batch dimension per sequence.
    Returns N."""
    _kv(codes, "ent_codes", per_seq, B, E * bits // 8, torch.uint8)
    N = codes.shape[-2]
    _need(scales, "ent_scales", torch.uint8, (B, N, E // 32) if per_seq else (N, E // 32))
    return N


def _sparse_attend_mx(bits, q, ent_codes, ent_scales, window, idx, q_pos=None, win_pos0=0, W=None,
                      scale=1.0, per_seq=False, out=None, lse=None, workspace=None, stream=None,
                      sink=None, norm_eps=None):
    """sparse_attend over MXFP4 entries: codes uint8 [N, 288] and E8M0
    scales uint8 [N, 18] (with a leading batch dimension per sequence); q,
    window and out are bf16."""
    _need(q, "q", torch.bfloat16, (None, None, E))
    B, H = q.shape[0], q.shape[1]
    N = _mx_entries(ent_codes, ent_scales, per_seq, B, bits)
    _kv(window, "window", per_seq, B, E, torch.bfloat16)
    _need(idx, "idx", torch.int32, (B, None))
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(out, "out", torch.bfloat16, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    k = idx.shape[1]
    win_rows = 0 if window is None else window.shape[-2]
    if W is None:
        W = win_rows
    need = library().cskv_sparse_attend_mxfp4_workspace_size(B, H, W, k)
    _need_ws(workspace, need)
    _dev(q, ent_codes, ent_scales, window, idx, q_pos, out, lse)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _call(f"cskv_sparse_attend_mxfp{bits}", _ptr(q), _ptr(ent_codes), _ptr(ent_scales), _ptr(window),
          _ptr(idx), B, H, N, W, k, N if per_seq else 0, win_rows * E if per_seq else 0, win_rows,
          _ptr(q_pos), int(win_pos0), float(scale), _sink(sink, H), _eps(norm_eps), _ptr(out),
          _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
    return out, lse


def _hca_attend_mx(bits, q, ent_codes, ent_scales, scale=1.0, per_seq=False, q_pos=None, m=None,
                   out=None, lse=None, workspace=None, stream=None, sink=None, norm_eps=None):
    """hca_attend over MXFP4 entries (codes [N, 288], scales [N, 18])."""
    if q_pos is not None and m is None:
        raise ValueError("hca_attend_mx: q_pos needs the block size m")
    _need(q, "q", torch.bfloat16, (None, None, E))
    B, H = q.shape[0], q.shape[1]
    N = _mx_entries(ent_codes, ent_scales, per_seq, B, bits)
    _need(q_pos, "q_pos", torch.int64, (B,))
    _need(out, "out", torch.bfloat16, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    need = library().cskv_hca_attend_mxfp4_workspace_size(B, H, N, int(per_seq))
    _need_ws(workspace, need)
    _dev(q, ent_codes, ent_scales, q_pos, out, lse)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _call(f"cskv_hca_attend_mxfp{bits}", _ptr(q), _ptr(ent_codes), _ptr(ent_scales), B, H, N,
          N if per_seq else 0, _ptr(q_pos), int(m) if q_pos is not None else 0, float(scale),
          _sink(sink, H), _eps(norm_eps), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
          _stream(stream))
    return out, lse


def sparse_attend_mxfp4(q, ent_codes, ent_scales, window, idx, **kw):
    """sparse_attend over MXFP4 entries: codes uint8 [N, 288] and E8M0
    scales uint8 [N, 18] (with a leading batch dimension per sequence); q,
    window and out are bf16; other arguments as sparse_attend."""
    return _sparse_attend_mx(4, q, ent_codes, ent_scales, window, idx, **kw)


def hca_attend_mxfp4(q, ent_codes, ent_scales, **kw):
    """hca_attend over MXFP4 entries (codes [N, 288], scales [N, 18])."""
    return _hca_attend_mx(4, q, ent_codes, ent_scales, **kw)


def sparse_attend_mxfp8(q, ent_codes, ent_scales, window, idx, **kw):
    """sparse_attend over MXFP8 entries: E4M3 codes uint8 [N, 576] and E8M0
    scales uint8 [N, 18] (with a leading batch dimension per sequence)."""
    return _sparse_attend_mx(8, q, ent_codes, ent_scales, window, idx, **kw)


def hca_attend_mxfp8(q, ent_codes, ent_scales, **kw):
    """hca_attend over MXFP8 entries (codes [N, 576], scales [N, 18])."""
    return _hca_attend_mx(8, q, ent_codes, ent_scales, **kw)


def merge(o_part, lse_part, dtype=torch.bfloat16, out=None, lse=None, stream=None, sink=None):
    """Merge split partials o_part [B, H, S, 512] fp32, lse_part [B, H, S]."""
    _need(lse_part, "lse_part", torch.float32, (None, None, None))
    B, H, S = lse_part.shape
    _need(o_part, "o_part", torch.float32, (B, H, S, D))
    if dtype not in _VAL_DT:
        raise ValueError(f"merge: output dtype {dtype}, expected float32 or bfloat16")
    _need(out, "out", dtype, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    _dev(o_part, lse_part, out, lse)
    if out is None:
        out = torch.empty((B, H, D), dtype=dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=o_part.device)
    _call("cskv_merge", _ptr(o_part), _ptr(lse_part), B, H, S, _sink(sink, H), _ptr(out),
          _ptr(lse), _dt(out), _stream(stream))
    return out, lse
