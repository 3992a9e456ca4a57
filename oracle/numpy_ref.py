"""Second formulation of the oracle in NumPy (TEST INFRASTRUCTURE ONLY).

Written from the same page passages as `cskv_oracle.c` but with library
primitives instead of loops: a sliding-window view and a softmax along the
window axis for compression, a matrix product for indexer scores, a
lexicographic sort for selection and a matrix-form softmax attention.  It is
used only to cross-check the C oracle; neither side calls the other.
"""
import numpy as np
from numpy.lib.stride_tricks import sliding_window_view


def compress(xv, zv, bias, m):
    """xv, zv: float64 [T, D] decoded values; bias float [2m, D].
    Windows of 2m tokens with stride m; entry i covers tokens [(i-1)m, (i+1)m).
    Absent tokens (before 0) are given weight 0 by a -inf logit."""
    T, Dd = xv.shape
    N = T // m
    pad = np.full((m, Dd), -np.inf)
    zp = np.concatenate([pad, zv[: N * m]], axis=0)              # [m + N*m, D]
    xp = np.concatenate([np.zeros((m, Dd)), xv[: N * m]], axis=0)
    zw = sliding_window_view(zp, 2 * m, axis=0)[::m]              # [N, D, 2m]
    xw = sliding_window_view(xp, 2 * m, axis=0)[::m]
    logits = zw + np.asarray(bias, dtype=np.float64).T[None, :, :]
    logits = logits - logits.max(axis=2, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=2, keepdims=True)
    return (w * xw).sum(axis=2)


def index_scores(qv, kv, scale=1.0):
    return scale * (qv @ kv.T)


def topk(scores, visible, k):
    B, N = scores.shape
    out = np.full((B, k), -1, dtype=np.int64)
    for b in range(B):
        ids = np.nonzero(visible[b])[0]
        order = np.lexsort((ids, -scores[b, ids]))                # score desc, then index asc
        sel = ids[order][:k]
        out[b, : len(sel)] = sel
    return out


def attend(qv, rows, Dv=512, scale=1.0, sink=None):
    """qv [H, E], rows [n, E] -> (out [H, Dv], lse [H]).  sink [H]: one more
    softmax column per head with that logit and a zero value."""
    logits = scale * (qv @ rows.T)
    values = rows[:, :Dv]
    if sink is not None:
        logits = np.concatenate([logits, np.asarray(sink, dtype=np.float64)[:, None]], axis=1)
        values = np.concatenate([values, np.zeros((1, Dv))], axis=0)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p / den) @ values, (mx + np.log(den))[:, 0]


def rms_normalize(x, eps):
    """x / sqrt(mean(x^2) + eps) along the last axis (unit root-mean-square)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
