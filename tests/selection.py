"""Check of a GPU top-k selection against the oracle's fp64 scores.

Where adjacent scores differ by less than 1e-3 relative several selections
are correct: the check takes the oracle's k-th score tau and accepts any set
of the right size whose members all score >= tau - 1e-3|tau| while every
visible non-member scores <= tau + 1e-3|tau|."""
import numpy as np


def check_selection(gpu_idx, scores, visible, k, rel=1e-3):
    gpu_idx = np.asarray(gpu_idx)
    B = scores.shape[0]
    exact = 0
    for b in range(B):
        vis = np.nonzero(visible[b])[0]
        n = min(k, len(vis))
        row = gpu_idx[b]
        sel = row[:n]
        assert (row[n:] == -1).all(), f"query {b}: padding"
        assert (sel >= 0).all() and len(np.unique(sel)) == n, f"query {b}: not {n} distinct entries"
        assert (np.diff(sel) > 0).all(), f"query {b}: not ascending"
        assert visible[b, sel].all(), f"query {b}: invisible entry selected"
        if n == len(vis):
            exact += 1
            continue
        s = scores[b]
        order = np.lexsort((vis, -s[vis]))
        ref = vis[order[:n]]
        tau = s[ref[-1]]
        band = rel * abs(tau)
        assert (s[sel] >= tau - band).all(), f"query {b}: member below the band"
        rest = np.setdiff1d(vis, sel, assume_unique=True)
        assert (s[rest] <= tau + band).all(), f"query {b}: non-member above the band"
        exact += int(np.array_equal(np.sort(ref), sel))
    return exact
