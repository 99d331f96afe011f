"""Per-row top-k selection (oracle; test infrastructure).

Follows the fallback top-k shown in review comment 3 of vime pull request #502
(``torch_dsa_topk`` after the suggested change): columns outside the row's
half-open window [row_starts, row_ends) are masked to -inf; k = min(topk, number
of columns); a selected -inf becomes -1; the row is padded with -1 up to topk.

Readings where the page leaves the result open (listed in the design notes):
* ties are broken by the lowest column index;
* -inf is never selected, +inf is; NaN in a window is a precondition violation;
  -0.0 and +0.0 compare equal;
* the selected columns are returned in ascending column order, followed by the
  -1 padding (the page returns score order; attention uses the row as a set).

This runs on the float32 score array exactly as handed to the kernel under test:
rounding fp64 scores to fp32 can create ties that the fp64 values do not have.
"""
from __future__ import annotations

import numpy as np


def topk_row(row_vals, start: int, end: int, k: int) -> np.ndarray:
    """Top-k columns of one row.  ``row_vals`` is indexable by global column."""
    out = np.full(k, -1, np.int32)
    if end <= start:
        return out
    cols = np.arange(start, end, dtype=np.int64)
    vals = np.asarray(row_vals[start:end], np.float64)
    if np.isnan(vals).any():
        raise ValueError("NaN score inside a window")
    keep = vals > -np.inf
    cols, vals = cols[keep], vals[keep]
    # order by score descending, then column ascending
    order = np.lexsort((cols, -vals))
    chosen = np.sort(cols[order[:k]])
    out[:chosen.size] = chosen
    return out


def topk(scores, row_starts, row_ends, k: int) -> np.ndarray:
    """[Nq, k] int32 for a dense [Nq, >=max(row_ends)] float32 score array."""
    nq = len(row_starts)
    out = np.empty((nq, k), np.int32)
    for t in range(nq):
        out[t] = topk_row(scores[t], int(row_starts[t]), int(row_ends[t]), k)
    return out


def topk_bruteforce_row(row_vals, start: int, end: int, k: int) -> list[int]:
    """Pure-Python selection for tiny rows: repeatedly take the best remaining
    (largest score, then smallest column) among finite-or-+inf candidates."""
    cand = [(float(row_vals[s]), s) for s in range(start, end) if float(row_vals[s]) > float("-inf")]
    picked = []
    for _ in range(min(k, len(cand))):
        best = None
        for v, s in cand:
            if s in picked:
                continue
            if best is None or v > best[0] or (v == best[0] and s < best[1]):
                best = (v, s)
        picked.append(best[1])
    return sorted(picked) + [-1] * (k - len(picked))
