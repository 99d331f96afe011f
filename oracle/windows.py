"""Row windows over packed (THD) sequences and the packed-offset rebase
(oracle; test infrastructure).

Windows: the fallback top-k in review comment 3 of vime pull request #502 keeps
column c of a row when row_starts <= c < row_ends (half-open).  Readings (listed
in the design notes): indices are global positions in the packed key buffer;
in causal mode the query at local position p of a sequence with q_len queries
and k_len keys sees keys [cu_k[b], cu_k[b] + k_len - q_len + p + 1), i.e. every
key up to and including its own position; otherwise it sees the whole sequence.

Rebase: review comment 1 of the same pull request adds a sample's packed offset
to every index that is not -1 and advances the offset by the sample's full
token length, so per-sample results line up with the packed key buffer.
"""
from __future__ import annotations

import numpy as np


def row_windows(cu_q, cu_k, causal: bool = True):
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    n = int(cu_q[-1])
    starts = np.empty(n, np.int32)
    ends = np.empty(n, np.int32)
    for b in range(len(cu_q) - 1):
        q_len = int(cu_q[b + 1] - cu_q[b])
        k_len = int(cu_k[b + 1] - cu_k[b])
        for p in range(q_len):
            t = int(cu_q[b]) + p
            starts[t] = cu_k[b]
            if causal:
                e = int(cu_k[b]) + k_len - q_len + p + 1
                ends[t] = max(int(cu_k[b]), min(e, int(cu_k[b + 1])))
            else:
                ends[t] = cu_k[b + 1]
    return starts, ends


def rebase(local_idx, offset: int) -> np.ndarray:
    """Add ``offset`` to every entry that is not -1."""
    local_idx = np.asarray(local_idx)
    return np.where(local_idx != -1, local_idx + offset, local_idx).astype(local_idx.dtype)


def rebase_packed(per_sample, token_lens):
    """Concatenate per-sample index rows, each rebased by the running offset,
    which advances by the sample's full token length."""
    out, offset = [], 0
    for local, n in zip(per_sample, token_lens):
        out.append(rebase(local, offset))
        offset += int(n)
    return np.concatenate(out, axis=0)
