"""Lightning-indexer scores, float64 (oracle; test infrastructure).

Definition (the formula of DeepSeek Sparse Attention's lightning indexer; on the
vLLM API page "vllm.models.kimi_k3.nvidia.dsa", ``KimiK3DSAIndexer.forward`` and
``score`` build its operands: per-head queries [T, H, D], ONE shared key per
token [T, D] and per-head weights [T, H], then call the scoring op):

    score[t, s] = k_scale[s] * sum_h w[t, h] * max(0, sum_d q[t, h, d] * k[s, d])

for every key s in the row's half-open window [row_starts[t], row_ends[t]).
``k_scale`` is 1 unless the keys are e4m3 codes with power-of-two scales; the
query scale is already folded into ``w`` (``score``: "folded into the weights").

Also returned on request: the conditioning scale
    c[t, s] = k_scale[s] * sum_h |w[t, h]| * sum_d |q[t, h, d] * k[s, d]|
used by the tests to state a relative tolerance that stays meaningful where the
head sum cancels.
"""
from __future__ import annotations

import numpy as np


def score_row(q_t, k_win, w_t, k_scale_win=None, with_cond: bool = False):
    """Scores of one query row against the keys of its window.

    q_t [H, D], k_win [n, D], w_t [H], k_scale_win [n] or None."""
    q_t = np.asarray(q_t, np.float64)
    k_win = np.asarray(k_win, np.float64)
    w_t = np.asarray(w_t, np.float64)
    logits = q_t @ k_win.T                               # [H, n]
    s = w_t @ np.maximum(logits, 0.0)                     # [n]
    if k_scale_win is not None:
        s = s * np.asarray(k_scale_win, np.float64)
    if not with_cond:
        return s
    c = np.abs(w_t) @ (np.abs(q_t) @ np.abs(k_win).T)    # [n]
    if k_scale_win is not None:
        c = c * np.asarray(k_scale_win, np.float64)
    return s, c


def scores_dense(q, k, w, row_starts, row_ends, k_scale=None, with_cond: bool = False,
                 fill=np.nan):
    """[Nq, Nk] float64 scores; entries outside each row's window are ``fill``."""
    nq, nk = q.shape[0], k.shape[0]
    S = np.full((nq, nk), fill, np.float64)
    C = np.full((nq, nk), fill, np.float64) if with_cond else None
    for t in range(nq):
        a, b = int(row_starts[t]), int(row_ends[t])
        if b <= a:
            continue
        ks = None if k_scale is None else k_scale[a:b]
        r = score_row(q[t], k[a:b], w[t], ks, with_cond)
        if with_cond:
            S[t, a:b], C[t, a:b] = r
        else:
            S[t, a:b] = r
    return (S, C) if with_cond else S


def scores_loops(q, k, w, row_starts, row_ends, k_scale=None):
    """The same definition as plain Python loops (small inputs only); an
    independent formulation the vectorised one is checked against."""
    nq, H, D = len(q), len(q[0]), len(q[0][0])
    out = {}
    for t in range(nq):
        for s in range(int(row_starts[t]), int(row_ends[t])):
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += float(q[t][h][d]) * float(k[s][d])
                if dot > 0.0:
                    tot += float(w[t][h]) * dot
            if k_scale is not None:
                tot *= float(k_scale[s])
            out[(t, s)] = tot
    return out
