"""Sparse MLA attention over the selected latent rows, float64 (oracle; test
infrastructure).

On the vLLM API page "vllm.models.kimi_k3.nvidia.dsa" (module docstring and
``KimiK3DSAAttention``) the MLA layers run with ``is_sparse=True`` so that the
sparse attention backend consumes the indexer's top-k indices: each query token
attends only to the latent KV rows its top-k row names.  In the absorbed MLA
form all heads share one latent row per key; the row holds the kv_lora_rank
latent dims followed by the rope dims.

Definition, per query row t and head h, with J_t = the entries of idx[t] that
are not -1, in list order:

    l_j   = sm_scale * sum_{d < d_qk} q[t, h, d] * kv[J_t[j], d]
    out   = sum_j exp(l_j - m) kv[J_t[j], :d_v] / sum_j exp(l_j - m),  m = max_j l_j
    lse   = m + log sum_j exp(l_j - m)

Readings (listed in the design notes): V is the first d_v dims of the same
latent row; an empty J_t gives out = 0 and lse = -inf; duplicate indices count
as often as they are listed; sm_scale is a runtime argument (the page's model
uses (qk_nope + qk_rope)^-0.5, times a YaRN factor when rope scaling is on).
"""
from __future__ import annotations

import numpy as np


def attend_row(q_t, kv, idx_t, sm_scale: float, d_v: int):
    """q_t [H, d_qk], kv [N, d_qk], idx_t [K] -> (out [H, d_v], lse [H])."""
    q_t = np.asarray(q_t, np.float64)
    H = q_t.shape[0]
    J = np.asarray(idx_t, np.int64)
    J = J[J != -1]
    if J.size == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    rows = np.asarray(kv[J], np.float64)                 # [n, d_qk]
    logits = sm_scale * (q_t @ rows.T)                   # [H, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    den = p.sum(axis=1, keepdims=True)
    out = (p @ rows[:, :d_v]) / den
    lse = m[:, 0] + np.log(den[:, 0])
    return out, lse


def sparse_mla(q, kv, idx, sm_scale: float, d_v: int, rows=None):
    """All (or the listed) query rows. Returns out [R, H, d_v], lse [R, H]."""
    rows = range(q.shape[0]) if rows is None else rows
    outs, lses = [], []
    for t in rows:
        o, l = attend_row(q[t], kv, idx[t], sm_scale, d_v)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
