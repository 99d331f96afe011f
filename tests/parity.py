"""Shared helpers of the GPU parity tests: device transfer of oracle arrays and
the tolerance checks (scores, end-to-end indices, attention outputs).

Tolerances (floating point):
  scores   |g - o| <= rtol * max(|o|, c/128), c = sum_h |w| sum_d |q k|; rtol 1e-3
           for fp32 inputs, 2e-2 for bf16 / fp8 inputs.  The c/128 floor only
           matters where the head sum cancels.
  indices  top-k on identical fp32 scores is bit-exact; end to end, the two
           selections may differ only in columns whose score is within
           tau(s) + tau(kth) of the k-th score, with the same number of -1.
  MLA      bf16: max|g - o| <= 2e-2 and, per row, <= 2e-2 * max|o[t]|;
           fp32: max|g - o| <= 1e-3.
           lse, per (row, head), a bound derived from the kernel's arithmetic
           (mla_lse_tol): the probabilities enter the row sum rounded to the
           input type (bf16: relative 2^-8 each, so at most 2^-8 in the log of
           their sum; fp32: 2^-24), each logit carries the fp32 accumulation
           error of its d_qk products (at most d_qk * 2^-24 * sum_d |q_d kv_d|,
           times sm_scale), and the lse itself is an fp32 value (a few ulp of
           |lse|).  No term scales with the largest lse of the batch.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.float32):
    """numpy (values exactly representable in dtype) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype in (torch.bfloat16, torch.float8_e4m3fn):
        t = t.to(torch.float32).to(dtype)
    else:
        t = t.to(dtype)
    return t.cuda()


def host(t) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
        t = t.float()
    return t.cpu().numpy()


def i32(x):
    return dev(np.asarray(x, np.int32), torch.int32)


def check_scores(g_row, o_row, c_row, rtol, what=""):
    g_row = np.asarray(g_row, np.float64)
    bound = rtol * np.maximum(np.abs(o_row), c_row / 128.0)
    err = np.abs(g_row - o_row)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} scores out of tolerance; worst col {i}: "
                             f"gpu {g_row[i]!r} oracle {o_row[i]!r} bound {bound[i]!r}")
    return float((err / np.maximum(np.abs(o_row), 1e-30)).max()) if err.size else 0.0


def check_topk_e2e(g, o, o_scores, tau, what=""):
    """g, o: index rows (int); o_scores/tau: dicts or arrays indexable by column."""
    g = np.asarray(g)
    o = np.asarray(o)
    assert (g == -1).sum() == (o == -1).sum(), f"{what}: different -1 counts"
    gs, os_ = set(g[g >= 0].tolist()), set(o[o >= 0].tolist())
    diff = gs ^ os_
    if not diff:
        return 0
    kth = min(os_, key=lambda s: (o_scores[s], -s))
    for s in diff:
        if abs(o_scores[s] - o_scores[kth]) > tau[s] + tau[kth]:
            raise AssertionError(f"{what}: column {s} (score {o_scores[s]}) differs, k-th score "
                                 f"{o_scores[kth]}, tolerance {tau[s] + tau[kth]}")
    return len(diff)


def mla_lse_tol(q, kv, idx, sm_scale: float, bf16: bool, o_lse):
    """Per (row, head) lse bound for the rows of q / idx (see the module text).

    q [R, H, d_qk] and kv [N, d_qk] hold the exact operand values (float64),
    idx [R, K] the selection (-1 skipped), o_lse [R, H] the oracle's lse."""
    q = np.asarray(q, np.float64)
    kv = np.asarray(kv, np.float64)
    R, H, d_qk = q.shape
    cond = np.zeros((R, H))
    for t in range(R):
        J = np.asarray(idx[t])
        J = J[(J >= 0) & (J < kv.shape[0])]
        if J.size:
            cond[t] = (np.abs(q[t]) @ np.abs(kv[J]).T).max(axis=1)
    u_p = 2.0 ** -8 if bf16 else 2.0 ** -24
    lse_abs = np.where(np.isfinite(o_lse), np.abs(o_lse), 0.0)
    return u_p + 4 * 2.0 ** -24 * lse_abs + sm_scale * d_qk * 2.0 ** -24 * cond


def check_mla(g_out, o_out, g_lse, o_lse, bf16: bool, what="", lse_tol=None):
    g_out = np.asarray(g_out, np.float64)
    err = np.abs(g_out - o_out)
    if bf16:
        assert err.max() <= 2e-2, f"{what}: max abs err {err.max()}"
        for t in range(o_out.shape[0]):
            scale = np.abs(o_out[t]).max()
            assert err[t].max() <= 2e-2 * scale + 1e-6, \
                f"{what}: row {t} err {err[t].max()} vs row max {scale}"
    else:
        assert err.max() <= 1e-3, f"{what}: max abs err {err.max()}"
    if g_lse is not None:
        assert lse_tol is not None, f"{what}: an lse check needs its bound (mla_lse_tol)"
        g_lse = np.asarray(g_lse, np.float64)
        fin = np.isfinite(o_lse)
        assert np.array_equal(np.isfinite(g_lse), fin), f"{what}: lse finiteness differs"
        lerr = np.abs(g_lse - np.where(fin, o_lse, 0.0))[fin]
        tol = np.broadcast_to(lse_tol, o_lse.shape)[fin]
        bad = lerr > tol
        assert not bad.any(), (f"{what}: {int(bad.sum())} lse out of bound; worst err "
                               f"{lerr.max()} (bound there {tol[np.argmax(lerr - tol)]})")
        say(f"  {what}: lse max err {lerr.max(initial=0):.2e} "
            f"(max |lse| {np.abs(o_lse[fin]).max(initial=0):.1f})")
    return float(err.max())
