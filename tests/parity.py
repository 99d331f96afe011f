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
           |lse_g - lse_o| <= 1e-3 (+ bf16 input rounding of the logits);
           fp32: max|g - o| <= 1e-3.
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


def check_mla(g_out, o_out, g_lse, o_lse, bf16: bool, what=""):
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
        g_lse = np.asarray(g_lse, np.float64)
        fin = np.isfinite(o_lse)
        assert np.array_equal(np.isfinite(g_lse), fin), f"{what}: lse finiteness differs"
        lerr = np.abs(g_lse[fin] - o_lse[fin])
        assert lerr.max(initial=0) <= 1e-3 + 2e-3 * np.abs(o_lse[fin]).max(initial=0), \
            f"{what}: lse err {lerr.max()}"
    return float(err.max())
