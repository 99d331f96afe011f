"""Pins for oracle.topk: the pages' semantics as hand-worked fixtures, pure-Python
brute force on tie-heavy rows, invariants, and set equality with torch.topk on
rows without ties."""
import os

import numpy as np
import torch

from oracle import topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    return float(x.replace("inf", "Infinity")) if "inf" in x else float(x)


def test_semantics_fixture():
    n = 0
    for line in open(os.path.join(GOLD, "topk_semantics.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        head, vals, exp = (p.split() for p in line.split("|"))
        k, a, b = map(int, head)
        row = np.array([_f(v) for v in vals], np.float32)
        got = topk.topk_row(row, a, b, k)
        assert got.tolist() == [int(e) for e in exp], line
        assert topk.topk_bruteforce_row(row, a, b, k) == [int(e) for e in exp], line
        n += 1
    assert n >= 10


def test_bruteforce_tie_heavy():
    g = np.random.default_rng(21)
    pool = np.array([-np.inf, -2.0, -0.0, 0.0, 1.0, 1.0, 3.0, np.inf], np.float32)
    for _ in range(300):
        n = int(g.integers(0, 40))
        row = pool[g.integers(0, len(pool), n)]
        a = int(g.integers(0, n + 1)); b = int(g.integers(a, n + 1))
        k = int(g.integers(1, 12))
        assert topk.topk_row(row, a, b, k).tolist() == topk.topk_bruteforce_row(row, a, b, k)


def _check_invariants(row, a, b, k, out):
    sel = out[out >= 0]
    n_sel = int(np.sum(np.asarray(row[a:b]) > -np.inf))
    assert sel.size == min(k, n_sel)
    assert np.all(out[sel.size:] == -1)
    assert np.all(np.diff(sel) > 0)                          # unique, ascending
    assert np.all((sel >= a) & (sel < b))
    if sel.size and sel.size < n_sel:
        chosen = set(sel.tolist())
        rest = [s for s in range(a, b) if s not in chosen and row[s] > -np.inf]
        vmin = min(row[s] for s in sel)
        vmax = max(row[s] for s in rest)
        assert vmin >= vmax
        if vmin == vmax:                                     # ties go to lower index
            assert max(s for s in sel if row[s] == vmin) < min(s for s in rest if row[s] == vmax)


def test_invariants_random():
    g = np.random.default_rng(22)
    for _ in range(100):
        n = int(g.integers(1, 500))
        row = g.standard_normal(n).astype(np.float32)
        if g.random() < 0.5:
            row = np.round(row * 2).astype(np.float32)       # many ties
        a = int(g.integers(0, n)); b = int(g.integers(a, n + 1))
        k = int(g.integers(1, 64))
        _check_invariants(row, a, b, k, topk.topk_row(row, a, b, k))


def test_matches_torch_topk_without_ties():
    g = np.random.default_rng(23)
    n, k = 1000, 100
    S = g.standard_normal((20, n)).astype(np.float32)
    rs = g.integers(0, 400, 20); re = rs + g.integers(150, 600, 20)
    out = topk.topk(S, rs, re, k)
    for t in range(20):
        m = torch.full((n,), float("-inf"))
        m[rs[t]:re[t]] = torch.from_numpy(S[t, rs[t]:re[t]])
        _, ti = torch.topk(m, k)
        assert set(ti.tolist()) == set(out[t].tolist())


def test_window_masks_garbage_and_padding():
    # +-1e4 garbage outside the window is never chosen; short windows pad with -1
    g = np.random.default_rng(24)
    row = np.where(g.random(300) < 0.5, 1e4, -1e4).astype(np.float32)
    row[100:110] = g.standard_normal(10).astype(np.float32)
    out = topk.topk_row(row, 100, 110, 16)
    assert out[:10].tolist() == list(range(100, 110))
    assert np.all(out[10:] == -1)
