"""Pins for oracle.indexer: hand-computed fixture, an independent loop
formulation, and closed-form special cases."""
import os

import numpy as np

from oracle import indexer, windows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load_hand():
    q = np.zeros((2, 2, 2)); k = np.zeros((2, 2)); w = np.zeros((2, 2)); exp = {}
    for line in open(os.path.join(GOLD, "indexer_hand.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "q":
            q[int(f[1]), int(f[2])] = [float(f[3]), float(f[4])]
        elif f[0] == "k":
            k[int(f[1])] = [float(f[2]), float(f[3])]
        elif f[0] == "w":
            w[int(f[1])] = [float(f[2]), float(f[3])]
        elif f[0] == "score":
            exp[(int(f[1]), int(f[2]))] = float(f[3])
    return q, k, w, exp


def test_hand_fixture():
    q, k, w, exp = _load_hand()
    rs, re = np.array([0, 0]), np.array([1, 2])
    S = indexer.scores_dense(q, k, w, rs, re)
    for (t, s), v in exp.items():
        assert S[t, s] == v
    assert np.isnan(S[0, 1])                   # outside the causal window
    loops = indexer.scores_loops(q, k, w, rs, re)
    assert loops == exp


def test_vectorised_vs_loops_tiny():
    g = np.random.default_rng(11)
    T, H, D = 24, 4, 32
    q = g.standard_normal((T, H, D)); k = g.standard_normal((T, D)); w = g.standard_normal((T, H))
    rs, re = windows.row_windows([0, T], [0, T], causal=True)
    S = indexer.scores_dense(q, k, w, rs, re)
    L = indexer.scores_loops(q, k, w, rs, re)
    assert len(L) == T * (T + 1) // 2
    for (t, s), v in L.items():
        np.testing.assert_allclose(S[t, s], v, rtol=1e-12, atol=1e-12)


def test_special_cases():
    g = np.random.default_rng(12)
    D = 16
    kk = g.standard_normal((1, D))
    # H=1, w=1, q=k: the score is |k|^2
    s = indexer.score_row(kk, kk, np.ones(1))
    np.testing.assert_allclose(s[0], kk[0] @ kk[0], rtol=1e-14)
    # q = -k: relu kills it
    assert indexer.score_row(-kk, kk, np.ones(1))[0] == 0.0
    # linear in w (including negative w)
    q = g.standard_normal((5, D)); k = g.standard_normal((7, D)); w = g.standard_normal(5)
    np.testing.assert_allclose(indexer.score_row(q, k, 3 * w), 3 * indexer.score_row(q, k, w), rtol=1e-12)
    np.testing.assert_allclose(indexer.score_row(q, k, -w), -indexer.score_row(q, k, w), rtol=1e-12)
    # heads add up
    w2 = g.standard_normal(5)
    np.testing.assert_allclose(indexer.score_row(q, k, w + w2),
                               indexer.score_row(q, k, w) + indexer.score_row(q, k, w2), rtol=1e-10, atol=1e-12)
    # key scale multiplies the score
    ks = 2.0 ** g.integers(-4, 4, 7)
    np.testing.assert_allclose(indexer.score_row(q, k, w, ks), ks * indexer.score_row(q, k, w), rtol=1e-14)


def test_conditioning_bounds_score():
    g = np.random.default_rng(13)
    q = g.standard_normal((6, 8)); k = g.standard_normal((9, 8)); w = g.standard_normal(6)
    s, c = indexer.score_row(q, k, w, with_cond=True)
    assert np.all(np.abs(s) <= c + 1e-12)
