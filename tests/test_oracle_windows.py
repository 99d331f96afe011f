"""Pins for oracle.windows: hand cases, the pages' rebase example, and the
packed-versus-per-sample identity (the rebase rule applied to the indexer and
top-k oracles end to end)."""
import os

import numpy as np

import synth
from oracle import indexer, topk, windows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_windows_hand():
    rs, re = windows.row_windows([0, 3, 5], [0, 3, 5], causal=True)
    assert rs.tolist() == [0, 0, 0, 3, 3]
    assert re.tolist() == [1, 2, 3, 4, 5]
    rs, re = windows.row_windows([0, 3, 5], [0, 3, 5], causal=False)
    assert re.tolist() == [3, 3, 3, 5, 5]
    # decode: one query per sequence sees its whole cache
    rs, re = windows.row_windows([0, 1, 2], [0, 7, 12], causal=True)
    assert rs.tolist() == [0, 7] and re.tolist() == [7, 12]


def test_rebase_fixture():
    samples, lens, expect = [], [], None
    for line in open(os.path.join(GOLD, "rebase_hand.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        parts = line.split("|")
        head = parts[0].split()
        rows = np.array([[int(v) for v in p.split()] for p in parts[1:]], np.int32)
        if head[0] == "sample":
            lens.append(int(head[1])); samples.append(rows)
        else:
            expect = rows
    got = windows.rebase_packed(samples, lens)
    np.testing.assert_array_equal(got, expect)
    # advancing by the local slice instead of token_len would give a different answer
    wrong = windows.rebase_packed(samples, [len(s) for s in samples])
    assert not np.array_equal(wrong, expect)


def test_packed_equals_per_sample_rebased():
    g = np.random.default_rng(41)
    lens = [5, 13, 1, 9]
    lay = synth.layout_from_lengths(lens)
    H, D, K = 3, 8, 4
    N = lay.n_k
    q = g.standard_normal((N, H, D)); k = g.standard_normal((N, D)); w = g.random((N, H))
    rs, re = windows.row_windows(lay.cu_q, lay.cu_k)
    S = indexer.scores_dense(q, k, w, rs, re, fill=np.nan).astype(np.float32)
    packed = topk.topk(S, rs, re, K)
    per = []
    cu = lay.cu_k
    for b in range(len(lens)):
        a, e = cu[b], cu[b + 1]
        lrs, lre = windows.row_windows([0, e - a], [0, e - a])
        Sl = indexer.scores_dense(q[a:e], k[a:e], w[a:e], lrs, lre).astype(np.float32)
        per.append(topk.topk(Sl, lrs, lre, K))
    np.testing.assert_array_equal(windows.rebase_packed(per, lens), packed)
