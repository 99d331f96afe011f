"""GPU parity of every entry point against the CPU oracle, on small and medium
seeded inputs that span several tiles and ragged tails, plus the edge cases
(empty and one-key windows, windows shorter than index_topk, ties, -inf,
garbage outside windows, rows longer than the LDS-resident limit).

All calls go through the C ABI (ctypes binding).  Oracle inputs come from
``synth`` and ``oracle.prep`` only; the HIP path gets the same canonical values."""
import numpy as np
import pytest
import torch

import synth
from oracle import indexer as o_idx
from oracle import mla as o_mla
from oracle import prep as o_prep
from oracle import topk as o_topk
from oracle import windows as o_win
from parity import check_mla, check_scores, check_topk_e2e, dev, host, i32, mla_lse_tol, say

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
P4K = synth.WORKLOADS["prefill4k"]


# ---------------------------------------------------------------------------
# input builders (oracle side)
# ---------------------------------------------------------------------------
def canonical_indexer(w, lay, dtype, signed=False, H=None, rope=True):
    H = w.n_heads if H is None else H
    q_raw = synth.index_q_raw(w, 0, lay.n_q)[:, :H]
    k_raw = synth.index_k_raw(w, 0, lay.n_k)
    wt = synth.index_weights(w, 0, lay.n_q, signed=signed)[:, :H]
    rd = w.rope_dim if rope else 0
    p = o_prep.prepare_indexer_inputs(q_raw, k_raw, wt, lay.positions(), lay.key_positions(),
                                      dtype, rd, w.rope_main_dim, w.rope_theta)
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k, causal=True)
    return p, rs, re


def to_device_indexer(p, dtype):
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]
    q, k = dev(p["q"], tdt), dev(p["k"], tdt)
    w = dev(p["w"])
    ks = None if p["k_scale"] is None else dev(p["k_scale"])
    return q, k, w, ks


def oracle_scores_f32(p, rs, re):
    S, C = o_idx.scores_dense(p["q"], p["k"], p["w"], rs, re, p["k_scale"], with_cond=True,
                              fill=np.nan)
    return S, C


# ---------------------------------------------------------------------------
# windows
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lens,decode", [([256], False), ([5, 1, 300, 77, 1024], False),
                                         ([17000, 3, 40000], True), ([0, 4, 0, 9], False)])
def test_row_windows(dsa, lens, decode):
    say(f"row_windows lens={lens} decode={decode}")
    lay = synth.layout_from_lengths(lens, decode)
    for causal in (True, False):
        rs, re = dsa.dsa_row_windows(i32(lay.cu_q), i32(lay.cu_k), lay.n_q, causal)
        ors, ore = o_win.row_windows(lay.cu_q, lay.cu_k, causal)
        np.testing.assert_array_equal(host(rs), ors)
        np.testing.assert_array_equal(host(re), ore)


# ---------------------------------------------------------------------------
# top-k (bit-exact on identical fp32 scores)
# ---------------------------------------------------------------------------
def _topk_case(dsa, S, rs, re, K, what):
    say(f"topk {what}: rows={S.shape[0]} cols={S.shape[1]} K={K}")
    g = host(dsa.dsa_topk(dev(S), i32(rs), i32(re), K))
    o = o_topk.topk(S, rs, re, K)
    bad = np.nonzero((g != o).any(axis=1))[0]
    assert bad.size == 0, f"{what}: rows differ, first {bad[:5]}: gpu {g[bad[0]][:12]} oracle {o[bad[0]][:12]}"


def test_topk_tiny_oracle_scores(dsa):
    lay = synth.layout(TINY)
    p, rs, re = canonical_indexer(TINY, lay, "f32")
    S, _ = oracle_scores_f32(p, rs, re)
    S32 = np.where(np.isnan(S), np.float32(-1e4), S).astype(np.float32)
    _topk_case(dsa, S32, rs, re, TINY.index_topk, "tiny")


def test_topk_ties_and_specials(dsa):
    g = np.random.default_rng(101)
    pool = np.array([-np.inf, -3.0, -0.0, 0.0, 1.0, 2.5, np.inf], np.float32)
    n_q, n = 300, 700
    S = pool[g.integers(0, len(pool), (n_q, n))]
    rs = g.integers(0, n, n_q).astype(np.int32)
    re = np.minimum(n, rs + g.integers(0, 500, n_q)).astype(np.int32)
    rs[:3] = [0, 5, 9]; re[:3] = [0, 5, 10]                 # empty, empty, one key
    for K in (1, 7, 64, 333, 2500):                          # 2500: every row whole, k past 2048
        _topk_case(dsa, S, rs, re, K, f"ties K={K}")


def test_topk_garbage_outside_windows(dsa):
    g = np.random.default_rng(102)
    lay = synth.layout_from_lengths([700, 1500, 3000, 90, 2100])
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k)
    S = np.where(g.random((lay.n_q, lay.n_k)) < 0.5, 1e4, -1e4).astype(np.float32)
    for t in range(lay.n_q):
        S[t, rs[t]:re[t]] = g.standard_normal(re[t] - rs[t]).astype(np.float32)
    _topk_case(dsa, S, rs, re, 1024, "thd garbage")


def test_topk_long_rows_split_path(dsa):
    # few rows over many columns: windows above the LDS-resident limit (8192) are
    # selected in up to 16 chunks and merged; shorter ones by one workgroup
    g = np.random.default_rng(103)
    n_q, n = 24, 70000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[::3] = np.round(S[::3] * 4) / 4                       # heavy ties on some rows
    S[1, 100:40000:7] = -np.inf                             # -inf inside a split window
    rs = np.zeros(n_q, np.int32)
    rs[5::6] = 777                                          # windows not starting at 0
    re = np.array([n, 8192, 8193, 9000, 30000, 65536] * 4, np.int32)
    assert dsa._lib_or_load().dsa_topk_workspace_size(n_q, n, 2048) > 0
    for K in (2048, 100, 1):
        _topk_case(dsa, S, rs, re, K, f"split K={K}")


def test_topk_split_few_candidates(dsa):
    # split-path windows where most keys are -inf: chunks emit fewer than K
    # candidates, the merged row is -1 padded
    g = np.random.default_rng(107)
    n_q, n = 6, 50000
    S = np.full((n_q, n), -np.inf, np.float32)
    for t in range(n_q):
        cols = g.choice(n, size=[10, 1500, 2047, 2048, 2049, 5000][t], replace=False)
        S[t, cols] = np.round(g.standard_normal(cols.size) * 2).astype(np.float32)
    rs = np.zeros(n_q, np.int32)
    re = np.full(n_q, n, np.int32)
    _topk_case(dsa, S, rs, re, 2048, "split sparse")


def test_topk_rows_longer_than_split(dsa):
    # windows above 16 * 8192 keys: one workgroup re-reads the row from memory
    g = np.random.default_rng(104)
    n_q, n = 3, 140000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[2] = np.round(S[2] * 3) / 3
    rs = np.array([0, 5, 1000], np.int32)
    re = np.array([n, 131073, 140000], np.int32)
    _topk_case(dsa, S, rs, re, 2048, "longer than split")


def test_topk_many_long_rows_stream_path(dsa):
    # more than 1024 rows over more than 8192 columns: one workgroup per row
    # streams a window of more than 8192 keys through LDS with its running
    # top-k and holds a shorter one whole
    g = np.random.default_rng(105)
    n_q, n = 1100, 9000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[::4] = np.round(S[::4] * 2) / 2                       # ties across pieces
    S[1::4, ::3] = -np.inf                                  # unselectable keys
    S[2::8] = -np.inf
    S[2::8, 4000:4100] = 1.0                                # fewer selectable keys than k
    rs = g.integers(0, 500, n_q).astype(np.int32)
    re = np.minimum(n, rs + g.integers(7000, 9000, n_q)).astype(np.int32)
    re[:6] = rs[:6] + np.array([0, 1, 4096, 4097, 8192, 8193])  # empty and boundary windows
    assert dsa._lib_or_load().dsa_topk_workspace_size(n_q, n, 2048) == 0
    for K in (2048, 333, 1):
        _topk_case(dsa, S, rs, re, K, f"stream K={K}")


def _select_path_rows(n, g):
    # rows built so that the k-th score falls, for k = 2048, into:
    #   0: a spread row (the boundary digit holds a few keys: ranks counted)
    #   1: a cluster of ~1000 keys inside one first digit (radix passes over the
    #      gathered keys)
    #   2: 2000 equal keys across the boundary (radix passes over all keys)
    #   3: equal keys only; 4: fewer selectable keys than k
    rows = np.empty((5, n), np.float32)
    rows[0] = g.uniform(0.0, 100.0, n)
    rows[1] = g.uniform(0.0, 100.0, n)
    top = rows[1] > 60.0
    rows[1][~top] = g.uniform(0.0, 50.0, int((~top).sum()))
    cl = g.choice(np.nonzero(~top)[0], 1000, replace=False)
    rows[1][cl] = 50.0 + g.uniform(0.0, 0.01, 1000).astype(np.float32)
    rows[2] = g.uniform(0.0, 100.0, n)
    rows[2][g.choice(n, 2000, replace=False)] = 70.0
    rows[3] = 3.25
    rows[4] = -np.inf
    rows[4][g.choice(n, 1500, replace=False)] = g.standard_normal(1500)
    return rows


def test_topk_select_paths(dsa):
    g = np.random.default_rng(107)
    n = 4096
    S = np.tile(_select_path_rows(n, g), (3, 1))
    n_q = S.shape[0]
    rs = np.zeros(n_q, np.int32)
    re = np.full(n_q, n, np.int32)
    for K in (2048, 1500):
        _topk_case(dsa, S, rs, re, K, f"select paths K={K}")


def test_topk_select_paths_stream_shrinks(dsa):
    # the same kinds of rows, 20480 keys wide, over > 1024 rows: the stream
    # kernel's shrinks see each kind of boundary digit
    g = np.random.default_rng(108)
    n = 20480
    base = _select_path_rows(n, g)
    S = np.repeat(base, 206, axis=0)[:1030]
    rs = np.zeros(S.shape[0], np.int32)
    re = np.full(S.shape[0], n, np.int32)
    assert dsa._lib_or_load().dsa_topk_workspace_size(S.shape[0], n, 2048) == 0
    _topk_case(dsa, S, rs, re, 2048, "select paths, stream")


def test_topk_many_long_rows_stream_shrinks(dsa):
    # windows of up to 40000 keys: the held keys are shrunk several times per
    # row, by the histogram floor and (on the rows of tied values) by the exact
    # select
    g = np.random.default_rng(106)
    n_q, n = 1030, 40000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[::3] = np.round(S[::3] * 4) / 4                       # crowded digits: many equal keys
    S[1::5, ::7] = -np.inf                                  # unselectable keys
    S[2::6] = np.linspace(-1.0, 3.0, n, dtype=np.float32)   # rising scores: a shrink per piece
    rs = g.integers(0, 2000, n_q).astype(np.int32)
    re = np.minimum(n, rs + g.integers(9000, 40000, n_q)).astype(np.int32)
    assert dsa._lib_or_load().dsa_topk_workspace_size(n_q, n, 2048) == 0
    for K in (2048, 100):
        _topk_case(dsa, S, rs, re, K, f"stream shrinks K={K}")


def test_topk_stream_path_wide_offsets(dsa):
    # more than 65536 columns: the stream kernel holds 32-bit window offsets (16-bit
    # ones up to 65536); windows start past 0 and run past offset 65535
    g = np.random.default_rng(109)
    n_q, n = 1030, 70000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[::3] = np.round(S[::3] * 4) / 4                       # crowded digits: many equal keys
    S[1::7, 60000:] += 2.0                                  # the top keys late in the window
    rs = g.integers(0, 3000, n_q).astype(np.int32)
    re = np.minimum(n, rs + g.integers(9000, 70000, n_q)).astype(np.int32)
    re[:4] = [n, n, 66000, 65537]
    rs[:4] = [0, 1, 0, 0]
    assert dsa._lib_or_load().dsa_topk_workspace_size(n_q, n, 2048) == 0
    _topk_case(dsa, S, rs, re, 2048, "stream, offsets past 65535")


def test_topk_many_rows_large_k_global_path(dsa):
    # k above 2048 over long windows: one workgroup per row re-reads from memory
    g = np.random.default_rng(106)
    n_q, n = 40, 12000
    S = g.standard_normal((n_q, n)).astype(np.float32)
    S[::3] = np.round(S[::3] * 3) / 3
    rs = np.zeros(n_q, np.int32)
    re = g.integers(9000, n, n_q).astype(np.int32)
    _topk_case(dsa, S, rs, re, 3000, "large k")


def test_topk_prefill4k_oracle_scores(dsa):
    # full prefill4k score matrix from the oracle (fp64 -> fp32), causal windows
    lay = synth.layout(P4K)
    p, rs, re = canonical_indexer(P4K, lay, "bf16")
    say("oracle scores prefill4k ...")
    S = np.full((lay.n_q, lay.n_k), -1e4, np.float32)
    for t in range(lay.n_q):
        S[t, :re[t]] = o_idx.score_row(p["q"][t], p["k"][:re[t]], p["w"][t])
    _topk_case(dsa, S, rs, re, P4K.index_topk, "prefill4k")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_topk_fused_matches_unfused(dsa, dtype):
    # few rows (decode shape): the fused call keeps the scores in LDS and must
    # return exactly the indices of dsa_indexer_scores + dsa_topk on the same
    # operands; windows cover the whole-row (<= 8192 keys), split (8193 ..
    # 131072) and streamed (> 131072) cases
    w = synth.WORKLOADS["decode" if dtype == "bf16" else "fp8_64k"]
    lay = synth.layout_from_lengths([5000, 33, 12000, 140000, 70000, 8192, 8193], decode=True)
    p, rs, re = canonical_indexer(w, lay, dtype, rope=False)
    q, k, wt, ks = to_device_indexer(p, dtype)
    say(f"indexer_topk fused vs unfused {dtype}: n_k={lay.n_k}")
    for K in (2048, 300):
        S = dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re), k_scale=ks)
        ref = host(dsa.dsa_topk(S, i32(rs), i32(re), K))
        got = host(dsa.dsa_indexer_topk(q, k, wt, i32(rs), i32(re), K, k_scale=ks))
        bad = np.nonzero((got != ref).any(axis=1))[0]
        assert bad.size == 0, f"fused differs on rows {bad}"
        # and the unfused selection is the oracle's on the GPU's fp32 scores
        o = o_topk.topk(host(S), rs, re, K)
        assert np.array_equal(ref, o)


# ---------------------------------------------------------------------------
# indexer scores
# ---------------------------------------------------------------------------
def _indexer_case(dsa, w, lay, dtype, what, signed=False, H=None, rope=True, rows=None):
    p, rs, re = canonical_indexer(w, lay, dtype, signed, H, rope)
    q, k, wt, ks = to_device_indexer(p, dtype)
    say(f"indexer {what}: n_q={lay.n_q} n_k={lay.n_k} H={q.shape[1]} dtype={dtype}")
    G = host(dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re), k_scale=ks))
    rtol = 1e-3 if dtype == "f32" else 2e-2
    rows = range(lay.n_q) if rows is None else rows
    worst = 0.0
    for t in rows:
        a, b = rs[t], re[t]
        ksw = None if p["k_scale"] is None else p["k_scale"][a:b]
        o, c = o_idx.score_row(p["q"][t], p["k"][a:b], p["w"][t], ksw, with_cond=True)
        worst = max(worst, check_scores(G[t, a:b], o, c, rtol, f"{what} row {t}"))
        assert np.isnan(G[t, :a]).all() and np.isnan(G[t, b:]).all(), f"{what}: wrote outside window"
    say(f"  max rel err {worst:.2e}")


def test_indexer_tiny_f32(dsa):
    _indexer_case(dsa, TINY, synth.layout(TINY), "f32", "tiny")


def test_indexer_bf16_prefill_small(dsa):
    _indexer_case(dsa, P4K, synth.layout_from_lengths([777]), "bf16", "bf16 T=777")


def test_indexer_bf16_thd_signed_weights(dsa):
    lay = synth.layout_from_lengths([33, 400, 1, 290])
    _indexer_case(dsa, P4K, lay, "bf16", "bf16 thd signed", signed=True)


def test_indexer_bf16_fewer_heads(dsa):
    _indexer_case(dsa, P4K, synth.layout_from_lengths([300, 45]), "bf16", "bf16 H=20", H=20)
    _indexer_case(dsa, P4K, synth.layout_from_lengths([300]), "bf16", "bf16 H=40", H=40)


def test_indexer_bf16_decode_rows(dsa):
    lay = synth.layout_from_lengths([5000, 33, 12000, 20001], decode=True)
    _indexer_case(dsa, P4K, lay, "bf16", "bf16 decode", rope=False)


def test_indexer_fp8_small(dsa):
    w = synth.WORKLOADS["fp8_64k"]
    _indexer_case(dsa, w, synth.layout_from_lengths([600]), "fp8", "fp8 T=600", rope=False)
    _indexer_case(dsa, w, synth.layout_from_lengths([3000], decode=True), "fp8", "fp8 decode",
                  rope=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_rows_random_windows(dsa, dtype):
    # > 256 rows (the row-block kernel) with unrelated windows in one block of 8
    # rows: empty, one key, starts and ends inside a 32-key tile, windows that
    # skip whole key pairs and chunks, and windows reaching the last key
    w = P4K if dtype == "bf16" else synth.WORKLOADS["fp8_64k"]
    lay = synth.layout_from_lengths([1000])
    p, _, _ = canonical_indexer(w, lay, dtype, signed=True, rope=dtype == "bf16")
    g = np.random.default_rng(11)
    n_q, n_k = lay.n_q, lay.n_k
    rs = g.integers(0, n_k, n_q).astype(np.int32)
    re = np.minimum(n_k, rs + g.integers(0, 700, n_q)).astype(np.int32)
    rs[:8] = [0, 5, 40, 63, 64, 300, 999, 700]
    re[:8] = [0, 6, 41, 65, 1000, 301, 1000, 690]   # empty, one key, ..., end < start
    rs[8:16] = np.arange(8) * 97
    re[8:16] = np.minimum(n_k, rs[8:16] + np.array([31, 32, 33, 63, 64, 65, 257, 513]))
    q, k, wt, ks = to_device_indexer(p, dtype)
    say(f"indexer random windows {dtype}: n_q={n_q} n_k={n_k}")
    G = host(dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re), k_scale=ks))
    worst = 0.0
    for t in range(n_q):
        a, b = int(rs[t]), max(int(rs[t]), int(re[t]))
        if b > a:
            ksw = None if p["k_scale"] is None else p["k_scale"][a:b]
            o, c = o_idx.score_row(p["q"][t], p["k"][a:b], p["w"][t], ksw, with_cond=True)
            worst = max(worst, check_scores(G[t, a:b], o, c, 2e-2, f"{dtype} row {t}"))
        assert np.isnan(G[t, :a]).all() and np.isnan(G[t, b:]).all(), f"row {t}: wrote outside window"
    say(f"  max rel err {worst:.2e}")


# ---------------------------------------------------------------------------
# fused indexer + top-k (end to end against oracle scores + oracle top-k)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lens,K", [([1200], 256), ([300, 900, 64], 128)])
def test_indexer_topk_end_to_end(dsa, lens, K):
    lay = synth.layout_from_lengths(lens)
    p, rs, re = canonical_indexer(P4K, lay, "bf16")
    q, k, wt, _ = to_device_indexer(p, "bf16")
    say(f"indexer_topk lens={lens} K={K}")
    G = host(dsa.dsa_indexer_topk(q, k, wt, i32(rs), i32(re), K))
    ndiff = 0
    for t in range(lay.n_q):
        a, b = rs[t], re[t]
        o, c = o_idx.score_row(p["q"][t], p["k"][a:b], p["w"][t], with_cond=True)
        full = np.full(lay.n_k, -np.inf); full[a:b] = o
        tau = np.zeros(lay.n_k); tau[a:b] = 2e-2 * np.maximum(np.abs(o), c / 128)
        oi = o_topk.topk_row(full.astype(np.float32), a, b, K)
        ndiff += check_topk_e2e(G[t], oi, full, tau, f"row {t}")
    say(f"  columns differing within tolerance: {ndiff}")


# ---------------------------------------------------------------------------
# sparse MLA
# ---------------------------------------------------------------------------
def _random_topk_rows(g, n_q, n_kv, K, windows=None, holes=False):
    """Index rows shaped like top-k output: ascending columns, then -1 padding."""
    out = np.full((n_q, K), -1, np.int32)
    for t in range(n_q):
        a, b = (0, n_kv) if windows is None else windows[t]
        n = min(K, b - a)
        n = int(g.integers(max(0, n // 2), n + 1)) if g.random() < 0.3 else n
        sel = np.sort(g.choice(np.arange(a, b), size=n, replace=False)) if n else np.zeros(0)
        out[t, :n] = sel
        if holes and n > 4:
            out[t, g.integers(0, n, 3)] = -1           # -1 inside the list too
    return out


def _mla_case(dsa, q, kv, idx, sm, d_v, bf16, what, rows=None, oracle_idx=None):
    """oracle_idx: the selection the oracle reads (default idx); the kernel reads idx."""
    tdt = torch.bfloat16 if bf16 else torch.float32
    qd, kvd = dev(q, tdt), dev(kv, tdt)
    say(f"mla {what}: n_q={q.shape[0]} H={q.shape[1]} n_kv={kv.shape[0]} K={idx.shape[1]}")
    out, lse = dsa.dsa_sparse_mla_fwd(qd, kvd, i32(idx), sm, d_v)
    rows = list(range(q.shape[0])) if rows is None else list(rows)
    oidx = idx if oracle_idx is None else oracle_idx
    oo, ol = o_mla.sparse_mla(q, kv, oidx, sm, d_v, rows=rows)
    tol = mla_lse_tol(q[rows], kv, oidx[rows], sm, bf16, ol)
    err = check_mla(host(out)[rows], oo, host(lse)[rows], ol, bf16, what, lse_tol=tol)
    say(f"  max abs err {err:.2e}")


def test_mla_tiny_f32(dsa):
    lay = synth.layout(TINY)
    p, rs, re = canonical_indexer(TINY, lay, "f32")
    S, _ = oracle_scores_f32(p, rs, re)
    idx = o_topk.topk(np.where(np.isnan(S), -np.inf, S).astype(np.float32), rs, re, TINY.index_topk)
    q = o_prep.round_f32(synth.mla_q(TINY, 0, lay.n_q))
    kv = o_prep.round_f32(synth.mla_kv(TINY, 0, lay.n_k))
    _mla_case(dsa, q, kv, idx, TINY.sm_scale, TINY.d_v, False, "tiny f32")


def test_mla_bf16_prefill_medium(dsa):
    g = np.random.default_rng(201)
    n_q, n_kv = 96, 3000
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = o_prep.round_bf16(synth.mla_kv(P4K, 0, n_kv))
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk, holes=True)
    idx[0] = -1                                            # empty row
    idx[1, 1:] = -1                                        # one key
    _mla_case(dsa, q, kv, idx, P4K.sm_scale, P4K.d_v, True, "bf16 prefill")


def test_mla_bf16_peaky_and_split(dsa):
    g = np.random.default_rng(202)
    n_q, n_kv = 6, 5000                                    # few queries: split-K path
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q) * 800.0)  # large logits: rescale path
    kv = o_prep.round_bf16(synth.mla_kv(P4K, 0, n_kv))
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk, holes=True)
    _mla_case(dsa, q, kv, idx, P4K.sm_scale, P4K.d_v, True, "bf16 split peaky")


def test_mla_bf16_large_logit_growth(dsa):
    # The logits rise by ~200 along the (ascending) key order while staying smooth
    # near the top (noise std ~0.5): far beyond the 2^32 slack over the first
    # tile's max that the softmax reference allows, so the workgroup runs its
    # query a second time against the true max.  The trend lives in a rope dim,
    # so values stay ~N(0, 0.01).
    g = np.random.default_rng(204)
    n_kv = 4096
    kv = synth.mla_kv(P4K, 0, n_kv)
    kv[:, 512] += np.linspace(0.0, 40.0, n_kv, dtype=np.float32)
    kv = o_prep.round_bf16(kv)
    for n_q, what in ((12, "split"), (200, "prefill")):
        q = synth.mla_q(P4K, 0, n_q)
        q[:, :, 512] += 120.0
        q = o_prep.round_bf16(q)
        idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk)
        _mla_case(dsa, q, kv, idx, P4K.sm_scale, P4K.d_v, True, f"bf16 logit growth {what}",
                  rows=range(0, n_q, 3))


@pytest.mark.parametrize("n_q,what", [(12, "split"), (200, "one workgroup per query")])
def test_mla_bf16_extreme_logits(dsa, n_q, what):
    # Logits of several hundred to ~2000 natural units (q scaled by 8000, value
    # rows scaled by 0.2 .. 3 along the cache): lse ~ 500 .. 1400, and a later
    # tile's max far above the first tile's, on the split path (few queries) and
    # on the one-workgroup-per-query launch.
    g = np.random.default_rng(205)
    n_kv = 4096
    kv = synth.mla_kv(P4K, 0, n_kv) * np.linspace(0.2, 3.0, n_kv, dtype=np.float32)[:, None]
    kv = o_prep.round_bf16(kv)
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q) * 8000.0)
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk)
    _mla_case(dsa, q, kv, idx, P4K.sm_scale, P4K.d_v, True, f"bf16 extreme logits {what}",
              rows=range(0, n_q, 1 if n_q < 50 else 7))


@pytest.mark.parametrize("n_q", [10, 300])
def test_mla_out_of_range_indices_are_skipped(dsa, n_q):
    # entries outside [0, n_kv) are skipped like -1: never gathered
    g = np.random.default_rng(206)
    n_kv = 900
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = o_prep.round_bf16(synth.mla_kv(P4K, 0, n_kv))
    idx = _random_topk_rows(g, n_q, n_kv, 512, holes=True)
    bad = idx.copy()
    pos = g.random(idx.shape) < 0.1
    junk = g.choice(np.array([n_kv, n_kv + 1, 2 ** 31 - 1, -2, -(2 ** 31)], np.int64), idx.shape)
    bad[pos] = junk[pos].astype(np.int32)
    bad[0, :] = n_kv + 5                                  # nothing in range: out 0, lse -inf
    oracle_idx = np.where((bad >= 0) & (bad < n_kv), bad, -1).astype(np.int32)
    _mla_case(dsa, q, kv, bad, P4K.sm_scale, P4K.d_v, True, f"bf16 out-of-range n_q={n_q}",
              oracle_idx=oracle_idx)
    qf = o_prep.round_f32(synth.mla_q(TINY, 0, 40))
    kvf = o_prep.round_f32(synth.mla_kv(TINY, 0, 50))
    idf = _random_topk_rows(g, 40, 50, 16, holes=True)
    idf[::3, 2] = 50
    idf[1::3, 5] = -7
    _mla_case(dsa, qf, kvf, idf, TINY.sm_scale, TINY.d_v, False, "f32 out-of-range",
              oracle_idx=np.where((idf >= 0) & (idf < 50), idf, -1).astype(np.int32))


def test_mla_bf16_fewer_heads(dsa):
    g = np.random.default_rng(203)
    n_q, n_kv = 40, 700
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q)[:, :96])
    kv = o_prep.round_bf16(synth.mla_kv(P4K, 0, n_kv))
    idx = _random_topk_rows(g, n_q, n_kv, 512)
    _mla_case(dsa, q, kv, idx, P4K.sm_scale, P4K.d_v, True, "bf16 H=96")


# ---------------------------------------------------------------------------
# sparse MLA over the fp8 latent cache (656-byte rows)
# ---------------------------------------------------------------------------
def _pack_mla_fp8(codes, scales, rope) -> np.ndarray:
    """Cache rows [N, 656] from the oracle's quantisation: 512 e4m3 code bytes,
    4 fp32 scales, 64 bf16 rope values (every value is exact in its format)."""
    N = codes.shape[0]
    c = torch.from_numpy(np.ascontiguousarray(codes, np.float32)).to(torch.float8_e4m3fn)
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float32))
    r = torch.from_numpy(np.ascontiguousarray(rope, np.float32)).to(torch.bfloat16)
    row = torch.cat([c.view(torch.uint8), s.view(torch.uint8).reshape(N, 16),
                     r.view(torch.uint8).reshape(N, 128)], dim=1)
    assert row.shape == (N, 656)
    return row.numpy()


def _fp8_cache(kv):
    """(cache bytes [N, 656], the dequantised rows [N, 576] the kernel reads)."""
    codes, s, rope = o_prep.mla_kv_quant(kv)
    return _pack_mla_fp8(codes, s, rope), o_prep.dequant_mla_kv(codes, s, rope)


def _mla_fp8_case(dsa, q, kv, idx, sm, what, rows=None, oracle_idx=None, cache=None):
    """q bf16 values [n_q, H, 576]; kv the latent rows before quantisation."""
    packed, kv_deq = _fp8_cache(kv)
    cache_d = torch.from_numpy(packed).cuda() if cache is None else cache
    qd = dev(q, torch.bfloat16)
    say(f"mla fp8 {what}: n_q={q.shape[0]} H={q.shape[1]} n_kv={kv.shape[0]} K={idx.shape[1]}")
    out, lse = dsa.dsa_sparse_mla_fwd(qd, cache_d, i32(idx), sm, 512)
    assert out.dtype == torch.bfloat16
    rows = list(range(q.shape[0])) if rows is None else list(rows)
    oidx = idx if oracle_idx is None else oracle_idx
    oo, ol = o_mla.sparse_mla(q, kv_deq, oidx, sm, 512, rows=rows)
    tol = mla_lse_tol(q[rows], kv_deq, oidx[rows], sm, True, ol)
    err = check_mla(host(out)[rows], oo, host(lse)[rows], ol, True, what, lse_tol=tol)
    say(f"  max abs err {err:.2e}")


def test_mla_fp8_prefill(dsa):
    g = np.random.default_rng(211)
    n_q, n_kv = 200, 3000                                  # one workgroup per query
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk, holes=True)
    idx[0] = -1                                            # empty row: out 0, lse -inf
    idx[1, 1:] = -1                                        # one key
    idx[2, 33:] = -1                                       # a ragged last tile
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, "prefill", rows=list(range(6)) +
                  list(range(6, n_q, 9)))


def test_mla_fp8_split_peaky(dsa):
    g = np.random.default_rng(212)
    n_q, n_kv = 6, 5000                                    # few queries: keys split
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q) * 800.0)
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk, holes=True)
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, "split peaky")


def test_mla_fp8_large_logit_growth(dsa):
    # a later tile's max far above the first one's: the second pass
    g = np.random.default_rng(213)
    n_kv = 4096
    kv = synth.mla_kv(P4K, 0, n_kv)
    kv[:, 512] += np.linspace(0.0, 40.0, n_kv, dtype=np.float32)
    for n_q, what in ((12, "split"), (200, "prefill")):
        q = synth.mla_q(P4K, 0, n_q)
        q[:, :, 512] += 120.0
        q = o_prep.round_bf16(q)
        idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk)
        _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, f"logit growth {what}",
                      rows=range(0, n_q, 3))


@pytest.mark.parametrize("n_q", [10, 300])
def test_mla_fp8_out_of_range_indices(dsa, n_q):
    g = np.random.default_rng(214)
    n_kv = 900
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _random_topk_rows(g, n_q, n_kv, 512, holes=True)
    bad = idx.copy()
    pos = g.random(idx.shape) < 0.1
    junk = g.choice(np.array([n_kv, n_kv + 1, 2 ** 31 - 1, -2, -(2 ** 31)], np.int64), idx.shape)
    bad[pos] = junk[pos].astype(np.int32)
    bad[0, :] = n_kv + 5
    oracle_idx = np.where((bad >= 0) & (bad < n_kv), bad, -1).astype(np.int32)
    _mla_fp8_case(dsa, q, kv, bad, P4K.sm_scale, f"out-of-range n_q={n_q}",
                  rows=range(0, n_q, 1 if n_q < 50 else 11), oracle_idx=oracle_idx)


@pytest.mark.parametrize("H", [96, 40])
def test_mla_fp8_fewer_heads(dsa, H):
    # 96: whole waves idle; 40: a wave with 8 of its 16 heads
    g = np.random.default_rng(215)
    n_q, n_kv = 30, 700
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q)[:, :H])
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _random_topk_rows(g, n_q, n_kv, 512)
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, f"H={H}")


@pytest.mark.parametrize("n_q,kv_fmt", [(40, "bf16"), (200, "bf16"), (40, "fp8"), (200, "fp8")])
def test_mla_more_heads_than_a_block(dsa, n_q, kv_fmt):
    # 160 heads: two head blocks of the grid, the second with one busy wave of
    # four; 40 queries run the split launch with its combine, 200 the direct one
    g = np.random.default_rng(216)
    n_kv, H = 700, 160
    q = np.concatenate([synth.mla_q(P4K, 0, n_q), synth.mla_q(P4K, 1000, 1000 + n_q)[:, :H - 128]],
                       axis=1)
    q = o_prep.round_bf16(q)
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _random_topk_rows(g, n_q, n_kv, 512, holes=True)
    rows = range(0, n_q, 1 if n_q < 50 else 9)
    if kv_fmt == "bf16":
        _mla_case(dsa, q, o_prep.round_bf16(kv), idx, P4K.sm_scale, P4K.d_v, True, f"bf16 H={H}",
                  rows=rows)
    else:
        _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, f"H={H}", rows=rows)


def test_mla_fp8_wide_value_range(dsa):
    # rows whose 128-dim tiles differ in magnitude by 2^-12 .. 2^6 (tiny tiles
    # quantise to e4m3 subnormals), an all-zero row and tiles of zeros
    g = np.random.default_rng(216)
    n_q, n_kv = 8, 1500
    kv = synth.mla_kv(P4K, 0, n_kv)
    tile_mag = 2.0 ** g.integers(-12, 7, size=(n_kv, 4))
    kv[:, :512] *= np.repeat(tile_mag, 128, axis=1).astype(np.float32)
    kv[5] = 0.0
    kv[7, 128:256] = 0.0
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk)
    idx[0, :3] = [5, 7, 9]
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, "wide value range")


def _tile_count_rows(g, n_q, n_kv, K):
    """Rows with 1 .. 9 tiles of selected keys (partial last tiles too), -1 after."""
    idx = np.full((n_q, K), -1, np.int32)
    for t in range(n_q):
        n = min(K, 32 * (t % 9 + 1) - (t % 3) * 7)
        idx[t, :n] = np.sort(g.choice(n_kv, size=n, replace=False))
    return idx


@pytest.mark.parametrize("n_q", [8, 200])
def test_mla_tile_counts(dsa, n_q):
    # every remainder of the tile loop's groups (four tiles for bf16 rows, three
    # for fp8 rows) on the one-workgroup-per-query launch and on split slices
    g = np.random.default_rng(219)
    n_kv = 2000
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = synth.mla_kv(P4K, 0, n_kv)
    idx = _tile_count_rows(g, n_q, n_kv, 512)
    rows = list(range(n_q)) if n_q < 50 else list(range(0, 27)) + list(range(100, 127))
    _mla_case(dsa, q, o_prep.round_bf16(kv), idx, P4K.sm_scale, P4K.d_v, True,
              f"tile counts bf16 n_q={n_q}", rows=rows)
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, f"tile counts n_q={n_q}", rows=rows)


@pytest.mark.parametrize("n_q", [8, 200])
def test_mla_index_width_not_a_tile_multiple(dsa, n_q):
    # index rows whose width is not a whole number of 32-key tiles: the row's
    # last tile runs past its end, and with few queries the split slices divide
    # a tile count that is not a multiple of the number of splits
    g = np.random.default_rng(223)
    n_kv = 3000
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    kv = synth.mla_kv(P4K, 0, n_kv)
    rows = list(range(n_q)) if n_q < 50 else list(range(0, 20)) + list(range(180, 200))
    for K in (100, 1007):
        idx = _random_topk_rows(g, n_q, n_kv, K, holes=True)
        assert (idx[rows, K - 1] >= 0).any()  # some rows use the row's last column
        _mla_case(dsa, q, o_prep.round_bf16(kv), idx, P4K.sm_scale, P4K.d_v, True,
                  f"width {K} bf16 n_q={n_q}", rows=rows)
        _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, f"width {K} n_q={n_q}", rows=rows)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_mla_kv_insert_bytes(dsa, src):
    # every written byte equals the oracle's quantisation; other slots untouched
    g = np.random.default_rng(217)
    n_tok, n_slots = 300, 700
    kv = synth.mla_kv(P4K, 0, n_tok)
    kv[:, :512] *= np.repeat(2.0 ** g.integers(-10, 8, size=(n_tok, 4)), 128, axis=1)
    kv[3] = 0.0
    kv[4, :128] = 0.0
    kv = o_prep.round_bf16(kv) if src == "bf16" else o_prep.round_f32(kv)
    slots = g.permutation(n_slots)[:n_tok].astype(np.int64)
    slots[::17] = -1
    slots[5] = n_slots + 3                                 # outside the cache: skipped
    tdt = torch.bfloat16 if src == "bf16" else torch.float32
    fill = g.integers(0, 256, size=(n_slots, 656)).astype(np.uint8)
    cache = torch.from_numpy(fill.copy()).cuda()
    say(f"mla kv insert {src}: n_tok={n_tok} n_slots={n_slots}")
    dsa.dsa_mla_kv_insert(dev(kv, tdt), torch.from_numpy(slots).cuda(), cache)
    got = cache.cpu().numpy()
    want = fill.copy()
    ok = (slots >= 0) & (slots < n_slots)
    want[slots[ok]] = _pack_mla_fp8(*o_prep.mla_kv_quant(kv[ok]))
    assert np.array_equal(got, want), f"{int((got != want).any(axis=1).sum())} rows differ"


def test_mla_fp8_decode_from_inserted_cache(dsa):
    # decode: the cache written by dsa_mla_kv_insert, read by the fp8 attention
    g = np.random.default_rng(218)
    n_q, n_kv = 4, 6000
    kv = o_prep.round_bf16(synth.mla_kv(P4K, 0, n_kv))
    cache = torch.zeros((n_kv, 656), dtype=torch.uint8, device="cuda")
    dsa.dsa_mla_kv_insert(dev(kv, torch.bfloat16), torch.arange(n_kv, device="cuda"), cache)
    q = o_prep.round_bf16(synth.mla_q(P4K, 0, n_q))
    idx = _random_topk_rows(g, n_q, n_kv, P4K.index_topk)
    _mla_fp8_case(dsa, q, kv, idx, P4K.sm_scale, "decode from inserted cache", cache=cache)


# ---------------------------------------------------------------------------
# input preparation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_indexer_prep(dsa, dtype):
    lay = synth.layout_from_lengths([300, 1000, 5000])
    w = P4K
    q_raw = synth.index_q_raw(w, 0, lay.n_q)
    k_raw = synth.index_k_raw(w, 0, lay.n_k)
    wt = synth.index_weights(w, 0, lay.n_q)
    rope = 0 if dtype == "fp8" else w.rope_dim
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]
    say(f"prep {dtype}")
    q, k, wo, ks = dsa.dsa_indexer_prep(dev(q_raw), dev(k_raw), dev(wt),
                                        i32(lay.positions()), i32(lay.key_positions()),
                                        out_dtype=tdt, rope_dim=rope, rope_main_dim=w.rope_main_dim,
                                        rope_theta=w.rope_theta)
    p = o_prep.prepare_indexer_inputs(q_raw, k_raw, wt, lay.positions(), lay.key_positions(),
                                      dtype, rope, w.rope_main_dim, w.rope_theta)
    gq, gk, gw = host(q), host(k), host(wo)
    if dtype == "f32":
        np.testing.assert_allclose(gq, p["q"], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(gk, p["k"], rtol=1e-5, atol=1e-5)
        np.testing.assert_array_equal(gw, p["w"])
    elif dtype == "bf16":
        # the device computes in fp32 and rounds once: apart by at most one bf16
        # step plus the fp32 rounding of the rotation (absolute, |x| ~ 1), which
        # dominates where the two rotated terms cancel
        for g_, o_ in ((gq, p["q"]), (gk, p["k"])):
            step = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_), 1e-30))) - 7)
            assert np.all(np.abs(g_ - o_) <= step * 1.0001 + 2e-6)
            assert np.mean(g_ != o_) < 0.02
        np.testing.assert_array_equal(gw, p["w"])
    else:
        np.testing.assert_array_equal(host(ks), p["k_scale"])          # scales identical
        np.testing.assert_array_equal(gq, p["q"])                      # no norm: codes identical
        np.testing.assert_array_equal(gw, p["w"])                      # folded weights identical
        mism = gk != p["k"]                                            # LayerNorm'd keys: fp32 vs fp64
        assert np.mean(mism) < 0.01
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(p["k"]), 2.0 ** -6))) - 3)
        assert np.all(np.abs(gk - p["k"])[mism] <= step[mism] * 1.0001)


# ---------------------------------------------------------------------------
# windows outside the keys are clamped to [0, n_k]; a caller's stream is used
# ---------------------------------------------------------------------------
def _clamp(rs, re, n):
    a = np.clip(rs, 0, None)
    b = np.minimum(re, n)
    return a.astype(np.int32), np.maximum(a, b).astype(np.int32)


@pytest.mark.parametrize("n_q", [40, 600])
def test_windows_clamped_to_keys(dsa, n_q):
    # row-split (few rows) and row-block indexer kernels, the top-k rows and
    # split paths, and the fused indexer + top-k: windows that start below 0 or
    # end past the last key behave as their clamped windows
    g = np.random.default_rng(301)
    lay = synth.layout_from_lengths([1500] if n_q == 600 else [1500], decode=False)
    p, _, _ = canonical_indexer(P4K, lay, "bf16", rope=False)
    n_k = lay.n_k
    p = dict(p, q=p["q"][:n_q], w=p["w"][:n_q])
    rs = g.integers(-3000, n_k, n_q).astype(np.int32)
    re = (rs + g.integers(0, 4000, n_q)).astype(np.int32)
    rs[:4] = [-(2 ** 31), 0, n_k - 1, n_k + 7]
    re[:4] = [2 ** 31 - 1, n_k + 1, n_k + 9000, n_k + 9]
    ca, cb = _clamp(rs, re, n_k)
    q, k, wt, _ = to_device_indexer(p, "bf16")
    say(f"clamped windows n_q={n_q} n_k={n_k}")
    G = host(dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re)))
    Gc = host(dsa.dsa_indexer_scores(q, k, wt, i32(ca), i32(cb)))
    np.testing.assert_array_equal(np.isnan(G), np.isnan(Gc))
    np.testing.assert_array_equal(G[~np.isnan(G)], Gc[~np.isnan(Gc)])
    for t in range(0, n_q, 13):
        a, b = int(ca[t]), int(cb[t])
        if b > a:
            o, c = o_idx.score_row(p["q"][t], p["k"][a:b], p["w"][t], with_cond=True)
            check_scores(G[t, a:b], o, c, 2e-2, f"clamped row {t}")
    S = np.where(np.isnan(Gc), np.float32(-1e4), Gc).astype(np.float32)
    for K in (64, 2048):
        got = host(dsa.dsa_topk(dev(S), i32(rs), i32(re), K))
        np.testing.assert_array_equal(got, o_topk.topk(S, ca, cb, K))
        fused = host(dsa.dsa_indexer_topk(q, k, wt, i32(rs), i32(re), K))
        ref = host(dsa.dsa_indexer_topk(q, k, wt, i32(ca), i32(cb), K))
        np.testing.assert_array_equal(fused, ref)
    # the split path of dsa_topk (few rows over more than 8192 columns)
    n = 20000
    S2 = g.standard_normal((12, n)).astype(np.float32)
    rs2 = np.array([-5, 0, 100, 19999, -100000, 5, 0, 0, 7, 8, 9, 10], np.int32)
    re2 = np.array([n + 3, 9000, 30000, 40000, 2 ** 31 - 1, 4, 0, n, 8193, 8200, 200, 12000],
                   np.int32)
    a2, b2 = _clamp(rs2, re2, n)
    assert dsa._lib_or_load().dsa_topk_workspace_size(12, n, 2048) > 0
    np.testing.assert_array_equal(host(dsa.dsa_topk(dev(S2), i32(rs2), i32(re2), 2048)),
                                  o_topk.topk(S2, a2, b2, 2048))


def test_calls_on_a_caller_stream(dsa):
    # every entry point enqueued on a non-default stream, with its workspace and
    # outputs allocated by the binding for that stream; results match the
    # default-stream calls
    g = np.random.default_rng(302)
    lay = synth.layout_from_lengths([20000], decode=True)
    lay2 = synth.layout_from_lengths([700, 20000, 9000], decode=True)
    p, rs, re = canonical_indexer(P4K, lay2, "bf16", rope=False)
    q, k, wt, _ = to_device_indexer(p, "bf16")
    mq = dev(o_prep.round_bf16(synth.mla_q(P4K, 0, 3)), torch.bfloat16)
    mkv = dev(o_prep.round_bf16(synth.mla_kv(P4K, 0, lay2.n_k)), torch.bfloat16)
    base_idx = dsa.dsa_indexer_topk(q, k, wt, i32(rs), i32(re), 2048)
    base_out, base_lse = dsa.dsa_sparse_mla_fwd(mq, mkv, base_idx, P4K.sm_scale, P4K.d_v)
    S = dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re))
    base_top = dsa.dsa_topk(S, i32(rs), i32(re), 2048)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    rsd, red = i32(rs), i32(re)
    torch.cuda.synchronize()
    idx = dsa.dsa_indexer_topk(q, k, wt, rsd, red, 2048, stream=s)
    top = dsa.dsa_topk(S, rsd, red, 2048, stream=s)
    out, lse = dsa.dsa_sparse_mla_fwd(mq, mkv, idx, P4K.sm_scale, P4K.d_v, stream=s)
    s.synchronize()
    assert torch.equal(idx, base_idx) and torch.equal(top, base_top)
    assert torch.equal(out, base_out) and torch.equal(lse, base_lse)
    del lay, g


# ---------------------------------------------------------------------------
# fused prefill indexer + top-k (more than 256 rows): candidates held in LDS
# ---------------------------------------------------------------------------
def _fused_vs_unfused(dsa, q, k, wt, ks, rs, re, K, what):
    S = dsa.dsa_indexer_scores(q, k, wt, rs, re, k_scale=ks)
    ref = dsa.dsa_topk(S, rs, re, K)
    need = dsa._lib_or_load().dsa_indexer_topk_workspace_size(q.shape[0], k.shape[0], q.shape[1],
                                                               q.shape[2], dsa._dtype_code(q), K)
    assert need == 0, f"{what}: the prefill path needs no workspace"
    got = dsa.dsa_indexer_topk(q, k, wt, rs, re, K, k_scale=ks)
    torch.cuda.synchronize()
    bad = torch.nonzero((got != ref).any(dim=1)).flatten().cpu().numpy()
    assert bad.size == 0, (f"{what}: fused differs on {bad.size} rows, first {bad[:5]}: "
                           f"{host(got[bad[0]])[:10]} vs {host(ref[bad[0]])[:10]}")
    return S, ref


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_topk_prefill_matches_unfused(dsa, dtype):
    # causal prefill and packed samples; windows from empty to 20000 keys (the
    # held candidates are shrunk several times per row); k from 1 to 2048
    w = P4K if dtype == "bf16" else synth.WORKLOADS["fp8_64k"]
    rope = dtype == "bf16"
    for lens, Ks in (([3000], (2048, 300)), ([700, 20000, 33, 1, 4100], (2048, 1, 777))):
        lay = synth.layout_from_lengths(lens)
        p, rs, re = canonical_indexer(w, lay, dtype, rope=rope)
        q, k, wt, ks = to_device_indexer(p, dtype)
        say(f"fused prefill {dtype} lens={lens}: n_q={lay.n_q}")
        for K in Ks:
            S, ref = _fused_vs_unfused(dsa, q, k, wt, ks, i32(rs), i32(re), K, f"{dtype} {lens} K={K}")
        # and the unfused selection is the oracle's on those fp32 scores (sampled rows)
        Sh = host(S)
        for t in list(range(0, lay.n_q, 997)) + [lay.n_q - 1]:
            np.testing.assert_array_equal(host(ref[t]), o_topk.topk_row(Sh[t], rs[t], re[t], Ks[-1]))


def test_indexer_topk_prefill_ties_and_signs(dsa):
    # rows whose weights are 0 (every score exactly 0: the first k columns win)
    # or negative (scores <= 0, with -0.0 == +0.0), and random windows inside
    # one block of four rows
    lay = synth.layout_from_lengths([6000])
    p, _, _ = canonical_indexer(P4K, lay, "bf16", signed=True)
    g = np.random.default_rng(303)
    n_q = 1500
    p = dict(p, q=p["q"][:n_q], w=p["w"][:n_q].copy())
    p["w"][0::5] = 0.0
    p["w"][1::5] = -np.abs(p["w"][1::5])
    rs = g.integers(0, 6000, n_q).astype(np.int32)
    re = np.minimum(6000, rs + g.integers(0, 6000, n_q)).astype(np.int32)
    rs[:8] = [0, 0, 5, 100, 0, 2999, 6000, 0]
    re[:8] = [6000, 1, 5, 2148, 2048, 5999, 6000, 2049]
    q, k, wt, _ = to_device_indexer(p, "bf16")
    for K in (2048, 64):
        _fused_vs_unfused(dsa, q, k, wt, None, i32(rs), i32(re), K, f"ties K={K}")


@pytest.mark.parametrize("n_q", [200, 1200])
def test_indexer_topk_short_windows(dsa, n_q):
    # windows of at most k keys: with no negative weight in the row every key is
    # selected and the fused kernels write the window without scoring it; a row
    # with one negative weight is scored.  200 rows take the decode kernel, 1200
    # the prefill kernel (blocks of four rows that are all short skip their loads)
    g = np.random.default_rng(305)
    n_k, K = 5000, 2048
    lay = synth.layout_from_lengths([n_k])
    p, _, _ = canonical_indexer(P4K, lay, "bf16", rope=False)
    p = dict(p, q=p["q"][:n_q], w=p["w"][:n_q].copy())
    rs = g.integers(0, n_k, n_q).astype(np.int32)
    re = np.minimum(n_k, rs + g.integers(0, K + 1, n_q)).astype(np.int32)  # at most K keys
    re[::7] = np.minimum(n_k, rs[::7] + g.integers(K + 1, n_k + 1, len(rs[::7])))  # some longer
    p["w"][3::11, 5] = -0.25  # one negative weight: scored
    q, k, wt, _ = to_device_indexer(p, "bf16")
    say(f"fused short windows: n_q={n_q}")
    _, ref = _fused_vs_unfused(dsa, q, k, wt, None, i32(rs), i32(re), K, f"short n_q={n_q}")
    r = host(ref)
    for t in range(n_q):
        n = re[t] - rs[t]
        if n <= K:
            np.testing.assert_array_equal(r[t, :n], np.arange(rs[t], re[t]))
            assert (r[t, n:] == -1).all()


def test_indexer_topk_prefill_wide_columns(dsa):
    # more than 65536 keys: the held columns are 32-bit
    g = np.random.default_rng(304)
    n_k, n_q = 70000, 300
    lay = synth.layout_from_lengths([n_k])
    p, _, _ = canonical_indexer(P4K, lay, "bf16", rope=False)
    p = dict(p, q=p["q"][:n_q], w=p["w"][:n_q])
    rs = g.integers(0, 10000, n_q).astype(np.int32)
    re = np.minimum(n_k, rs + g.integers(1, n_k, n_q)).astype(np.int32)
    rs[:3], re[:3] = [0, 0, 4], [n_k, 65537, 65541]
    q, k, wt, _ = to_device_indexer(p, "bf16")
    say(f"fused prefill wide: n_q={n_q} n_k={n_k}")
    _fused_vs_unfused(dsa, q, k, wt, None, i32(rs), i32(re), 2048, "wide")


# ---------------------------------------------------------------------------
# fp8 index-key cache: fused norm -> quant -> insert, and decode scoring from it
# ---------------------------------------------------------------------------
def _e4m3_step(o):
    a = np.abs(o)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))


def _check_cache(g_codes, g_scales, o_codes, o_scales, rows, what):
    np.testing.assert_array_equal(g_scales[rows], o_scales[rows], err_msg=f"{what}: scales")
    d = np.abs(g_codes[rows] - o_codes[rows])
    assert np.all(d <= _e4m3_step(o_codes[rows]) * 1.0001), f"{what}: a code off by more than one step"
    frac = np.mean(d > 0)
    assert frac < 0.01, f"{what}: {frac:.3%} of the codes differ"
    return frac


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_k_cache_insert(dsa, in_dtype):
    g = np.random.default_rng(401)
    n_tok, n_slots, D = 2000, 2600, 128
    k_raw = synth.index_k_raw(P4K, 0, n_tok) * 3.0 + 0.5
    if in_dtype == "bf16":
        k_raw = o_prep.round_bf16(k_raw)
    wgt = o_prep.round_f32(1.0 + 0.3 * g.standard_normal(D))
    bias = o_prep.round_f32(0.1 * g.standard_normal(D))
    slots = g.permutation(n_slots)[:n_tok].astype(np.int64)
    slots[::37] = -1                                      # padding tokens
    slots[5] = n_slots + 3                                # past the cache: ignored
    k_raw[7] = 0.0                                        # an all-zero row
    sentinel = 0x7E                                       # e4m3 448
    cache = torch.full((n_slots, D), sentinel, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_slots,), -1.0, dtype=torch.float32, device="cuda")
    tdt = torch.float32 if in_dtype == "f32" else torch.bfloat16
    say(f"k cache insert {in_dtype}: {n_tok} tokens into {n_slots} slots")
    dsa.dsa_indexer_k_insert(dev(k_raw, tdt), dev(slots, torch.int64), cache, scales,
                             norm_weight=dev(wgt), norm_bias=dev(bias), eps=1e-6)
    g_codes = cache.view(torch.float8_e4m3fn).float().cpu().numpy().astype(np.float64)
    g_scales = host(scales).astype(np.float64)
    o_codes = np.full((n_slots, D), 448.0)
    o_scales = np.full(n_slots, -1.0)
    o_prep.k_norm_quant_insert(k_raw, wgt, bias, 1e-6, slots, o_codes, o_scales)
    written = np.zeros(n_slots, bool)
    written[slots[(slots >= 0) & (slots < n_slots)]] = True
    assert np.all(host(cache)[~written] == sentinel) and np.all(g_scales[~written] == -1.0)
    frac = _check_cache(g_codes, g_scales, o_codes, o_scales, written, f"insert {in_dtype}")
    # an all-zero raw key normalises to 0: what is written is the bias
    np.testing.assert_array_equal(g_codes[slots[7]] * g_scales[slots[7]],
                                  o_codes[slots[7]] * o_scales[slots[7]])
    say(f"  {frac:.4%} of the codes one e4m3 step from the oracle's")


def test_decode_scores_from_fp8_key_cache(dsa):
    # a decode step over caches filled by two inserts (the prompt, then each
    # sequence's newest token), scored and selected straight from the cache
    w8 = synth.WORKLOADS["fp8_64k"]
    lens = [20000, 9000, 70000, 300, 8193]
    lay = synth.layout_from_lengths(lens, decode=True)
    k_raw = o_prep.round_bf16(synth.index_k_raw(w8, 0, lay.n_k))
    q_raw = synth.index_q_raw(w8, 0, lay.n_q)
    wt = synth.index_weights(w8, 0, lay.n_q)
    g = np.random.default_rng(402)
    wgt = o_prep.round_f32(1.0 + 0.2 * g.standard_normal(128))
    bias = o_prep.round_f32(0.05 * g.standard_normal(128))
    last = lay.cu_k[1:] - 1
    first = np.setdiff1d(np.arange(lay.n_k), last)
    batches = [first, np.concatenate([last, [-1, -1]])]   # the step batch has two padding tokens
    cache = torch.zeros((lay.n_k, 128), dtype=torch.uint8, device="cuda")
    scales = torch.zeros(lay.n_k, dtype=torch.float32, device="cuda")
    o_codes, o_scales = np.zeros((lay.n_k, 128)), np.zeros(lay.n_k)
    for bt in batches:
        rows = np.where(bt >= 0, bt, 0)
        kb = k_raw[rows]
        dsa.dsa_indexer_k_insert(dev(kb, torch.bfloat16), dev(bt.astype(np.int64), torch.int64),
                                 cache, scales, norm_weight=dev(wgt), norm_bias=dev(bias))
        o_prep.k_norm_quant_insert(kb, wgt, bias, 1e-6, bt, o_codes, o_scales)
    torch.cuda.synchronize()
    g_codes = cache.view(torch.float8_e4m3fn).float().cpu().numpy().astype(np.float64)
    _check_cache(g_codes, host(scales).astype(np.float64), o_codes, o_scales,
                 np.ones(lay.n_k, bool), "decode cache")
    # fp8 queries with the query scale folded into the weights (no keys to prepare)
    q8, _, w_f, _ = dsa.dsa_indexer_prep(dev(q_raw), None, dev(wt), out_dtype=torch.float8_e4m3fn)
    pq = o_prep.prepare_indexer_inputs(q_raw, np.zeros((1, 128)), wt, np.zeros(lay.n_q),
                                       np.zeros(1), "fp8")
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k)
    kc = cache.view(torch.float8_e4m3fn)
    say(f"decode from the fp8 cache: n_k={lay.n_k}")
    G = host(dsa.dsa_indexer_scores(q8, kc, w_f, i32(rs), i32(re), k_scale=scales))
    idx = host(dsa.dsa_indexer_topk(q8, kc, w_f, i32(rs), i32(re), 2048, k_scale=scales))
    ndiff = 0
    for t in range(lay.n_q):
        a, b = int(rs[t]), int(re[t])
        o, c = o_idx.score_row(pq["q"][t], o_codes[a:b], pq["w"][t], o_scales[a:b], with_cond=True)
        check_scores(G[t, a:b], o, c, 2e-2, f"fp8 cache row {t}")
        full = np.full(lay.n_k, -np.inf)
        full[a:b] = o
        tau = np.zeros(lay.n_k)
        tau[a:b] = 2e-2 * np.maximum(np.abs(o), c / 128)
        oi = o_topk.topk_row(full.astype(np.float32), a, b, 2048)
        ndiff += check_topk_e2e(idx[t], oi, full, tau, f"fp8 cache row {t}")
    say(f"  selection differs from the oracle's in {ndiff} columns (within tolerance)")


# ---------------------------------------------------------------------------
# MXFP4 indexer (e2m1 values, E8M0 scale per 32 dims, scaled MFMA)
# ---------------------------------------------------------------------------
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_codes(v):
    """e2m1 values -> 4-bit codes (sign in bit 3)."""
    v = np.asarray(v, np.float64)
    mag = np.searchsorted(_E2M1, np.abs(v))
    assert np.all(_E2M1[mag] == np.abs(v)), "not an e2m1 value"
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def _e2m1_values(c):
    c = np.asarray(c, np.uint8)
    return np.where(c & 8, -1.0, 1.0) * _E2M1[c & 7]


def _pack_rows(codes):  # [..., D] e2m1 values -> [..., D/2] bytes, even element low
    c = _e2m1_codes(codes)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _unpack_rows(b):
    b = np.asarray(b, np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.float64)
    out[..., 0::2] = _e2m1_values(b & 15)
    out[..., 1::2] = _e2m1_values(b >> 4)
    return out


def mxfp4_device(p):
    """The oracle's MXFP4 operands in the library's layout: q per token = its H
    code rows then its H scale groups; k codes; k E8M0 bytes."""
    n_q, H, D = p["q_codes"].shape
    qb = _pack_rows(p["q_codes"]).reshape(n_q, H * D // 2)
    qs = (p["q_exp"] + 127).astype(np.uint8).reshape(n_q, H * D // 32)
    q = np.concatenate([qb, qs], axis=1)
    k = _pack_rows(p["k_codes"])
    ks = (p["k_exp"] + 127).astype(np.uint8)
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return u8(q), u8(k), dev(p["w"]), u8(ks)


def test_indexer_prep_mxfp4(dsa):
    lay = synth.layout_from_lengths([300, 1000])
    w = synth.WORKLOADS["fp8_64k"]
    q_raw = synth.index_q_raw(w, 0, lay.n_q)
    k_raw = synth.index_k_raw(w, 0, lay.n_k)
    wt = synth.index_weights(w, 0, lay.n_q)
    say("prep mxfp4")
    q, k, wo, ks = dsa.dsa_indexer_prep(dev(q_raw), dev(k_raw), dev(wt), out_dtype="mxfp4")
    p = o_prep.prepare_indexer_inputs(q_raw, k_raw, wt, np.zeros(lay.n_q), np.zeros(lay.n_k),
                                      "mxfp4")
    H, D = w.n_heads, w.head_dim
    gq = host(q).reshape(lay.n_q, -1)
    np.testing.assert_array_equal(_unpack_rows(gq[:, :H * D // 2].reshape(lay.n_q, H, D // 2)),
                                  p["q_codes"])                     # no norm: codes identical
    np.testing.assert_array_equal(gq[:, H * D // 2:].reshape(lay.n_q, H, D // 32).astype(int) - 127,
                                  p["q_exp"])
    np.testing.assert_array_equal(host(wo), p["w"])
    gk = _unpack_rows(host(k))
    ge = host(ks).astype(int) - 127
    same_e = ge == p["k_exp"]
    assert np.mean(same_e) > 0.999                                   # fp32 vs fp64 norm
    mism = gk != p["k_codes"]
    assert np.mean(mism) < 0.01
    rows_ok = same_e.all(axis=1)
    # a differing code is the neighbour on the e2m1 grid
    idx = lambda v: np.searchsorted(_E2M1, np.abs(v)) * np.sign(v + 0.0)
    assert np.all(np.abs(idx(gk[rows_ok]) - idx(p["k_codes"][rows_ok]))[mism[rows_ok]] <= 1)


@pytest.mark.parametrize("lens,decode", [([777], False), ([5000, 33, 12000, 20001], True)])
def test_indexer_scores_mxfp4(dsa, lens, decode):
    # the oracle's canonical MXFP4 operands on the GPU (row-block and row-split
    # kernels) against the oracle's scores on the dequantised values
    w = synth.WORKLOADS["fp8_64k"]
    lay = synth.layout_from_lengths(lens, decode=decode)
    p, rs, re = canonical_indexer(w, lay, "mxfp4", signed=True, rope=False)
    q, k, wt, ks = mxfp4_device(p)
    say(f"indexer mxfp4 lens={lens}: n_q={lay.n_q} n_k={lay.n_k}")
    G = host(dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re), k_scale=ks))
    worst = 0.0
    for t in range(0, lay.n_q, 1 if decode else 7):
        a, b = rs[t], re[t]
        o, c = o_idx.score_row(p["q"][t], p["k"][a:b], p["w"][t], with_cond=True)
        worst = max(worst, check_scores(G[t, a:b], o, c, 2e-2, f"mxfp4 row {t}"))
        assert np.isnan(G[t, :a]).all() and np.isnan(G[t, b:]).all()
    say(f"  max rel err {worst:.2e}")


@pytest.mark.parametrize("lens,decode", [([3000, 700], False), ([70000, 9000, 300], True)])
def test_indexer_topk_mxfp4(dsa, lens, decode):
    w = synth.WORKLOADS["fp8_64k"]
    lay = synth.layout_from_lengths(lens, decode=decode)
    p, rs, re = canonical_indexer(w, lay, "mxfp4", rope=False)
    q, k, wt, ks = mxfp4_device(p)
    for K in (2048, 100):
        S = dsa.dsa_indexer_scores(q, k, wt, i32(rs), i32(re), k_scale=ks)
        ref = host(dsa.dsa_topk(S, i32(rs), i32(re), K))
        got = host(dsa.dsa_indexer_topk(q, k, wt, i32(rs), i32(re), K, k_scale=ks))
        assert np.array_equal(got, ref), f"mxfp4 fused differs (K={K})"
        Sh = host(S)
        for t in list(range(0, lay.n_q, 251)) + [lay.n_q - 1]:
            np.testing.assert_array_equal(ref[t], o_topk.topk_row(Sh[t], rs[t], re[t], K))
