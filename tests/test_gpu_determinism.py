"""Every entry point run twice on the same inputs gives the same bits.

No kernel accumulates through atomics or in an order that depends on timing:
the indexer and the attention accumulate in a fixed order, the top-k's
atomics only count (the selection is decided by the key values), the split
attention is merged in split order.  This checks it on prefill and decode
shapes, composed and fused, direct and split launches, bf16 and fp8 operands,
and the cache inserts."""
import numpy as np
import pytest
import torch

import synth
from parity import dev, i32, say

pytestmark = pytest.mark.gpu

P4K = synth.WORKLOADS["prefill4k"]


def _same(run, what):
    a = run()
    torch.cuda.synchronize()
    a = [x.clone() for x in a]
    b = run()
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), \
            f"{what}: output {i} differs between two runs"


@pytest.mark.parametrize("lens,decode", [([5000], False), ([3000, 9000], True)])
def test_indexer_topk_deterministic(dsa, lens, decode):
    say(f"determinism indexer/top-k lens={lens} decode={decode}")
    w = P4K
    lay = synth.layout_from_lengths(lens, decode)
    q_raw = dev(synth.index_q_raw(w, 0, lay.n_q))
    k_raw = dev(synth.index_k_raw(w, 0, lay.n_k))
    wt = dev(synth.index_weights(w, 0, lay.n_q))
    pos_q, pos_k = i32(lay.positions()), i32(lay.key_positions())
    rs, re = dsa.dsa_row_windows(i32(lay.cu_q), i32(lay.cu_k), lay.n_q)
    K = 2048
    for dt in (torch.bfloat16, torch.float8_e4m3fn):
        rope = w.rope_dim if dt == torch.bfloat16 else 0
        _same(lambda: [t for t in dsa.dsa_indexer_prep(q_raw, k_raw, wt, pos_q, pos_k, dt, rope,
                                                       w.rope_main_dim, w.rope_theta)
                       if t is not None], f"prep {dt}")
        q, k, wd, ks = dsa.dsa_indexer_prep(q_raw, k_raw, wt, pos_q, pos_k, dt, rope,
                                            w.rope_main_dim, w.rope_theta)
        S = torch.full((lay.n_q, lay.n_k), float("-inf"), dtype=torch.float32, device="cuda")

        def scores():
            dsa.dsa_indexer_scores(q, k, wd, rs, re, k_scale=ks, scores=S)
            return [S]
        _same(scores, f"scores {dt}")
        _same(lambda: [dsa.dsa_topk(S, rs, re, K)], f"top-k {dt}")
        _same(lambda: [dsa.dsa_indexer_topk(q, k, wd, rs, re, K, k_scale=ks)], f"fused {dt}")


@pytest.mark.parametrize("n_q", [8, 300])
def test_sparse_mla_deterministic(dsa, n_q):
    # 8 queries: the split launch and its combine; 300: one workgroup per query
    say(f"determinism sparse MLA n_q={n_q}")
    g = np.random.default_rng(611)
    n_kv, K = 6000, 2048
    q = dev(synth.mla_q(P4K, 0, n_q), torch.bfloat16)
    kv = dev(synth.mla_kv(P4K, 0, n_kv), torch.bfloat16)
    idx = np.sort(g.integers(0, n_kv, (n_q, K)), axis=1).astype(np.int32)
    idx[:, K - 100:] = -1  # -1 padding at the end, as top-k writes it
    idx = i32(idx)
    cache = torch.empty((n_kv, dsa.MLA_FP8_ROW_BYTES), dtype=torch.uint8, device="cuda")
    slots = torch.arange(n_kv, dtype=torch.int64, device="cuda")

    def insert():
        dsa.dsa_mla_kv_insert(kv, slots, cache)
        return [cache]
    _same(insert, "latent insert")
    for rows in (kv, cache):
        _same(lambda: list(dsa.dsa_sparse_mla_fwd(q, rows, idx, P4K.sm_scale, P4K.d_v)),
              f"sparse MLA ({'bf16' if rows is kv else 'fp8'} rows)")


def test_key_insert_deterministic(dsa):
    say("determinism key insert")
    n = 5000
    k_raw = dev(synth.index_k_raw(P4K, 0, n), torch.bfloat16)
    slots = torch.arange(n, dtype=torch.int64, device="cuda")
    kc = torch.empty((n, 128), dtype=torch.float8_e4m3fn, device="cuda")
    ksc = torch.empty(n, dtype=torch.float32, device="cuda")

    def run():
        dsa.dsa_indexer_k_insert(k_raw, slots, kc, ksc)
        return [kc, ksc]
    _same(run, "key insert")
