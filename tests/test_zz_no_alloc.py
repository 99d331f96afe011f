"""dsa_indexer_topk_noalloc (the library's own scratch array as workspace)
against dsa_indexer_topk (a caller workspace): identical indices, on two calls
in a row, the second with a smaller input, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from oracle import prep as o_prep
from oracle import windows as o_win
from parity import dev, i32, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["decode"]


def _operands(lens, dtype):
    lay = synth.layout_from_lengths(lens, decode=True)
    q_raw = synth.index_q_raw(W, 0, lay.n_q)
    k_raw = synth.index_k_raw(W, 0, lay.n_k)
    wt = synth.index_weights(W, 0, lay.n_q)
    p = o_prep.prepare_indexer_inputs(q_raw, k_raw, wt, lay.positions(), lay.key_positions(), dtype)
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float8_e4m3fn
    ks = None if p["k_scale"] is None else dev(p["k_scale"])
    return dev(p["q"], tdt), dev(p["k"], tdt), dev(p["w"]), ks, i32(rs), i32(re)


def test_noalloc_matches_workspace_call(dsa):
    lib = dsa._lib_or_load()
    # windows longer than 8192 keys take the split path, whose candidates live
    # in the workspace; the second call is smaller and reuses the array
    calls = [([70000, 9000, 300, 20000, 131072, 8193] * 4, "bf16", 2048),
             ([12000, 50, 9000], "fp8", 700)]
    for lens, dtype, K in calls:
        q, k, w, ks, rs, re = _operands(lens, dtype)
        need = lib.dsa_indexer_topk_workspace_size(q.shape[0], k.shape[0], q.shape[1], q.shape[2],
                                                   dsa._dtype_code(q), K)
        say(f"noalloc {dtype}: n_q={q.shape[0]} n_k={k.shape[0]} K={K} workspace {need} B")
        assert 0 < need <= lib_scratch_bytes()
        ref = dsa.dsa_indexer_topk(q, k, w, rs, re, K, k_scale=ks)
        got = dsa.dsa_indexer_topk_noalloc(q, k, w, rs, re, K, k_scale=ks)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert (got.cpu().numpy() >= -1).all()
    # a call that needs no workspace at all (windows of at most 8192 keys)
    q, k, w, ks, rs, re = _operands([5000, 17, 8192], "bf16")
    ref = dsa.dsa_indexer_topk(q, k, w, rs, re, 2048)
    got = dsa.dsa_indexer_topk_noalloc(q, k, w, rs, re, 2048)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_noalloc_rejects_more_than_the_array(dsa):
    # 256 decode rows over windows of more than 8192 keys: 256 x 262208 B > 64 MiB
    # (more rows take the prefill kernel, which needs no workspace)
    q, k, w, ks, rs, re = _operands([9000] * 256, "bf16")
    out = torch.full((256, 2048), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DSAError, match="workspace"):
        dsa.dsa_indexer_topk_noalloc(q, k, w, rs, re, 2048, out=out)
    torch.cuda.synchronize()
    assert (out == -7).all()                                   # nothing was enqueued


def lib_scratch_bytes():
    return 64 << 20
