"""CPU oracle for the DSA hot path (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``sparse_attention_08_amd``) and imports nothing from it.

Each function is the plain definition of one step, written out in float64:

* ``prep``     index-key LayerNorm, index RoPE, bf16 / e4m3 rounding, power-of-two
               (UE8M0) block scales, query-scale fold into the head weights.
* ``indexer``  lightning-indexer scores over each row's key window.
* ``topk``     per-row top-k with window masking, lowest-index ties, -inf
               excluded, ascending-index output and -1 padding.
* ``mla``      softmax attention restricted to the selected latent rows.
* ``windows``  per-row key windows from cu_seqlens, and the packed-offset rebase.

Sources are the three pages this method is described on: the vime docs page
"Day-0 Model Plugins", the vime pull request #502 with its review comments, and
the vLLM API page "vllm.models.kimi_k3.nvidia.dsa".  Where the pages leave a step
open the reading adopted is stated in the function's docstring.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or hand-computed fixtures;
none is "parity unpinned".
"""
from . import prep, indexer, topk, mla, windows  # noqa: F401
