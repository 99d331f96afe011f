"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse MLA).

This module only draws random numbers and lays out the packed-sequence
structure (sequence lengths, cu_seqlens, per-sample positions).  It holds none
of the method's arithmetic: the key LayerNorm, RoPE, quantisation, scoring,
selection and attention all live on each side separately (the CPU oracle and
the HIP library).  Both sides take their raw inputs from here.

Every tensor is generated in row blocks of ``BLOCK_ROWS`` rows from its own
numpy Generator seeded with ``[0xD5A, config_id, tensor_id, block]``, so any row
range can be regenerated on its own without materialising the whole tensor.

Workloads (shapes follow the DeepSeek-V3.2-style DSA layer described on the
vLLM API page "vllm.models.kimi_k3.nvidia.dsa": one shared index key per token,
per-head index weights, index_topk selected keys, MLA over a 512+64 latent row):

* ``tiny``     one causal sequence T=256, fp32; indexer 4 heads x 32 dims,
               index_topk 16; MLA 8 heads, d_qk 64, d_v 32.
* ``prefill4k`` one causal sequence T=4096, bf16; indexer 64 x 128 with RoPE on
               the leading 64 dims; index_topk 2048; MLA 128 heads, 576/512.
* ``thd``      8 packed sequences with lengths ~U{512..8192}, bf16, otherwise
               as prefill4k; invalid score columns hold +-1e4 garbage.
* ``decode``   64 single-token queries with their own caches of ~U{16384..131072}
               keys, bf16; no RoPE.
* ``fp8_64k``  one causal sequence T=65536; indexer q/k quantised to e4m3 with
               power-of-two scales; MLA in bf16.
"""
from __future__ import annotations

import dataclasses
import numpy as np

BLOCK_ROWS = 4096
SEED_ROOT = 0xD5A

# tensor ids inside a config's seed
T_LENGTHS, T_IDX_Q, T_IDX_K, T_IDX_W, T_MLA_Q, T_MLA_KV, T_GARBAGE, T_SIGN = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    dtype: str                 # "f32" | "bf16" | "fp8"  (indexer input type)
    mla_dtype: str             # "f32" | "bf16"
    n_heads: int               # index heads H
    head_dim: int              # index head dim D
    index_topk: int            # K
    mla_heads: int             # Hm
    d_qk: int
    d_v: int
    rope_dim: int              # leading index dims that get RoPE (0 = none)
    rope_main_dim: int         # rotary dim of the main attention cache
    rope_theta: float
    mla_scale: float           # std of MLA q / kv draws
    decode: bool               # one query per sequence, window = whole cache
    fixed_len: int = 0         # single causal sequence length
    n_seqs: int = 1
    len_lo: int = 0
    len_hi: int = 0
    garbage: bool = False      # pre-fill invalid score columns with +-1e4

    @property
    def sm_scale(self) -> float:
        return float(self.d_qk) ** -0.5


WORKLOADS = {
    "tiny": Workload("tiny", 1, "f32", "f32", 4, 32, 16, 8, 64, 32, 0, 0, 1e4,
                     1.0, False, fixed_len=256),
    "prefill4k": Workload("prefill4k", 2, "bf16", "bf16", 64, 128, 2048, 128, 576, 512,
                          64, 64, 1e4, 0.1, False, fixed_len=4096),
    "thd": Workload("thd", 3, "bf16", "bf16", 64, 128, 2048, 128, 576, 512,
                    64, 64, 1e4, 0.1, False, n_seqs=8, len_lo=512, len_hi=8192,
                    garbage=True),
    "decode": Workload("decode", 4, "bf16", "bf16", 64, 128, 2048, 128, 576, 512,
                       0, 0, 1e4, 0.1, True, n_seqs=64, len_lo=16384, len_hi=131072),
    "fp8_64k": Workload("fp8_64k", 5, "fp8", "bf16", 64, 128, 2048, 128, 576, 512,
                        0, 0, 1e4, 0.1, False, fixed_len=65536),
}


def rng(config_id: int, tensor_id: int, block: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, config_id, tensor_id, block])


# ----------------------------------------------------------------------------
# packed-sequence structure
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Layout:
    """Packed (THD) layout of one workload.

    ``k_lens[b]`` keys and ``q_lens[b]`` queries per sequence; the queries of a
    sequence are its last ``q_lens[b]`` tokens.  ``cu_q``/``cu_k`` are the
    exclusive prefix sums (int32, length n_seqs+1).
    """
    q_lens: np.ndarray
    k_lens: np.ndarray

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.k_lens)]).astype(np.int32)

    @property
    def n_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def n_k(self) -> int:
        return int(self.k_lens.sum())

    def positions(self) -> np.ndarray:
        """Position of every query token inside its own sequence (int64)."""
        out = np.empty(self.n_q, np.int64)
        cq = self.cu_q
        for b in range(len(self.q_lens)):
            ql, kl = int(self.q_lens[b]), int(self.k_lens[b])
            out[cq[b]:cq[b + 1]] = np.arange(kl - ql, kl)
        return out

    def key_positions(self) -> np.ndarray:
        out = np.empty(self.n_k, np.int64)
        ck = self.cu_k
        for b in range(len(self.k_lens)):
            out[ck[b]:ck[b + 1]] = np.arange(int(self.k_lens[b]))
        return out


def layout(w: Workload, n_seqs: int | None = None) -> Layout:
    if w.fixed_len:
        lens = np.array([w.fixed_len], np.int64)
    else:
        ns = w.n_seqs if n_seqs is None else n_seqs
        lens = rng(w.config_id, T_LENGTHS).integers(w.len_lo, w.len_hi + 1, size=w.n_seqs)
        lens = lens[:ns].astype(np.int64)
    if w.decode:
        return Layout(np.ones_like(lens), lens)
    return Layout(lens.copy(), lens)


def layout_from_lengths(lens, decode: bool = False) -> Layout:
    lens = np.asarray(lens, np.int64)
    return Layout(np.ones_like(lens) if decode else lens.copy(), lens)


# ----------------------------------------------------------------------------
# row-blocked draws
# ----------------------------------------------------------------------------
def _blocked(config_id, tensor_id, r0, r1, row_shape, draw):
    """Rows [r0, r1) of a tensor drawn block by block (float32)."""
    out = np.empty((r1 - r0,) + tuple(row_shape), np.float32)
    b0, b1 = r0 // BLOCK_ROWS, (r1 - 1) // BLOCK_ROWS if r1 > r0 else -1
    for b in range(b0, b1 + 1):
        g = rng(config_id, tensor_id, b)
        blk = draw(g, (BLOCK_ROWS,) + tuple(row_shape))
        lo, hi = max(r0, b * BLOCK_ROWS), min(r1, (b + 1) * BLOCK_ROWS)
        out[lo - r0:hi - r0] = blk[lo - b * BLOCK_ROWS:hi - b * BLOCK_ROWS]
    return out


def _normal(g, shape):
    return g.standard_normal(shape, dtype=np.float32)


def _uniform(g, shape):
    return g.random(shape, dtype=np.float32)


def index_q_raw(w: Workload, r0: int, r1: int) -> np.ndarray:
    """Raw index queries [rows, H, D] ~ N(0,1), float32."""
    return _blocked(w.config_id, T_IDX_Q, r0, r1, (w.n_heads, w.head_dim), _normal)


def index_k_raw(w: Workload, r0: int, r1: int) -> np.ndarray:
    """Raw (pre-LayerNorm) index keys [rows, D] ~ N(0,1), float32."""
    return _blocked(w.config_id, T_IDX_K, r0, r1, (w.head_dim,), _normal)


def index_weights(w: Workload, r0: int, r1: int, signed: bool = False) -> np.ndarray:
    """Per-head index weights [rows, H] ~ U(0,1) (or N(0,1) when ``signed``)."""
    if signed:
        return _blocked(w.config_id, T_SIGN, r0, r1, (w.n_heads,), _normal)
    return _blocked(w.config_id, T_IDX_W, r0, r1, (w.n_heads,), _uniform)


def mla_q(w: Workload, r0: int, r1: int) -> np.ndarray:
    """MLA queries [rows, Hm, d_qk] ~ N(0,1)*scale, float32."""
    x = _blocked(w.config_id, T_MLA_Q, r0, r1, (w.mla_heads, w.d_qk), _normal)
    if w.mla_scale != 1.0:
        x *= np.float32(w.mla_scale)
    return x


def mla_kv(w: Workload, r0: int, r1: int) -> np.ndarray:
    """Latent KV rows [rows, d_qk] (latent dims then rope dims) ~ N(0,1)*scale."""
    x = _blocked(w.config_id, T_MLA_KV, r0, r1, (w.d_qk,), _normal)
    if w.mla_scale != 1.0:
        x *= np.float32(w.mla_scale)
    return x


def garbage(w: Workload, r0: int, r1: int, n_cols: int) -> np.ndarray:
    """+-1e4 with random sign, [rows, n_cols] float32 (invalid score columns)."""
    g = rng(w.config_id, T_GARBAGE, r0)
    s = g.integers(0, 2, size=(r1 - r0, n_cols), dtype=np.int8)
    return np.where(s == 1, np.float32(1e4), np.float32(-1e4)).astype(np.float32)


def sample_rows(n_rows: int, index_topk: int, seed: int, n_random: int = 256,
                starts=(0,)) -> np.ndarray:
    """Stratified row sample: first rows, rows around index_topk and the last
    row of each sequence start, plus ``n_random`` seeded random rows."""
    picks = set()
    for s0 in starts:
        for r in (0, 1, 2, index_topk - 2, index_topk - 1, index_topk, index_topk + 1):
            if 0 <= s0 + r < n_rows:
                picks.add(s0 + r)
    picks.add(n_rows - 1)
    g = np.random.default_rng([SEED_ROOT, 99, seed])
    picks.update(int(x) for x in g.integers(0, n_rows, size=min(n_random, n_rows)))
    return np.array(sorted(picks), np.int64)


# ----------------------------------------------------------------------------
# device-side draws for large tensors (torch's counter-based Philox generator,
# seeded per config and tensor).  Both sides read the same device tensor: the
# kernels directly, the oracle through a host copy of the rows it checks.
# ----------------------------------------------------------------------------
def _torch_seed(config_id: int, tensor_id: int, salt: int = 0) -> int:
    return (SEED_ROOT << 32) ^ (config_id << 20) ^ (tensor_id << 8) ^ salt


def device_normal(w: Workload, tensor_id: int, shape, device, scale: float = 1.0, salt: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(w.config_id, tensor_id, salt))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x


def device_uniform(w: Workload, tensor_id: int, shape, device, salt: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(w.config_id, tensor_id, salt))
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)


def device_inputs(w: Workload, device, lay: Layout | None = None, mla: bool = True,
                  signed_weights: bool = False):
    """Raw fp32 device tensors of a workload: index q [Nq,H,D], index k [Nk,D],
    weights [Nq,H], MLA q [Nq,Hm,d_qk] and latent kv [Nk,d_qk] (when ``mla``)."""
    lay = layout(w) if lay is None else lay
    out = dict(layout=lay)
    out["q_raw"] = device_normal(w, T_IDX_Q, (lay.n_q, w.n_heads, w.head_dim), device)
    out["k_raw"] = device_normal(w, T_IDX_K, (lay.n_k, w.head_dim), device)
    out["w"] = (device_normal(w, T_SIGN, (lay.n_q, w.n_heads), device) if signed_weights
                else device_uniform(w, T_IDX_W, (lay.n_q, w.n_heads), device))
    if mla:
        out["mla_q"] = device_normal(w, T_MLA_Q, (lay.n_q, w.mla_heads, w.d_qk), device, w.mla_scale)
        out["mla_kv"] = device_normal(w, T_MLA_KV, (lay.n_k, w.d_qk), device, w.mla_scale)
    return out


def device_garbage(w: Workload, shape, device):
    """+-1e4 with random sign (device tensor): what a score buffer holds outside
    the rows' windows before the indexer writes the in-window entries."""
    import torch
    u = device_uniform(w, T_GARBAGE, shape, device)
    return torch.where(u < 0.5, torch.tensor(1e4, device=device), torch.tensor(-1e4, device=device))
