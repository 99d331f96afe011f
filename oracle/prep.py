"""Input preparation before the indexer, float64 (oracle; test infrastructure).

Follows the vLLM API page "vllm.models.kimi_k3.nvidia.dsa":

* ``KimiK3DSAIndexerKNorm``: the shared index key goes through a LayerNorm with
  weight 1 and bias 0 (the page computes it in fp32 and casts back; here it is
  computed in float64 and rounded once to the target format).
* ``KimiK3DSAIndexer._apply_index_rope``: RoPE on the leading ``index_rope_dim``
  dims of each head, half-split ("neox") pairing, frequencies taken from the
  leading ``index_rope_dim/2`` frequencies of the main attention's rotary cache,
  applied after the key norm.
* ``KimiK3DSAIndexer.__init__`` (scale format comment) and ``score``: index
  scales are powers of two ("ue8m0"), one per ``index_head_dim`` block, read as
  fp32; the query scale is folded into the per-head weights.

Readings where the page is silent (each listed in the design notes):
* LayerNorm uses the biased variance and eps = 1e-6.
* A power-of-two scale is the smallest power of two s with amax <= 448*s (so no
  element saturates); an all-zero block gets s = 1.  Elements are rounded to
  OCP E4M3FN (max 448) with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ----------------------------------------------------------------------------
# rounding to narrow formats (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def _round_format(x, mant_bits: int, emin: int) -> np.ndarray:
    """Round float64 values to a binary format with ``mant_bits`` stored
    mantissa bits and minimum normal exponent ``emin`` (no overflow handling).

    The spacing of representable values around x is 2**(max(e, emin) - mant_bits)
    with e = floor(log2|x|); scaling by that power of two is exact in float64, so
    ``np.rint`` (ties to even) performs the rounding exactly."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e - 1, emin)             # floor(log2|x|), clamped to subnormals
    q = (e - mant_bits).astype(np.float64)
    return np.rint(np.ldexp(x, (-q).astype(np.int64))) * np.exp2(q)


def round_bf16(x) -> np.ndarray:
    """bfloat16 (8 significant bits, fp32 exponent range), RNE."""
    return _round_format(x, 7, -126)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def round_e2m1(x) -> np.ndarray:
    """OCP FP4 E2M1 (the MXFP4 element type): 1 mantissa bit, min normal 1,
    subnormal step 0.5, max 6; values are clamped to +-6 before rounding
    (the MX conversion saturates)."""
    x = np.clip(np.asarray(x, np.float64), -6.0, 6.0)
    return _round_format(x, 1, 0)


def round_e4m3(x) -> np.ndarray:
    """OCP E4M3FN: 3 mantissa bits, min normal 2**-6, subnormal step 2**-9,
    max 448.  Values are clamped to +-448 before rounding."""
    x = np.clip(np.asarray(x, np.float64), -E4M3_MAX, E4M3_MAX)
    return _round_format(x, 3, -6)


# ----------------------------------------------------------------------------
# LayerNorm (KimiK3DSAIndexerKNorm)
# ----------------------------------------------------------------------------
def layer_norm(x, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm over the last axis with weight 1, bias 0, biased variance."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    d = x - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    return d / np.sqrt(var + eps)


def layer_norm_affine(x, weight=None, bias=None, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm over the last axis followed by the per-dim weight and bias
    (KimiK3DSAIndexerKNorm holds both; weight None = 1, bias None = 0)."""
    y = layer_norm(x, eps)
    if weight is not None:
        y = y * np.asarray(weight, np.float64)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y


# ----------------------------------------------------------------------------
# RoPE on the leading dims, half-split pairing (_apply_index_rope)
# ----------------------------------------------------------------------------
def rope_inv_freq(rope_dim: int, rope_main_dim: int, theta: float) -> np.ndarray:
    """Leading rope_dim/2 frequencies of a rotary cache of dim rope_main_dim:
    inv_freq[i] = theta ** (-2 i / rope_main_dim)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / rope_main_dim)


def rope_leading(x, positions, rope_dim: int, rope_main_dim: int, theta: float) -> np.ndarray:
    """Rotate dims [0, rope_dim) of the last axis; dim i pairs with i + rope_dim/2.

    ``x`` is [T, ..., D]; ``positions`` is [T].  Dims >= rope_dim are unchanged."""
    x = np.array(x, np.float64, copy=True)
    if rope_dim == 0:
        return x
    half = rope_dim // 2
    ang = np.asarray(positions, np.float64)[:, None] * rope_inv_freq(rope_dim, rope_main_dim, theta)[None, :]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    a, b = x[..., :half].copy(), x[..., half:rope_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rope_dim] = b * c + a * s
    return x


# ----------------------------------------------------------------------------
# power-of-two block scales + e4m3 (score(): fp8 query, scale folded into weights)
# ----------------------------------------------------------------------------
def ue8m0_scale(amax) -> np.ndarray:
    """Smallest power of two s with amax <= 448*s; 1 where amax == 0."""
    amax = np.asarray(amax, np.float64)
    r = amax / E4M3_MAX
    m, e = np.frexp(np.where(r > 0, r, 1.0))
    # r = m * 2**e with 0.5 <= m < 1: r is itself a power of two iff m == 0.5
    p = np.where(m == 0.5, e - 1, e)
    s = np.exp2(p.astype(np.float64))
    # guard the division rounding: make sure amax <= 448*s and s/2 would not do
    s = np.where(amax > E4M3_MAX * s, s * 2, s)
    s = np.where((amax > 0) & (amax <= E4M3_MAX * s / 2), s / 2, s)
    return np.where(amax > 0, s, 1.0)


def quant_e4m3_blocks(x, block: int):
    """Quantise the last axis in blocks of ``block`` elements.

    Returns (codes, scales): ``codes`` holds the e4m3 values (as float64),
    ``scales`` [..., D/block] the power-of-two scales; x ~= codes * scale."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    assert D % block == 0
    xb = x.reshape(x.shape[:-1] + (D // block, block))
    s = ue8m0_scale(np.abs(xb).max(axis=-1))
    codes = round_e4m3(xb / s[..., None])
    return codes.reshape(x.shape), s


def mx_scale_exponent(amax) -> np.ndarray:
    """MXFP4 shared scale (OCP Microscaling format, block of 32): X = 2^e with
    e = floor(log2 amax) - 2 (2 = the largest exponent of E2M1); amax = 0 gives
    e = 0.  The E8M0 byte is e + 127."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # amax = m 2^e, 0.5 <= m < 1
    return np.where(amax > 0, (e - 1) - 2, 0).astype(np.int64)


def quant_mxfp4_blocks(x, block: int = 32):
    """MXFP4 along the last axis: returns (codes, scale_exp) with codes the E2M1
    values (float64) and scale_exp [..., D/block] the scale exponents;
    x ~= codes * 2^scale_exp per block (values of |x| / 2^e in [6, 8) saturate)."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    assert D % block == 0
    xb = x.reshape(x.shape[:-1] + (D // block, block))
    e = mx_scale_exponent(np.abs(xb).max(axis=-1))
    codes = round_e2m1(xb / np.exp2(e)[..., None].astype(np.float64))
    return codes.reshape(x.shape), e


def fold_q_scale(w, q_scale) -> np.ndarray:
    """score() folds the per-(token, head) query scale into the head weights."""
    return np.asarray(w, np.float64) * np.asarray(q_scale, np.float64)


# ----------------------------------------------------------------------------
# whole-workload preparation (what the indexer consumes)
# ----------------------------------------------------------------------------
def prepare_indexer_inputs(q_raw, k_raw, w, positions_q, positions_k, dtype: str,
                           rope_dim: int = 0, rope_main_dim: int = 0,
                           theta: float = 1e4, eps: float = 1e-6):
    """key LayerNorm -> RoPE (q and k) -> round to ``dtype``.

    dtype "f32"/"bf16": returns dict(q, k, w, k_scale=None), values exactly
    representable in that format (float64 arrays).
    dtype "fp8": q and k are e4m3 codes, ``k_scale`` [Nk] and the folded
    weights w*q_scale [Nq, H]; the score is k_scale[s] * sum_h w'[t,h] relu(q8.k8).
    """
    k = layer_norm(k_raw, eps)
    q = np.asarray(q_raw, np.float64)
    if rope_dim:
        q = rope_leading(q, positions_q, rope_dim, rope_main_dim, theta)
        k = rope_leading(k, positions_k, rope_dim, rope_main_dim, theta)
    w = np.asarray(w, np.float64)
    if dtype == "f32":
        return dict(q=round_f32(q), k=round_f32(k), w=round_f32(w), k_scale=None)
    if dtype == "bf16":
        return dict(q=round_bf16(q), k=round_bf16(k), w=round_f32(w), k_scale=None)
    if dtype == "fp8":
        D = q.shape[-1]
        q8, sq = quant_e4m3_blocks(q, D)          # sq [Nq, H, 1]
        k8, sk = quant_e4m3_blocks(k, D)          # sk [Nk, 1]
        wf = round_f32(fold_q_scale(w, sq[..., 0]))
        return dict(q=q8, k=k8, w=wf, k_scale=sk[:, 0])
    if dtype == "mxfp4":
        # block scales per 32 dims on both sides (not foldable into per-head
        # weights): the operands are handed over dequantised, with the codes
        # and scale exponents alongside
        q4, eq = quant_mxfp4_blocks(q)            # eq [Nq, H, D/32]
        k4, ek = quant_mxfp4_blocks(k)            # ek [Nk, D/32]
        qd = q4 * np.repeat(np.exp2(eq.astype(np.float64)), 32, axis=-1)
        kd = k4 * np.repeat(np.exp2(ek.astype(np.float64)), 32, axis=-1)
        return dict(q=qd, k=kd, w=round_f32(w), k_scale=None, q_codes=q4, q_exp=eq,
                    k_codes=k4, k_exp=ek)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# the fp8 index-key cache and its fused insert
# ----------------------------------------------------------------------------
def k_norm_quant_insert(k_raw, weight, bias, eps, slot_mapping, cache_codes, cache_scales):
    """The index-key cache insert of KimiK3DSAIndexer._fused_k_insert (vLLM API
    page "vllm.models.kimi_k3.nvidia.dsa"): each new key row goes through the
    key LayerNorm (with the norm's weight and bias; the fused insert is used
    only without index rope), is quantised to e4m3 with one power-of-two
    ("ue8m0") scale for its index_head_dim block, and is written to the cache
    slot slot_mapping[i].

    Readings: a negative slot is a padding token and writes nothing; so does a
    slot past the cache (the insert never writes outside it); every other slot
    keeps its contents; two tokens never share a slot.  cache_codes [n_slots, D]
    (e4m3 values as float64) and cache_scales [n_slots] are updated in place
    and returned."""
    y = layer_norm_affine(k_raw, weight, bias, eps)
    codes, s = quant_e4m3_blocks(y, y.shape[-1])
    slots = np.asarray(slot_mapping, np.int64)
    ok = (slots >= 0) & (slots < cache_codes.shape[0])
    cache_codes[slots[ok]] = codes[ok]
    cache_scales[slots[ok]] = s[ok, 0]
    return cache_codes, cache_scales


# ----------------------------------------------------------------------------
# the fp8 latent KV cache of the sparse MLA ("fp8_ds_mla")
# ----------------------------------------------------------------------------
def mla_kv_quant(kv, d_latent: int = 512, block: int = 128):
    """A latent row in the fp8 cache format that KimiK3DSAAttention selects with
    kv_cache_dtype "fp8_ds_mla" (vLLM API page "vllm.models.kimi_k3.nvidia.dsa";
    the page names the format, not its layout).

    Readings: the d_latent latent dims (the value, and the first d_latent dims
    of the key) are e4m3 codes with one fp32 scale per `block` dims, chosen by
    the power-of-two rule of the index cache (the smallest power of two s with
    amax <= 448 s); the rope dims after them stay bf16.  Returns (codes
    [N, d_latent], scales [N, d_latent/block], rope [N, d_qk - d_latent]); the
    row the attention reads is dequant_mla_kv(codes, scales, rope)."""
    kv = np.asarray(kv, np.float64)
    codes, s = quant_e4m3_blocks(kv[:, :d_latent], block)
    return codes, s, round_bf16(kv[:, d_latent:])


def dequant_mla_kv(codes, scales, rope, block: int = 128) -> np.ndarray:
    """The latent row the attention reads: codes * scale of each block, then the
    rope dims."""
    lat = np.asarray(codes, np.float64) * np.repeat(np.asarray(scales, np.float64), block, axis=-1)
    return np.concatenate([lat, np.asarray(rope, np.float64)], axis=-1)
