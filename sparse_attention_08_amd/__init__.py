"""Python binding of the DSA hot-path library (``libdsa.so``, HIP for gfx950).

Argument marshalling only: every step of the path runs in the library's
kernels.  Tensors are torch CUDA (HIP) tensors; each call is enqueued on the
current torch stream.  The entry points carry the names of the C ABI in
``include/dsa.h``:

    dsa_row_windows, dsa_indexer_prep, dsa_indexer_k_insert, dsa_indexer_scores,
    dsa_topk, dsa_indexer_topk, dsa_indexer_topk_noalloc, dsa_mla_kv_insert,
    dsa_sparse_mla_fwd (+ workspace-size queries)

A nonzero status raises ``DSAError``.  Importing this package does not load
the library; ``load()`` does, and fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3, DTYPE_MXFP4 = 0, 1, 2, 3

_lib = None


class DSAError(RuntimeError):
    pass


def _hip_runtimes_in_process():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def load(path: str = LIB_PATH):
    """Load libdsa.so (after torch, so that it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime the tensors come from)
    if not os.path.exists(path):
        raise DSAError(f"{path} not found: build it with python -m sparse_attention_08_amd._build")
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_in_process()
    if len(runtimes) > 1:
        raise DSAError(f"more than one HIP runtime loaded: {runtimes}")
    _declare(lib)
    _lib = lib
    return lib


def _declare(lib):
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dsa_version": (ctypes.c_int, []),
        "dsa_row_windows": (ctypes.c_int, [P, P, I32, I64, I32, P, P, P]),
        "dsa_indexer_prep": (ctypes.c_int, [P, P, P, P, P, I64, I64, I32, I32, I32, I32, F32, F32,
                                            I32, P, P, P, P, P]),
        "dsa_indexer_k_insert": (ctypes.c_int, [P, I32, P, P, F32, P, I64, I32, P, P, I64, P]),
        "dsa_mla_kv_insert": (ctypes.c_int, [P, I32, P, I64, I32, P, I64, P]),
        "dsa_indexer_scores": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I32, I32, I32, P, I64, P]),
        "dsa_topk_workspace_size": (SZ, [I64, I64, I32]),
        "dsa_topk": (ctypes.c_int, [P, I64, P, P, I64, I64, I32, P, P, SZ, P]),
        "dsa_indexer_topk_workspace_size": (SZ, [I64, I64, I32, I32, I32, I32]),
        "dsa_indexer_topk": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I32, I32, I32, I32, P, P,
                                            SZ, P]),
        "dsa_indexer_topk_noalloc": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I32, I32, I32,
                                                    I32, P, P]),
        "dsa_sparse_mla_workspace_size": (SZ, [I64, I32, I32, I32, I32, I32]),
        "dsa_sparse_mla_fwd": (ctypes.c_int, [P, P, P, I64, I64, I32, I32, I32, I32, F32, I32, P, P,
                                              P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


EXPORTS = ("dsa_status_string", "dsa_version", "dsa_row_windows", "dsa_indexer_prep",
           "dsa_indexer_k_insert", "dsa_indexer_scores", "dsa_topk_workspace_size", "dsa_topk",
           "dsa_indexer_topk_workspace_size", "dsa_indexer_topk", "dsa_indexer_topk_noalloc",
           "dsa_mla_kv_insert", "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_fwd")


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise DSAError("expected a device tensor")
    if not t.is_contiguous():
        raise DSAError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream=None):
    """Context in which outputs and workspaces are allocated: the stream the
    kernels run on, so that torch's caching allocator does not hand a workspace
    to another stream's allocation while the kernels still use it."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check(status: int, what: str):
    if status != 0:
        msg = _lib.dsa_status_string(status).decode()
        raise DSAError(f"{what} failed: {msg} ({status})")


def _dtype_code(t) -> int:
    """Operand format of a tensor; MXFP4 operands are uint8 buffers."""
    import torch
    return {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16,
            torch.float8_e4m3fn: DTYPE_FP8_E4M3, torch.uint8: DTYPE_MXFP4}[t.dtype]


def _indexer_dims(q, k, w):
    """(n_q, n_heads, head_dim): from q [n_q, H, D], or for MXFP4 (uint8 q of
    H * (D/2 + D/32) bytes per token) from w [n_q, H] and k [n_k, D/2]."""
    import torch
    if q.dtype == torch.uint8:
        return q.shape[0], w.shape[1], k.shape[1] * 2
    return q.shape


def _lib_or_load():
    return _lib if _lib is not None else load()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def dsa_row_windows(cu_seqlens_q, cu_seqlens_k, n_rows: int, causal: bool = True,
                    row_starts=None, row_ends=None, stream=None):
    import torch
    lib = _lib_or_load()
    dev = cu_seqlens_q.device
    with _on(stream):
        rs = torch.empty(n_rows, dtype=torch.int32, device=dev) if row_starts is None else row_starts
        re = torch.empty(n_rows, dtype=torch.int32, device=dev) if row_ends is None else row_ends
    _check(lib.dsa_row_windows(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1,
                               n_rows, int(causal), _ptr(rs), _ptr(re), _stream(stream)),
           "dsa_row_windows")
    return rs, re


def dsa_indexer_prep(q_raw, k_raw, w, pos_q=None, pos_k=None, out_dtype=None, rope_dim: int = 0,
                     rope_main_dim: int = 0, rope_theta: float = 1e4, eps: float = 1e-6,
                     stream=None):
    """Returns (q, k, w_out, k_scale) in out_dtype (k_scale is None unless fp8 or
    mxfp4; k and k_scale are None when k_raw is None: queries only, e.g. a
    decode step over a key cache).  out_dtype "mxfp4": q uint8 [n_q, H*(D/2+D/32)],
    k uint8 [n_k, D/2], k_scale uint8 [n_k, D/32] (E8M0)."""
    import torch
    lib = _lib_or_load()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    n_q, H, D = q_raw.shape
    n_k = 0 if k_raw is None else k_raw.shape[0]
    dev_ = q_raw.device
    with _on(stream):
        if out_dtype == "mxfp4":
            code = DTYPE_MXFP4
            q = torch.empty((n_q, H * (D // 2 + D // 32)), dtype=torch.uint8, device=dev_)
            k = None if k_raw is None else torch.empty((n_k, D // 2), dtype=torch.uint8, device=dev_)
            ks = None if k_raw is None else torch.empty((n_k, D // 32), dtype=torch.uint8, device=dev_)
        else:
            q = torch.empty((n_q, H, D), dtype=out_dtype, device=dev_)
            code = _dtype_code(q)
            k = None if k_raw is None else torch.empty((n_k, D), dtype=out_dtype, device=dev_)
            ks = torch.empty(n_k, dtype=torch.float32, device=dev_) \
                if out_dtype == torch.float8_e4m3fn and k_raw is not None else None
        w_out = torch.empty((n_q, H), dtype=torch.float32, device=dev_)
    _check(lib.dsa_indexer_prep(_ptr(q_raw), _ptr(k_raw), _ptr(w), _ptr(pos_q), _ptr(pos_k),
                                n_q, n_k, H, D, rope_dim, rope_main_dim, rope_theta, eps,
                                code, _ptr(q), _ptr(k), _ptr(w_out), _ptr(ks),
                                _stream(stream)), "dsa_indexer_prep")
    return q, k, w_out, ks


def dsa_indexer_k_insert(k_raw, slot_mapping, k_cache, k_scale_cache, norm_weight=None,
                         norm_bias=None, eps: float = 1e-6, stream=None):
    """LayerNorm -> e4m3 + power-of-two scale -> cache rows slot_mapping[i]
    (k_cache uint8 / float8_e4m3fn [n_slots, D], k_scale_cache f32 [n_slots],
    updated in place; negative slots are skipped)."""
    lib = _lib_or_load()
    n_tok, D = k_raw.shape
    _check(lib.dsa_indexer_k_insert(_ptr(k_raw), _dtype_code(k_raw), _ptr(norm_weight),
                                    _ptr(norm_bias), eps, _ptr(slot_mapping), n_tok, D,
                                    _ptr(k_cache), _ptr(k_scale_cache), k_cache.shape[0],
                                    _stream(stream)), "dsa_indexer_k_insert")
    return k_cache, k_scale_cache


MLA_FP8_ROW_BYTES = 656  # 512 e4m3 latent codes, 4 fp32 scales, 64 bf16 rope values


def dsa_mla_kv_insert(kv, slot_mapping, kv_cache, stream=None):
    """Latent rows kv [n, 576] (f32 / bf16) -> fp8 cache rows slot_mapping[i] of
    kv_cache uint8 [n_slots, 656], updated in place; negative slots are skipped."""
    lib = _lib_or_load()
    n_tok, d_qk = kv.shape
    if kv_cache.dim() != 2 or kv_cache.shape[1] != MLA_FP8_ROW_BYTES:
        raise DSAError("kv_cache must be uint8 [n_slots, 656]")
    _check(lib.dsa_mla_kv_insert(_ptr(kv), _dtype_code(kv), _ptr(slot_mapping), n_tok, d_qk,
                                 _ptr(kv_cache), kv_cache.shape[0], _stream(stream)),
           "dsa_mla_kv_insert")
    return kv_cache


def dsa_indexer_scores(q, k, w, row_starts, row_ends, k_scale=None, scores=None, ld=None,
                       stream=None):
    """scores [n_q, ld] fp32; only in-window entries are written."""
    import torch
    lib = _lib_or_load()
    n_q, H, D = _indexer_dims(q, k, w)
    n_k = k.shape[0]
    if scores is None:
        ld = n_k if ld is None else ld
        with _on(stream):
            scores = torch.full((n_q, ld), float("nan"), dtype=torch.float32, device=q.device)
    ld = scores.shape[1]
    _check(lib.dsa_indexer_scores(_ptr(q), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(row_starts),
                                  _ptr(row_ends), n_q, n_k, H, D, _dtype_code(q), _ptr(scores), ld,
                                  _stream(stream)), "dsa_indexer_scores")
    return scores


def dsa_topk(scores, row_starts, row_ends, index_topk: int, n_cols=None, out=None, stream=None):
    import torch
    lib = _lib_or_load()
    n_q, ld = scores.shape
    n_cols = ld if n_cols is None else n_cols
    ws_bytes = lib.dsa_topk_workspace_size(n_q, n_cols, index_topk)
    with _on(stream):
        if out is None:
            out = torch.empty((n_q, index_topk), dtype=torch.int32, device=scores.device)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device) if ws_bytes else None
    _check(lib.dsa_topk(_ptr(scores), ld, _ptr(row_starts), _ptr(row_ends), n_q, n_cols,
                        index_topk, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)), "dsa_topk")
    return out


def indexer_topk_workspace(n_q, n_k, n_heads, head_dim, dtype_code, index_topk) -> int:
    return _lib_or_load().dsa_indexer_topk_workspace_size(n_q, n_k, n_heads, head_dim, dtype_code,
                                                          index_topk)


def dsa_indexer_topk(q, k, w, row_starts, row_ends, index_topk: int, k_scale=None, out=None,
                     workspace=None, stream=None):
    import torch
    lib = _lib_or_load()
    n_q, H, D = _indexer_dims(q, k, w)
    n_k = k.shape[0]
    need = lib.dsa_indexer_topk_workspace_size(n_q, n_k, H, D, _dtype_code(q), index_topk)
    with _on(stream):
        if out is None:
            out = torch.empty((n_q, index_topk), dtype=torch.int32, device=q.device)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_indexer_topk(_ptr(q), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(row_starts),
                                _ptr(row_ends), n_q, n_k, H, D, _dtype_code(q), index_topk,
                                _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "dsa_indexer_topk")
    return out


def dsa_indexer_topk_noalloc(q, k, w, row_starts, row_ends, index_topk: int, k_scale=None,
                             out=None, stream=None):
    """dsa_indexer_topk with the library's own scratch array as its workspace
    (no device allocation by the library; out is allocated here unless given)."""
    import torch
    lib = _lib_or_load()
    n_q, H, D = _indexer_dims(q, k, w)
    n_k = k.shape[0]
    if out is None:
        with _on(stream):
            out = torch.empty((n_q, index_topk), dtype=torch.int32, device=q.device)
    _check(lib.dsa_indexer_topk_noalloc(_ptr(q), _ptr(k), _ptr(k_scale), _ptr(w),
                                        _ptr(row_starts), _ptr(row_ends), n_q, n_k, H, D,
                                        _dtype_code(q), index_topk, _ptr(out), _stream(stream)),
           "dsa_indexer_topk_noalloc")
    return out


def sparse_mla_workspace(n_q, n_heads, d_qk, d_v, index_topk, dtype_code) -> int:
    return _lib_or_load().dsa_sparse_mla_workspace_size(n_q, n_heads, d_qk, d_v, index_topk,
                                                        dtype_code)


def dsa_sparse_mla_fwd(q, kv, topk_idx, sm_scale: float, d_v: int, out=None, lse=None,
                       want_lse: bool = True, workspace=None, stream=None):
    import torch
    lib = _lib_or_load()
    n_q, H, d_qk = q.shape
    n_kv = kv.shape[0]
    K = topk_idx.shape[1]
    # a uint8 kv [n_kv, 656] is the fp8 latent cache (bf16 q and out)
    fp8_kv = kv.dtype == torch.uint8
    if fp8_kv and (kv.dim() != 2 or kv.shape[1] != MLA_FP8_ROW_BYTES):
        raise DSAError("an fp8 latent cache must be uint8 [n_kv, 656]")
    code = DTYPE_FP8_E4M3 if fp8_kv else _dtype_code(q)
    need = lib.dsa_sparse_mla_workspace_size(n_q, H, d_qk, d_v, K, code)
    with _on(stream):
        if out is None:
            out = torch.empty((n_q, H, d_v), dtype=q.dtype, device=q.device)
        if lse is None and want_lse:
            lse = torch.empty((n_q, H), dtype=torch.float32, device=q.device)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_mla_fwd(_ptr(q), _ptr(kv), _ptr(topk_idx), n_q, n_kv, H, d_qk, d_v, K,
                                  sm_scale, code, _ptr(out), _ptr(lse), _ptr(workspace),
                                  nbytes, _stream(stream)), "dsa_sparse_mla_fwd")
    return out, lse
