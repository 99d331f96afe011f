"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/dsa.h declares, and rejects invalid arguments before
anything is enqueued (those calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_08_amd", "libdsa.so")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    import torch  # noqa: F401  load torch's HIP runtime first, as the binding does
    import sparse_attention_08_amd as b
    return b.load(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_indexer_topk", "dsa_sparse_mla_fwd",
              "dsa_row_windows"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    import sparse_attention_08_amd as b
    assert sorted(b.EXPORTS) == declared_functions()


def test_status_strings_and_version(lib):
    assert lib.dsa_version() >= 100
    assert lib.dsa_status_string(0) == b"ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.dsa_status_string(s) not in (b"ok", b"unknown status")


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
FAKE32 = ctypes.c_void_p(0x2000)


def test_topk_rejects_bad_arguments(lib):
    # index_topk < 1
    assert lib.dsa_topk(FAKE, 16, FAKE, FAKE, 4, 16, 0, FAKE, None, 0, None) == INVALID
    # ld < n_cols
    assert lib.dsa_topk(FAKE, 8, FAKE, FAKE, 4, 16, 4, FAKE, None, 0, None) == INVALID
    # null scores
    assert lib.dsa_topk(None, 16, FAKE, FAKE, 4, 16, 4, FAKE, None, 0, None) == INVALID
    # negative sizes
    assert lib.dsa_topk(FAKE, 16, FAKE, FAKE, -1, 16, 4, FAKE, None, 0, None) == INVALID
    # empty problem is fine and enqueues nothing
    assert lib.dsa_topk(None, 16, None, None, 0, 16, 4, None, None, 0, None) == 0


def test_indexer_rejects_bad_arguments(lib):
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", FAKE32), ("k", FAKE32), ("ks", None), ("w", FAKE), ("rs", FAKE), ("re", FAKE),
        ("nq", 4), ("nk", 8), ("h", 64), ("d", 128), ("dt", 1), ("sc", FAKE), ("ld", 8), ("st", None))]
    assert lib.dsa_indexer_scores(*args(h=65)) == UNSUPPORTED
    assert lib.dsa_indexer_scores(*args(d=64)) == UNSUPPORTED
    assert lib.dsa_indexer_scores(*args(ld=7)) == INVALID
    assert lib.dsa_indexer_scores(*args(dt=2)) == INVALID            # fp8 needs k_scale
    assert lib.dsa_indexer_scores(*args(ks=FAKE)) == INVALID         # bf16 must not get k_scale
    assert lib.dsa_indexer_scores(*args(dt=7)) == INVALID
    assert lib.dsa_indexer_scores(*args(q=ctypes.c_void_p(0x1008))) == UNSUPPORTED  # misaligned
    assert lib.dsa_indexer_scores(*args(w=None)) == INVALID
    assert lib.dsa_indexer_scores(*args(dt=0, d=300)) == UNSUPPORTED


def test_indexer_topk_workspace_is_checked(lib):
    # few rows over more than 8192 keys (fused: candidate workspace) and many
    # rows with index_topk above 2048 (scores go through the workspace)
    for n_q, n_k, K in ((4, 10000, 4), (2000, 8, 3000)):
        need = lib.dsa_indexer_topk_workspace_size(n_q, n_k, 64, 128, 1, K)
        assert need > 0
        st = lib.dsa_indexer_topk(FAKE32, FAKE32, None, FAKE, FAKE, FAKE, n_q, n_k, 64, 128, 1, K,
                                  FAKE, None, 0, None)
        assert st == WORKSPACE
        st = lib.dsa_indexer_topk(FAKE32, FAKE32, None, FAKE, FAKE, FAKE, n_q, n_k, 64, 128, 1, K,
                                  FAKE, FAKE32, need - 1, None)
        assert st == WORKSPACE
    # fused with every window inside 8192 keys needs none, nor does prefill
    assert lib.dsa_indexer_topk_workspace_size(4, 8192, 64, 128, 1, 4) == 0
    assert lib.dsa_indexer_topk_workspace_size(2000, 100000, 64, 128, 1, 2048) == 0


def test_topk_workspace_is_checked(lib):
    need = lib.dsa_topk_workspace_size(4, 10000, 2048)
    assert need == 4 * 16 * 2048 * 8 + 4 * 16 * 4
    assert lib.dsa_topk_workspace_size(4, 8192, 2048) == 0       # windows fit one workgroup
    assert lib.dsa_topk_workspace_size(2000, 10000, 2048) == 0   # many rows: one per workgroup
    st = lib.dsa_topk(FAKE32, 10000, FAKE, FAKE, 4, 10000, 2048, FAKE, None, 0, None)
    assert st == WORKSPACE


def test_mla_rejects_bad_arguments(lib):
    base = dict(q=FAKE32, kv=FAKE32, idx=FAKE, nq=4, nkv=16, h=128, dqk=576, dv=512, k=2048,
                sm=0.04, dt=1, out=FAKE32, lse=None, ws=None, wsb=0, st=None)
    def call(**kw):
        a = dict(base, **kw)
        return lib.dsa_sparse_mla_fwd(*a.values())
    assert call(dqk=512) == UNSUPPORTED
    assert call(h=100) == UNSUPPORTED
    assert call(dv=600) == INVALID
    assert call(dt=2, dqk=512) == UNSUPPORTED               # the fp8 latent cache: 576 only
    assert call(dt=2, out=ctypes.c_void_p(FAKE32.value + 4)) == UNSUPPORTED  # out 8-aligned
    assert call(dt=5) == INVALID
    assert call(k=0) == INVALID
    assert call(out=None) == INVALID
    # decode-sized call needs split workspace
    need = lib.dsa_sparse_mla_workspace_size(4, 128, 576, 512, 2048, 1)
    assert need == 4 * 16 * 128 * (512 * 2 + 4)     # 16 splits: bf16 partial o, fp32 partial lse
    assert call() == WORKSPACE
    # the fp8 latent cache splits the same way
    assert lib.dsa_sparse_mla_workspace_size(4, 128, 576, 512, 2048, 2) == need
    assert call(dt=2) == WORKSPACE


def test_mla_kv_insert_rejects_bad_arguments(lib):
    a = [FAKE32, 1, FAKE, 4, 576, FAKE32, 8, None]
    def call(i, v):
        b = list(a)
        b[i] = v
        return lib.dsa_mla_kv_insert(*b)
    assert call(4, 512) == UNSUPPORTED                    # rows are 512 latent + 64 rope
    assert call(1, 2) == UNSUPPORTED                      # fp8 input rows
    assert call(1, 7) == INVALID
    assert call(0, None) == INVALID
    assert call(2, None) == INVALID
    assert call(5, None) == INVALID
    assert call(3, -1) == INVALID
    assert call(5, ctypes.c_void_p(FAKE32.value + 8)) == UNSUPPORTED  # cache 16-aligned


def test_windows_and_prep_reject_bad_arguments(lib):
    assert lib.dsa_row_windows(FAKE, FAKE, 0, 4, 1, FAKE, FAKE, None) == INVALID
    assert lib.dsa_row_windows(FAKE, FAKE, 1, 4, 2, FAKE, FAKE, None) == INVALID
    assert lib.dsa_row_windows(None, FAKE, 1, 4, 1, FAKE, FAKE, None) == INVALID
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 2, 128, 63, 64, 1e4, 1e-6, 1, FAKE, FAKE, FAKE, None, None]
    assert lib.dsa_indexer_prep(*a) == INVALID                      # odd rope_dim
    a[9] = 64; a[13] = 2
    assert lib.dsa_indexer_prep(*a) == INVALID                      # fp8 needs k_scale_out


def test_noalloc_rejects_a_workspace_beyond_its_array(lib):
    # 256 decode rows over long windows need 256 * (16 * 2048 * 8 + 64) bytes of
    # candidates, more than the 64 MiB array: refused before any device call
    need = lib.dsa_indexer_topk_workspace_size(256, 100000, 64, 128, 1, 2048)
    assert need > (64 << 20)
    assert lib.dsa_indexer_topk_noalloc(FAKE, FAKE, None, FAKE32, FAKE, FAKE, 256, 100000, 64,
                                        128, 1, 2048, FAKE, None) == WORKSPACE
    # prefill rows keep their candidates on chip: no workspace at all
    assert lib.dsa_indexer_topk_workspace_size(65536, 65536, 64, 128, 2, 2048) == 0
    assert lib.dsa_indexer_topk_workspace_size(257, 1 << 20, 64, 128, 1, 2048) == 0
