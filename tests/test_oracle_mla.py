"""Pins for oracle.mla: hand fixture, dense causal attention through torch's
scaled_dot_product_attention (library routine) when the selection covers the
whole causal window, and closed-form special cases."""
import os

import numpy as np
import scipy.special
import torch

from oracle import mla

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_fixture():
    rows = {}
    kv = []
    for line in open(os.path.join(GOLD, "mla_hand.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "kv":
            kv.append([float(v) for v in f[1:]])
        else:
            rows[f[0]] = [float(v) for v in f[1:]]
    q = np.array([rows["q"]])
    idx = np.array([int(v) for v in rows["idx"]])
    out, lse = mla.attend_row(q, np.array(kv), idx, 1.0, 1)
    np.testing.assert_allclose(out[0, 0], rows["out"][0], rtol=1e-14)
    np.testing.assert_allclose(lse[0], rows["lse"][0], rtol=1e-14)


def test_full_selection_equals_dense_causal_attention():
    g = np.random.default_rng(31)
    T, H, dqk, dv = 20, 3, 16, 8
    q = g.standard_normal((T, H, dqk)); kv = g.standard_normal((T, dqk))
    K = 32                                                  # >= every window
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)
    sm = dqk ** -0.5
    out, lse = mla.sparse_mla(q, kv, idx, sm, dv)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]         # [1, H, T, dqk]
    kt = torch.from_numpy(kv)[None, None].expand(1, H, T, dqk)
    vt = torch.from_numpy(kv[:, :dv])[None, None].expand(1, H, T, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=sm)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    logits = np.einsum("thd,sd->ths", q, kv) * sm
    mask = np.tril(np.ones((T, T), bool))
    ref_lse = scipy.special.logsumexp(np.where(mask[:, None, :], logits, -np.inf), axis=2)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_special_cases():
    g = np.random.default_rng(32)
    H, dqk, dv, N = 4, 12, 6, 30
    kv = g.standard_normal((N, dqk))
    idx = np.array([3, 17, -1, 8, 25, -1])
    # q = 0: uniform weights -> mean of the selected V rows, lse = log n
    o, l = mla.attend_row(np.zeros((H, dqk)), kv, idx, 0.5, dv)
    np.testing.assert_allclose(o, np.broadcast_to(kv[[3, 17, 8, 25], :dv].mean(0), (H, dv)), rtol=1e-13)
    np.testing.assert_allclose(l, np.log(4.0), rtol=1e-14)
    # one key: that V row, lse = its logit
    q = g.standard_normal((H, dqk))
    o, l = mla.attend_row(q, kv, np.array([-1, 11, -1]), 0.3, dv)
    np.testing.assert_allclose(o, np.broadcast_to(kv[11, :dv], (H, dv)), rtol=1e-13)
    np.testing.assert_allclose(l, 0.3 * q @ kv[11], rtol=1e-12, atol=1e-15)
    # order of the selection does not matter
    o1, l1 = mla.attend_row(q, kv, idx, 0.7, dv)
    o2, l2 = mla.attend_row(q, kv, idx[::-1].copy(), 0.7, dv)
    np.testing.assert_allclose(o1, o2, rtol=1e-12); np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # empty selection
    o, l = mla.attend_row(q, kv, np.full(5, -1), 0.7, dv)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # a shift of every logit by a constant does not change the output
    o3, l3 = mla.attend_row(q, kv + 0.0, idx, 0.7, dv)
    np.testing.assert_allclose(o3, o1)
