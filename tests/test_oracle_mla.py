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
    # a shift of every logit by a constant: one more dim with kv = 1 on every row
    # and q = c on every head adds c * sm_scale to each logit (the value dims are
    # untouched); the output is unchanged and the lse moves by c * sm_scale
    c = np.linspace(-40.0, 25.0, H)
    q_ext = np.concatenate([q, c[:, None]], axis=1)
    kv_ext = np.concatenate([kv, np.ones((N, 1))], axis=1)
    o3, l3 = mla.attend_row(q_ext, kv_ext, idx, 0.7, dv)
    np.testing.assert_allclose(o3, o1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l3, l1 + 0.7 * c, rtol=1e-13)
    # a logit that grows by 200 across the selection: the largest key dominates,
    # lse = its logit + log(1 + sum of the others' e^(l - l_max))
    kv_big = kv.copy()
    kv_big[:, 0] = np.arange(N) * 10.0
    qb = np.zeros((1, dqk)); qb[0, 0] = 1.0
    o4, l4 = mla.attend_row(qb, kv_big, np.array([29, 3, 28]), 1.0, dv)
    np.testing.assert_allclose(l4[0], 290.0 + np.log1p(np.exp(-10.0) + np.exp(-260.0)), rtol=1e-15)
    w29 = 1.0 / (1.0 + np.exp(-10.0) + np.exp(-260.0))
    np.testing.assert_allclose(o4[0], w29 * kv_big[29, :dv] + (1 - w29) * kv_big[28, :dv]
                               + np.exp(-260.0) * w29 * (kv_big[3, :dv] - kv_big[28, :dv]),
                               rtol=1e-12, atol=1e-15)


def test_fp8_latent_cache_rows():
    # the fp8 latent row: e4m3 codes with a power-of-two scale per 128 latent
    # dims, rope dims in bf16; dequantised rows are exact in bf16 (e4m3 times a
    # power of two), and attention on them is attention on those rows
    from oracle import prep
    g = np.random.default_rng(33)
    kv = prep.round_bf16(g.standard_normal((40, 576)) * 0.1 * np.exp2(g.integers(-3, 4, (40, 1))))
    codes, sc, rope = prep.mla_kv_quant(kv)
    assert codes.shape == (40, 512) and sc.shape == (40, 4) and rope.shape == (40, 64)
    np.testing.assert_array_equal(rope, kv[:, 512:])
    m, _ = np.frexp(sc)
    assert np.all(m == 0.5)
    amax = np.abs(kv[:, :512].reshape(40, 4, 128)).max(-1)
    assert np.all(amax <= 448 * sc) and np.all(amax > 224 * sc)
    deq = prep.dequant_mla_kv(codes, sc, rope)
    np.testing.assert_array_equal(prep.round_bf16(deq), deq)
    big = np.abs(codes) >= 2 ** -6
    rel = np.abs(deq[:, :512] - kv[:, :512])[big] / np.abs(kv[:, :512])[big]
    assert rel.max() <= 2 ** -4
    # rows already on the grid come back exactly: e4m3 codes whose block maximum
    # is 448 (which fixes the scale) times a power of two per block
    codes0 = prep.round_e4m3(g.standard_normal((6, 4, 128)) * 100.0)
    codes0[:, :, 0] = 448.0 * np.sign(g.standard_normal((6, 4)) + 0.5)
    e = g.integers(-12, 3, (6, 4)).astype(np.float64)
    lat = (codes0 * np.exp2(e)[..., None]).reshape(6, 512)
    rope0 = prep.round_bf16(g.standard_normal((6, 64)))
    c2, s2, r2 = prep.mla_kv_quant(np.concatenate([lat, rope0], axis=1))
    np.testing.assert_array_equal(c2, codes0.reshape(6, 512))
    np.testing.assert_array_equal(s2, np.exp2(e))
    np.testing.assert_array_equal(prep.dequant_mla_kv(c2, s2, r2)[:, :512], lat)
