"""Pins for oracle.prep: LayerNorm, RoPE, bf16 / e4m3 rounding, power-of-two
scales.  Each check compares against something other than the oracle itself:
closed forms, a library routine (torch CPU casts and layer_norm), or a
hand-computed fixture."""
import os

import numpy as np
import pytest
import torch

from oracle import prep

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_layernorm_closed_form():
    # each output row has mean 0 and biased variance var/(var+eps)
    g = np.random.default_rng(1)
    x = g.standard_normal((64, 128)) * 3 + 1.5
    eps = 1e-6
    y = prep.layer_norm(x, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_layernorm_vs_torch():
    g = np.random.default_rng(2)
    x = g.standard_normal((32, 128))
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    np.testing.assert_allclose(prep.layer_norm(x, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_layernorm_large_eps_changes_scale():
    # a dropped eps would fail this: constant-free row of variance 1 -> 1/sqrt(1+eps)
    x = np.array([[1.0, -1.0, 1.0, -1.0]])
    y = prep.layer_norm(x, eps=3.0)
    np.testing.assert_allclose(y, x / 2.0, rtol=1e-15)


def test_rope_hand_fixture():
    rows = {l.split()[0]: l.split()[1:] for l in open(os.path.join(GOLD, "rope_hand.txt"))
            if l.strip() and not l.startswith("#")}
    x = np.array([[float(v) for v in rows["x"]]])
    pos = np.array([int(rows["pos"][0])])
    out = prep.rope_leading(x, pos, rope_dim=4, rope_main_dim=4, theta=1e4)
    np.testing.assert_allclose(out[0], [float(v) for v in rows["out"]], rtol=1e-14)


def test_rope_properties():
    g = np.random.default_rng(3)
    D, R = 128, 64
    q = g.standard_normal((5, 3, D))
    k = g.standard_normal((5, D))
    # position 0 is the identity
    np.testing.assert_array_equal(prep.rope_leading(q, np.zeros(5), R, 64, 1e4), q)
    pos = np.array([0, 1, 17, 500, 4095])
    qr = prep.rope_leading(q, pos, R, 64, 1e4)
    # every (i, i+R/2) pair keeps its norm; dims beyond R are untouched
    half = R // 2
    n0 = q[..., :half] ** 2 + q[..., half:R] ** 2
    n1 = qr[..., :half] ** 2 + qr[..., half:R] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    np.testing.assert_array_equal(qr[..., R:], q[..., R:])
    # dot products over the rotated dims depend only on the position difference
    a, b = g.standard_normal(D), g.standard_normal(D)
    def dot(m, n):
        ra = prep.rope_leading(a[None], np.array([m]), R, 64, 1e4)[0]
        rb = prep.rope_leading(b[None], np.array([n]), R, 64, 1e4)[0]
        return ra @ rb
    np.testing.assert_allclose(dot(10, 3), dot(107, 100), rtol=1e-9)
    np.testing.assert_allclose(dot(3, 10), dot(1003, 1010), rtol=1e-9)
    assert abs(dot(10, 3) - dot(10, 4)) > 1e-6


def test_round_bf16_vs_torch():
    g = np.random.default_rng(4)
    x = np.concatenate([g.standard_normal(100000) * 10.0 ** g.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 3.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 2 ** -130]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(prep.round_bf16(x.astype(np.float64)), ref)


def test_round_e4m3_vs_torch():
    g = np.random.default_rng(5)
    x = np.concatenate([g.uniform(-448, 448, 50000), g.standard_normal(50000) * 2.0 ** -6,
                        [0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(prep.round_e4m3(x.astype(np.float64)), ref)


def test_ue8m0_scale_properties():
    g = np.random.default_rng(6)
    amax = np.concatenate([np.abs(g.standard_normal(10000)) * 10.0 ** g.integers(-8, 8, 10000),
                           448.0 * 2.0 ** np.arange(-10, 10), [448.0 * (1 + 2 ** -40)]])
    s = prep.ue8m0_scale(amax)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)                     # powers of two
    assert np.all(amax <= 448.0 * s)            # no saturation
    assert np.all(amax > 448.0 * s / 2)         # smallest such power
    assert prep.ue8m0_scale(np.array([0.0]))[0] == 1.0
    np.testing.assert_array_equal(prep.ue8m0_scale(448.0 * 2.0 ** np.arange(-3, 4)), 2.0 ** np.arange(-3, 4))


def test_quant_roundtrip_and_idempotent():
    g = np.random.default_rng(7)
    x = g.standard_normal((50, 4, 128))
    codes, s = prep.quant_e4m3_blocks(x, 128)
    assert np.all(np.abs(codes) <= 448)
    # codes are e4m3 values
    np.testing.assert_array_equal(prep.round_e4m3(codes), codes)
    deq = codes * np.repeat(s, 128, axis=-1)
    # relative error of e4m3 rounding is at most 2^-4 for normal codes
    big = np.abs(codes) >= 2 ** -6
    assert np.all(np.abs(deq - x)[big] <= 2 ** -4 * np.abs(x)[big] + 1e-300)
    codes2, s2 = prep.quant_e4m3_blocks(deq, 128)
    np.testing.assert_array_equal(codes2 * np.repeat(s2, 128, axis=-1), deq)


def test_fp8_fold_equals_dequantised_definition():
    # score(q8, k8, w*sq, sk) equals the definition on dequantised values because
    # the scales are positive and relu is positively homogeneous
    from oracle import indexer
    g = np.random.default_rng(8)
    H, D, N = 4, 128, 6
    q = g.standard_normal((1, H, D))
    k = g.standard_normal((N, D))
    w = g.random((1, H)).astype(np.float32).astype(np.float64)   # fp32 weights: the fold is exact
    p = prep.prepare_indexer_inputs(q, k, w, np.zeros(1), np.zeros(N), "fp8")
    q8, sq = prep.quant_e4m3_blocks(q, D)
    kn = prep.layer_norm(k)
    k8, sk = prep.quant_e4m3_blocks(kn, D)
    deq_q = q8 * sq
    deq_k = k8 * sk
    ref = indexer.score_row(deq_q[0], deq_k, w[0])
    got = indexer.score_row(p["q"][0], p["k"], p["w"][0], p["k_scale"])
    np.testing.assert_allclose(got, ref, rtol=1e-12)


# ---------------------------------------------------------------------------
# the composed preparation: LayerNorm -> RoPE -> rounding, positions per sample
# ---------------------------------------------------------------------------
def _prep_fixture():
    rows = {l.split()[0]: [float(v) for v in l.split()[1:]]
            for l in open(os.path.join(GOLD, "prep_hand.txt")) if l.strip() and not l.startswith("#")}
    return rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prepare_composed_hand_fixture(dtype):
    # norm, then rope (half-split pairs), then one rounding to the operand format:
    # a rope applied before the norm, interleaved pairs, or a normed query fail it
    f = _prep_fixture()
    q_raw = np.array(f["q_raw"]).reshape(1, 1, 6)
    k_raw = np.array(f["k_raw"]).reshape(1, 6)
    w = np.array([f["w"]])
    p = prep.prepare_indexer_inputs(q_raw, k_raw, w, np.array([int(f["q_pos"][0])]),
                                    np.array([int(f["k_pos"][0])]), dtype, rope_dim=4,
                                    rope_main_dim=4, theta=1e4, eps=1e-6)
    want_k, want_q = np.array(f["k_out"]), np.array(f["q_out"])
    if dtype == "f32":
        np.testing.assert_allclose(p["k"][0], want_k, rtol=1.2e-7, atol=0)
        np.testing.assert_allclose(p["q"][0, 0], want_q, rtol=1.2e-7, atol=0)
    else:
        to_bf16 = lambda x: torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(p["k"][0], to_bf16(want_k))
        np.testing.assert_array_equal(p["q"][0, 0], to_bf16(want_q))
    np.testing.assert_array_equal(p["w"], w)
    assert p["k_scale"] is None


def test_positions_restart_per_sample():
    # review comment 1 of vime pull request #502 keeps per-sample positions and
    # rebases only the indices; the rope angle uses the position inside the sample
    import synth
    lay = synth.layout_from_lengths([3, 2])
    np.testing.assert_array_equal(lay.positions(), [0, 1, 2, 0, 1])
    np.testing.assert_array_equal(lay.key_positions(), [0, 1, 2, 0, 1])
    dec = synth.layout_from_lengths([5, 3], decode=True)       # the query is the last token
    np.testing.assert_array_equal(dec.positions(), [4, 2])
    # a sample that repeats the first tokens of another one gets identical operands
    g = np.random.default_rng(9)
    q_raw = g.standard_normal((5, 2, 8))
    k_raw = g.standard_normal((5, 8))
    q_raw[3:5], k_raw[3:5] = q_raw[0:2], k_raw[0:2]
    w = g.random((5, 2))
    p = prep.prepare_indexer_inputs(q_raw, k_raw, w, lay.positions(), lay.key_positions(), "f32",
                                    rope_dim=4, rope_main_dim=4)
    np.testing.assert_array_equal(p["q"][3:5], p["q"][0:2])
    np.testing.assert_array_equal(p["k"][3:5], p["k"][0:2])
    # and the first token of each sample is not rotated (position 0)
    p0 = prep.prepare_indexer_inputs(q_raw, k_raw, w, lay.positions(), lay.key_positions(), "f32")
    np.testing.assert_array_equal(p["q"][[0, 3]], p0["q"][[0, 3]])
    np.testing.assert_array_equal(p["k"][[0, 3]], p0["k"][[0, 3]])
    assert np.abs(p["q"][[1, 2, 4]] - p0["q"][[1, 2, 4]]).max() > 1e-3


def test_same_position_pair_is_rope_invariant():
    # q and k of one token are rotated by the same angle, so their dot product
    # over the rotated dims is unchanged: the diagonal scores of a prefill and a
    # decode query's score against its own cache entry equal the unrotated ones
    # (up to the fp32 rounding of the operands).  Rotating q and k at different
    # positions breaks this.
    import synth
    from oracle import indexer
    g = np.random.default_rng(10)
    for lay in (synth.layout_from_lengths([6, 4]), synth.layout_from_lengths([7, 3], decode=True)):
        H, D = 3, 16
        q_raw = g.standard_normal((lay.n_q, H, D)) * 3.0
        k_raw = g.standard_normal((lay.n_k, D))
        w = g.standard_normal((lay.n_q, H))
        args = (q_raw, k_raw, w, lay.positions(), lay.key_positions(), "f32")
        pr = prep.prepare_indexer_inputs(*args, rope_dim=8, rope_main_dim=8)
        pn = prep.prepare_indexer_inputs(*args)
        cu_q, cu_k = lay.cu_q, lay.cu_k
        for b in range(len(lay.q_lens)):
            for j in range(int(lay.q_lens[b])):
                t = int(cu_q[b]) + j
                s = int(cu_k[b + 1]) - int(lay.q_lens[b]) + j      # the query's own token
                dr = pr["q"][t] @ pr["k"][s]
                dn = pn["q"][t] @ pn["k"][s]
                np.testing.assert_allclose(dr, dn, rtol=1e-5, atol=1e-5)
                sr = indexer.score_row(pr["q"][t], pr["k"][s:s + 1], pr["w"][t])
                sn = indexer.score_row(pn["q"][t], pn["k"][s:s + 1], pn["w"][t])
                np.testing.assert_allclose(sr, sn, rtol=1e-5, atol=1e-5)
        # an off-diagonal pair does change (the rope is not a no-op here)
        t, s = lay.n_q - 1, 0
        assert abs(pr["q"][t] @ pr["k"][s] - pn["q"][t] @ pn["k"][s]).max() > 1e-3


# ---------------------------------------------------------------------------
# the fp8 index-key cache insert (norm -> quant -> slot)
# ---------------------------------------------------------------------------
def test_layer_norm_affine_vs_torch():
    g = np.random.default_rng(20)
    x = g.standard_normal((16, 128)) * 2 + 0.3
    wgt, b = g.standard_normal(128), g.standard_normal(128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(wgt),
                                         torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(prep.layer_norm_affine(x, wgt, b, 1e-6), ref, rtol=1e-12, atol=1e-12)
    # weight 1 and bias 0 (the defaults) are the plain norm
    np.testing.assert_array_equal(prep.layer_norm_affine(x, None, None), prep.layer_norm(x))


def test_k_insert_slots_and_quantisation():
    g = np.random.default_rng(21)
    n_slots, D = 12, 128
    codes = np.full((n_slots, D), 7.0)
    scales = np.full(n_slots, 3.0)
    k = g.standard_normal((5, D)) * np.array([1.0, 50.0, 1e-3, 0.0, 2.0])[:, None]
    slots = np.array([3, -1, 11, 0, 12])          # a padding token and a slot past the cache
    prep.k_norm_quant_insert(k, None, None, 1e-6, slots, codes, scales)
    untouched = [i for i in range(n_slots) if i not in (3, 11, 0)]
    assert np.all(codes[untouched] == 7.0) and np.all(scales[untouched] == 3.0)
    # a zero row normalises to zero: codes 0 with scale 1
    assert np.all(codes[0] == 0.0) and scales[0] == 1.0
    for src, dst in ((0, 3), (2, 11)):
        y = prep.layer_norm(k[src])
        s = scales[dst]
        m, _ = np.frexp(s)
        assert m == 0.5 and np.abs(y).max() <= 448 * s < 2 * np.abs(y).max()
        # the codes are e4m3 values and each is the nearest one to y / s
        np.testing.assert_array_equal(prep.round_e4m3(codes[dst]), codes[dst])
        ref = torch.from_numpy(y / s).to(torch.float8_e4m3fn).double().numpy()
        np.testing.assert_array_equal(codes[dst], ref)
    # the norm makes the insert invariant to an affine change of the raw key
    c2, s2 = np.zeros((1, D)), np.zeros(1)
    prep.k_norm_quant_insert(k[2:3] * 1e4 + 5.0, None, None, 0.0, [0], c2, s2)
    c3, s3 = np.zeros((1, D)), np.zeros(1)
    prep.k_norm_quant_insert(k[2:3], None, None, 0.0, [0], c3, s3)
    np.testing.assert_array_equal(c2 * s2[:, None], c3 * s3[:, None])


# ---------------------------------------------------------------------------
# MXFP4 (OCP microscaling: E2M1 elements, E8M0 scale per 32)
# ---------------------------------------------------------------------------
def test_round_e2m1_grid_and_ties():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    np.testing.assert_array_equal(prep.round_e2m1(grid), grid)
    np.testing.assert_array_equal(prep.round_e2m1(-grid), -grid)
    # ties go to the even mantissa bit (0.5 = 0.1b: odd; 1, 2, 4: even)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    np.testing.assert_array_equal(prep.round_e2m1(ties), [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    np.testing.assert_array_equal(prep.round_e2m1([0.26, 0.74, 1.26, 2.6, 5.01, 6.5, 7.99, 1e9]),
                                  [0.5, 0.5, 1.5, 3.0, 6.0, 6.0, 6.0, 6.0])   # saturates at 6
    # every value rounds to a nearest grid point
    g = np.random.default_rng(30)
    x = g.uniform(-6, 6, 20000)
    r = prep.round_e2m1(x)
    full = np.concatenate([-grid[::-1], grid])
    best = np.abs(x[:, None] - full[None, :]).min(axis=1)
    np.testing.assert_allclose(np.abs(x - r), best, rtol=0, atol=1e-15)


def test_mxfp4_block_scales():
    g = np.random.default_rng(31)
    x = g.standard_normal((20, 4, 128)) * 10.0 ** g.integers(-4, 4, (20, 4, 1))
    x[0, 0, :32] = 0.0                          # an all-zero block: exponent 0
    codes, e = prep.quant_mxfp4_blocks(x)
    assert e.shape == (20, 4, 4) and e[0, 0, 0] == 0 and np.all(codes[0, 0, :32] == 0)
    amax = np.abs(x.reshape(20, 4, 4, 32)).max(-1)
    nz = amax > 0
    # 2^e <= amax / 4 < 2^(e+1): the largest element lands in [4, 8) before saturation
    assert np.all(np.exp2(e[nz] + 2.0) <= amax[nz]) and np.all(amax[nz] < np.exp2(e[nz] + 3.0))
    np.testing.assert_array_equal(prep.round_e2m1(codes), codes)
    deq = codes * np.repeat(np.exp2(e.astype(float)), 32, axis=-1)
    # error: within half a grid step of the element's binade, or the saturation
    # (at most 2 steps of 2^e below 8 2^e)
    ok = np.abs(deq - x) <= np.maximum(0.25, 0.5 * np.exp2(np.floor(np.log2(np.maximum(
        np.abs(x) / np.repeat(np.exp2(e.astype(float)), 32, -1), 1.0))) - 1)) \
        * np.repeat(np.exp2(e.astype(float)), 32, -1) + 1e-300
    sat = np.abs(x) >= 6 * np.repeat(np.exp2(e.astype(float)), 32, -1)
    assert np.all(ok | sat)
    assert np.all(np.abs(deq[sat]) == 6 * np.repeat(np.exp2(e.astype(float)), 32, -1)[sat])


def test_mxfp4_prepared_operands_score_as_dequantised():
    from oracle import indexer
    g = np.random.default_rng(32)
    q = g.standard_normal((3, 4, 128))
    k = g.standard_normal((9, 128))
    w = g.random((3, 4)).astype(np.float32).astype(np.float64)
    p = prep.prepare_indexer_inputs(q, k, w, np.zeros(3), np.zeros(9), "mxfp4")
    kn = prep.layer_norm(k)
    k4, ek = prep.quant_mxfp4_blocks(kn)
    np.testing.assert_array_equal(p["k_codes"], k4)
    np.testing.assert_array_equal(p["k"], k4 * np.repeat(np.exp2(ek.astype(float)), 32, axis=-1))
    # the score is the definition on the dequantised operands (no key scale)
    ref = indexer.score_row(p["q"][1], p["k"], w[1])
    manual = np.array([sum(w[1, h] * max(0.0, float(p["q"][1, h] @ p["k"][s])) for h in range(4))
                       for s in range(9)])
    np.testing.assert_allclose(ref, manual, rtol=1e-13)
