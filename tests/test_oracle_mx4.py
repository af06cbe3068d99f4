"""Pins of the oracle's MXFP4 arithmetic (fp4 e2m1 codes with e8m0 block
scales of 32 along the contraction) to facts outside it.  torch has no fp4
conversion on the CPU, so the e2m1 grid is pinned through torch's float8_e4m3fn
(every e2m1 value is an e4m3 value whose two low mantissa bits are zero, within
the e2m1 exponent range), through the format constants the OCP microscaling
specification states (largest normal 6, smallest normal 1, one subnormal 0.5),
and by brute force: nearest-value search over all 16 codes, loops over codes
and scales for every GEMM operand orientation, and the K-major block-by-block
sums that fix each expert product's quantisation axis."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

CODES = np.arange(16, dtype=np.uint8)


def test_e2m1_grid_is_the_one_mantissa_bit_slice_of_e4m3():
    # e4m3 values (decoded by torch) with exponent in [0, 2] and mantissa bits xx0 0 -> 1 mantissa bit
    e4 = torch.arange(0x80, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    codes = np.arange(0x80)
    exp = (codes >> 3) & 15
    one_bit = (codes & 3) == 0
    normals = np.sort(e4[(exp >= 7) & (exp <= 9) & one_bit])
    want = np.concatenate([[0.0, 0.5], normals])
    np.testing.assert_array_equal(O.e2m1_decode(CODES[:8]), want)
    np.testing.assert_array_equal(want, [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e2m1_spec_constants_and_sign():
    mags = O.e2m1_decode(CODES[:8])
    assert mags.max() == O.E2M1_MAX == 6.0                  # largest normal
    assert mags[mags >= 1.0].min() == 1.0                    # smallest normal
    assert list(mags[(mags > 0) & (mags < 1.0)]) == [0.5]    # the one subnormal
    assert np.all(np.diff(mags) > 0)
    np.testing.assert_array_equal(O.e2m1_decode(CODES[8:]), -mags)
    assert np.signbit(O.e2m1_decode([8])[0])                 # code 8 is -0


def _brute_encode(v):
    """nearest e2m1 value by scanning all 16 codes; ties to the even code;
    beyond 6 saturates; -0 and negative values round to the negative codes"""
    vals = O.e2m1_decode(CODES)
    out = []
    for x in np.asarray(v, np.float64):
        best = None
        for c in CODES:
            if (c >= 8) != bool(np.signbit(x)):
                continue
            dist = abs(min(abs(x), 6.0) - abs(vals[c]))
            if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (dist, c)
        out.append(best[1])
    return np.array(out, np.uint8)


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(0)
    mags = O.e2m1_decode(CODES[:8])
    mids = (mags[:-1] + mags[1:]) / 2
    v = np.concatenate([rng.uniform(-7, 7, 3000), rng.normal(0, 1, 2000), mids, -mids, mags, -mags,
                        [0.0, -0.0, 6.0, 6.5, 100.0, -1e9, 0.25, -0.25, 0.2499]])
    np.testing.assert_array_equal(O.e2m1_encode(v), _brute_encode(v))
    # the midpoints go to the even code of each pair: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    np.testing.assert_array_equal(O.e2m1_decode(O.e2m1_encode(mids)), [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])


def test_e2m1_encode_inverts_decode():
    np.testing.assert_array_equal(O.e2m1_encode(O.e2m1_decode(CODES)), CODES)


def test_nibble_packing():
    np.testing.assert_array_equal(O.pack_e2m1(np.array([1, 2, 15, 0], np.uint8)), np.array([0x21, 0x0F], np.uint8))
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    np.testing.assert_array_equal(O.unpack_e2m1(O.pack_e2m1(c)), c)


def test_fp4_scale_rule_is_minimal_and_never_clips():
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.exp2(rng.uniform(-100, 100, 5000)), 6.0 * np.exp2(np.arange(-20, 20.0)),
                           4.0 * np.exp2(np.arange(-20, 20.0))])
    e = O.mx_scale_exp(amax, "e2m1").astype(np.float64)
    assert np.all(6.0 * np.exp2(e) >= amax)
    assert np.all(6.0 * np.exp2(e - 1) < amax)
    assert O.mx_scale_exp([0.0], "e2m1")[0] == -127
    blk = rng.normal(0, 3, (200, 32))
    codes, sb = O.mx_quantize(blk, 1, "e2m1")
    top = np.max(np.abs(O.e2m1_decode(codes)), axis=1)       # the block's largest magnitude lands in (3, 6]
    assert np.all((top >= 3.0) & (top <= 6.0))
    np.testing.assert_array_equal(sb[:, 0], O.mx_scale_exp(np.abs(blk).max(1), "e2m1") + 127)


def _brute_dot4(ca, sa, cb, sb, i, j, K):
    tot = 0.0
    for k in range(K):
        av = O.e2m1_decode([ca[i, k]])[0] * 2.0 ** (int(sa[i, k // 32]) - 127)
        bv = O.e2m1_decode([cb[j, k]])[0] * 2.0 ** (int(sb[j, k // 32]) - 127)
        tot += av * bv
    return tot


@pytest.mark.parametrize("axis_a,axis_b", [(1, 1), (0, 0), (1, 0), (0, 1)])
def test_mx4_gemm_matches_brute_force_over_codes(axis_a, axis_b):
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 70
    a = rng.normal(0, 1, (M, K)) * np.exp2(rng.integers(-6, 6, (M, K)))
    b = rng.normal(0, 1, (N, K)) * np.exp2(rng.integers(-6, 6, (N, K)))
    a_st = a if axis_a == 1 else a.T.copy()
    b_st = b if axis_b == 1 else b.T.copy()
    qa = O.mx_qdq(a_st, axis_a, "e2m1")
    qb = O.mx_qdq(b_st, axis_b, "e2m1")
    C = (qa if axis_a == 1 else qa.T) @ (qb if axis_b == 1 else qb.T).T
    ca, sa = O.mx_quantize(a, 1, "e2m1")
    cb, sb = O.mx_quantize(b, 1, "e2m1")
    for i in range(M):
        for j in range(N):
            assert C[i, j] == pytest.approx(_brute_dot4(ca, sa, cb, sb, i, j, K), rel=1e-12, abs=1e-300)


def test_mx4_forward_equals_bf16_forward_on_grid_inputs():
    """Blocks whose values are e2m1 values times one power of two, with a 6 or
    a 4 in every block so the scale rule picks that power: quantisation is
    lossless and the MXFP4 expert's H, U, A equal the bf16 expert's."""
    rng = np.random.default_rng(4)
    grid = np.array([-6.0, -3.0, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 4.0, 6.0])
    n, d, f = 6, 64, 32

    def on_grid(shape, s):
        a = rng.choice(grid, shape)
        a[..., ::32] = 6.0                      # one full-scale value per 32-block along the last axis
        return a * s
    x = on_grid((n, d), 0.25)
    w13 = on_grid((2 * f, d), 1.0 / 64)
    w2 = on_grid((d, f), 1.0 / 64)
    np.testing.assert_array_equal(O.mx_qdq(x, 1, "e2m1"), x)
    np.testing.assert_array_equal(O.mx_qdq(w13, 1, "e2m1"), w13)
    a = O.swiglu_ffn_fwd_mx(x, w13, w2, "bf16", fmt="e2m1")
    b = O.swiglu_ffn_fwd(x, w13, w2, "bf16")
    np.testing.assert_array_equal(a["H"], b["H"])
    np.testing.assert_array_equal(a["U"], b["U"])
    np.testing.assert_array_equal(a["A"], b["A"])


def test_mx4_backward_moves_more_than_mx8():
    """The e2m1 step is 2^-1 relative at the bottom of a binade: every MXFP4
    gradient sits farther from the bf16 expert's than the MXFP8 one does, and
    within 60% relative L2."""
    rng = np.random.default_rng(5)
    n, d, f = 48, 64, 96
    x = O.round_bf16(rng.normal(0, 1, (n, d)))
    w13 = O.round_bf16(rng.normal(0, 0.1, (2 * f, d)))
    w2 = O.round_bf16(rng.normal(0, 0.1, (d, f)))
    dy = O.round_bf16(rng.normal(0, 1, (n, d)))
    fa = O.swiglu_ffn_fwd(x, w13, w2, "bf16")
    ga = O.swiglu_ffn_bwd(x, fa["H"], fa["U"], fa["A"], dy, w13, w2, "bf16")
    g8 = O.swiglu_ffn_bwd_mx(x, fa["H"], fa["U"], fa["A"], dy, w13, w2, "bf16", fmt="e4m3")
    g4 = O.swiglu_ffn_bwd_mx(x, fa["H"], fa["U"], fa["A"], dy, w13, w2, "bf16", fmt="e2m1")
    for k in ("dH", "dU", "dX", "dW13", "dW2"):
        r8 = np.linalg.norm(g8[k] - ga[k]) / np.linalg.norm(ga[k])
        r4 = np.linalg.norm(g4[k] - ga[k]) / np.linalg.norm(ga[k])
        assert r8 < r4 < 0.6, (k, r8, r4)


def _kmajor_product4(P, Q):
    cp, sp = O.mx_quantize(P, 1, "e2m1")
    cq, sq = O.mx_quantize(Q, 1, "e2m1")
    vp, vq = O.e2m1_decode(cp), O.e2m1_decode(cq)
    C = np.zeros((P.shape[0], Q.shape[0]))
    for k in range(P.shape[1]):
        a = vp[:, k] * np.exp2(sp[:, k // 32].astype(np.float64) - 127)
        b = vq[:, k] * np.exp2(sq[:, k // 32].astype(np.float64) - 127)
        C += np.outer(a, b)
    return C


def _with_outliers(a, rng, n=2, big=600.0):
    a = a.copy()
    for _ in range(n):
        i, j = rng.integers(0, a.shape[0]), rng.integers(0, a.shape[1])
        a[i, j] = big * (1 if rng.random() < 0.5 else -1)
    return a


def _assert_product(got, want, what):
    err = np.max(np.abs(got - want)) / np.max(np.abs(want))
    assert err < 1e-12, f"{what}: max error {err:.3e} relative to the largest output"


def test_mx4_forward_gemms_quantise_along_their_contraction():
    rng = np.random.default_rng(21)
    n, d, f = 40, 96, 64
    x = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    w13 = _with_outliers(rng.normal(0, 0.05, (2 * f, d)), rng, big=30.0)
    w2 = _with_outliers(rng.normal(0, 0.05, (d, f)), rng, big=30.0)
    o = O.swiglu_ffn_fwd_mx(x, w13, w2, "f64", fmt="e2m1")
    _assert_product(o["H"], _kmajor_product4(x, w13[:f]), "H")
    _assert_product(o["U"], _kmajor_product4(x, w13[f:]), "U")
    _assert_product(o["Y"], _kmajor_product4(o["A"], w2), "Y")


def test_mx4_backward_gemms_quantise_along_their_contraction():
    rng = np.random.default_rng(22)
    n, d, f = 40, 96, 64
    x = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    w13 = _with_outliers(rng.normal(0, 0.05, (2 * f, d)), rng, big=30.0)
    w2 = _with_outliers(rng.normal(0, 0.05, (d, f)), rng, big=30.0)
    H = rng.normal(0, 1, (n, f))
    U = _with_outliers(rng.normal(0, 1, (n, f)), rng)
    A = _with_outliers(rng.normal(0, 1, (n, f)), rng)
    dY = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    o = O.swiglu_ffn_bwd_mx(x, H, U, A, dY, w13, w2, "f64", fmt="e2m1")
    dHU = np.concatenate([o["dH"], o["dU"]], axis=1)
    _assert_product(o["dA"], _kmajor_product4(dY, w2.T), "dA")
    _assert_product(o["dW2"], _kmajor_product4(dY.T, A.T), "dW2")
    _assert_product(o["dX32"], _kmajor_product4(dHU, w13.T), "dX")
    _assert_product(o["dW13"], _kmajor_product4(dHU.T, x.T), "dW13")


def test_mx4_layer_runs_through_the_layer_oracle():
    """The layer oracle takes the MXFP4 expert for an mxfp4 layer: its output
    differs from the same layer in MXFP8 and from bf16, and equals the MXFP4
    expert applied row block by row block."""
    import moe_inputs as mi
    cfg = mi.MoEConfig("t4", T=40, d=64, E=4, k=2, f=64, dtype="mxfp4", expert_std=0.1, backward=True)
    inp = mi.make_inputs(cfg, seed=3, with_grad_inputs=True)
    f4 = O.layer_forward(inp, cfg)
    f8 = O.layer_forward(inp, cfg.with_(dtype="mxfp8"))
    fb = O.layer_forward(inp, cfg.with_(dtype="bf16"))
    assert not np.array_equal(f4["y"], f8["y"]) and not np.array_equal(f4["y"], fb["y"])
    e = int(np.argmax(np.diff(f4["offsets"])))
    lo, hi = int(f4["offsets"][e]), int(f4["offsets"][e + 1])
    o = O.swiglu_ffn_fwd_mx(f4["Xp"][lo:hi], O._np(inp["w13"][e]), O._np(inp["w2"][e]), "bf16", fmt="e2m1")
    np.testing.assert_array_equal(f4["Yp"][lo:hi], o["Y"])
    b4 = O.layer_backward(inp, f4, cfg)
    assert np.all(np.isfinite(b4["dx"]))
