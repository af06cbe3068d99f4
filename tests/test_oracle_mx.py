"""Pins of the oracle's MXFP8 arithmetic (fp8 e4m3fn codes with e8m0 block
scales of 32 along the contraction) to facts outside it: torch's float8_e4m3fn
conversions (a library routine), the format's definition on all 256 codes,
constructed round-to-nearest-even midpoints, the scale rule's inequalities, and
brute-force loops over codes and scales for the block layout of every GEMM
operand orientation the layer uses."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_all_codes_match_torch():
    mine, ref = O.e4m3_decode(ALL), _torch_decode(ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert O.e4m3_decode([0x7E])[0] == 448.0 and O.e4m3_decode([0x01])[0] == 2.0 ** -9


def test_e4m3_encode_inverts_decode():
    ok = ~np.isnan(O.e4m3_decode(ALL))
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(ALL[ok])), ALL[ok])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000),
                        rng.normal(0, 0.01, 2000), np.exp2(rng.uniform(-12, 8.7, 2000))])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(v), ref)


def test_e4m3_rne_midpoints_and_saturation():
    vals = O.e4m3_decode(np.arange(0x7E, dtype=np.uint8))      # 0 .. 416 ascending
    mids = (vals[:-1] + vals[1:]) / 2
    got = O.e4m3_encode(mids)
    lo = np.arange(0x7D, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)    # the even code of the pair
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(O.e4m3_encode([448.0, 460.0, 1e6, -1e6]), [0x7E, 0x7E, 0x7E, 0xFE])
    np.testing.assert_array_equal(O.e4m3_encode([0.0, -0.0, 2.0 ** -11]), [0x00, 0x80, 0x00])


def test_scale_rule_is_minimal_and_never_clips():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.exp2(rng.uniform(-100, 100, 5000)), 448.0 * np.exp2(np.arange(-20, 20.0))])
    e = O.mx_scale_exp(amax).astype(np.float64)
    assert np.all(448.0 * np.exp2(e) >= amax)
    assert np.all(448.0 * np.exp2(e - 1) < amax)
    assert O.mx_scale_exp([0.0])[0] == -127
    assert O.mx_scale_exp([1e-300])[0] == -127 and O.mx_scale_exp([1e300])[0] == 127
    # a block's largest magnitude lands in [224, 448] (scaled amax in (224, 448],
    # then rounded): the top of the range, no saturation
    blk = rng.normal(0, 3, (200, 32))
    codes, sb = O.mx_quantize(blk, 1)
    top = np.max(np.abs(O.e4m3_decode(codes)), axis=1)
    assert np.all((top >= 224) & (top <= 448)) and np.all(sb[:, 0] == O.mx_scale_exp(np.abs(blk).max(1)) + 127)


def _brute_dot(ca, sa, cb, sb, i, j, K):
    """sum_k dec(a[i,k]) 2^(sa[i,k//32]-127) * dec(b[j,k]) 2^(sb[j,k//32]-127), one term at a time"""
    tot = 0.0
    for k in range(K):
        av = O.e4m3_decode([ca[i, k]])[0] * 2.0 ** (int(sa[i, k // 32]) - 127)
        bv = O.e4m3_decode([cb[j, k]])[0] * 2.0 ** (int(sb[j, k // 32]) - 127)
        tot += av * bv
    return tot


@pytest.mark.parametrize("axis_a,axis_b", [(1, 1), (0, 0), (1, 0), (0, 1)])
def test_mx_gemm_matches_brute_force_over_codes(axis_a, axis_b):
    """C = qdq(A along K) . qdq(B along K) for each storage orientation of the
    operands (K-contiguous = axis 1, row-index-contiguous = axis 0), checked
    element by element against loops over the codes and scales."""
    rng = np.random.default_rng(2)
    M, N, K = 3, 4, 70                                     # K not a multiple of 32: a padded last block
    a = rng.normal(0, 1, (M, K)) * np.exp2(rng.integers(-6, 6, (M, K)))
    b = rng.normal(0, 1, (N, K)) * np.exp2(rng.integers(-6, 6, (N, K)))
    a_st = a if axis_a == 1 else a.T.copy()                # how the operand lies in memory
    b_st = b if axis_b == 1 else b.T.copy()
    qa = O.mx_qdq(a_st, axis_a)
    qb = O.mx_qdq(b_st, axis_b)
    C = (qa if axis_a == 1 else qa.T) @ (qb if axis_b == 1 else qb.T).T
    ca, sa = O.mx_quantize(a, 1)
    cb, sb = O.mx_quantize(b, 1)
    for i in range(M):
        for j in range(N):
            assert C[i, j] == pytest.approx(_brute_dot(ca, sa, cb, sb, i, j, K), rel=1e-12, abs=1e-300)


def test_row_blocks_restart_at_the_range_start():
    """Quantising an expert's 40 rows along the rows uses blocks [0, 32) and
    [32, 40) of that range (rows past its end count as zero), not blocks of the
    whole buffer."""
    rng = np.random.default_rng(3)
    full = rng.normal(0, 1, (100, 5))
    full[50] = 1000.0                                      # a huge row inside the expert's first block
    lo, hi = 45, 85
    q = O.mx_qdq(full[lo:hi], 0)
    # block 1 of the range (rows 77..84) is independent of row 50
    own = O.mx_qdq(full[lo + 32:hi], 0)
    np.testing.assert_array_equal(q[32:], own)
    # block 0 holds row 50, so its small rows quantise coarsely (flushed to zero at 1000/448 scale)
    assert np.abs(q[:32][np.abs(full[lo:lo + 32]) < 0.005]).max(initial=0.0) == 0.0


def test_mx_forward_equals_bf16_forward_on_grid_inputs():
    """With inputs whose every 32-block is exactly representable (values on the
    e4m3 grid times a power-of-two block scale), MXFP8 quantisation of X and W is
    lossless, so H and U of the MX expert equal those of the bf16 expert."""
    rng = np.random.default_rng(4)
    grid = np.array([-2.0, -1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0, 2.0])
    n, d, f = 6, 64, 32
    x = rng.choice(grid, (n, d))
    w13 = rng.choice(grid, (2 * f, d)) / 8
    w2 = rng.choice(grid, (d, f)) / 8
    np.testing.assert_array_equal(O.mx_qdq(x, 1), x)
    np.testing.assert_array_equal(O.mx_qdq(w13, 1), w13)
    a = O.swiglu_ffn_fwd_mx(x, w13, w2, "bf16")
    b = O.swiglu_ffn_fwd(x, w13, w2, "bf16")
    np.testing.assert_array_equal(a["H"], b["H"])
    np.testing.assert_array_equal(a["U"], b["U"])
    np.testing.assert_array_equal(a["A"], b["A"])


def test_mx_backward_is_close_to_bf16_backward():
    """MXFP8 moves each GEMM by a few percent (the e4m3 step is 2^-3 relative at
    the bottom of a binade, 2^-4 at the top): the MX expert's gradients differ
    from the bf16 expert's by more than bf16 rounding and by less than 10%
    relative L2 (dX goes through two MX GEMMs)."""
    rng = np.random.default_rng(5)
    n, d, f = 48, 64, 96
    x = O.round_bf16(rng.normal(0, 1, (n, d)))
    w13 = O.round_bf16(rng.normal(0, 0.1, (2 * f, d)))
    w2 = O.round_bf16(rng.normal(0, 0.1, (d, f)))
    dy = O.round_bf16(rng.normal(0, 1, (n, d)))
    fa = O.swiglu_ffn_fwd(x, w13, w2, "bf16")
    ga = O.swiglu_ffn_bwd(x, fa["H"], fa["U"], fa["A"], dy, w13, w2, "bf16")
    gm = O.swiglu_ffn_bwd_mx(x, fa["H"], fa["U"], fa["A"], dy, w13, w2, "bf16")
    for k in ("dH", "dU", "dX", "dW13", "dW2"):
        rel = np.linalg.norm(gm[k] - ga[k]) / np.linalg.norm(ga[k])
        assert 1e-4 < rel < 1e-1, (k, rel)


# ---------------------------------------------------------------------------
# Quantisation axis of every GEMM of the MXFP8 expert.  Each product
# C[i, j] = sum_k P[i, k] Q[j, k] must see both operands quantised in blocks
# of 32 along its contraction index k (the tensor layouts per GEMM of the
# figures page, Figure 31).  The reference below writes each operand in its
# K-major form, quantises it along that K, and sums one k at a time with the
# block index k // 32 spelled out.  Inputs carry one large outlier per
# operand: in the right blocks it only coarsens its own 32-value block, in a
# block laid along the other axis it flushes the small values of 31 other
# rows to zero, which moves whole rows of the product.
# ---------------------------------------------------------------------------
def _kmajor_product(P, Q):
    """sum_k deq(P)[i, k] deq(Q)[j, k] with P [M, K], Q [N, K] quantised along K."""
    cp, sp = O.mx_quantize(P, 1)
    cq, sq = O.mx_quantize(Q, 1)
    vp, vq = O.e4m3_decode(cp), O.e4m3_decode(cq)
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


def test_mx_forward_gemms_quantise_along_their_contraction():
    """H, U = X W13^T contract over d (X and W13 blocked along d); Y = A W2^T
    contracts over f (A and W2 blocked along f).  The oracle runs unrounded
    ("f64" storage) so that each product is compared exactly."""
    rng = np.random.default_rng(21)
    n, d, f = 40, 96, 64                         # 40 rows: a short last row block
    x = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    w13 = _with_outliers(rng.normal(0, 0.05, (2 * f, d)), rng, big=30.0)
    w2 = _with_outliers(rng.normal(0, 0.05, (d, f)), rng, big=30.0)
    o = O.swiglu_ffn_fwd_mx(x, w13, w2, "f64")
    _assert_product(o["H"], _kmajor_product(x, w13[:f]), "H")
    _assert_product(o["U"], _kmajor_product(x, w13[f:]), "U")
    _assert_product(o["Y"], _kmajor_product(o["A"], w2), "Y")


def test_mx_backward_gemms_quantise_along_their_contraction():
    """dA = dY W2 contracts over d (dY along d, W2 along its rows d);
    dW2 = dY^T A and dW13 = dHU^T X contract over the expert's rows (blocks of
    32 rows from its first row); dX = dHU W13 contracts over 2f (dHU along 2f,
    W13 along its rows).  The outliers sit in X, dY, A, W13, W2 and in U
    (which carries one into dH)."""
    rng = np.random.default_rng(22)
    n, d, f = 40, 96, 64
    x = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    w13 = _with_outliers(rng.normal(0, 0.05, (2 * f, d)), rng, big=30.0)
    w2 = _with_outliers(rng.normal(0, 0.05, (d, f)), rng, big=30.0)
    H = rng.normal(0, 1, (n, f))
    U = _with_outliers(rng.normal(0, 1, (n, f)), rng)
    A = _with_outliers(rng.normal(0, 1, (n, f)), rng)
    dY = _with_outliers(rng.normal(0, 1, (n, d)), rng)
    o = O.swiglu_ffn_bwd_mx(x, H, U, A, dY, w13, w2, "f64")
    dHU = np.concatenate([o["dH"], o["dU"]], axis=1)
    assert np.max(np.abs(o["dH"])) > 50 * np.median(np.abs(o["dH"]))     # U's outlier reached dH
    _assert_product(o["dA"], _kmajor_product(dY, w2.T), "dA")
    _assert_product(o["dW2"], _kmajor_product(dY.T, A.T), "dW2")
    _assert_product(o["dX32"], _kmajor_product(dHU, w13.T), "dX")
    _assert_product(o["dW13"], _kmajor_product(dHU.T, x.T), "dW13")
