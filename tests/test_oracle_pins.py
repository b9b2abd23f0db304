"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself (exact rational arithmetic, numpy/scipy library routines,
algebraic identities, closed-form special cases, the pages' printed sizes).

Chosen so that a plausible mistake -- a dropped zero-point term, a wrong sign,
a transposed operand, a flipped filter, a missing padding check, an FMA where
two roundings are defined -- fails at least one of them.
"""
from fractions import Fraction
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# binary16 decoder
# --------------------------------------------------------------------------
def test_f16_decoder_all_bit_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)  # numpy's own conversion
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_decoder_hand_values(oracle):
    # textbook binary16 values
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3555: 0.333251953125, 0x8000: -0.0}
    for b, v in cases.items():
        assert oracle.f16_to_f64(np.array([b], np.uint16))[0] == v


# --------------------------------------------------------------------------
# O1 fp16 GEMM
# --------------------------------------------------------------------------
def _frac_gemm(A, Bt):
    M, K = A.shape
    N = Bt.shape[0]
    Af = [[Fraction(float(v)) for v in row] for row in A.astype(np.float64)]
    Bf = [[Fraction(float(v)) for v in row] for row in Bt.astype(np.float64)]
    return [[sum((Af[m][k] * Bf[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 7, 3)])
def test_gemm_f16_brute_force_exact(oracle, M, N, K):
    rng = np.random.default_rng(100 + M * 64 + N * 8 + K)
    A = synth.f16_uniform(rng, (M, K))
    Bt = synth.f16_uniform(rng, (N, K))
    R = oracle.gemm_f16(A, Bt)
    exact = _frac_gemm(A, Bt)
    for m in range(M):
        for n in range(N):
            bound = sum(abs(float(A[m, k]) * float(Bt[n, k])) for k in range(K)) * K * 2.0 ** -52
            assert abs(Fraction(R[m, n]) - exact[m][n]) <= Fraction(bound), (m, n)


def test_gemm_f16_integer_valued_exact(oracle):
    rng = np.random.default_rng(7)
    A = synth.f16_small_ints(rng, (37, 96))
    Bt = synth.f16_small_ints(rng, (29, 96))
    R = oracle.gemm_f16(A, Bt)
    ref = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert np.array_equal(R, ref.astype(np.float64))


def test_gemm_f16_vs_numpy_float64(oracle):
    rng = np.random.default_rng(8)
    A = synth.f16_normal(rng, (61, 203))
    Bt = synth.f16_normal(rng, (45, 203))
    R = oracle.gemm_f16(A, Bt)
    ref = A.astype(np.float64) @ Bt.astype(np.float64).T
    assert np.max(np.abs(R - ref)) <= 1e-12 * np.max(np.abs(ref))
    # a transposed operand would fail this (non-square, distinct shapes)
    assert R.shape == (61, 45)


def test_gemm_f16_transpose_invariant(oracle):
    rng = np.random.default_rng(9)
    A = synth.f16_uniform(rng, (13, 40))
    Bt = synth.f16_uniform(rng, (21, 40))
    assert np.array_equal(oracle.gemm_f16(A, Bt), oracle.gemm_f16(Bt, A).T)


def test_gemm_f16_identity(oracle):
    rng = np.random.default_rng(10)
    A = synth.f16_uniform(rng, (9, 16))
    I = np.eye(16, dtype=np.float16)
    assert np.array_equal(oracle.gemm_f16(A, I), A.astype(np.float64))


# --------------------------------------------------------------------------
# O2 / O3 u8 x i8 with zero points
# --------------------------------------------------------------------------
def _py_int_gemm(A, zA, Bt, zB):
    M, K = A.shape
    N = Bt.shape[0]
    return [[sum((int(A[m, k]) - zA) * (int(Bt[n, k]) - zB) for k in range(K)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("zA,zB", [(128, 3), (128, 0), (0, 0), (17, -5), (255, 127), (3, -128)])
def test_int_naive_brute_force(oracle, zA, zB):
    rng = np.random.default_rng(abs(zA * 131 + zB))
    A = synth.u8_uniform(rng, (6, 8))
    Bt = synth.i8_uniform(rng, (7, 8), lo=-128, hi=127)
    C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
    assert C.tolist() == _py_int_gemm(A, zA, Bt, zB)


@pytest.mark.parametrize("zA,zB", [(128, 3), (128, 0), (0, 0), (17, -5), (255, 127), (200, -128)])
def test_int_closed_form_equals_naive(oracle, zA, zB):
    rng = np.random.default_rng(1000 + zA + 7 * (zB + 128))
    A = synth.u8_uniform(rng, (33, 77))
    Bt = synth.i8_uniform(rng, (19, 77), lo=-128, hi=127)
    assert np.array_equal(oracle.gemm_u8i8_naive(A, zA, Bt, zB), oracle.gemm_u8i8_closed(A, zA, Bt, zB))


def test_int_vs_numpy_int64(oracle):
    rng = np.random.default_rng(11)
    A = synth.u8_uniform(rng, (50, 300))
    Bt = synth.i8_uniform(rng, (40, 300))
    zA, zB = 128, 3
    ref = (A.astype(np.int64) - zA) @ (Bt.astype(np.int64) - zB).T
    assert np.array_equal(oracle.gemm_u8i8_naive(A, zA, Bt, zB), ref)
    assert np.array_equal(oracle.gemm_u8i8_closed(A, zA, Bt, zB), ref)


@pytest.mark.parametrize("a,b", [(255, -128), (0, 127), (255, 127), (0, -128)])
def test_int_extreme_constant_inputs(oracle, a, b):
    K = 33
    A = np.full((4, K), a, np.uint8)
    Bt = np.full((3, K), b, np.int8)
    for zA, zB in [(128, 3), (0, 0), (255, -128)]:
        want = K * (a - zA) * (b - zB)
        assert np.all(oracle.gemm_u8i8_naive(A, zA, Bt, zB) == want)
        assert np.all(oracle.gemm_u8i8_closed(A, zA, Bt, zB) == want)


def test_int_special_cases(oracle):
    rng = np.random.default_rng(12)
    K = 24
    Bt = synth.i8_uniform(rng, (5, K))
    A = np.full((4, K), 77, np.uint8)
    assert np.all(oracle.gemm_u8i8_closed(A, 77, Bt, 9) == 0)        # A == zA
    A2 = synth.u8_uniform(rng, (4, K))
    Bz = np.full((5, K), -4, np.int8)
    assert np.all(oracle.gemm_u8i8_closed(A2, 128, Bz, -4) == 0)     # B == zB
    # K = 1: outer product
    a1 = synth.u8_uniform(rng, (6, 1))
    b1 = synth.i8_uniform(rng, (7, 1))
    outer = np.outer(a1[:, 0].astype(np.int64) - 10, b1[:, 0].astype(np.int64) + 2)
    assert np.array_equal(oracle.gemm_u8i8_closed(a1, 10, b1, -2), outer)
    # B = identity (zB = 0): C = A - zA
    A3 = synth.u8_uniform(rng, (5, 16))
    I = np.eye(16, dtype=np.int8)
    assert np.array_equal(oracle.gemm_u8i8_closed(A3, 128, I, 0), A3.astype(np.int64) - 128)


def test_int_row_col_sums(oracle):
    rng = np.random.default_rng(13)
    A = synth.u8_uniform(rng, (9, 31))
    Bt = synth.i8_uniform(rng, (8, 31), lo=-128, hi=127)
    assert np.array_equal(oracle.u8_rowsum(A), A.astype(np.int64).sum(1))
    assert np.array_equal(oracle.i8_colsum(Bt), Bt.astype(np.int64).sum(1))


# --------------------------------------------------------------------------
# O4 dequant / O5 requant
# --------------------------------------------------------------------------
def test_dequant_matches_numpy_float32(oracle):
    rng = np.random.default_rng(14)
    C = rng.integers(-(2 ** 31), 2 ** 31, size=(17, 23), dtype=np.int64)
    D = oracle.dequant(C, 0.02, 0.01)
    s = np.float32(np.float32(0.02) * np.float32(0.01))
    assert oracle.dequant_scale(0.02, 0.01) == s
    ref = C.astype(np.float32) * s  # int64 -> float32 is RNE in numpy; one fp32 product
    assert np.array_equal(D, ref)


def test_dequant_large_ints_round_once(oracle):
    # 2^24 + 1 is not representable in fp32: the conversion rounds to even.
    C = np.array([[2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 24 + 1)]], np.int64)
    D = oracle.dequant(C, 1.0, 1.0)
    assert D.tolist() == [[16777216.0, 16777220.0, -16777216.0]]


def test_dequant_hand_cases(oracle):
    """Hand-worked binary32 cases, two of them where the reading taken,
    fl32(fl32(C) * fl32(sA*sB)), differs from multiplying by sA and sB in
    turn."""
    with open(os.path.join(GOLDEN, "dequant_cases.json")) as f:
        cases = json.load(f)["cases"]
    differing = 0
    for c in cases:
        sA, sB = float.fromhex(c["sA"]), float.fromhex(c["sB"])
        assert np.float32(sA) == sA and np.float32(sB) == sB, c  # the scales are binary32 values
        D = oracle.dequant(np.array([[c["C"]]], np.int64), sA, sB)
        assert float(D[0, 0]) == float.fromhex(c["D"]), c
        if "other_order" in c:
            assert float.fromhex(c["other_order"]) != float.fromhex(c["D"])
            differing += 1
    assert differing >= 2


def test_requant_hand_cases(oracle):
    with open(os.path.join(GOLDEN, "requant_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert oracle.requant_one(c["acc"], c["scale"], c["bias"]) == c["q"], c


def test_requant_matches_numpy(oracle):
    rng = np.random.default_rng(15)
    C = rng.integers(-(2 ** 27), 2 ** 27, size=(31, 40), dtype=np.int64)
    scale = rng.uniform(1e-7, 2e-6, size=40).astype(np.float32)
    bias = rng.standard_normal(40).astype(np.float32)
    Q = oracle.requant(C, scale, bias)
    t = C.astype(np.float32) * scale[None, :]
    y = t + bias[None, :]
    ref = np.clip(np.rint(y), -128, 127).astype(np.int8)  # numpy rint: half to even
    assert np.array_equal(Q, ref)
    assert np.count_nonzero((ref > -128) & (ref < 127)) > 100  # exercised unsaturated


def test_requant_differs_from_fused_multiply_add(oracle):
    # Search (with numpy's IEEE float32 arithmetic) for inputs where the
    # two-rounding form fl(fl(c*s)+b) and a fused c*s+b requantize to different
    # int8 values; the oracle must give the two-rounding answer on every one.
    rng = np.random.default_rng(16)
    n = 4_000_000
    C = rng.integers(-40000, 40000, size=n)
    s = rng.uniform(0.001, 0.003, size=n).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    two = (C.astype(np.float32) * s) + b
    fused = (C.astype(np.float64) * s.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    q_two = np.clip(np.rint(two), -128, 127)
    q_fused = np.clip(np.rint(fused), -128, 127)
    idx = np.nonzero(q_two != q_fused)[0]
    assert idx.size >= 1
    for i in idx:
        got = oracle.requant_one(int(C[i]), s[i], b[i])
        assert got == int(q_two[i]) != int(q_fused[i])


# --------------------------------------------------------------------------
# O6 / O7 convolution
# --------------------------------------------------------------------------
CONV_SHAPES = [
    # Nb, H, W, C, Kout, R, S, stride, pad
    (2, 5, 6, 3, 4, 3, 3, (1, 1), (1, 1)),
    (1, 7, 5, 2, 3, 3, 2, (2, 1), (1, 0)),
    (3, 4, 4, 5, 2, 1, 1, (1, 1), (0, 0)),
    (1, 6, 6, 4, 3, 5, 5, (1, 1), (2, 2)),
    (2, 9, 8, 3, 2, 3, 3, (2, 2), (1, 1)),
]


@pytest.mark.parametrize("shape", CONV_SHAPES)
def test_conv_direct_equals_im2col_gemm(oracle, shape):
    Nb, H, W, C, Kout, R, S, st, pd = shape
    rng = np.random.default_rng(sum(shape[:7]))
    x = synth.f16_normal(rng, (Nb, H, W, C))
    w = synth.f16_normal(rng, (Kout, R, S, C))
    yd = oracle.conv2d_direct(x, w, st, pd)
    yi = oracle.conv2d_im2col(x, w, st, pd)
    assert np.array_equal(yd, yi)  # same (r, s, c) order -> identical doubles


@pytest.mark.parametrize("shape", CONV_SHAPES)
def test_conv_direct_vs_scipy_correlate(oracle, shape):
    from scipy.signal import correlate2d

    Nb, H, W, C, Kout, R, S, (sh, sw), (ph, pw) = shape
    rng = np.random.default_rng(7 * sum(shape[:7]))
    x = synth.f16_normal(rng, (Nb, H, W, C))
    w = synth.f16_normal(rng, (Kout, R, S, C))
    y = oracle.conv2d_direct(x, w, (sh, sw), (ph, pw))
    xd = np.pad(x.astype(np.float64), ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    P, Q = y.shape[1], y.shape[2]
    ref = np.zeros_like(y)
    for n in range(Nb):
        for k in range(Kout):
            acc = sum(correlate2d(xd[n, :, :, c], w[k, :, :, c].astype(np.float64), mode="valid")
                      for c in range(C))
            ref[n, :, :, k] = acc[::sh, ::sw][:P, :Q]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_conv_impulse_pins_orientation_and_padding(oracle):
    Nb, H, W, C, Kout, R, S = 1, 6, 7, 3, 2, 3, 3
    rng = np.random.default_rng(17)
    w = synth.f16_normal(rng, (Kout, R, S, C))
    h0, w0, c0 = 0, 4, 1
    x = np.zeros((Nb, H, W, C), np.float16)
    x[0, h0, w0, c0] = 1.0
    y = oracle.conv2d_direct(x, w, (1, 1), (1, 1))
    want = np.zeros_like(y)
    for r in range(R):
        for s in range(S):
            p, q = h0 + 1 - r, w0 + 1 - s
            if 0 <= p < H and 0 <= q < W:
                want[0, p, q, :] = w[:, r, s, c0].astype(np.float64)
    assert np.array_equal(y, want)


def test_conv_all_ones_border_sums(oracle):
    Nb, H, W, C, Kout = 1, 5, 5, 2, 3
    rng = np.random.default_rng(18)
    w = synth.f16_small_ints(rng, (Kout, 3, 3, C), -3, 3)
    x = np.ones((Nb, H, W, C), np.float16)
    y = oracle.conv2d_direct(x, w, (1, 1), (1, 1))
    wi = w.astype(np.int64)
    # corner (0,0) sees taps r,s in {1,2}; interior sees all 9
    assert np.array_equal(y[0, 0, 0], wi[:, 1:, 1:, :].sum((1, 2, 3)).astype(np.float64))
    assert np.array_equal(y[0, 2, 2], wi.sum((1, 2, 3)).astype(np.float64))
    assert np.array_equal(y[0, 4, 2], wi[:, :2, :, :].sum((1, 2, 3)).astype(np.float64))


def test_conv_1x1_equals_gemm(oracle):
    rng = np.random.default_rng(19)
    x = synth.f16_normal(rng, (2, 3, 4, 16))
    w = synth.f16_normal(rng, (5, 1, 1, 16))
    y = oracle.conv2d_direct(x, w)
    g = oracle.gemm_f16(x.reshape(-1, 16), w.reshape(5, 16))
    assert np.array_equal(y.reshape(-1, 5), g)


def test_conv_direct_at_matches_full(oracle):
    rng = np.random.default_rng(20)
    x = synth.f16_normal(rng, (2, 5, 5, 4))
    w = synth.f16_normal(rng, (3, 3, 3, 4))
    full = oracle.conv2d_direct(x, w, (1, 1), (1, 1)).reshape(-1, 3)
    pix = [0, 7, 24, 25, 49]
    assert np.array_equal(oracle.conv2d_direct_at(x, w, pix, (1, 1), (1, 1)), full[pix])


def test_conv_sizes_match_printed_tutorial_sizes(oracle):
    with open(os.path.join(GOLDEN, "conv_tutorial_sizes.json")) as f:
        g = json.load(f)
    c = g["problem"]
    P = oracle.conv_out_dim(c["height"], c["kernel_h"], c["stride_h"], c["pad_h"])
    Q = oracle.conv_out_dim(c["width"], c["kernel_w"], c["stride_w"], c["pad_w"])
    assert P * Q == g["printed"]["grid_z_extent"]
    assert c["batch"] * c["height"] * c["width"] * c["in_channels"] == g["printed"]["input_elements"]
    assert c["kernel_h"] * c["kernel_w"] * c["in_channels"] * c["out_channels"] == g["printed"]["weight_elements"]
    assert c["batch"] * P * Q * c["out_channels"] == g["printed"]["output_elements"]
    wl = synth.workload("c4", scale_down=256)  # same geometry, batch 1
    d = wl.dims
    assert (d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"]) == (
        c["height"], c["width"], c["in_channels"], c["out_channels"], c["kernel_h"], c["kernel_w"])


# --------------------------------------------------------------------------
# O8: quantized convolution (u8 activations x i8 weights, zero points; the
# padding holds the zero point, i.e. the real value 0)
# --------------------------------------------------------------------------
QCONV_CASES = [
    # Nb, H, W, C, Kout, R, S, stride, pad, zA, zB
    (2, 5, 6, 3, 4, 3, 3, (1, 1), (1, 1), 128, 3),
    (1, 7, 5, 2, 3, 3, 2, (2, 1), (1, 0), 37, -5),
    (3, 4, 4, 5, 2, 1, 1, (1, 1), (0, 0), 0, 0),
    (1, 6, 6, 4, 3, 5, 5, (1, 1), (2, 2), 255, 127),
    (2, 9, 8, 3, 2, 3, 3, (2, 2), (1, 1), 100, -128),
]


def _qconv_inputs(rng, case):
    Nb, H, W, C, Kout, R, S = case[:7]
    x = synth.u8_uniform(rng, (Nb, H, W, C))
    w = rng.integers(-128, 128, (Kout, R, S, C)).astype(np.int8)
    return x, w


@pytest.mark.parametrize("case", QCONV_CASES)
def test_qconv_equals_zero_point_im2col_then_naive_gemm(oracle, case):
    Nb, H, W, C, Kout, R, S, st, pd, zA, zB = case
    rng = np.random.default_rng(sum(case[:7]) + zA)
    x, w = _qconv_inputs(rng, case)
    y = oracle.conv2d_u8i8_direct(x, zA, w, zB, st, pd)
    col = oracle.im2col_u8(x, zA, R, S, st, pd)
    ref = oracle.gemm_u8i8_naive(col, zA, w.reshape(Kout, R * S * C), zB)
    assert np.array_equal(y.reshape(-1, Kout), ref)


@pytest.mark.parametrize("case", QCONV_CASES)
def test_qconv_vs_scipy_correlate_of_shifted_values(oracle, case):
    # the real-valued view: (x - zA) zero-padded, correlated with (w - zB)
    from scipy.signal import correlate2d

    Nb, H, W, C, Kout, R, S, (sh, sw), (ph, pw), zA, zB = case
    rng = np.random.default_rng(5 * sum(case[:7]) + zA)
    x, w = _qconv_inputs(rng, case)
    y = oracle.conv2d_u8i8_direct(x, zA, w, zB, (sh, sw), (ph, pw))
    xd = np.pad(x.astype(np.float64) - zA, ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    wd = w.astype(np.float64) - zB
    P, Q = y.shape[1], y.shape[2]
    ref = np.zeros(y.shape, np.float64)
    for n in range(Nb):
        for k in range(Kout):
            acc = sum(correlate2d(xd[n, :, :, c], wd[k, :, :, c], mode="valid") for c in range(C))
            ref[n, :, :, k] = acc[::sh, ::sw][:P, :Q]
    assert np.array_equal(y.astype(np.float64), ref)  # integers far below 2^53: exact


def test_qconv_brute_force_python_ints(oracle):
    Nb, H, W, C, Kout, R, S, (sh, sw), (ph, pw), zA, zB = 1, 4, 3, 2, 2, 3, 3, (1, 1), (1, 1), 77, 9
    rng = np.random.default_rng(99)
    x, w = _qconv_inputs(rng, (Nb, H, W, C, Kout, R, S))
    y = oracle.conv2d_u8i8_direct(x, zA, w, zB, (sh, sw), (ph, pw))
    for p in range(y.shape[1]):
        for q in range(y.shape[2]):
            for k in range(Kout):
                acc = 0
                for r in range(R):
                    for s in range(S):
                        h, ww = p * sh + r - ph, q * sw + s - pw
                        for c in range(C):
                            xv = int(x[0, h, ww, c]) if 0 <= h < H and 0 <= ww < W else zA
                            acc += (xv - zA) * (int(w[k, r, s, c]) - zB)
                assert int(y[0, p, q, k]) == acc


def test_qconv_special_cases(oracle):
    Nb, H, W, C, Kout, R, S = 2, 5, 4, 3, 3, 3, 3
    rng = np.random.default_rng(31)
    x, w = _qconv_inputs(rng, (Nb, H, W, C, Kout, R, S))
    # activations at the zero point, or weights at theirs: exactly zero
    assert not oracle.conv2d_u8i8_direct(np.full_like(x, 61), 61, w, 4, (1, 1), (1, 1)).any()
    assert not oracle.conv2d_u8i8_direct(x, 61, np.full_like(w, -7), -7, (1, 1), (1, 1)).any()
    # x - zA = 1 and w - zB = 1 everywhere: each output counts its in-image
    # taps times C (the padded taps contribute nothing, not (0 - zA)(w - zB))
    y = oracle.conv2d_u8i8_direct(np.full_like(x, 201), 200, np.full_like(w, -3), -4, (1, 1), (1, 1))
    rows = np.array([min(p + 1, H - 1) - max(p - 1, 0) + 1 for p in range(H)])
    cols = np.array([min(q + 1, W - 1) - max(q - 1, 0) + 1 for q in range(W)])
    want = (rows[:, None] * cols[None, :] * C).astype(np.int64)
    assert np.array_equal(y, np.broadcast_to(want[None, :, :, None], y.shape))
    # 1x1 filter, no padding: the u8 x i8 GEMM of the pixels
    w1 = w[:, :1, :1, :]
    y1 = oracle.conv2d_u8i8_direct(x, 90, w1, -2, (1, 1), (0, 0))
    ref = oracle.gemm_u8i8_naive(x.reshape(-1, C), 90, w1.reshape(Kout, C), -2)
    assert np.array_equal(y1.reshape(-1, Kout), ref)
    # a listed subset of pixels equals those rows of the whole output
    pix = np.array([0, 7, 19, Nb * H * W - 1])
    at = oracle.conv2d_u8i8_direct_at(x, 13, w, 5, pix, (1, 1), (1, 1))
    assert np.array_equal(at, oracle.conv2d_u8i8_direct(x, 13, w, 5, (1, 1), (1, 1)).reshape(-1, Kout)[pix])


# ----------------------------------------------------------------- O9: blocked NHWCnc layout
def blk_x_to_nhwc(xb):
    """[Nb/16][H][W][C/16][16n][16c] -> [Nb][H][W][C] (numpy permutation only)."""
    NB, H, W, CB = xb.shape[:4]
    return xb.transpose(0, 4, 1, 2, 3, 5).reshape(NB * 16, H, W, CB * 16)


def blk_w_to_krsc(wb):
    """[R][S][C/16][K/16][16c][16k] -> [K][R][S][C]."""
    R, S, CB, OB = wb.shape[:4]
    return wb.transpose(3, 5, 0, 1, 2, 4).reshape(OB * 16, R, S, CB * 16)


def blk_y_to_nhwc(yb):
    """[Nb/16][P][Q][K/16][16n][16k] -> [Nb][P][Q][K]."""
    NB, P, Q, OB = yb.shape[:4]
    return yb.transpose(0, 4, 1, 2, 3, 5).reshape(NB * 16, P, Q, OB * 16)


@pytest.mark.parametrize("NB,H,W,CB,OB,R,S,stride,pad", [
    (1, 5, 4, 2, 1, 3, 3, (1, 1), (1, 1)),
    (2, 3, 6, 1, 2, 2, 3, (2, 1), (0, 2)),
    (1, 4, 4, 3, 1, 1, 1, (1, 1), (0, 0)),
])
def test_conv_nhwcnc_equals_direct_nhwc(oracle, NB, H, W, CB, OB, R, S, stride, pad):
    """O9 on blocked tensors is O6 on the same logical tensors, bit for bit
    (same (r, s, c) summation order; the layouts differ only by a
    permutation of axes)."""
    rng = np.random.default_rng(NB * 100 + H * 10 + W)
    xb = synth.f16_normal(rng, (NB, H, W, CB, 16, 16))
    wb = synth.f16_normal(rng, (R, S, CB, OB, 16, 16), std=0.1)
    yb = oracle.conv2d_nhwcnc_direct(xb, wb, stride, pad)
    y = oracle.conv2d_direct(blk_x_to_nhwc(xb), blk_w_to_krsc(wb), stride, pad)
    assert np.array_equal(blk_y_to_nhwc(yb), y)


def test_conv_nhwcnc_brute_force_from_the_blocked_formula(oracle):
    """Pure-Python integer evaluation of the blocked definition:
    Conv[nb,p,q,ob,nn,oo] = sum_{kh,kw,ic,ii} Apad[nb, p*sh+kh, q*sw+kw, ic, nn, ii]
                            * W[kh, kw, ic, ob, ii, oo]."""
    rng = np.random.default_rng(91)
    NB, H, W, CB, OB, R, S, sh, sw, ph, pw = 1, 2, 3, 1, 1, 2, 2, 1, 1, 1, 1
    xb = synth.f16_small_ints(rng, (NB, H, W, CB, 16, 16), -3, 3)
    wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16), -3, 3)
    P, Q = (H + 2 * ph - R) // sh + 1, (W + 2 * pw - S) // sw + 1
    A = xb.astype(np.int64).tolist()
    Wt = wb.astype(np.int64).tolist()
    yb = oracle.conv2d_nhwcnc_direct(xb, wb, (sh, sw), (ph, pw))
    for nb in range(NB):
        for p in range(P):
            for q in range(Q):
                for ob in range(OB):
                    for nn in range(16):
                        for oo in range(16):
                            acc = 0
                            for kh in range(R):
                                for kw in range(S):
                                    h, w = p * sh + kh - ph, q * sw + kw - pw
                                    if not (0 <= h < H and 0 <= w < W):
                                        continue  # Apad is 0 in the padding
                                    for ic in range(CB):
                                        for ii in range(16):
                                            acc += A[nb][h][w][ic][nn][ii] * Wt[kh][kw][ic][ob][ii][oo]
                            assert yb[nb, p, q, ob, nn, oo] == acc


def test_conv_nhwcnc_impulse(oracle):
    """One 1 at image n0, pixel (h0, w0), channel c0 of a blocked input: the
    output at image n0, pixel (h0 + ph - r, w0 + pw - s), channel k is the
    weight W[r, s, c0, k] -- cross-correlation orientation and block indexing."""
    NB, H, W, CB, OB, R, S = 1, 5, 6, 2, 1, 3, 3
    n0, h0, w0, c0 = 9, 2, 4, 21
    xb = np.zeros((NB, H, W, CB, 16, 16), np.float16)
    xb[n0 // 16, h0, w0, c0 // 16, n0 % 16, c0 % 16] = 1.0
    rng = np.random.default_rng(92)
    wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16))
    yb = oracle.conv2d_nhwcnc_direct(xb, wb, (1, 1), (1, 1))
    y = blk_y_to_nhwc(yb)
    for r in range(R):
        for s in range(S):
            p, q = h0 + 1 - r, w0 + 1 - s
            if 0 <= p < H and 0 <= q < W:
                for k in range(16 * OB):
                    assert y[n0, p, q, k] == float(wb[r, s, c0 // 16, k // 16, c0 % 16, k % 16])
    assert np.count_nonzero(y) <= R * S * 16 * OB
    assert np.count_nonzero(y[np.arange(16) != n0]) == 0


def test_blocked_workload_has_the_tutorials_shapes():
    with open(os.path.join(GOLDEN, "conv_tutorial_sizes.json")) as f:
        g = json.load(f)
    b, pr = g["blocked_layout"], g["printed"]
    wl = synth.workload("b4")
    assert list(wl.arrays["x"].shape) == b["data_shape"]
    assert list(wl.arrays["w"].shape) == b["kernel_shape"]
    assert int(np.prod(b["data_shape"])) == pr["input_elements"]
    assert int(np.prod(b["kernel_shape"])) == pr["weight_elements"]
    assert int(np.prod(b["output_shape"])) == pr["output_elements"]
