"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (int32 C, requantized int8 Q) and the dequantized fp32 D are
compared bit-exactly; fp32 outputs of the fp16 paths within the FP_TOL gate of
gpu_util.fp_rel_err.  Integer-valued fp16 inputs make the fp16 paths exact too,
which pins layouts, strides and data movement bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import FP_TOL, empty_dev, fp_rel_err, strided, to_dev, to_host, workspace_for

pytestmark = pytest.mark.gpu

VARIANTS = ["0", "1", "2", "4"]  # 256x256, 128x128, 64x64, 224x256 tiles


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    return m


@pytest.fixture(autouse=True)
def _default_tuning(igc):
    """Every test starts and ends with the library's default tuning."""
    igc.set_tuning(-1, 1)
    yield
    igc.set_tuning(-1, 1)


@pytest.fixture
def variant(request, igc):
    v = getattr(request, "param", None)
    igc.set_tuning(-1 if v is None else int(v), 1)
    return v


def run_f16(igc, A, Bt, lda=None, ldb=None, ldc=None, sentinel=np.nan):
    import torch

    M, K = A.shape
    N = Bt.shape[0]
    lda = lda or K
    ldb = ldb or K
    ldc = ldc or N
    dA = to_dev(strided(A, lda)) if M else empty_dev((0,), torch.float16)
    dB = to_dev(strided(Bt, ldb)) if N else empty_dev((0,), torch.float16)
    dC = to_dev(np.full((M, ldc), sentinel, np.float32))
    igc.gemm_f16f32(M, N, K, dA, lda, dB, ldb, dC, ldc, workspace=workspace_for(igc.gemm_f16f32_workspace_size(M, N, K)))
    C = to_host(dC)
    if ldc > N:  # columns past N are never written
        pad = C[:, N:]
        assert np.all(np.isnan(pad)) if np.isnan(sentinel) else np.all(pad == sentinel)
    return C[:, :N]


# ----------------------------------------------------------------- fp16 GEMM
F16_EXACT_SHAPES = [(64, 64, 64), (256, 256, 256), (300, 200, 264), (1, 1, 8), (33, 65, 136),
                    (513, 257, 192), (128, 384, 8)]


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("M,N,K", F16_EXACT_SHAPES)
def test_f16_integer_valued_bit_exact(igc, oracle, variant, M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = run_f16(igc, A, Bt)
    ref = oracle.gemm_f16(A, Bt)
    assert np.array_equal(C.astype(np.float64), ref)


# The LDS-bypass fp16 kernel (forced): 32x32 or 16x16 tiles, one wave each,
# operands loaded straight into the MFMA registers.
@pytest.mark.parametrize("bv", [5, 6])
@pytest.mark.parametrize("M,N,K", F16_EXACT_SHAPES + [(256, 256, 1024), (70, 33, 520)])
def test_f16_bypass_integer_valued_bit_exact(igc, oracle, bv, M, N, K):
    igc.set_tuning(bv, 1)
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = run_f16(igc, A, Bt)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f16(A, Bt))


@pytest.mark.parametrize("bv", [5, 6])
@pytest.mark.parametrize("M,N,K,ldc", [(256, 256, 256, 256), (200, 300, 1000, 301), (64, 48, 4096, 48)])
def test_f16_bypass_random_tolerance(igc, oracle, bv, M, N, K, ldc):
    igc.set_tuning(bv, 1)
    rng = np.random.default_rng(M + N + K + 5)
    A = synth.f16_uniform(rng, (M, K))
    Bt = synth.f16_uniform(rng, (N, K))
    C = run_f16(igc, A, Bt, ldc=ldc)
    assert fp_rel_err(C, oracle.gemm_f16(A, Bt)) <= FP_TOL


# Small tiles in grids of one round of 256 compute units or less (ragged
# edges, long K loops) and of several rounds (289-1156 tiles).
@pytest.mark.parametrize("variant,M,N,K", [("2", 1088, 1088, 264), ("1", 2176, 2176, 136),
                                           ("2", 200, 136, 2056), ("1", 300, 260, 1160)])
def test_f16_small_tiles_one_and_several_rounds(igc, oracle, variant, M, N, K):
    igc.set_tuning(int(variant), 1)
    rng = np.random.default_rng(M + N + K + 1)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = run_f16(igc, A, Bt)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f16(A, Bt))


@pytest.mark.parametrize("variant,M,N,K", [("2", 1088, 1088, 400), ("1", 2176, 2176, 144),
                                           ("2", 130, 70, 3000), ("1", 300, 260, 2064)])
def test_u8i8_small_tiles_one_and_several_rounds(igc, oracle, variant, M, N, K):
    igc.set_tuning(int(variant), 1)
    rng = np.random.default_rng(M + N + K + 2)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    got = run_u8i8(igc, A, 37, Bt, -5, outputs=("C",))
    assert np.array_equal(got["C"].astype(np.int64), oracle.gemm_u8i8_naive(A, 37, Bt, -5))


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("M,N,K", [(256, 256, 1024), (200, 300, 1000), (512, 128, 2048)])
def test_f16_random_tolerance(igc, oracle, variant, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = synth.f16_normal(rng, (M, K))
    Bt = synth.f16_normal(rng, (N, K))
    C = run_f16(igc, A, Bt)
    assert fp_rel_err(C, oracle.gemm_f16(A, Bt)) <= FP_TOL


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (70, 50, 7, 7, 7, 50),        # K not a multiple of 8: element-wise loaders
    (65, 33, 13, 15, 21, 37),     # odd leading dimensions
    (130, 260, 72, 80, 96, 261),  # aligned K, padded rows, odd ldc (scalar stores)
    (256, 256, 128, 136, 128, 260),
])
def test_f16_strides_and_unaligned(igc, oracle, M, N, K, lda, ldb, ldc):
    rng = np.random.default_rng(lda * ldb + ldc)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = run_f16(igc, A, Bt, lda, ldb, ldc)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f16(A, Bt))


def test_f16_misaligned_pointer(igc, oracle):
    import torch

    rng = np.random.default_rng(5)
    M, N, K = 40, 24, 64
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    flatA = np.concatenate([np.zeros(1, np.float16), A.ravel()])  # +2 bytes
    dA = to_dev(flatA)
    dB = to_dev(Bt)
    dC = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA.data_ptr() + 2, K, dB, K, dC, N)
    assert np.array_equal(to_host(dC).astype(np.float64), oracle.gemm_f16(A, Bt))


def test_f16_k_zero_and_empty(igc):
    import torch

    dC = to_dev(np.full((5, 7), np.nan, np.float32))
    igc.gemm_f16f32(5, 7, 0, 0, 0, 0, 0, dC, 7)
    assert np.all(to_host(dC) == 0)
    assert igc.gemm_f16f32(0, 7, 16, 0, 16, 0, 16, 0, 7) == igc.IGC_OK
    assert igc.gemm_f16f32(7, 0, 16, 0, 16, 0, 16, 0, 0) == igc.IGC_OK
    del torch


# ----------------------------------------------------------------- u8 x i8
def run_u8i8(igc, A, zA, Bt, zB, outputs=("C", "D", "Q"), scale=None, bias=None, dq=0.0,
             lda=None, ldb=None, colsum_B=None):
    import torch

    M, K = A.shape
    N = Bt.shape[0]
    lda = lda or K
    ldb = ldb or K
    dA = to_dev(strided(A, lda))
    dB = to_dev(strided(Bt, ldb))
    out = {}
    kw = dict(dq_scale=dq, colsum_B=colsum_B)
    if "C" in outputs:
        out["C"] = empty_dev((M, N), torch.int32)
        kw.update(C_i32=out["C"], ldc=N)
    if "D" in outputs:
        out["D"] = empty_dev((M, N), torch.float32)
        kw.update(D_f32=out["D"], ldd=N)
    if "Q" in outputs:
        out["Q"] = empty_dev((M, N), torch.int8)
        dS = to_dev(scale.astype(np.float32))
        dBi = to_dev(bias.astype(np.float32))
        out["_keep"] = (dS, dBi)
        kw.update(Q_i8=out["Q"], ldq=N, scale_n=dS, bias_n=dBi)
    igc.gemm_u8i8_zp(M, N, K, dA, lda, zA, dB, ldb, zB,
                     workspace=workspace_for(igc.gemm_u8i8_zp_workspace_size(M, N, K)), **kw)
    return {k: to_host(v) for k, v in out.items() if not k.startswith("_")}


def check_u8i8(oracle, got, A, zA, Bt, zB, scale=None, bias=None, sA=0.02, sB=0.01):
    C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
    if "C" in got:
        assert np.array_equal(got["C"].astype(np.int64), C)
    if "D" in got:
        assert np.array_equal(got["D"], oracle.dequant(C, sA, sB))
    if "Q" in got:
        assert np.array_equal(got["Q"], oracle.requant(C, scale, bias))


def q_params(rng, N, K):
    # a scale near 1/sigma(acc) so most requantized outputs are not saturated
    sigma = 74.0 * 74.0 * np.sqrt(K)  # std of one product of centred operands, times sqrt(K)
    scale = (rng.uniform(0.5, 2.0, N) * 40.0 / sigma).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    return scale, bias


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (300, 200, 272), (256, 256, 1024), (17, 260, 16),
                                   (520, 72, 400)])
@pytest.mark.parametrize("zA,zB", [(128, 3), (128, 0), (0, 0), (37, -5), (255, 127)])
def test_u8i8_bit_exact(igc, oracle, variant, M, N, K, zA, zB):
    rng = np.random.default_rng(M * 131 + N * 17 + K + zA * 3 + zB)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K), lo=-128, hi=127)
    scale, bias = q_params(rng, N, K)
    s = oracle.dequant_scale(0.02, 0.01)
    got = run_u8i8(igc, A, zA, Bt, zB, scale=scale, bias=bias, dq=float(s))
    check_u8i8(oracle, got, A, zA, Bt, zB, scale, bias)


@pytest.mark.parametrize("M,N,K,lda,ldb", [(50, 40, 13, 13, 13), (33, 17, 100, 103, 101),
                                           (64, 64, 48, 64, 48)])
def test_u8i8_unaligned_and_tails(igc, oracle, M, N, K, lda, ldb):
    rng = np.random.default_rng(K * lda + ldb)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K), lo=-128, hi=127)
    scale, bias = q_params(rng, N, K)
    for zA, zB in [(128, 3), (7, -100)]:
        got = run_u8i8(igc, A, zA, Bt, zB, scale=scale, bias=bias,
                       dq=float(oracle.dequant_scale(0.02, 0.01)), lda=lda, ldb=ldb)
        check_u8i8(oracle, got, A, zA, Bt, zB, scale, bias)


@pytest.mark.parametrize("outputs", [("C",), ("D",), ("Q",), ("C", "Q"), ("D", "Q")])
def test_u8i8_output_subsets(igc, oracle, outputs):
    rng = np.random.default_rng(len(outputs) * 10 + ord(outputs[0][0]))
    M, N, K = 96, 80, 256
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale, bias = q_params(rng, N, K)
    got = run_u8i8(igc, A, 128, Bt, 3, outputs=outputs, scale=scale, bias=bias,
                   dq=float(oracle.dequant_scale(0.02, 0.01)))
    assert set(got) == set(outputs)
    check_u8i8(oracle, got, A, 128, Bt, 3, scale, bias)


# Requantized int8 as the only output: whole tiles requantize in registers and
# stage packed int8, edge tiles take the staged int32 path; 520 x 520 mixes
# both for every tile size, and the zero points select each sums mask.
@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("zA,zB", [(128, 0), (128, 3), (37, 0), (37, -5)])
def test_u8i8_requant_only_whole_and_edge_tiles(igc, oracle, variant, zA, zB):
    M, N, K = 520, 520, 384
    rng = np.random.default_rng(zA * 7 + zB + 1000)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale, bias = q_params(rng, N, K)
    got = run_u8i8(igc, A, zA, Bt, zB, outputs=("Q",), scale=scale, bias=bias)
    C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
    ref = oracle.requant(C, scale, bias)
    assert np.count_nonzero((ref > -128) & (ref < 127)) > ref.size // 2  # mostly unsaturated
    assert np.array_equal(got["Q"], ref)


# Every tile whole, requantized int8 the only output: the 256-column tiles
# take the kernels compiled with the requantize-in-registers epilogue alone
# (all four zero-point sums masks), for the GEMM and the convolution.
@pytest.mark.parametrize("v,M", [(0, 512), (4, 448)])
@pytest.mark.parametrize("zA,zB", [(128, 0), (128, 3), (37, 0), (37, -5)])
def test_u8i8_requant_whole_tiles(igc, oracle, v, M, zA, zB):
    N, K = 512, 384
    rng = np.random.default_rng(zA * 11 + zB + v + 2000)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale, bias = q_params(rng, N, K)
    igc.set_tuning(v, 1)
    try:
        got = run_u8i8(igc, A, zA, Bt, zB, outputs=("Q",), scale=scale, bias=bias)
    finally:
        igc.set_tuning(-1, 1)
    ref = oracle.requant(oracle.gemm_u8i8_naive(A, zA, Bt, zB), scale, bias)
    assert np.count_nonzero((ref > -128) & (ref < 127)) > ref.size // 2
    assert np.array_equal(got["Q"], ref)


# (the uniform-tap u8 convolution runs its 256-row tile as the 224-row one)
@pytest.mark.parametrize("v,Nb,HW", [(4, 14, 4), (4, 7, 8), (0, 7, 8)])  # M = Nb*HW*HW = 224 / 448
@pytest.mark.parametrize("zA,zB", [(100, 0), (0, 3)])
def test_qconv_requant_whole_tiles(igc, oracle, v, Nb, HW, zA, zB):
    C, Kout = 128, 256
    rng = np.random.default_rng(v * 13 + zA + zB)
    x = synth.u8_uniform(rng, (Nb, HW, HW, C))
    w = synth.i8_uniform(rng, (Kout, 3, 3, C))
    scale, bias = q_params(rng, Kout, 9 * C)
    igc.set_tuning(v, 1)
    try:
        got = run_qconv(igc, x, zA, w, zB, (1, 1), (1, 1), outputs=("Q",), scale=scale, bias=bias)
    finally:
        igc.set_tuning(-1, 1)
    C32 = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * HW * HW), (1, 1), (1, 1))
    ref = oracle.requant(C32, scale, bias)
    assert np.count_nonzero((ref > -128) & (ref < 127)) > ref.size // 2
    assert np.array_equal(got["Q"], ref)


# Requantize rounding at exact halves: scale 0.5 and bias 0 put every odd
# accumulator on a tie (round half to even), and 127.5 / -128.5 at the
# saturation bounds; whole tiles (the in-register path) and edge tiles (the
# staged path).
@pytest.mark.parametrize("v,M,N", [(0, 256, 256), (4, 448, 256), (0, 260, 250)])
def test_u8i8_requant_ties_to_even(igc, oracle, v, M, N):
    K = 16
    rng = np.random.default_rng(M + N + v)
    A = synth.u8_uniform(rng, (M, K))
    Bt = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scale = np.full(N, 0.5, np.float32)
    bias = np.zeros(N, np.float32)
    igc.set_tuning(v, 1)
    try:
        got = run_u8i8(igc, A, 128, Bt, 0, outputs=("Q",), scale=scale, bias=bias)
    finally:
        igc.set_tuning(-1, 1)
    C = oracle.gemm_u8i8_naive(A, 128, Bt, 0)
    ref = oracle.requant(C, scale, bias)
    assert np.count_nonzero((C % 2 == 1) & (np.abs(C) < 256)) > C.size // 10  # ties, unsaturated
    assert np.count_nonzero(np.isin(C, (255, -257))) > 0  # 127.5 and -128.5
    assert np.array_equal(got["Q"], ref)


def test_u8i8_colsum(igc, oracle):
    import torch

    for N, K, ldb in [(512, 2304, 2304), (37, 1000, 1003), (3, 1, 1), (256, 33025, 33025)]:
        rng = np.random.default_rng(N + K)
        Bt = synth.i8_uniform(rng, (N, K))
        dB = to_dev(strided(Bt, ldb))
        out = empty_dev((N,), torch.int32)
        igc.u8i8_colsum(N, K, dB, ldb, out)
        assert np.array_equal(to_host(out).astype(np.int64), oracle.i8_colsum(Bt))


# The caller's column sums (colsum_B): used by whole requantize-only tiles
# (the kernels then form no column sums), ignored elsewhere; the results are
# the same either way.
@pytest.mark.parametrize("v,M,N,outputs", [(0, 512, 512, ("Q",)), (4, 448, 256, ("Q",)),
                                           (0, 520, 300, ("Q",)), (4, 448, 256, ("C", "Q")),
                                           (1, 512, 512, ("Q",))])
@pytest.mark.parametrize("zA,zB", [(37, 0), (200, -5), (128, 3)])
def test_u8i8_precomputed_colsum(igc, oracle, v, M, N, outputs, zA, zB):
    import torch

    K = 384
    rng = np.random.default_rng(M + N + zA + v)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale, bias = q_params(rng, N, K)
    cs = empty_dev((N,), torch.int32)
    igc.u8i8_colsum(N, K, to_dev(Bt), K, cs)
    igc.set_tuning(v, 1)
    try:
        got = run_u8i8(igc, A, zA, Bt, zB, outputs=outputs, scale=scale, bias=bias, colsum_B=cs)
    finally:
        igc.set_tuning(-1, 1)
    C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
    assert np.array_equal(got["Q"], oracle.requant(C, scale, bias))
    if "C" in outputs:
        assert np.array_equal(got["C"].astype(np.int64), C)


@pytest.mark.parametrize("v,Nb,HW", [(4, 7, 8), (-1, 4, 14)])
@pytest.mark.parametrize("zA,zB", [(100, 0), (0, 3)])
def test_qconv_precomputed_colsum(igc, oracle, v, Nb, HW, zA, zB):
    import torch

    C, Kout, R, S = 128, 256, 3, 3
    rng = np.random.default_rng(v + zA + zB + 7)
    x = synth.u8_uniform(rng, (Nb, HW, HW, C))
    w = synth.i8_uniform(rng, (Kout, R, S, C))
    scale, bias = q_params(rng, Kout, R * S * C)
    cs = empty_dev((Kout,), torch.int32)
    igc.u8i8_colsum(Kout, R * S * C, to_dev(w), R * S * C, cs)
    igc.set_tuning(v, 1)
    try:
        got = run_qconv(igc, x, zA, w, zB, (1, 1), (1, 1), outputs=("Q",), scale=scale, bias=bias, colsum_B=cs)
    finally:
        igc.set_tuning(-1, 1)
    C32 = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * HW * HW), (1, 1), (1, 1))
    assert np.array_equal(got["Q"], oracle.requant(C32, scale, bias))


@pytest.mark.parametrize("K", [33024, 33025])
def test_u8i8_extreme_values_at_overflow_bound(igc, oracle, K):
    # |C| = 255 * 255 * K reaches 2,147,450,625 at K = 33025 (just below 2^31).
    M, N = 64, 64
    A = np.full((M, K), 255, np.uint8)
    Bt = np.full((N, K), -128, np.int8)
    got = run_u8i8(igc, A, 0, Bt, 127, outputs=("C",))
    assert np.all(got["C"].astype(np.int64) == 255 * (-255) * K)
    A2 = np.zeros((M, K), np.uint8)
    got = run_u8i8(igc, A2, 255, Bt, 127, outputs=("C",))
    assert np.all(got["C"].astype(np.int64) == (-255) * (-255) * K)


def test_u8i8_deterministic(igc):
    rng = np.random.default_rng(3)
    A = synth.u8_uniform(rng, (512, 512))
    Bt = synth.i8_uniform(rng, (512, 512))
    r1 = run_u8i8(igc, A, 128, Bt, 3, outputs=("C",))
    r2 = run_u8i8(igc, A, 128, Bt, 3, outputs=("C",))
    assert np.array_equal(r1["C"], r2["C"])


# ----------------------------------------------------------------- conv
def run_conv(igc, x, w, stride, pad):
    import torch

    Nb, H, W, C = x.shape
    Kout, R, S, _ = w.shape
    P = (H + 2 * pad[0] - R) // stride[0] + 1
    Q = (W + 2 * pad[1] - S) // stride[1] + 1
    dx = to_dev(x)
    dw = to_dev(w)
    dy = empty_dev((Nb, P, Q, Kout), torch.float32)
    dims = (Nb, H, W, C, Kout, R, S, stride[0], stride[1], pad[0], pad[1])
    igc.conv2d_implicit_gemm(*dims, dx, dw, dy,
                             workspace=workspace_for(igc.conv2d_implicit_gemm_workspace_size(*dims)))
    return to_host(dy)


CONV_CASES = [
    # Nb, H, W, C, Kout, R, S, stride, pad
    (4, 3, 3, 64, 24, 3, 3, (1, 1), (0, 0)),      # 1x1 output: P*Q = Q = 1
    (1, 14, 14, 256, 512, 3, 3, (1, 1), (1, 1)),   # one image of the 256-batch workload
    (2, 9, 11, 64, 96, 3, 3, (1, 1), (1, 1)),
    (3, 8, 8, 16, 24, 1, 1, (1, 1), (0, 0)),
    (2, 13, 10, 32, 40, 5, 5, (2, 2), (2, 2)),
    (1, 7, 9, 3, 13, 3, 3, (1, 2), (1, 0)),       # C % 8 != 0, odd Kout
    (2, 6, 6, 24, 20, 3, 2, (2, 1), (0, 1)),
    (1, 30, 30, 8, 300, 3, 3, (1, 1), (1, 1)),    # M = 900 rows, N ragged
    # C % 64 == 0 and R*S <= 31: the uniform-tap loader
    (2, 13, 10, 64, 40, 5, 5, (2, 2), (2, 2)),
    (1, 12, 12, 128, 64, 3, 3, (2, 1), (0, 1)),
    (1, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0)),
    (1, 9, 9, 64, 32, 7, 7, (1, 1), (3, 3)),      # R*S = 49: the general loader
]


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_integer_valued_bit_exact(igc, oracle, variant, case):
    Nb, H, W, C, Kout, R, S, st, pd = case
    # |x|, |w| <= 4: every partial sum is an integer below 16*R*S*C < 2^24, so exact.
    rng = np.random.default_rng(sum(case[:7]))
    x = synth.f16_small_ints(rng, (Nb, H, W, C), -4, 4)
    w = synth.f16_small_ints(rng, (Kout, R, S, C), -4, 4)
    y = run_conv(igc, x, w, st, pd)
    assert np.array_equal(y.astype(np.float64), oracle.conv2d_direct(x, w, st, pd))


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_random_tolerance(igc, oracle, variant, case):
    Nb, H, W, C, Kout, R, S, st, pd = case
    rng = np.random.default_rng(3 * sum(case[:7]))
    x = synth.f16_normal(rng, (Nb, H, W, C))
    w = synth.f16_normal(rng, (Kout, R, S, C), std=0.05)
    y = run_conv(igc, x, w, st, pd)
    assert fp_rel_err(y, oracle.conv2d_direct(x, w, st, pd)) <= FP_TOL


def test_conv_impulse(igc):
    Nb, H, W, C, Kout = 1, 6, 7, 16, 8
    rng = np.random.default_rng(17)
    w = synth.f16_normal(rng, (Kout, 3, 3, C))
    x = np.zeros((Nb, H, W, C), np.float16)
    h0, w0, c0 = 0, 4, 5
    x[0, h0, w0, c0] = 1.0
    y = run_conv(igc, x, w, (1, 1), (1, 1))
    want = np.zeros_like(y)
    for r in range(3):
        for s in range(3):
            p, q = h0 + 1 - r, w0 + 1 - s
            if 0 <= p < H and 0 <= q < W:
                want[0, p, q, :] = w[:, r, s, c0].astype(np.float32)
    assert np.array_equal(y, want)


# ----------------------------------------------------------------- stream-K
# More 256x256 tiles than one round of compute units, not a whole number of
# rounds: the last tiles are shared between workgroups and summed through the
# workspace.  The shared tiles are the last ones in the tile order, i.e. the
# last tile rows here.
def _sk_run(igc, A, Bt, on):
    # (stream-K runs on the 256x256 tiles; at these shapes the default choice
    # would be 224x256 tiles)
    igc.set_tuning(0, 2 if on else 0)
    if on:
        M, K = A.shape
        assert igc.gemm_f16f32_workspace_size(M, Bt.shape[0], K) > 0
    return run_f16(igc, A, Bt)


@pytest.mark.parametrize("M,N,K", [
    (6144, 4096, 512),   # 384 tiles: 128 shared, two workgroups each
    (4352, 4096, 1024),  # 272 tiles: 16 shared, four workgroups each
    (4352, 4096, 648),   # partial K tile first, 11 K tiles
])
def test_streamk_integer_valued_exact(igc, oracle, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = _sk_run(igc, A, Bt, True)
    C0 = _sk_run(igc, A, Bt, False)
    assert np.array_equal(C, C0)
    rows = np.array(sorted({4095, 4096, 4097, M - 1} | set(rng.integers(4096, M, 24).tolist())
                           | set(rng.integers(0, 4096, 8).tolist())))
    assert np.array_equal(C[rows].astype(np.float64), oracle.gemm_f16(A[rows], Bt))


def test_streamk_random_tolerance_and_deterministic(igc, oracle):
    M, N, K = 6144, 4096, 1024
    rng = np.random.default_rng(17)
    A = synth.f16_normal(rng, (M, K))
    Bt = synth.f16_normal(rng, (N, K))
    C1 = _sk_run(igc, A, Bt, True)
    C2 = _sk_run(igc, A, Bt, True)
    assert np.array_equal(C1, C2)
    rows = np.array(sorted({4096, M - 1} | set(rng.integers(4096, M, 16).tolist())))
    assert fp_rel_err(C1[rows], oracle.gemm_f16(A[rows], Bt)) <= FP_TOL


def test_streamk_workspace_contract(igc, oracle):
    """The split needs the caller's workspace: a workspace smaller than the
    query's size is rejected before anything is launched, no workspace runs
    the whole-tile path (same results), and one zero-filled workspace serves
    consecutive calls (the kernel leaves its counters at zero)."""
    import torch

    M, N, K = 4352, 4096, 1024
    rng = np.random.default_rng(23)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    igc.set_tuning(0, 2)
    need = igc.gemm_f16f32_workspace_size(M, N, K)
    assert need > 0
    dA, dB = to_dev(A), to_dev(Bt)
    dC = empty_dev((M, N), torch.float32)
    small = workspace_for(need - 16)
    st = igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N, workspace=small, check=False)
    assert st == igc.IGC_EINVAL and "workspace" in igc.last_error()
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N)  # no workspace: whole tiles
    C0 = to_host(dC).copy()
    ws = workspace_for(need)
    for _ in range(3):
        dC.fill_(float("nan"))
        igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N, workspace=ws)
        assert np.array_equal(to_host(dC), C0)
    rows = np.array(sorted({4095, 4096, M - 1} | set(rng.integers(4096, M, 12).tolist())))
    assert np.array_equal(C0[rows].astype(np.float64), oracle.gemm_f16(A[rows], Bt))


# ----------------------------------------------------------------- quantized conv
def run_qconv(igc, x, zA, w, zB, stride, pad, outputs=("C",), scale=None, bias=None, dq=0.0, colsum_B=None):
    import torch

    Nb, H, W, C = x.shape
    Kout, R, S, _ = w.shape
    P = (H + 2 * pad[0] - R) // stride[0] + 1
    Q = (W + 2 * pad[1] - S) // stride[1] + 1
    M = Nb * P * Q
    dx, dw = to_dev(x), to_dev(w)
    out, kw = {}, dict(dq_scale=dq, colsum_B=colsum_B)
    if "C" in outputs:
        out["C"] = empty_dev((M, Kout), torch.int32)
        kw.update(C_i32=out["C"], ldc=Kout)
    if "D" in outputs:
        out["D"] = empty_dev((M, Kout), torch.float32)
        kw.update(D_f32=out["D"], ldd=Kout)
    if "Q" in outputs:
        out["Q"] = empty_dev((M, Kout), torch.int8)
        dS, dBi = to_dev(scale.astype(np.float32)), to_dev(bias.astype(np.float32))
        out["_keep"] = (dS, dBi)
        kw.update(Q_i8=out["Q"], ldq=Kout, scale_n=dS, bias_n=dBi)
    dims = (Nb, H, W, C, Kout, R, S, stride[0], stride[1], pad[0], pad[1])
    igc.conv2d_u8i8_zp(*dims, dx, zA, dw, zB, workspace=workspace_for(igc.conv2d_u8i8_zp_workspace_size(*dims)),
                       **kw)
    return {k: to_host(v) for k, v in out.items() if not k.startswith("_")}


QCONV_CASES = [
    # Nb, H, W, C, Kout, R, S, stride, pad, zA, zB
    (4, 3, 3, 128, 24, 3, 3, (1, 1), (0, 0), 61, 2),  # 1x1 output: P*Q = Q = 1
    (1, 14, 14, 256, 512, 3, 3, (1, 1), (1, 1), 100, 0),    # one image of the 256-batch shape
    (2, 9, 11, 128, 96, 3, 3, (1, 1), (1, 1), 128, 3),      # uniform taps, zA' = 0
    (2, 13, 10, 128, 40, 5, 5, (2, 2), (2, 2), 37, -5),
    (1, 12, 12, 256, 64, 3, 3, (2, 1), (0, 1), 255, 127),
    (3, 8, 8, 128, 24, 1, 1, (1, 1), (0, 0), 0, -128),
    (2, 9, 11, 64, 96, 3, 3, (1, 1), (1, 1), 90, 2),        # C % 128 != 0: element-wise
    (1, 7, 9, 3, 13, 3, 3, (1, 2), (1, 0), 200, -1),
    (1, 9, 9, 128, 32, 7, 7, (1, 1), (3, 3), 17, 4),        # R*S = 49: element-wise
    (2, 9, 11, 128, 96, 3, 3, (1, 1), (1, 1), 0, 5),        # zA = 0: padding needs no rewrite
    (1, 7, 9, 16, 13, 3, 3, (1, 2), (1, 1), 0, 0),          # zA = 0, element-wise
]


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", QCONV_CASES)
def test_qconv_int32_bit_exact(igc, oracle, variant, case):
    Nb, H, W, C, Kout, R, S, st, pd, zA, zB = case
    rng = np.random.default_rng(sum(case[:7]) + zA)
    x = synth.u8_uniform(rng, (Nb, H, W, C))
    w = synth.i8_uniform(rng, (Kout, R, S, C))
    got = run_qconv(igc, x, zA, w, zB, st, pd)
    P = (H + 2 * pd[0] - R) // st[0] + 1
    Q = (W + 2 * pd[1] - S) // st[1] + 1
    ref = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * P * Q), st, pd)
    assert np.array_equal(got["C"].astype(np.int64), ref)


@pytest.mark.parametrize("case", [QCONV_CASES[0], QCONV_CASES[1], QCONV_CASES[3], QCONV_CASES[6]])
def test_qconv_dequant_and_requant_bit_exact(igc, oracle, case):
    Nb, H, W, C, Kout, R, S, st, pd, zA, zB = case
    rng = np.random.default_rng(3 * sum(case[:7]) + zA)
    x = synth.u8_uniform(rng, (Nb, H, W, C))
    w = synth.i8_uniform(rng, (Kout, R, S, C))
    # scales near 1/sigma(C), so most requantized outputs are not saturated
    scale = (rng.uniform(0.5, 2.0, Kout) * 40.0 / (74.0 * 74.0 * np.sqrt(R * S * C))).astype(np.float32)
    bias = rng.standard_normal(Kout).astype(np.float32)
    got = run_qconv(igc, x, zA, w, zB, st, pd, outputs=("C", "D", "Q"), scale=scale, bias=bias,
                    dq=float(oracle.dequant_scale(0.02, 0.01)))
    P = (H + 2 * pd[0] - R) // st[0] + 1
    Q = (W + 2 * pd[1] - S) // st[1] + 1
    Cref = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * P * Q), st, pd)
    assert np.array_equal(got["C"].astype(np.int64), Cref)
    assert np.array_equal(got["D"], oracle.dequant(Cref, 0.02, 0.01))
    assert np.array_equal(got["Q"], oracle.requant(Cref, scale, bias))


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", [QCONV_CASES[1], QCONV_CASES[3], QCONV_CASES[5]])
def test_qconv_requant_only(igc, oracle, variant, case):
    Nb, H, W, C, Kout, R, S, st, pd, zA, zB = case
    rng = np.random.default_rng(7 * sum(case[:7]) + zA)
    x = synth.u8_uniform(rng, (Nb, H, W, C))
    w = synth.i8_uniform(rng, (Kout, R, S, C))
    scale = (rng.uniform(0.5, 2.0, Kout) * 40.0 / (74.0 * 74.0 * np.sqrt(R * S * C))).astype(np.float32)
    bias = rng.standard_normal(Kout).astype(np.float32)
    got = run_qconv(igc, x, zA, w, zB, st, pd, outputs=("Q",), scale=scale, bias=bias)
    P = (H + 2 * pd[0] - R) // st[0] + 1
    Q = (W + 2 * pd[1] - S) // st[1] + 1
    Cref = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * P * Q), st, pd)
    assert np.array_equal(got["Q"], oracle.requant(Cref, scale, bias))


# ----------------------------------------------------------------- blocked NHWCnc conv
def run_conv_nhwcnc(igc, xb, wb, stride, pad, x_offset=0):
    """x_offset: bytes by which x is shifted from a 16-byte boundary (the
    element-wise loader)."""
    import torch

    NB, H, W, CB = xb.shape[:4]
    R, S, _, OB = wb.shape[:4]
    dims = (16 * NB, H, W, 16 * CB, 16 * OB, R, S, stride[0], stride[1], pad[0], pad[1])
    P = (H + 2 * pad[0] - R) // stride[0] + 1
    Q = (W + 2 * pad[1] - S) // stride[1] + 1
    if x_offset:
        raw = empty_dev((xb.size + 8,), torch.float16)
        raw[x_offset // 2: x_offset // 2 + xb.size].copy_(to_dev(xb.reshape(-1)))
        dx = raw.data_ptr() + x_offset
        keep = raw
    else:
        keep = dx = to_dev(xb)
    dy = to_dev(np.full((NB, P, Q, OB, 16, 16), np.nan, np.float32))
    ws = workspace_for(igc.conv2d_implicit_gemm_nhwcnc_workspace_size(*dims))
    igc.conv2d_implicit_gemm_nhwcnc(*dims, dx, to_dev(wb), dy, workspace=ws)
    del keep
    return to_host(dy)


NHWCNC_CASES = [
    # NB, H, W, CB, OB, R, S, stride, pad
    (1, 14, 14, 16, 32, 3, 3, (1, 1), (1, 1)),  # 16 images of the 256x14x14 conv: uniform-tap path
    (1, 9, 11, 4, 6, 3, 3, (1, 1), (1, 1)),     # C = 64
    (2, 6, 7, 2, 3, 3, 3, (2, 1), (1, 0)),      # C = 32: 8-channel chunks across taps
    (1, 8, 8, 1, 2, 1, 1, (1, 1), (0, 0)),      # C = 16, 1x1
    (1, 13, 10, 3, 2, 5, 5, (2, 2), (2, 2)),    # C = 48
]


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", NHWCNC_CASES)
def test_conv_nhwcnc_integer_valued_bit_exact(igc, oracle, variant, case):
    NB, H, W, CB, OB, R, S, stride, pad = case
    rng = np.random.default_rng(NB * 1000 + H * 100 + W * 10 + CB)
    xb = synth.f16_small_ints(rng, (NB, H, W, CB, 16, 16), -4, 4)
    wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16), -4, 4)
    y = run_conv_nhwcnc(igc, xb, wb, stride, pad)
    assert np.array_equal(y.astype(np.float64), oracle.conv2d_nhwcnc_direct(xb, wb, stride, pad))


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("case", [NHWCNC_CASES[0], NHWCNC_CASES[2], NHWCNC_CASES[4]])
def test_conv_nhwcnc_random_tolerance(igc, oracle, variant, case):
    NB, H, W, CB, OB, R, S, stride, pad = case
    rng = np.random.default_rng(7 + H + CB)
    xb = synth.f16_normal(rng, (NB, H, W, CB, 16, 16))
    wb = synth.f16_normal(rng, (R, S, CB, OB, 16, 16), std=0.05)
    y = run_conv_nhwcnc(igc, xb, wb, stride, pad)
    assert fp_rel_err(y, oracle.conv2d_nhwcnc_direct(xb, wb, stride, pad)) <= FP_TOL


@pytest.mark.parametrize("case", [NHWCNC_CASES[1], NHWCNC_CASES[2]])
def test_conv_nhwcnc_misaligned_input(igc, oracle, case):
    """x two bytes past a 16-byte boundary: the element-wise loader."""
    NB, H, W, CB, OB, R, S, stride, pad = case
    rng = np.random.default_rng(11 + CB)
    xb = synth.f16_small_ints(rng, (NB, H, W, CB, 16, 16), -4, 4)
    wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16), -4, 4)
    y = run_conv_nhwcnc(igc, xb, wb, stride, pad, x_offset=2)
    assert np.array_equal(y.astype(np.float64), oracle.conv2d_nhwcnc_direct(xb, wb, stride, pad))


def test_conv_nhwcnc_split_tiles_across_xcds(igc, oracle):
    """Regression: 64x64 tiles with the partial round split (320 tiles over
    256 compute units, each split tile shared by two workgroups on different
    XCDs).  While the arrival count was a relaxed atomic, the last contributor
    could read the other's partial slot still zero-filled: hundreds of wrong
    outputs per call, a different set each call.  Several calls, bit-exact."""
    NB, H, W, CB, OB, R, S, stride, pad = 2, 16, 16, 8, 8, 3, 1, (1, 1), (1, 2)
    rng = np.random.default_rng(334)
    xb = synth.f16_small_ints(rng, (NB, H, W, CB, 16, 16), -4, 4)
    wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16), -4, 4)
    ref = oracle.conv2d_nhwcnc_direct(xb, wb, stride, pad)
    igc.set_tuning(2, 2)  # 64x64 tiles, split wherever tiles leave compute units idle
    try:
        for rep in range(4):
            y = run_conv_nhwcnc(igc, xb, wb, stride, pad).astype(np.float64)
            assert np.array_equal(y, ref), (rep, int(np.sum(y != ref)))
    finally:
        igc.set_tuning(-1, 1)


def test_conv_nhwcnc_matches_the_nhwc_path(igc):
    """The same logical convolution through both entry points gives the same
    fp32 values (same tiles, same K order)."""
    import torch

    rng = np.random.default_rng(5)
    NB, H, W, CB, OB = 1, 9, 11, 4, 6
    xb = synth.f16_normal(rng, (NB, H, W, CB, 16, 16))
    wb = synth.f16_normal(rng, (3, 3, CB, OB, 16, 16), std=0.05)
    yb = run_conv_nhwcnc(igc, xb, wb, (1, 1), (1, 1))
    x = np.ascontiguousarray(xb.transpose(0, 4, 1, 2, 3, 5).reshape(16 * NB, H, W, 16 * CB))
    w = np.ascontiguousarray(wb.transpose(3, 5, 0, 1, 2, 4).reshape(16 * OB, 3, 3, 16 * CB))
    y = run_conv(igc, x, w, (1, 1), (1, 1))
    assert np.array_equal(yb.transpose(0, 4, 1, 2, 3, 5).reshape(y.shape), y)


# ----------------------------------------------------------------- split tiles on small grids
# Grids smaller than one round of compute units with long K loops: every
# tile's K-tile iterations are shared between workgroups (forced here; the
# default splits where the idle part of the round is large).  The integer
# kernels publish each segment's zero-point-corrected share and add
# K*zA'*zB once, so the results stay exact.
@pytest.mark.parametrize("v", ["1", "2"])
@pytest.mark.parametrize("M,N,K", [(200, 136, 2064), (64, 64, 4096), (300, 260, 1040), (17, 260, 3008)])
@pytest.mark.parametrize("zA,zB", [(128, 3), (0, 0), (37, -5), (255, 127), (128, 0)])
def test_u8i8_split_tiles_bit_exact(igc, oracle, v, M, N, K, zA, zB):
    igc.set_tuning(int(v), 2)
    assert igc.gemm_u8i8_zp_workspace_size(M, N, K) > 0
    rng = np.random.default_rng(M + 3 * N + 7 * K + zA - zB)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K), lo=-128, hi=127)
    scale, bias = q_params(rng, N, K)
    s = oracle.dequant_scale(0.02, 0.01)
    got = run_u8i8(igc, A, zA, Bt, zB, scale=scale, bias=bias, dq=float(s))
    check_u8i8(oracle, got, A, zA, Bt, zB, scale, bias)


@pytest.mark.parametrize("v", ["1", "2"])
def test_u8i8_split_tiles_requant_only_and_deterministic(igc, oracle, v):
    igc.set_tuning(int(v), 2)
    M, N, K = 256, 192, 4096
    rng = np.random.default_rng(31)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale, bias = q_params(rng, N, K)
    g1 = run_u8i8(igc, A, 100, Bt, -7, outputs=("Q",), scale=scale, bias=bias)
    g2 = run_u8i8(igc, A, 100, Bt, -7, outputs=("Q",), scale=scale, bias=bias)
    assert np.array_equal(g1["Q"], g2["Q"])
    check_u8i8(oracle, g1, A, 100, Bt, -7, scale, bias)


@pytest.mark.parametrize("v", ["1", "2"])
@pytest.mark.parametrize("case", [QCONV_CASES[2], QCONV_CASES[3], QCONV_CASES[4], QCONV_CASES[9]])
def test_qconv_split_tiles_bit_exact(igc, oracle, v, case):
    Nb, H, W, C, Kout, R, S, stride, pad, zA, zB = case
    igc.set_tuning(int(v), 2)
    rng = np.random.default_rng(Nb + H + C + zA)
    x = synth.u8_uniform(rng, (Nb, H, W, C))
    w = synth.i8_uniform(rng, (Kout, R, S, C), lo=-128, hi=127)
    scale, bias = q_params(rng, Kout, R * S * C)
    got = run_qconv(igc, x, zA, w, zB, stride, pad, outputs=("C", "Q"), scale=scale, bias=bias)
    P = (H + 2 * pad[0] - R) // stride[0] + 1
    Q = (W + 2 * pad[1] - S) // stride[1] + 1
    ref = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * P * Q), stride, pad)
    assert np.array_equal(got["C"].astype(np.int64), ref)
    assert np.array_equal(got["Q"], oracle.requant(ref, scale, bias))


@pytest.mark.parametrize("v", ["1", "2"])
@pytest.mark.parametrize("M,N,K", [(512, 128, 2048), (70, 33, 4104), (256, 256, 1024)])
def test_f16_split_tiles_integer_valued_exact(igc, oracle, v, M, N, K):
    igc.set_tuning(int(v), 2)
    rng = np.random.default_rng(M + N + K + 9)
    A = synth.f16_small_ints(rng, (M, K))
    Bt = synth.f16_small_ints(rng, (N, K))
    C = run_f16(igc, A, Bt)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f16(A, Bt))


@pytest.mark.parametrize("v", ["1", "2"])
@pytest.mark.parametrize("case", [CONV_CASES[1], CONV_CASES[3]])
def test_conv_split_tiles_integer_valued_exact(igc, oracle, v, case):
    Nb, H, W, C, Kout, R, S, stride, pad = case
    igc.set_tuning(int(v), 2)
    rng = np.random.default_rng(Nb * 7 + H + C)
    x = synth.f16_small_ints(rng, (Nb, H, W, C), -4, 4)
    w = synth.f16_small_ints(rng, (Kout, R, S, C), -4, 4)
    y = run_conv(igc, x, w, stride, pad)
    assert np.array_equal(y.astype(np.float64), oracle.conv2d_direct(x, w, stride, pad))
