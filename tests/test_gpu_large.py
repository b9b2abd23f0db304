"""Operands at the input-size limits of the loaders (GPU).

The uniform-tap and 16-byte im2col loaders address x with 32-bit byte
offsets from one buffer base, so the host takes them only while those
offsets stay below 2^31 bytes: the uniform-tap loader needs x plus the
padding's offset ((pad_h * W + pad_w) * C elements) below 2^31 bytes, the
16-byte loader x itself below 2^31 bytes; beyond that the element-wise
loader (64-bit element index) runs.  Each case sits just past one of these
switch points.  Operands are small integers in fp16, so every output is exact
in fp32 and compared bit for bit with the oracle at sampled pixels: the
first and last rows of the image, its corners and random pixels (the last
rows read the highest offsets of x).  The GEMMs take an A of 2.25 GB,
compared on its first, last and random rows, and two outputs have more
than 2^31 elements."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import empty_dev, to_dev, workspace_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    m.set_tuning(-1, 1)
    yield m


CASES = [
    # H = W, C, Kout, R = S, pad; x bytes = H*W*C*2
    # 4095^2 x 64 fp16 plus the padding's offset (4095 + 1)*64*2 is
    # 2,146,959,488 bytes < 2^31: the uniform-tap loader at its largest input
    pytest.param(4095, 64, 16, 3, 1, id="uniform_taps_largest_input"),
    # 4100^2 x 64 fp16 = 2,151,680,000 bytes >= 2^31: element-wise loader
    pytest.param(4100, 64, 16, 3, 1, id="x_past_2GiB_elementwise"),
    # 4095^2 x 64 fp16 = 2,146,435,200 bytes < 2^31, but with the padding's
    # offset (2*4095 + 2)*64*2 = 1,048,576 bytes it passes 2^31: the 16-byte
    # loader instead of the uniform-tap one
    pytest.param(4095, 64, 16, 5, 2, id="x_plus_padding_past_2GiB_16byte"),
]


@pytest.mark.parametrize("HW, C, Kout, RS, pad", CASES)
def test_conv_f16_at_loader_limits(igc, oracle, HW, C, Kout, RS, pad):
    import torch

    rng = np.random.default_rng(HW)
    print(f"conv f16 1x{HW}x{HW}x{C} * {Kout}x{RS}x{RS}x{C} pad {pad}", flush=True)
    x = synth.i8_uniform(rng, (1, HW, HW, C), -8, 8).astype(np.float16)
    w = synth.i8_uniform(rng, (Kout, RS, RS, C), -8, 8).astype(np.float16)
    P = Q = HW + 2 * pad - RS + 1
    M = P * Q
    dims = (1, HW, HW, C, Kout, RS, RS, 1, 1, pad, pad)
    dx, dw = to_dev(x), to_dev(w)
    dy = empty_dev((M, Kout), torch.float32)
    igc.conv2d_implicit_gemm(*dims, dx, dw, dy,
                             workspace=workspace_for(igc.conv2d_implicit_gemm_workspace_size(*dims)))
    torch.cuda.synchronize()
    pix = {0, Q - 1, (P - 1) * Q, M - 1, M // 2}
    pix |= set(range(0, 40)) | set(range(M - 40, M))
    pix |= set(rng.integers(0, M, 200).tolist())
    pix = np.array(sorted(pix), dtype=np.int64)
    got = dy[torch.from_numpy(pix).cuda()].cpu().numpy().astype(np.float64)
    del dx, dy
    ref = oracle.conv2d_direct_at(x, w, pix, (1, 1), (pad, pad))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:10]


QCASES = [
    # H = W, C, Kout, R = S, pad; x bytes = H*W*C
    # 4095^2 x 128 u8 plus (4095 + 1)*128 is 2,146,959,488 bytes < 2^31: the
    # uniform-tap loader at its largest input
    pytest.param(4095, 128, 16, 3, 1, id="uniform_taps_largest_input"),
    # with (2*4095 + 2)*128 it is 2,147,483,776 >= 2^31: the element-wise loader
    pytest.param(4095, 128, 16, 5, 2, id="x_plus_padding_past_2GiB_elementwise"),
]


@pytest.mark.parametrize("HW, C, Kout, RS, pad", QCASES)
def test_conv_u8i8_at_loader_limits(igc, oracle, HW, C, Kout, RS, pad):
    """The quantized convolution at the same limits, int32 output, with zero
    points on both sides (the padding holds zA)."""
    import torch

    rng = np.random.default_rng(HW + RS)
    zA, zB = 100, -3
    print(f"conv u8i8 1x{HW}x{HW}x{C} * {Kout}x{RS}x{RS}x{C} pad {pad}", flush=True)
    x = synth.u8_uniform(rng, (1, HW, HW, C))
    w = synth.i8_uniform(rng, (Kout, RS, RS, C))
    P = Q = HW + 2 * pad - RS + 1
    M = P * Q
    dims = (1, HW, HW, C, Kout, RS, RS, 1, 1, pad, pad)
    dx, dw = to_dev(x), to_dev(w)
    dC = empty_dev((M, Kout), torch.int32)
    igc.conv2d_u8i8_zp(*dims, dx, zA, dw, zB, C_i32=dC, ldc=Kout,
                       workspace=workspace_for(igc.conv2d_u8i8_zp_workspace_size(*dims)))
    torch.cuda.synchronize()
    pix = {0, Q - 1, (P - 1) * Q, M - 1, M // 2}
    pix |= set(range(0, 40)) | set(range(M - 40, M))
    pix |= set(rng.integers(0, M, 200).tolist())
    pix = np.array(sorted(pix), dtype=np.int64)
    got = dC[torch.from_numpy(pix).cuda()].cpu().numpy().astype(np.int64)
    del dx, dC
    ref = oracle.conv2d_u8i8_direct_at(x, zA, w, zB, pix, (1, 1), (pad, pad))
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:10]


def _rows_sample(rng, M):
    rows = set(range(0, 40)) | set(range(M - 40, M)) | {M // 2}
    rows |= set(rng.integers(0, M, 100).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def test_gemm_f16_operand_past_2GiB(igc, oracle):
    """fp16 GEMM whose A (1,100,000 x 1024) spans 2.25 GB: each tile's loads
    are addressed from its own first row (64-bit base), so the whole-matrix
    size never enters a 32-bit offset.  Integer-valued operands: exact."""
    import torch

    M, N, K = 1_100_000, 64, 1024
    rng = np.random.default_rng(7)
    print(f"gemm f16 M={M} N={N} K={K}", flush=True)
    A = synth.i8_uniform(rng, (M, K), -8, 8).astype(np.float16)
    Bt = synth.i8_uniform(rng, (N, K), -8, 8).astype(np.float16)
    dA, dB = to_dev(A), to_dev(Bt)
    dC = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N, workspace=workspace_for(igc.gemm_f16f32_workspace_size(M, N, K)))
    torch.cuda.synchronize()
    rows = _rows_sample(rng, M)
    got = dC[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, oracle.gemm_f16(A[rows], Bt))


def test_gemm_u8i8_operand_past_2GiB(igc, oracle):
    """u8 x i8 GEMM whose A (2,200,000 x 1024) spans 2.25 GB, int32 and
    requantized int8 outputs, zero points on both sides."""
    import torch

    M, N, K = 2_200_000, 64, 1024
    zA, zB = 77, 5
    rng = np.random.default_rng(8)
    print(f"gemm u8i8 M={M} N={N} K={K}", flush=True)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale = rng.uniform(0.0005, 0.002, size=N).astype(np.float32)
    bias = (rng.standard_normal(N) * 4).astype(np.float32)
    dA, dB = to_dev(A), to_dev(Bt)
    dS, dBi = to_dev(scale), to_dev(bias)
    dC = empty_dev((M, N), torch.int32)
    dQ = empty_dev((M, N), torch.int8)
    igc.gemm_u8i8_zp(M, N, K, dA, K, zA, dB, K, zB, C_i32=dC, ldc=N, Q_i8=dQ, ldq=N, scale_n=dS, bias_n=dBi,
                     workspace=workspace_for(igc.gemm_u8i8_zp_workspace_size(M, N, K)))
    torch.cuda.synchronize()
    rows = _rows_sample(rng, M)
    idx = torch.from_numpy(rows).cuda()
    C = dC[idx].cpu().numpy().astype(np.int64)
    Q = dQ[idx].cpu().numpy()
    ref = oracle.gemm_u8i8_naive(A[rows], zA, Bt, zB)
    assert np.array_equal(C, ref)
    assert np.array_equal(Q, oracle.requant(ref, scale, bias))


def test_gemm_f16_output_past_2G_elements(igc, oracle):
    """fp32 C of 65,536 x 32,800 = 2,149,580,800 elements (8.6 GB), ragged in
    N: every output address is a 64-bit row offset.  Compared on sampled rows
    (the last ones hold the highest addresses)."""
    import torch

    M, N, K = 65_536, 32_800, 64
    rng = np.random.default_rng(9)
    print(f"gemm f16 M={M} N={N} K={K}", flush=True)
    A = synth.i8_uniform(rng, (M, K), -8, 8).astype(np.float16)
    Bt = synth.i8_uniform(rng, (N, K), -8, 8).astype(np.float16)
    dA, dB = to_dev(A), to_dev(Bt)
    dC = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N, workspace=workspace_for(igc.gemm_f16f32_workspace_size(M, N, K)))
    torch.cuda.synchronize()
    rows = _rows_sample(rng, M)
    got = dC[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    del dC
    assert np.array_equal(got, oracle.gemm_f16(A[rows], Bt))


def test_gemm_u8i8_requant_output_past_2G_elements(igc, oracle):
    """Requantized int8 Q of 65,536 x 32,800 elements (2.15 GB), ragged in N."""
    import torch

    M, N, K = 65_536, 32_800, 256
    zA, zB = 128, 0
    rng = np.random.default_rng(10)
    print(f"gemm u8i8 requant M={M} N={N} K={K}", flush=True)
    A = synth.u8_uniform(rng, (M, K))
    Bt = synth.i8_uniform(rng, (N, K))
    scale = rng.uniform(0.001, 0.01, size=N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    dA, dB = to_dev(A), to_dev(Bt)
    dS, dBi = to_dev(scale), to_dev(bias)
    dQ = empty_dev((M, N), torch.int8)
    igc.gemm_u8i8_zp(M, N, K, dA, K, zA, dB, K, zB, Q_i8=dQ, ldq=N, scale_n=dS, bias_n=dBi,
                     workspace=workspace_for(igc.gemm_u8i8_zp_workspace_size(M, N, K)))
    torch.cuda.synchronize()
    rows = _rows_sample(rng, M)
    Q = dQ[torch.from_numpy(rows).cuda()].cpu().numpy()
    del dQ
    assert np.array_equal(Q, oracle.requant(oracle.gemm_u8i8_naive(A[rows], zA, Bt, zB), scale, bias))
