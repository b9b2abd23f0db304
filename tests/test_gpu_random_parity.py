"""Randomized parity (GPU): seeded random shapes, zero points, outputs, tile
variants, split modes and leading dimensions for the five entry points,
every output compared with the oracle bit for bit (integer-valued fp16
operands, whose sums are exact in fp32; u8 x i8 int32, dequantized fp32 and
requantized int8 outputs).  The fixed-case
tests pin chosen corners; these cover their combinations."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from test_gpu_parity import run_conv, run_conv_nhwcnc, run_f16, run_qconv, run_u8i8

pytestmark = pytest.mark.gpu

KINDS = ("gemm_u8i8", "conv_u8i8", "gemm_f16", "conv_f16", "conv_nhwcnc")
LD_PAD = (0, 0, 0, 8, 16, 3, 64)  # leading dimension = extent + one of these


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    m.set_tuning(-1, 1)
    yield m
    m.set_tuning(-1, 1)


def _conv_shape(rng, channels):
    while True:
        Nb, H, W = int(rng.integers(1, 4)), int(rng.integers(1, 17)), int(rng.integers(1, 17))
        C = int(rng.choice(channels))
        Kout = int(rng.integers(1, 300))
        R, S = int(rng.choice([1, 3, 3, 5])), int(rng.choice([1, 3, 3, 5]))
        st = (int(rng.choice([1, 1, 2])), int(rng.choice([1, 1, 2])))
        pd = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        if H + 2 * pd[0] >= R and W + 2 * pd[1] >= S:
            return Nb, H, W, C, Kout, R, S, st, pd


def _gemm_shape(rng, m_max, n_max, big):
    if rng.random() < 0.4:
        return int(rng.choice(big[0])), int(rng.choice(big[1])), int(rng.choice(big[2]))
    return int(rng.integers(1, m_max)), int(rng.integers(1, n_max)), int(rng.integers(1, 1300))


def _one_case(igc, oracle, rng):
    import torch

    kind = KINDS[int(rng.integers(0, len(KINDS)))]
    v = int(rng.choice([-1, -1, -1, 0, 1, 2, 3, 4]))  # by shape, or a forced tile
    sk = int(rng.choice([1, 1, 0, 2]))  # split where it pays, never, always
    igc.set_tuning(v, sk)
    try:
        if kind == "gemm_f16":
            M, N, K = _gemm_shape(rng, 700, 600, ([256, 512, 1024], [256, 512], [64, 512, 1024]))
            A, Bt = synth.f16_small_ints(rng, (M, K)), synth.f16_small_ints(rng, (N, K))
            lda, ldb, ldc = (int(x + rng.choice(LD_PAD)) for x in (K, K, N))
            desc = f"{kind} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} variant={v} split={sk}"
            print(desc, flush=True)
            got = run_f16(igc, A, Bt, lda=lda, ldb=ldb, ldc=ldc)
            assert np.array_equal(got.astype(np.float64), oracle.gemm_f16(A, Bt)), desc
            return kind
        if kind == "conv_f16":
            Nb, H, W, C, Kout, R, S, st, pd = _conv_shape(rng, [64, 128, 256, int(rng.integers(1, 100))])
            x, w = synth.f16_small_ints(rng, (Nb, H, W, C)), synth.f16_small_ints(rng, (Kout, R, S, C))
            desc = f"{kind} {Nb}x{H}x{W}x{C} * {Kout}x{R}x{S} stride={st} pad={pd} variant={v} split={sk}"
            print(desc, flush=True)
            assert np.array_equal(run_conv(igc, x, w, st, pd).astype(np.float64),
                                  oracle.conv2d_direct(x, w, st, pd)), desc
            return kind
        if kind == "conv_nhwcnc":
            # blocked layout: 16 images x 16 channels innermost (the shape's
            # batch, channels and output channels are block counts)
            _, H, W, _, _, R, S, st, pd = _conv_shape(rng, [16])
            NB, CB, OB = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3, 4, 8])), int(rng.integers(1, 9))
            xb = synth.f16_small_ints(rng, (NB, H, W, CB, 16, 16), -4, 4)
            wb = synth.f16_small_ints(rng, (R, S, CB, OB, 16, 16), -4, 4)
            desc = (f"{kind} {16 * NB}x{H}x{W}x{16 * CB} * {16 * OB}x{R}x{S} stride={st} pad={pd} "
                    f"variant={v} split={sk}")
            print(desc, flush=True)
            assert np.array_equal(run_conv_nhwcnc(igc, xb, wb, st, pd).astype(np.float64),
                                  oracle.conv2d_nhwcnc_direct(xb, wb, st, pd)), desc
            return kind
        outs = [("Q",), ("C",), ("C", "Q"), ("Q",), ("D",), ("C", "D", "Q")][int(rng.integers(0, 6))]
        zA = int(rng.choice([0, 128, int(rng.integers(0, 256))]))
        zB = int(rng.choice([0, int(rng.integers(-128, 128))]))
        sA, sB = float(rng.uniform(0.001, 0.1)), float(rng.uniform(0.001, 0.1))
        use_cs = "C" not in outs and rng.random() < 0.5
        if kind == "gemm_u8i8":
            M, N, K = _gemm_shape(rng, 600, 520, ([224, 256, 448, 512], [256, 512], [128, 256, 384, 1024]))
            A, Bt = synth.u8_uniform(rng, (M, K)), synth.i8_uniform(rng, (N, K))
            scale = rng.uniform(0.001, 0.05, size=N).astype(np.float32)
            bias = (rng.standard_normal(N) * 4).astype(np.float32)
            cs = torch.from_numpy(oracle.i8_colsum(Bt).astype(np.int32)).cuda() if use_cs else None
            lda, ldb = (int(K + rng.choice(LD_PAD)) for _ in range(2))
            desc = (f"{kind} M={M} N={N} K={K} lda={lda} ldb={ldb} zA={zA} zB={zB} outputs={outs} "
                    f"colsum={use_cs} variant={v} split={sk}")
            print(desc, flush=True)
            got = run_u8i8(igc, A, zA, Bt, zB, outputs=outs, scale=scale, bias=bias, colsum_B=cs,
                           dq=float(oracle.dequant_scale(sA, sB)), lda=lda, ldb=ldb)
            C32 = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
        else:
            Nb, H, W, C, Kout, R, S, st, pd = _conv_shape(rng, [128, 256, 128, int(rng.integers(1, 200))])
            x, w = synth.u8_uniform(rng, (Nb, H, W, C)), synth.i8_uniform(rng, (Kout, R, S, C))
            scale = rng.uniform(0.0001, 0.01, size=Kout).astype(np.float32)
            bias = (rng.standard_normal(Kout) * 4).astype(np.float32)
            cs = (torch.from_numpy(oracle.i8_colsum(w.reshape(Kout, -1)).astype(np.int32)).cuda()
                  if use_cs else None)
            desc = (f"{kind} {Nb}x{H}x{W}x{C} * {Kout}x{R}x{S} stride={st} pad={pd} zA={zA} zB={zB} "
                    f"outputs={outs} colsum={use_cs} variant={v} split={sk}")
            print(desc, flush=True)
            got = run_qconv(igc, x, zA, w, zB, st, pd, outputs=outs, scale=scale, bias=bias, colsum_B=cs,
                            dq=float(oracle.dequant_scale(sA, sB)))
            C32 = oracle.conv2d_u8i8_direct(x, zA, w, zB, st, pd).reshape(-1, Kout)
        if "C" in got:
            assert np.array_equal(got["C"].astype(np.int64), C32), desc
        if "D" in got:
            assert np.array_equal(got["D"], oracle.dequant(C32, sA, sB)), desc
        if "Q" in got:
            assert np.array_equal(got["Q"], oracle.requant(C32, scale, bias)), desc
        return kind
    finally:
        igc.set_tuning(-1, 1)


@pytest.mark.parametrize("seed", [101, 102, 103])
def test_random_cases_match_the_oracle(igc, oracle, seed):
    rng = np.random.default_rng(seed)
    seen = [_one_case(igc, oracle, rng) for _ in range(50)]
    assert set(seen) == set(KINDS)


def _medium_case(igc, oracle, rng, kind):
    """GEMMs of about 600-2500 x 256-1500 and convolutions of up to 16 x 28 x 28
    x 256 -> 512: the shapes where the default plan picks the large tiles and,
    in the partial last round, the split; bit-exact like the small cases."""
    sk = int(rng.choice([1, 1, 2]))
    igc.set_tuning(-1, sk)
    try:
        if kind == "gemm_f16":
            M, N, K = int(rng.integers(600, 2500)), int(rng.integers(256, 1500)), int(rng.choice([64, 256, 512, 1000, 1024]))
            A, Bt = synth.f16_small_ints(rng, (M, K), -4, 4), synth.f16_small_ints(rng, (N, K), -4, 4)
            desc = f"{kind} M={M} N={N} K={K} split={sk}"
            print(desc, flush=True)
            assert np.array_equal(run_f16(igc, A, Bt).astype(np.float64), oracle.gemm_f16(A, Bt)), desc
        elif kind == "gemm_u8i8":
            M, N, K = int(rng.integers(600, 2500)), int(rng.integers(256, 1500)), int(rng.choice([128, 256, 512, 1024]))
            zA, zB = int(rng.choice([128, 0, 77])), int(rng.choice([0, -9]))
            A, Bt = synth.u8_uniform(rng, (M, K)), synth.i8_uniform(rng, (N, K))
            scale = rng.uniform(0.0005, 0.005, N).astype(np.float32)
            bias = rng.standard_normal(N).astype(np.float32)
            outs = [("Q",), ("C",), ("C", "D", "Q")][int(rng.integers(0, 3))]
            desc = f"{kind} M={M} N={N} K={K} zA={zA} zB={zB} outputs={outs} split={sk}"
            print(desc, flush=True)
            got = run_u8i8(igc, A, zA, Bt, zB, outputs=outs, scale=scale, bias=bias,
                           dq=float(oracle.dequant_scale(0.02, 0.01)))
            C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
            if "C" in got:
                assert np.array_equal(got["C"].astype(np.int64), C), desc
            if "D" in got:
                assert np.array_equal(got["D"], oracle.dequant(C, 0.02, 0.01)), desc
            if "Q" in got:
                assert np.array_equal(got["Q"], oracle.requant(C, scale, bias)), desc
        else:
            Nb, HW = int(rng.choice([4, 8, 16])), int(rng.choice([7, 14, 28]))
            C = int(rng.choice([128, 256])) if kind == "conv_u8i8" else int(rng.choice([64, 128, 256]))
            Kout, RS = int(rng.choice([64, 128, 256, 512])), int(rng.choice([1, 3]))
            st = int(rng.choice([1, 1, 2]))
            pd = int(rng.choice([0, 1])) if RS == 3 else 0
            desc = f"{kind} {Nb}x{HW}x{HW}x{C} * {Kout}x{RS}x{RS} stride={st} pad={pd} split={sk}"
            print(desc, flush=True)
            if kind == "conv_f16":
                x = synth.f16_small_ints(rng, (Nb, HW, HW, C), -4, 4)
                w = synth.f16_small_ints(rng, (Kout, RS, RS, C), -4, 4)
                assert np.array_equal(run_conv(igc, x, w, (st, st), (pd, pd)).astype(np.float64),
                                      oracle.conv2d_direct(x, w, (st, st), (pd, pd))), desc
            elif kind == "conv_nhwcnc":
                xb = synth.f16_small_ints(rng, (max(1, Nb // 8), HW, HW, C // 16, 16, 16), -4, 4)
                wb = synth.f16_small_ints(rng, (RS, RS, C // 16, Kout // 16, 16, 16), -4, 4)
                assert np.array_equal(run_conv_nhwcnc(igc, xb, wb, (st, st), (pd, pd)).astype(np.float64),
                                      oracle.conv2d_nhwcnc_direct(xb, wb, (st, st), (pd, pd))), desc
            else:
                x, w = synth.u8_uniform(rng, (Nb, HW, HW, C)), synth.i8_uniform(rng, (Kout, RS, RS, C))
                zA = int(rng.choice([100, 128, 0]))
                scale = rng.uniform(0.0001, 0.002, Kout).astype(np.float32)
                bias = rng.standard_normal(Kout).astype(np.float32)
                got = run_qconv(igc, x, zA, w, 0, (st, st), (pd, pd), outputs=("C", "Q"), scale=scale, bias=bias)
                Cr = oracle.conv2d_u8i8_direct(x, zA, w, 0, (st, st), (pd, pd)).reshape(-1, Kout)
                assert np.array_equal(got["C"].astype(np.int64), Cr), desc
                assert np.array_equal(got["Q"], oracle.requant(Cr, scale, bias)), desc
    finally:
        igc.set_tuning(-1, 1)


@pytest.mark.parametrize("seed", [201, 202])
def test_medium_random_cases_match_the_oracle(igc, oracle, seed):
    rng = np.random.default_rng(seed)
    for i in range(30):
        _medium_case(igc, oracle, rng, KINDS[i % len(KINDS)])


def test_long_k_random_cases_match_the_oracle(igc, oracle):
    """Small outputs over a long K (fp16 up to 16384, u8 x i8 up to the 33025
    limit): few tiles, so the split shares each tile's K range between many
    workgroups (the u8 x i8 split arithmetic is 32-bit)."""
    rng = np.random.default_rng(301)
    for i in range(10):
        v, sk = int(rng.choice([-1, -1, 1, 2])), int(rng.choice([1, 2]))
        igc.set_tuning(v, sk)
        try:
            if i % 2 == 0:
                M, N, K = int(rng.integers(64, 1024)), int(rng.integers(64, 1024)), int(rng.integers(2048, 16385))
                A, Bt = synth.f16_small_ints(rng, (M, K), -2, 2), synth.f16_small_ints(rng, (N, K), -2, 2)
                desc = f"gemm_f16 M={M} N={N} K={K} variant={v} split={sk}"
                print(desc, flush=True)
                assert np.array_equal(run_f16(igc, A, Bt).astype(np.float64), oracle.gemm_f16(A, Bt)), desc
            else:
                M, N = int(rng.integers(64, 768)), int(rng.integers(64, 768))
                K = [33025, 33024, int(rng.integers(2048, 33026))][i // 2 % 3]
                zA, zB = int(rng.choice([128, 0, 255])), int(rng.choice([0, 127, -128]))
                A, Bt = synth.u8_uniform(rng, (M, K)), synth.i8_uniform(rng, (N, K), -128, 127)
                scale = rng.uniform(1e-6, 1e-4, N).astype(np.float32)
                bias = rng.standard_normal(N).astype(np.float32)
                desc = f"gemm_u8i8 M={M} N={N} K={K} zA={zA} zB={zB} variant={v} split={sk}"
                print(desc, flush=True)
                got = run_u8i8(igc, A, zA, Bt, zB, outputs=("C", "Q"), scale=scale, bias=bias)
                C = oracle.gemm_u8i8_naive(A, zA, Bt, zB)
                assert np.array_equal(got["C"].astype(np.int64), C), desc
                assert np.array_equal(got["Q"], oracle.requant(C, scale, bias)), desc
        finally:
            igc.set_tuning(-1, 1)
