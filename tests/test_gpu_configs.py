"""The five workloads, and the quantized convolution q4, at their full sizes
in the launch configuration the benchmark times (default tuning), against the
oracle on every output element.

Integer outputs are compared bit for bit.  fp32 outputs use the gate of
gpu_util.fp_rel_err; the unfloored element-wise maximum and the normwise
error max|x - r| / max|r| are printed beside it (reported, not gated).
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import FP_TOL, empty_dev, fp_errors, fp_rel_err, to_dev, to_host, workspace_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    m.set_tuning(-1, 1)
    yield m
    m.set_tuning(-1, 1)


def report(name, got, ref):
    gate, unfloored, normwise = fp_errors(got, ref)
    print(f"{name}: gated rel err {gate:.3e} (limit {FP_TOL}), unfloored element-wise {unfloored:.3e}, "
          f"normwise {normwise:.3e}", flush=True)
    return gate


def run_gemm_f16(igc, wl):
    import torch

    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    dA, dB = to_dev(wl.arrays["A"]), to_dev(wl.arrays["Bt"])
    dC = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N,
                    workspace=workspace_for(igc.gemm_f16f32_workspace_size(M, N, K)))
    return dC


def test_c1_full(igc, oracle):
    wl = synth.workload("c1")
    C = to_host(run_gemm_f16(igc, wl))
    ref = oracle.gemm_f16(wl.arrays["A"], wl.arrays["Bt"])
    assert report("c1", C, ref) <= FP_TOL


def test_c3_full(igc, oracle):
    wl = synth.workload("c3")
    C = to_host(run_gemm_f16(igc, wl))
    ref = oracle.gemm_f16(wl.arrays["A"], wl.arrays["Bt"])
    assert report("c3 (all 4096 x 4096 outputs)", C, ref) <= FP_TOL


def u8i8_outputs(igc, wl, outputs=None):
    import torch

    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    pr = wl.params
    outputs = pr["outputs"] if outputs is None else outputs
    dA, dB = to_dev(wl.arrays["A"]), to_dev(wl.arrays["Bt"])
    out, kw = {}, {}
    if "C_i32" in outputs:
        out["C"] = empty_dev((M, N), torch.int32)
        kw.update(C_i32=out["C"], ldc=N)
    if "D_f32" in outputs:
        out["D"] = empty_dev((M, N), torch.float32)
        s = np.float32(np.float32(pr["sA"]) * np.float32(pr["sB"]))
        kw.update(D_f32=out["D"], ldd=N, dq_scale=float(s))
    if "Q_i8" in outputs:
        out["Q"] = empty_dev((M, N), torch.int8)
        dS, dBi = to_dev(wl.arrays["scale"]), to_dev(wl.arrays["bias"])
        out["_keep"] = (dS, dBi)
        kw.update(Q_i8=out["Q"], ldq=N, scale_n=dS, bias_n=dBi)
    igc.gemm_u8i8_zp(M, N, K, dA, K, pr["zA"], dB, K, pr["zB"],
                     workspace=workspace_for(igc.gemm_u8i8_zp_workspace_size(M, N, K)), **kw)
    return {k: (to_host(v) if k != "_keep" else v) for k, v in out.items()}


def test_c2_full(igc, oracle):
    wl = synth.workload("c2")
    out = u8i8_outputs(igc, wl)
    pr = wl.params
    C = oracle.gemm_u8i8_naive(wl.arrays["A"], pr["zA"], wl.arrays["Bt"], pr["zB"])
    assert np.array_equal(out["C"].astype(np.int64), C)
    assert np.array_equal(out["D"], oracle.dequant(C, pr["sA"], pr["sB"]))


def test_c5_full(igc, oracle):
    """Every requantized output of the 8192^3 int8 GEMM in the benchmark's
    launch (int8 output only), and every int32 accumulator from a second
    launch that writes C as well: saturated outputs (about 95% at these
    scales) would hide accumulator errors."""
    wl = synth.workload("c5")
    pr = wl.params
    Q = u8i8_outputs(igc, wl)["Q"]
    C_gpu = u8i8_outputs(igc, wl, outputs=("C_i32",))["C"]
    C = oracle.gemm_u8i8_naive(wl.arrays["A"], pr["zA"], wl.arrays["Bt"], pr["zB"])
    assert np.array_equal(C_gpu.astype(np.int64), C), "int32 accumulators differ"
    del C_gpu
    ref = oracle.requant(C, wl.arrays["scale"], wl.arrays["bias"])
    unsat = int(np.count_nonzero((ref > -128) & (ref < 127)))
    print(f"c5: {unsat} of {ref.size} requantized outputs unsaturated", flush=True)
    assert unsat >= ref.size // 100
    assert np.array_equal(Q, ref)


def run_c4(igc, wl):
    import torch

    d = wl.dims
    dims = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"], d["stride_w"],
            d["pad_h"], d["pad_w"])
    dx, dw = to_dev(wl.arrays["x"]), to_dev(wl.arrays["w"])
    dy = empty_dev((d["M"], d["Kout"]), torch.float32)
    igc.conv2d_implicit_gemm(*dims, dx, dw, dy,
                             workspace=workspace_for(igc.conv2d_implicit_gemm_workspace_size(*dims)))
    return to_host(dy)


def test_c4_full(igc, oracle):
    wl = synth.workload("c4")
    y = run_c4(igc, wl)
    ref = oracle.conv2d_direct(wl.arrays["x"], wl.arrays["w"], (1, 1), (1, 1)).reshape(wl.dims["M"], -1)
    assert report("c4 (all 50176 x 512 outputs)", y, ref) <= FP_TOL


def test_c4_streamk_sampled_pixels(igc, oracle):
    """The c4 convolution on 256x256 tiles with the last round's tiles shared
    between workgroups (stream-K, forced): tile rows 128.. of the 196 hold
    the shared tiles (392 tiles on 256 compute units)."""
    wl = synth.workload("c4")
    d = wl.dims
    M = d["M"]
    igc.set_tuning(0, 2)
    try:
        dims = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"], d["stride_w"],
                d["pad_h"], d["pad_w"])
        assert igc.conv2d_implicit_gemm_workspace_size(*dims) > 0
        y = run_c4(igc, wl)
    finally:
        igc.set_tuning(-1, 1)
    rng = np.random.default_rng(44)
    pix = {0, 13, 14, 195, 196, 223, 224, 255, 256, M - 1, M - 196, M - 224, 14 * 14 * 128 + 7 * 14 + 7,
           128 * 256, 128 * 256 - 1, 150 * 256 + 77, 170 * 256 + 255, 190 * 256 + 1}
    pix |= set(rng.integers(128 * 256, M, 200).tolist())
    pix = np.array(sorted(pix))
    ref = oracle.conv2d_direct_at(wl.arrays["x"], wl.arrays["w"], pix, (1, 1), (1, 1))
    assert report(f"c4 stream-K, {len(pix)} sampled pixels", y[pix], ref) <= FP_TOL


@pytest.mark.parametrize("precomputed_colsum", [True, False])
def test_q4_full(igc, oracle, precomputed_colsum):
    """The quantized convolution at the 256x14x14 conv shape, requantized
    int8, on every output: with the weights' column sums formed once and
    passed in (as the benchmark runs it), and formed in the K loop."""
    import torch

    wl = synth.workload("q4")
    d, pr = wl.dims, wl.params
    x, w = wl.arrays["x"], wl.arrays["w"]
    scale, bias = wl.arrays["scale"], wl.arrays["bias"]
    M, N = d["M"], d["N"]
    dims = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"], d["stride_w"],
            d["pad_h"], d["pad_w"])
    dQ = empty_dev((M, N), torch.int8)
    dS, dBi = to_dev(scale), to_dev(bias)
    dx, dw = to_dev(x), to_dev(w)
    cs = None
    if precomputed_colsum:
        Kd = d["R"] * d["S"] * d["C"]
        cs = empty_dev((N,), torch.int32)
        igc.u8i8_colsum(N, Kd, dw, Kd, cs)
    igc.conv2d_u8i8_zp(*dims, dx, pr["zA"], dw, pr["zB"], Q_i8=dQ, ldq=N, scale_n=dS, bias_n=dBi,
                       workspace=workspace_for(igc.conv2d_u8i8_zp_workspace_size(*dims)), colsum_B=cs)
    Q = to_host(dQ)
    C = oracle.conv2d_u8i8_direct_at(x, pr["zA"], w, pr["zB"], np.arange(M), (1, 1), (1, 1))
    ref = oracle.requant(C, scale, bias)
    print(f"q4: {int(np.count_nonzero((ref > -128) & (ref < 127)))} of {ref.size} outputs unsaturated",
          flush=True)
    assert np.array_equal(Q, ref)


def run_b4(igc, wl):
    import torch

    d = wl.dims
    dims = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"], d["stride_w"],
            d["pad_h"], d["pad_w"])
    dx, dw = to_dev(wl.arrays["x"]), to_dev(wl.arrays["w"])
    dy = empty_dev((d["Nb"] // 16, 14, 14, d["Kout"] // 16, 16, 16), torch.float32)
    igc.conv2d_implicit_gemm_nhwcnc(*dims, dx, dw, dy,
                                    workspace=workspace_for(igc.conv2d_implicit_gemm_nhwcnc_workspace_size(*dims)))
    return to_host(dy)


def test_b4_full(igc, oracle):
    """The 256x14x14 convolution in the tutorial's blocked NHWCnc layout, every output."""
    wl = synth.workload("b4")
    y = run_b4(igc, wl)
    ref = oracle.conv2d_nhwcnc_direct(wl.arrays["x"], wl.arrays["w"], (1, 1), (1, 1))
    assert report("b4 (all 256x14x14x512 outputs, blocked)", y, ref) <= FP_TOL


def test_b4_streamk_full(igc, oracle):
    """The same on 256x256 tiles with the last round's tiles shared (stream-K,
    forced).  Whole tiles sum every output in the same K order whatever their
    size, so the split is seen as the shared tiles' outputs differing from an
    unsplit run on the same tiles in their last bits."""
    wl = synth.workload("b4")
    igc.set_tuning(0, 0)
    try:
        y0 = run_b4(igc, wl)
        igc.set_tuning(0, 2)
        y = run_b4(igc, wl)
    finally:
        igc.set_tuning(-1, 1)
    assert np.any(y != y0), "the forced split left every output as the whole-tile run"
    ref = oracle.conv2d_nhwcnc_direct(wl.arrays["x"], wl.arrays["w"], (1, 1), (1, 1))
    assert report("b4 stream-K (all outputs, blocked)", y, ref) <= FP_TOL
