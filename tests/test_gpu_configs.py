"""The five workloads at their full sizes, in the launch configuration the
benchmark times (default variant choice), against the oracle.  Where the full
oracle would take minutes, whole output rows (GEMM) or whole output pixels
(conv) are sampled: first, last, tile and workgroup boundaries, and random ones.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import FP_TOL, empty_dev, fp_rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    return m


@pytest.fixture(autouse=True)
def _default_variant(monkeypatch):
    monkeypatch.delenv("IGC_FORCE_VARIANT", raising=False)


def sample_rows(M, rng, extra=8, tile=256):
    rows = {0, 1, M - 1, M // 2, tile - 1, tile, min(M - 1, 2 * tile + 3)}
    rows |= set(rng.integers(0, M, extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M))


def run_gemm_f16(igc, wl):
    import torch

    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    dA, dB = to_dev(wl.arrays["A"]), to_dev(wl.arrays["Bt"])
    dC = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N)
    return dC


def test_c1_full(igc, oracle):
    wl = synth.workload("c1")
    C = to_host(run_gemm_f16(igc, wl))
    ref = oracle.gemm_f16(wl.arrays["A"], wl.arrays["Bt"])
    assert fp_rel_err(C, ref) <= FP_TOL


def test_c3_sampled_rows(igc, oracle):
    wl = synth.workload("c3")
    dC = run_gemm_f16(igc, wl)
    rows = sample_rows(wl.dims["M"], np.random.default_rng(33))
    C = to_host(dC[rows.tolist()])
    ref = oracle.gemm_f16(wl.arrays["A"][rows], wl.arrays["Bt"])
    err = fp_rel_err(C, ref)
    print(f"c3 sampled rows {len(rows)}: max rel err {err:.3e}")
    assert err <= FP_TOL


def u8i8_outputs(igc, wl):
    import torch

    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    pr = wl.params
    dA, dB = to_dev(wl.arrays["A"]), to_dev(wl.arrays["Bt"])
    out, kw = {}, {}
    if "C_i32" in pr["outputs"]:
        out["C"] = empty_dev((M, N), torch.int32)
        kw.update(C_i32=out["C"], ldc=N)
    if "D_f32" in pr["outputs"]:
        out["D"] = empty_dev((M, N), torch.float32)
        s = np.float32(np.float32(pr["sA"]) * np.float32(pr["sB"]))
        kw.update(D_f32=out["D"], ldd=N, dq_scale=float(s))
    if "Q_i8" in pr["outputs"]:
        out["Q"] = empty_dev((M, N), torch.int8)
        dS, dBi = to_dev(wl.arrays["scale"]), to_dev(wl.arrays["bias"])
        out["_keep"] = (dS, dBi)
        kw.update(Q_i8=out["Q"], ldq=N, scale_n=dS, bias_n=dBi)
    igc.gemm_u8i8_zp(M, N, K, dA, K, pr["zA"], dB, K, pr["zB"], **kw)
    return out


def test_c2_full(igc, oracle):
    wl = synth.workload("c2")
    out = u8i8_outputs(igc, wl)
    pr = wl.params
    C = oracle.gemm_u8i8_naive(wl.arrays["A"], pr["zA"], wl.arrays["Bt"], pr["zB"])
    assert np.array_equal(to_host(out["C"]).astype(np.int64), C)
    assert np.array_equal(to_host(out["D"]), oracle.dequant(C, pr["sA"], pr["sB"]))


def test_c5_sampled_rows(igc, oracle):
    wl = synth.workload("c5")
    out = u8i8_outputs(igc, wl)
    pr = wl.params
    rows = sample_rows(wl.dims["M"], np.random.default_rng(55), extra=6)
    Q = to_host(out["Q"][rows.tolist()])
    C = oracle.gemm_u8i8_naive(wl.arrays["A"][rows], pr["zA"], wl.arrays["Bt"], pr["zB"])
    ref = oracle.requant(C, wl.arrays["scale"], wl.arrays["bias"])
    unsat = np.count_nonzero((ref > -128) & (ref < 127))
    print(f"c5 sampled rows {len(rows)}: {unsat} of {ref.size} outputs unsaturated")
    assert np.array_equal(Q, ref)


# default: 224x256 tiles (448 tiles, two full rounds on 256 compute units);
# forced: 256x256 tiles with the last round's tiles shared (stream-K)
@pytest.mark.parametrize("variant,streamk", [(None, "1"), ("0", "2")])
def test_c4_sampled_pixels(igc, oracle, monkeypatch, variant, streamk):
    import torch

    if variant is not None:
        monkeypatch.setenv("IGC_FORCE_VARIANT", variant)
    monkeypatch.setenv("IGC_STREAMK", streamk)
    wl = synth.workload("c4")
    d = wl.dims
    x, w = wl.arrays["x"], wl.arrays["w"]
    dx, dw = to_dev(x), to_dev(w)
    dy = empty_dev((d["Nb"], 14, 14, d["Kout"]), torch.float32)
    igc.conv2d_implicit_gemm(d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"],
                             d["stride_h"], d["stride_w"], d["pad_h"], d["pad_w"], dx, dw, dy)
    M = d["M"]
    rng = np.random.default_rng(44)
    # (with the split forced, tile rows 128.. of the 196 hold the tiles shared
    # between workgroups: 392 tiles on 256 compute units)
    pix = {0, 13, 14, 195, 196, 223, 224, 255, 256, M - 1, M - 196, M - 224, 14 * 14 * 128 + 7 * 14 + 7,
           128 * 256, 128 * 256 - 1, 150 * 256 + 77, 170 * 256 + 255, 190 * 256 + 1}
    pix |= set(rng.integers(0, M, 40).tolist())
    pix = np.array(sorted(pix))
    y = to_host(dy.reshape(M, d["Kout"])[pix.tolist()])
    ref = oracle.conv2d_direct_at(x, w, pix, (1, 1), (1, 1))
    err = fp_rel_err(y, ref)
    print(f"c4 sampled pixels {len(pix)}: max rel err {err:.3e}")
    assert err <= FP_TOL


def test_q4_sampled_pixels(igc, oracle):
    """The quantized convolution at the 256x14x14 conv shape, requantized int8,
    bit-exact on sampled output pixels (borders and interior of several images)."""
    import torch

    wl = synth.workload("q4")
    d, pr = wl.dims, wl.params
    x, w = wl.arrays["x"], wl.arrays["w"]
    scale, bias = wl.arrays["scale"], wl.arrays["bias"]
    M, N = d["M"], d["N"]
    dQ = empty_dev((M, N), torch.int8)
    dS, dBi = to_dev(scale), to_dev(bias)
    dx, dw = to_dev(x), to_dev(w)
    igc.conv2d_u8i8_zp(d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"],
                       d["stride_w"], d["pad_h"], d["pad_w"], dx, pr["zA"], dw, pr["zB"],
                       Q_i8=dQ, ldq=N, scale_n=dS, bias_n=dBi)
    rng = np.random.default_rng(45)
    pix = {0, 13, 14, 195, 196, 223, 224, 255, 256, M - 1, M - 196, M - 224, 14 * 14 * 128 + 7 * 14 + 7}
    pix |= set(rng.integers(0, M, 40).tolist())
    pix = np.array(sorted(pix))
    Q = to_host(dQ[pix.tolist()])
    C = oracle.conv2d_u8i8_direct_at(x, pr["zA"], w, pr["zB"], pix, (1, 1), (1, 1))
    assert np.array_equal(Q, oracle.requant(C, scale, bias))
