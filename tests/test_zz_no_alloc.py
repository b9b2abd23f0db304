"""gemm_f16f32_noalloc: the fp16 GEMM with its stream-K workspace in the
library's static device array instead of a caller-owned one.  Checked
against gemm_f16f32 (with a caller-owned workspace) on two calls in a row,
the second smaller, with the split forced so the array is used; and against
the oracle on integer-valued inputs, where every correct result is exact."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import FP_TOL, empty_dev, fp_rel_err, to_dev, to_host, workspace_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    yield m
    m.set_tuning(-1, 1)


def _both(igc, A, Bt):
    import torch

    M, K = A.shape
    N = Bt.shape[0]
    dA, dB = to_dev(A), to_dev(Bt)
    need = igc.gemm_f16f32_workspace_size(M, N, K)
    ref = empty_dev((M, N), torch.float32)
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, ref, N, workspace=workspace_for(need))
    got = to_dev(np.full((M, N), np.nan, np.float32))
    igc.gemm_f16f32_noalloc(M, N, K, dA, K, dB, K, got, N)
    return need, to_host(got), to_host(ref)


def test_noalloc_matches_gemm_f16f32_twice_second_smaller(igc, oracle):
    igc.set_tuning(0, 2)  # 256x256 tiles, the last round's tiles shared
    try:
        rng = np.random.default_rng(77)
        # 272 tiles on 256 compute units: 16 shared, K = 512 -> 8 K tiles each
        A = synth.f16_normal(rng, (4352, 512))
        Bt = synth.f16_normal(rng, (4096, 512))
        need, got, ref = _both(igc, A, Bt)
        assert 0 < need <= 32 << 20
        assert fp_rel_err(got, ref) <= FP_TOL
        rows = np.array(sorted({0, 4095, 4096, 4351} | set(rng.integers(4096, 4352, 10).tolist())))
        assert fp_rel_err(got[rows], oracle.gemm_f16(A[rows], Bt)) <= FP_TOL
        # smaller: 270 tiles, 14 shared, K = 256 -> 4 K tiles each; integer
        # values, so every correct result is exact
        A2 = synth.f16_small_ints(rng, (4608, 256))
        B2 = synth.f16_small_ints(rng, (3840, 256))
        need2, got2, ref2 = _both(igc, A2, B2)
        assert 0 < need2 < need
        assert np.array_equal(got2, ref2)
        rows = np.array(sorted({0, 4095, 4096, 4607} | set(rng.integers(4096, 4608, 10).tolist())))
        assert np.array_equal(got2[rows].astype(np.float64), oracle.gemm_f16(A2[rows], B2))
    finally:
        igc.set_tuning(-1, 1)


def test_noalloc_default_tuning_and_too_large_split(igc):
    import torch

    # default tuning: no split at this shape, nothing of the array is used
    rng = np.random.default_rng(78)
    A = synth.f16_small_ints(rng, (300, 136))
    Bt = synth.f16_small_ints(rng, (200, 136))
    need, got, ref = _both(igc, A, Bt)
    assert need == 0
    assert np.array_equal(got, ref)
    # a forced split over 256 workgroups needs 128 MiB: rejected, nothing launched
    igc.set_tuning(0, 2)
    try:
        M, N, K = 4352, 4096, 2048
        assert igc.gemm_f16f32_workspace_size(M, N, K) > 32 << 20
        dA = empty_dev((M, K), torch.float16)
        dB = empty_dev((N, K), torch.float16)
        dC = empty_dev((M, N), torch.float32)
        st = igc.gemm_f16f32_noalloc(M, N, K, dA, K, dB, K, dC, N, check=False)
        assert st == igc.IGC_EUNSUPPORTED and "scratch" in igc.last_error()
    finally:
        igc.set_tuning(-1, 1)
