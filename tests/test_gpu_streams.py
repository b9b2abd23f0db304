"""Calls on different streams at once (GPU).

The entry points enqueue on the caller's stream and keep no state between
calls but the caller's workspace, so launches on two streams, each with its
own workspace, may overlap in time.  Here split-tile (stream-K) GEMMs and
quantized convolutions alternate over two default-priority streams without
synchronizing in between, and from two host threads; every result must equal
the oracle bit for bit."""
from __future__ import annotations

import threading

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    m.set_tuning(-1, 2)  # split wherever the tiles leave compute units idle
    yield m
    m.set_tuning(-1, 1)


def _problems(oracle, n):
    """n integer-valued fp16 GEMMs of distinct shapes (each splits) and their
    exact products."""
    out = []
    for i in range(n):
        rng = np.random.default_rng(700 + i)
        M, N, K = int(rng.integers(300, 700)), int(rng.integers(200, 600)), int(rng.choice([1024, 2048]))
        A, Bt = synth.f16_small_ints(rng, (M, K), -4, 4), synth.f16_small_ints(rng, (N, K), -4, 4)
        out.append((M, N, K, A, Bt, oracle.gemm_f16(A, Bt)))
    return out


def _launch_f16(igc, torch, prob, stream):
    M, N, K, A, Bt, _ = prob
    nws = igc.gemm_f16f32_workspace_size(M, N, K)
    assert nws > 0  # these shapes split
    with torch.cuda.stream(stream):
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(Bt).cuda()
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    igc.gemm_f16f32(M, N, K, dA, K, dB, K, dC, N, stream=stream, workspace=ws)
    return dC, (dA, dB, ws)


def test_split_gemms_alternating_over_two_streams(igc, oracle):
    import torch

    probs = _problems(oracle, 8)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [_launch_f16(igc, torch, p, streams[i % 2]) for i, p in enumerate(probs)]
    torch.cuda.synchronize()
    for (dC, _), p in zip(outs, probs):
        assert np.array_equal(dC.cpu().numpy().astype(np.float64), p[5]), p[:3]


def test_split_gemms_and_quantized_convs_from_two_threads(igc, oracle):
    import torch

    probs = _problems(oracle, 6)
    rng = np.random.default_rng(17)
    x = synth.u8_uniform(rng, (4, 14, 14, 128))
    w = synth.i8_uniform(rng, (96, 3, 3, 128))
    zA, zB = 100, -3
    ref_q = oracle.conv2d_u8i8_direct(x, zA, w, zB, (1, 1), (1, 1)).reshape(-1, 96)
    results, errors = {}, []

    def gemms():
        try:
            s = torch.cuda.Stream()
            results["gemm"] = [_launch_f16(igc, torch, p, s) for p in probs]
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    def convs():
        try:
            s = torch.cuda.Stream()
            dims = (4, 14, 14, 128, 96, 3, 3, 1, 1, 1, 1)
            outs = []
            for _ in range(6):
                with torch.cuda.stream(s):
                    dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
                    dC = torch.empty((4 * 14 * 14, 96), dtype=torch.int32, device="cuda")
                    nws = igc.conv2d_u8i8_zp_workspace_size(*dims)
                    ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device="cuda")
                igc.conv2d_u8i8_zp(*dims, dx, zA, dw, zB, C_i32=dC, ldc=96, stream=s, workspace=ws,
                                   ws_bytes=nws)
                outs.append((dC, (dx, dw, ws)))
            s.synchronize()
            results["conv"] = outs
        except Exception as e:
            errors.append(e)

    threads = [threading.Thread(target=gemms), threading.Thread(target=convs)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for (dC, _), p in zip(results["gemm"], probs):
        assert np.array_equal(dC.cpu().numpy().astype(np.float64), p[5]), p[:3]
    for dC, _ in results["conv"]:
        assert np.array_equal(dC.cpu().numpy().astype(np.int64), ref_q)
