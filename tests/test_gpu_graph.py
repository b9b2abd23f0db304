"""HIP-graph capture of the entry points (GPU).

The library only enqueues kernels on the caller's stream (no allocation, copy
or synchronization), so a caller may capture its calls into a graph.  Each
graph here is replayed several times, with eager work and synchronizations
between the replays and the outputs overwritten before each one; every replay
must reproduce the eager call bit for bit.  The split-tile (stream-K) case
also checks that its arrival counters are left at zero from one replay to the
next (the workspace is zero-filled once, before capture)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def igc():
    import torch

    assert torch.cuda.is_available()
    import implicit_gemm_convolution_amd as m

    assert m.device_check() == m.IGC_OK, m.last_error()
    m.set_tuning(-1, 1)
    yield m
    m.set_tuning(-1, 1)


def _check_replays(run, outs):
    import torch

    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # a warm-up call on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        run()
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(7)
        other.mul_(1.0001)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {rep} differs from the eager call"
    # and eager again after the replays
    for o in outs:
        o.fill_(7)
    run()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)


def _f16(rng, shape):
    import torch

    return torch.from_numpy(rng.uniform(-1, 1, size=shape).astype(np.float16)).cuda()


def test_graph_gemm_f16_bypass(igc):
    import torch

    rng = np.random.default_rng(11)
    n = 256
    A, B = _f16(rng, (n, n)), _f16(rng, (n, n))
    C = torch.empty((n, n), dtype=torch.float32, device="cuda")
    _check_replays(lambda: igc.gemm_f16f32(n, n, n, A, n, B, n, C, n), [C])


def test_graph_gemm_f16_streamk(igc):
    import torch

    rng = np.random.default_rng(12)
    M = N = 640
    K = 1024
    A, B = _f16(rng, (M, K)), _f16(rng, (N, K))
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    igc.set_tuning(-1, 2)  # split wherever the tiles leave compute units idle
    try:
        nws = igc.gemm_f16f32_workspace_size(M, N, K)
        assert nws > 0
        ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
        _check_replays(lambda: igc.gemm_f16f32(M, N, K, A, K, B, K, C, N, workspace=ws, ws_bytes=nws), [C])
    finally:
        igc.set_tuning(-1, 1)


def test_graph_gemm_u8i8(igc):
    import torch

    rng = np.random.default_rng(13)
    n = 1024
    A = torch.from_numpy(rng.integers(0, 256, size=(n, n), dtype=np.uint8)).cuda()
    B = torch.from_numpy(rng.integers(-128, 128, size=(n, n), dtype=np.int8)).cuda()
    C = torch.empty((n, n), dtype=torch.int32, device="cuda")
    D = torch.empty((n, n), dtype=torch.float32, device="cuda")
    _check_replays(lambda: igc.gemm_u8i8_zp(n, n, n, A, n, 128, B, n, 3, C_i32=C, ldc=n, D_f32=D, ldd=n,
                                            dq_scale=0.0002), [C, D])


def test_graph_conv_u8i8_requant(igc):
    import torch

    rng = np.random.default_rng(14)
    Nb, H, W, Cin, Kout, R, S = 2, 14, 14, 128, 128, 3, 3
    zA, zB = 100, 0
    x = torch.from_numpy(rng.integers(0, 256, size=(Nb, H, W, Cin), dtype=np.uint8)).cuda()
    w = torch.from_numpy(rng.integers(-127, 128, size=(Kout, R, S, Cin), dtype=np.int8)).cuda()
    scale = torch.from_numpy(rng.uniform(0.001, 0.01, size=Kout).astype(np.float32)).cuda()
    bias = torch.from_numpy(rng.standard_normal(Kout).astype(np.float32)).cuda()
    M = Nb * H * W
    Q = torch.empty((M, Kout), dtype=torch.int8, device="cuda")
    _check_replays(lambda: igc.conv2d_u8i8_zp(Nb, H, W, Cin, Kout, R, S, 1, 1, 1, 1, x, zA, w, zB,
                                              Q_i8=Q, ldq=Kout, scale_n=scale, bias_n=bias), [Q])


def test_graph_gemm_u8i8_streamk(igc):
    import torch

    rng = np.random.default_rng(15)
    M, N, K = 384, 320, 4096
    A = torch.from_numpy(rng.integers(0, 256, size=(M, K), dtype=np.uint8)).cuda()
    B = torch.from_numpy(rng.integers(-128, 128, size=(N, K), dtype=np.int8)).cuda()
    C = torch.empty((M, N), dtype=torch.int32, device="cuda")
    igc.set_tuning(-1, 2)  # split wherever the tiles leave compute units idle
    try:
        nws = igc.gemm_u8i8_zp_workspace_size(M, N, K)
        assert nws > 0
        ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
        _check_replays(lambda: igc.gemm_u8i8_zp(M, N, K, A, K, 90, B, K, 5, C_i32=C, ldc=N,
                                                workspace=ws, ws_bytes=nws), [C])
        assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0  # arrival counters back at zero
    finally:
        igc.set_tuning(-1, 1)
