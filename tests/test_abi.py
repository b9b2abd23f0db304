"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before touching the HIP runtime."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "igc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def igc():
    import implicit_gemm_convolution_amd as m

    if not os.path.exists(m.LIB_PATH):
        from implicit_gemm_convolution_amd import build

        build.build()
    m.load()
    return m


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("gemm_f16f32", "gemm_u8i8_zp", "conv2d_implicit_gemm", "conv2d_u8i8_zp"):
        assert name in fns
        assert name + "_workspace_size" in fns


def test_library_allocates_no_device_memory():
    """The caller owns every device buffer: no HIP allocation, free, memset,
    copy or synchronization appears in the library's sources."""
    csrc = os.path.join(ROOT, "implicit_gemm_convolution_amd", "csrc")
    banned = re.compile(r"\bhip(Malloc\w*|Free\w*|Memset\w*|Memcpy\w*|StreamSynchronize|DeviceSynchronize"
                        r"|HostMalloc|MallocManaged|ExtMallocWithFlags)\s*\(")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"//[^\n]*", "", text)
        assert not banned.search(text), (name, banned.search(text).group(0))


def test_library_exports_every_declared_symbol(igc):
    lib = ctypes.CDLL(igc.LIB_PATH)
    fns = declared_functions()
    assert set(fns) == set(igc.EXPORTED)
    for name in fns:
        assert hasattr(lib, name), name


def test_one_hip_runtime_in_process(igc):
    maps = open("/proc/self/maps").read()
    paths = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(paths) == 1, paths


def test_status_strings(igc):
    for st in (0, -1, -2, -3, -4, -5):
        assert igc.status_string(st).startswith("IGC_")


def test_gemm_f16_validation(igc):
    E = igc.IGC_EINVAL
    f = lambda *a: igc.gemm_f16f32(*a, check=False)  # noqa: E731
    assert f(-1, 4, 4, 1, 4, 1, 4, 1, 4) == E
    assert f(4, 4, 4, 0, 4, 1, 4, 1, 4) == E          # A NULL
    assert f(4, 4, 4, 1, 4, 0, 4, 1, 4) == E          # B NULL
    assert f(4, 4, 4, 1, 4, 1, 4, 0, 4) == E          # C NULL
    assert f(4, 4, 8, 1, 4, 1, 8, 1, 4) == E          # lda < K
    assert f(4, 4, 8, 1, 8, 1, 7, 1, 4) == E          # ldb < K
    assert f(4, 5, 8, 1, 8, 1, 8, 1, 4) == E          # ldc < N
    assert "ldc" in igc.last_error()
    # empty problems succeed without any device work
    assert f(0, 4, 4, 0, 4, 0, 4, 0, 4) == igc.IGC_OK
    assert f(4, 0, 4, 0, 4, 0, 4, 0, 0) == igc.IGC_OK


def test_gemm_u8i8_validation(igc):
    E = igc.IGC_EINVAL

    def f(M=4, N=4, K=16, A=1, lda=16, zA=128, B=1, ldb=16, zB=0, **kw):
        kw.setdefault("C_i32", 1)
        kw.setdefault("ldc", N)
        return igc.gemm_u8i8_zp(M, N, K, A, lda, zA, B, ldb, zB, check=False, **kw)

    assert f(zA=-1) == E
    assert f(zA=256) == E
    assert f(zB=128) == E
    assert f(zB=-129) == E
    assert f(C_i32=None) == E                          # no output requested
    assert f(ldc=3) == E
    assert f(C_i32=None, D_f32=1, ldd=2) == E
    assert f(C_i32=None, Q_i8=1, ldq=4) == E           # Q without scale/bias
    assert f(A=None) == E
    assert f(lda=15) == E
    assert f(K=33026, lda=33026, ldb=33026) == igc.IGC_EOVERFLOW
    assert f(M=0) == igc.IGC_OK
    st = igc.load().gemm_u8i8_zp(4, 4, 16, 1, 16, 128, 1, 16, 0, None, None)
    assert st == E                                     # NULL epilogue descriptor
    assert f(colsum_B=0x1002) == E                     # colsum_B not 4-byte aligned


def test_colsum_validation(igc):
    E = igc.IGC_EINVAL

    def f(N=4, K=16, B=16, ldb=16, out=16):
        return igc.u8i8_colsum(N, K, B, ldb, out, check=False)

    assert f(N=-1) == E
    assert f(K=-1) == E
    assert f(ldb=15) == E
    assert f(B=None) == E
    assert f(out=None) == E
    assert f(K=33026, ldb=33026) == igc.IGC_EOVERFLOW
    assert f(N=0, B=None, out=None) == igc.IGC_OK


def test_conv_validation(igc):
    E = igc.IGC_EINVAL

    def f(Nb=1, H=4, W=4, C=8, Kout=8, R=3, S=3, sh=1, sw=1, ph=1, pw=1, x=1, w=1, y=1):
        return igc.conv2d_implicit_gemm(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, x, w, y, check=False)

    assert f(Nb=0) == E
    assert f(C=-1) == E
    assert f(sh=0) == E
    assert f(ph=-1) == E
    assert f(x=None) == E
    assert f(R=7, ph=1) == E                           # filter larger than the padded input
    assert f(Nb=1 << 20, H=1 << 10, W=1 << 10, C=8) == igc.IGC_EUNSUPPORTED
    # coordinates of 2^15 or more do not fit the loaders' 16-bit halves
    U = igc.IGC_EUNSUPPORTED
    assert f(H=1, W=40000, C=8, R=1, S=3, ph=0, pw=1) == U
    assert f(H=32768, W=1, C=8, R=3, S=1, ph=1, pw=0) == U
    assert f(H=4, W=4, ph=32768, pw=0, R=3, S=3) == U
    assert f(H=4, W=4, ph=0, pw=40000, R=3, S=3) == U
    assert "32768" in igc.last_error()


def test_conv_nhwcnc_validation(igc):
    E = igc.IGC_EINVAL

    def f(Nb=16, H=4, W=4, C=16, Kout=16, R=3, S=3, sh=1, sw=1, ph=1, pw=1, x=16, w=16, y=16, ws=256, nws=1 << 20):
        return igc.conv2d_implicit_gemm_nhwcnc(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, x, w, y,
                                               workspace=ws, ws_bytes=nws, check=False)

    assert f(Nb=8) == E                                # blocks of 16 images
    assert f(C=24) == E                                # blocks of 16 channels
    assert f(Kout=40) == E
    assert f(x=None) == E
    assert f(ws=None, nws=0) == E                      # the workspace is required
    assert "workspace" in igc.last_error()
    assert f(w=24) == E                                # misaligned weights
    assert f(R=7) == E                                 # filter larger than the padded input
    out = ctypes.c_size_t(0)
    L = igc.load()
    assert L.conv2d_implicit_gemm_nhwcnc_workspace_size(8, 4, 4, 16, 16, 3, 3, 1, 1, 1, 1, ctypes.byref(out)) == E


def test_qconv_validation(igc):
    E = igc.IGC_EINVAL

    def f(Nb=1, H=4, W=4, C=128, Kout=8, R=3, S=3, sh=1, sw=1, ph=1, pw=1, x=1, zA=128, w=1, zB=0, **kw):
        kw.setdefault("C_i32", 1)
        kw.setdefault("ldc", Kout)
        return igc.conv2d_u8i8_zp(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, x, zA, w, zB, check=False, **kw)

    assert f(Nb=0) == E
    assert f(sh=0) == E
    assert f(R=7, ph=1) == E                           # filter larger than the padded input
    assert f(x=None) == E
    assert f(w=None) == E
    assert f(zA=256) == E
    assert f(zB=-129) == E
    assert f(C_i32=None) == E                          # no output requested
    assert f(ldc=7) == E
    assert f(C_i32=None, Q_i8=1, ldq=8) == E           # Q without scale/bias
    assert f(C=3670, R=3, S=3) == igc.IGC_EOVERFLOW    # K = 33030
    assert f(Nb=1 << 20, H=1 << 10, W=1 << 10, C=8) == igc.IGC_EUNSUPPORTED
    assert f(H=1, W=40000, C=8, R=1, S=3, ph=0, pw=1) == igc.IGC_EUNSUPPORTED
    st = igc.load().conv2d_u8i8_zp(1, 4, 4, 128, 8, 3, 3, 1, 1, 1, 1, 1, 128, 1, 0, None, None)
    assert st == E                                     # NULL epilogue descriptor


def test_set_tuning_validation(igc):
    E = igc.IGC_EINVAL
    assert igc.set_tuning(-2, 1, check=False) == E
    assert igc.set_tuning(7, 1, check=False) == E
    assert igc.set_tuning(-1, 3, check=False) == E
    assert igc.set_tuning(-1, -1, check=False) == E
    for v in range(-1, 7):
        for sk in range(3):
            assert igc.set_tuning(v, sk, check=False) == igc.IGC_OK
    assert igc.set_tuning(-1, 1, check=False) == igc.IGC_OK


def test_workspace_size_validation(igc):
    L = igc.load()
    out = ctypes.c_size_t(7)
    E = igc.IGC_EINVAL
    assert L.gemm_f16f32_workspace_size(-1, 4, 4, ctypes.byref(out)) == E
    assert L.gemm_u8i8_zp_workspace_size(4, 4, -4, ctypes.byref(out)) == E
    assert L.gemm_f16f32_workspace_size(4, 4, 4, None) == E
    # an empty problem needs nothing and no device
    assert L.gemm_f16f32_workspace_size(0, 4, 4, ctypes.byref(out)) == igc.IGC_OK
    assert out.value == 0
    conv = (1, 4, 4, 8, 8, 3, 3, 1, 1, 1, 1)
    bad = (1, 4, 4, 8, 8, 7, 3, 1, 1, 1, 1)  # filter larger than the padded input
    assert L.conv2d_implicit_gemm_workspace_size(*bad, ctypes.byref(out)) == E
    assert L.conv2d_u8i8_zp_workspace_size(*bad, ctypes.byref(out)) == E
    assert L.conv2d_u8i8_zp_workspace_size(*conv, None) == E


def test_valid_call_without_gpu_reports_nodev(igc):
    try:
        import torch

        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert igc.gemm_f16f32(4, 4, 8, 16, 8, 16, 8, 16, 4, check=False) == igc.IGC_ENODEV
    assert igc.u8i8_colsum(4, 16, 16, 16, 16, check=False) == igc.IGC_ENODEV
    assert igc.device_check() == igc.IGC_ENODEV
    out = ctypes.c_size_t(0)
    assert igc.load().gemm_f16f32_workspace_size(4096, 4096, 4096, ctypes.byref(out)) == igc.IGC_ENODEV
