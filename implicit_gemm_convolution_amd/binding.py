"""Thin ctypes binding of libigc.so (include/igc.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Device buffers are passed either as raw device addresses (ints) or
as torch tensors on a ROCm device (their ``data_ptr()`` is taken); streams as
a raw ``hipStream_t`` (int) or a ``torch.cuda.Stream``.  When no stream is
given, torch's current stream is used if torch is loaded, else the null
stream.

The library must already be built (``python -m implicit_gemm_convolution_amd.build``
or ``__graft_entry__.build()``); a missing library raises, there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libigc.so")

IGC_OK = 0
IGC_EINVAL = -1
IGC_EUNSUPPORTED = -2
IGC_EOVERFLOW = -3
IGC_EHIP = -4
IGC_ENODEV = -5

# Every symbol include/igc.h declares.
EXPORTED = ("gemm_f16f32", "gemm_u8i8_zp", "conv2d_implicit_gemm", "conv2d_u8i8_zp",
            "gemm_f16f32_workspace_size", "gemm_u8i8_zp_workspace_size",
            "conv2d_implicit_gemm_workspace_size", "conv2d_u8i8_zp_workspace_size",
            "gemm_f16f32_noalloc", "conv2d_implicit_gemm_nhwcnc", "conv2d_implicit_gemm_nhwcnc_workspace_size",
            "u8i8_colsum",
            "igc_status_string", "igc_last_error", "igc_device_check", "igc_set_tuning")


class IGCError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


class Epilogue(ctypes.Structure):
    """igc_u8i8_epilogue."""
    _fields_ = [
        ("C_i32", ctypes.c_void_p),
        ("ldc", ctypes.c_int),
        ("D_f32", ctypes.c_void_p),
        ("ldd", ctypes.c_int),
        ("dq_scale", ctypes.c_float),
        ("Q_i8", ctypes.c_void_p),
        ("ldq", ctypes.c_int),
        ("scale_n", ctypes.c_void_p),
        ("bias_n", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
        ("colsum_B", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libigc.so once.  torch (when installed) is imported first so that
    the library binds to the HIP runtime torch already uses."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is not built; run `python -m implicit_gemm_convolution_amd.build`")
    try:  # one HIP runtime per process: let torch's copy be the one that is loaded
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    i, p, z = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    pz = ctypes.POINTER(ctypes.c_size_t)
    L.gemm_f16f32.argtypes = [i, i, i, p, i, p, i, p, i, p, z, p]
    L.gemm_f16f32.restype = i
    L.gemm_f16f32_noalloc.argtypes = [i, i, i, p, i, p, i, p, i, p]
    L.gemm_f16f32_noalloc.restype = i
    L.gemm_u8i8_zp.argtypes = [i, i, i, p, i, i, p, i, i, ctypes.POINTER(Epilogue), p]
    L.gemm_u8i8_zp.restype = i
    L.conv2d_implicit_gemm.argtypes = [i] * 11 + [p, p, p, p, z, p]
    L.conv2d_implicit_gemm.restype = i
    L.conv2d_u8i8_zp.argtypes = [i] * 11 + [p, i, p, i, ctypes.POINTER(Epilogue), p]
    L.conv2d_implicit_gemm_nhwcnc.argtypes = [i] * 11 + [p, p, p, p, z, p]
    L.conv2d_implicit_gemm_nhwcnc.restype = i
    L.conv2d_u8i8_zp.restype = i
    for name in ("gemm_f16f32_workspace_size", "gemm_u8i8_zp_workspace_size"):
        getattr(L, name).argtypes = [i, i, i, pz]
        getattr(L, name).restype = i
    for name in ("conv2d_implicit_gemm_workspace_size", "conv2d_u8i8_zp_workspace_size",
                 "conv2d_implicit_gemm_nhwcnc_workspace_size"):
        getattr(L, name).argtypes = [i] * 11 + [pz]
        getattr(L, name).restype = i
    L.u8i8_colsum.argtypes = [i, i, p, i, p, p]
    L.u8i8_colsum.restype = i
    L.igc_set_tuning.argtypes = [i, i]
    L.igc_set_tuning.restype = i
    L.igc_status_string.argtypes = [i]
    L.igc_status_string.restype = ctypes.c_char_p
    L.igc_last_error.argtypes = []
    L.igc_last_error.restype = ctypes.c_char_p
    L.igc_device_check.argtypes = []
    L.igc_device_check.restype = i
    _lib = L
    return L


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"expected a device address or a tensor, got {type(x)}")


def _stream(s) -> int | None:
    if s is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"expected a hipStream_t or a torch stream, got {type(s)}")


def _check(status: int, where: str) -> int:
    if status != IGC_OK:
        L = load()
        detail = L.igc_last_error().decode() or L.igc_status_string(status).decode()
        raise IGCError(status, where, detail)
    return status


def status_string(status: int) -> str:
    return load().igc_status_string(status).decode()


def last_error() -> str:
    return load().igc_last_error().decode()


def device_check(raise_on_error: bool = False) -> int:
    st = load().igc_device_check()
    return _check(st, "igc_device_check") if raise_on_error else st


def set_tuning(force_variant: int = -1, streamk_mode: int = 1, *, check=True) -> int:
    """Process-wide overrides (tests, sweeps): a forced tile variant (-1 = by
    shape) and the stream-K mode (0 off, 1 where it pays, 2 always)."""
    st = load().igc_set_tuning(int(force_variant), int(streamk_mode))
    return _check(st, "igc_set_tuning") if check else st


def _ws_query(name, *args) -> int:
    out = ctypes.c_size_t(0)
    _check(getattr(load(), name)(*args, ctypes.byref(out)), name)
    return int(out.value)


def gemm_f16f32_workspace_size(M, N, K) -> int:
    return _ws_query("gemm_f16f32_workspace_size", M, N, K)


def gemm_u8i8_zp_workspace_size(M, N, K) -> int:
    return _ws_query("gemm_u8i8_zp_workspace_size", M, N, K)


def conv2d_implicit_gemm_workspace_size(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w) -> int:
    return _ws_query("conv2d_implicit_gemm_workspace_size", Nb, H, W, C, Kout, R, S, stride_h, stride_w,
                     pad_h, pad_w)


def conv2d_u8i8_zp_workspace_size(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w) -> int:
    return _ws_query("conv2d_u8i8_zp_workspace_size", Nb, H, W, C, Kout, R, S, stride_h, stride_w,
                     pad_h, pad_w)


def conv2d_implicit_gemm_nhwcnc_workspace_size(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w) -> int:
    return _ws_query("conv2d_implicit_gemm_nhwcnc_workspace_size", Nb, H, W, C, Kout, R, S, stride_h, stride_w,
                     pad_h, pad_w)


def _ws_bytes(workspace, ws_bytes):
    if ws_bytes is None:
        ws_bytes = int(workspace.numel() * workspace.element_size()) if hasattr(workspace, "numel") else 0
    return ws_bytes


def gemm_f16f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None, *, workspace=None, ws_bytes=None,
                check=True) -> int:
    st = load().gemm_f16f32(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _addr(workspace),
                            _ws_bytes(workspace, ws_bytes), _stream(stream))
    return _check(st, "gemm_f16f32") if check else st


def gemm_f16f32_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=None, *, check=True) -> int:
    """gemm_f16f32 with its workspace in the library's static device array
    (allocates nothing; calls that overlap on one GPU race)."""
    st = load().gemm_f16f32_noalloc(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _stream(stream))
    return _check(st, "gemm_f16f32_noalloc") if check else st


def u8i8_colsum(N, K, B, ldb, colsum, stream=None, *, check=True) -> int:
    """colsum[n] = sum_k B[n*ldb + k] (int32), for the colsum_B argument."""
    st = load().u8i8_colsum(N, K, _addr(B), ldb, _addr(colsum), _stream(stream))
    return _check(st, "u8i8_colsum") if check else st


def gemm_u8i8_zp(M, N, K, A, lda, zA, B, ldb, zB, *, C_i32=None, ldc=0, D_f32=None, ldd=0,
                 dq_scale=0.0, Q_i8=None, ldq=0, scale_n=None, bias_n=None, stream=None,
                 workspace=None, ws_bytes=None, colsum_B=None, check=True) -> int:
    ep = Epilogue(_addr(C_i32), ldc, _addr(D_f32), ldd, float(dq_scale), _addr(Q_i8), ldq,
                  _addr(scale_n), _addr(bias_n), _addr(workspace), _ws_bytes(workspace, ws_bytes),
                  _addr(colsum_B))
    st = load().gemm_u8i8_zp(M, N, K, _addr(A), lda, zA, _addr(B), ldb, zB, ctypes.byref(ep),
                             _stream(stream))
    return _check(st, "gemm_u8i8_zp") if check else st


def conv2d_implicit_gemm(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, x, w, y,
                         stream=None, *, workspace=None, ws_bytes=None, check=True) -> int:
    st = load().conv2d_implicit_gemm(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w,
                                     _addr(x), _addr(w), _addr(y), _addr(workspace),
                                     _ws_bytes(workspace, ws_bytes), _stream(stream))
    return _check(st, "conv2d_implicit_gemm") if check else st


def conv2d_implicit_gemm_nhwcnc(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, x, w, y,
                                stream=None, *, workspace=None, ws_bytes=None, check=True) -> int:
    """The convolution on blocked NHWCnc tensors (block 16); the workspace is required."""
    st = load().conv2d_implicit_gemm_nhwcnc(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w,
                                            _addr(x), _addr(w), _addr(y), _addr(workspace),
                                            _ws_bytes(workspace, ws_bytes), _stream(stream))
    return _check(st, "conv2d_implicit_gemm_nhwcnc") if check else st


def conv2d_u8i8_zp(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, x, zA, w, zB, *,
                   C_i32=None, ldc=0, D_f32=None, ldd=0, dq_scale=0.0, Q_i8=None, ldq=0,
                   scale_n=None, bias_n=None, stream=None, workspace=None, ws_bytes=None,
                   colsum_B=None, check=True) -> int:
    ep = Epilogue(_addr(C_i32), ldc, _addr(D_f32), ldd, float(dq_scale), _addr(Q_i8), ldq,
                  _addr(scale_n), _addr(bias_n), _addr(workspace), _ws_bytes(workspace, ws_bytes),
                  _addr(colsum_B))
    st = load().conv2d_u8i8_zp(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, _addr(x), zA,
                               _addr(w), zB, ctypes.byref(ep), _stream(stream))
    return _check(st, "conv2d_u8i8_zp") if check else st
