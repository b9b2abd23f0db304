"""CPU oracle for the GEMM / implicit-GEMM convolution path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product library
(``implicit_gemm_convolution_amd``) never imports, links or calls it, and it
never imports the product.  The two sides share nothing except the seeded
input generators in ``synth.py``, which hold none of the method's arithmetic.

The arithmetic is plain C in ``oracle.c`` (fp64 / int64 reductions in a fixed
order); this module only marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` next to it."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_decode.argtypes = [_p, _p, _i64]
        L.oracle_gemm_f16.argtypes = [_i64] * 3 + [_p, _i64, _p, _i64, _p, _i64]
        L.oracle_gemm_u8i8_naive.argtypes = [_i64] * 3 + [_p, _i64, _i64, _p, _i64, _i64, _p, _i64]
        L.oracle_gemm_u8i8_closed.argtypes = [_i64] * 3 + [_p, _i64, _i64, _p, _i64, _i64, _p, _i64]
        L.oracle_u8_rowsum.argtypes = [_i64, _i64, _p, _i64, _p]
        L.oracle_i8_colsum.argtypes = [_i64, _i64, _p, _i64, _p]
        L.oracle_dequant_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_dequant_scale.restype = ctypes.c_float
        L.oracle_dequant.argtypes = [_i64, _i64, _p, _i64, ctypes.c_float, ctypes.c_float, _p, _i64]
        L.oracle_requant_one.argtypes = [_i64, ctypes.c_float, ctypes.c_float]
        L.oracle_requant_one.restype = ctypes.c_int8
        L.oracle_requant.argtypes = [_i64, _i64, _p, _i64, _p, _p, _p, _i64]
        conv_args = [_i64] * 11
        L.oracle_conv2d_direct.argtypes = conv_args + [_p, _p, _p]
        L.oracle_conv2d_direct_at.argtypes = conv_args + [_p, _p, _p, _i64, _p]
        L.oracle_conv2d_im2col.argtypes = conv_args + [_p, _p, _p]
        L.oracle_im2col_f16.argtypes = [_i64] * 10 + [_p, _p]
        L.oracle_conv2d_u8i8_direct_at.argtypes = conv_args + [_p, _i64, _p, _i64, _p, _i64, _p]
        L.oracle_im2col_u8.argtypes = [_i64] * 10 + [_p, _i64, _p]
        L.oracle_conv2d_nhwcnc_direct.argtypes = conv_args + [_p, _p, _p]
        L.oracle_conv_out_dim.argtypes = [_i64] * 4
        L.oracle_conv_out_dim.restype = _i64
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _rows(a: np.ndarray, dtype) -> np.ndarray:
    """2-D C-contiguous view with the given element type (no value change)."""
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.ndim == 2
    return a


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode binary16 bit patterns (uint16 or float16 array) to float64."""
    b = np.ascontiguousarray(bits).view(np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().oracle_f16_decode(_ptr(b), _ptr(out), b.size)
    return out


def gemm_f16(A: np.ndarray, Bt: np.ndarray) -> np.ndarray:
    """O1: R = A @ Bt.T in float64.  A is M x K fp16, Bt is N x K fp16 (B column-major)."""
    A = _rows(A, np.float16)
    Bt = _rows(Bt, np.float16)
    M, K = A.shape
    N, K2 = Bt.shape
    assert K == K2
    R = np.empty((M, N), np.float64)
    lib().oracle_gemm_f16(M, N, K, _ptr(A), K, _ptr(Bt), K, _ptr(R), N)
    return R


def gemm_u8i8_naive(A: np.ndarray, zA: int, Bt: np.ndarray, zB: int) -> np.ndarray:
    """O2: C[m,n] = sum_k (A[m,k]-zA)(B[k,n]-zB) in int64.  Bt is N x K int8."""
    A = _rows(A, np.uint8)
    Bt = _rows(Bt, np.int8)
    M, K = A.shape
    N, K2 = Bt.shape
    assert K == K2
    C = np.empty((M, N), np.int64)
    lib().oracle_gemm_u8i8_naive(M, N, K, _ptr(A), K, int(zA), _ptr(Bt), K, int(zB), _ptr(C), N)
    return C


def gemm_u8i8_closed(A: np.ndarray, zA: int, Bt: np.ndarray, zB: int) -> np.ndarray:
    """O3: the four-term expansion of O2, computed by its own loops."""
    A = _rows(A, np.uint8)
    Bt = _rows(Bt, np.int8)
    M, K = A.shape
    N, K2 = Bt.shape
    assert K == K2
    C = np.empty((M, N), np.int64)
    lib().oracle_gemm_u8i8_closed(M, N, K, _ptr(A), K, int(zA), _ptr(Bt), K, int(zB), _ptr(C), N)
    return C


def u8_rowsum(A: np.ndarray) -> np.ndarray:
    A = _rows(A, np.uint8)
    out = np.empty(A.shape[0], np.int64)
    lib().oracle_u8_rowsum(A.shape[0], A.shape[1], _ptr(A), A.shape[1], _ptr(out))
    return out


def i8_colsum(Bt: np.ndarray) -> np.ndarray:
    Bt = _rows(Bt, np.int8)
    out = np.empty(Bt.shape[0], np.int64)
    lib().oracle_i8_colsum(Bt.shape[0], Bt.shape[1], _ptr(Bt), Bt.shape[1], _ptr(out))
    return out


def dequant_scale(sA: float, sB: float) -> np.float32:
    return np.float32(lib().oracle_dequant_scale(np.float32(sA), np.float32(sB)))


def dequant(C: np.ndarray, sA: float, sB: float) -> np.ndarray:
    """O4: D = fl32(fl32(C) * fl32(sA*sB))."""
    C = _rows(C.astype(np.int64, copy=False), np.int64)
    M, N = C.shape
    D = np.empty((M, N), np.float32)
    lib().oracle_dequant(M, N, _ptr(C), N, np.float32(sA), np.float32(sB), _ptr(D), N)
    return D


def requant_one(c: int, scale: float, bias: float) -> int:
    return int(lib().oracle_requant_one(int(c), np.float32(scale), np.float32(bias)))


def requant(C: np.ndarray, scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """O5: q = clamp(rne(fl32(fl32(fl32(C)*scale[n]) + bias[n])), -128, 127)."""
    C = _rows(C.astype(np.int64, copy=False), np.int64)
    M, N = C.shape
    scale = np.ascontiguousarray(scale, np.float32)
    bias = np.ascontiguousarray(bias, np.float32)
    assert scale.shape == (N,) and bias.shape == (N,)
    Q = np.empty((M, N), np.int8)
    lib().oracle_requant(M, N, _ptr(C), N, _ptr(scale), _ptr(bias), _ptr(Q), N)
    return Q


def conv_out_dim(n: int, k: int, stride: int, pad: int) -> int:
    return int(lib().oracle_conv_out_dim(n, k, stride, pad))


def _conv_shapes(x, w, stride, pad):
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert x.dtype == np.float16 and w.dtype == np.float16
    Nb, H, W, C = x.shape
    Kout, R, S, C2 = w.shape
    assert C == C2
    sh, sw = stride
    ph, pw = pad
    return x, w, (Nb, H, W, C, Kout, R, S, sh, sw, ph, pw)


def conv2d_direct(x: np.ndarray, w: np.ndarray, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """O6: direct 7-loop conv. x NHWC fp16, w KRSC fp16 -> y NHWC float64."""
    x, w, dims = _conv_shapes(x, w, stride, pad)
    Nb, H, W, C, Kout, R, S, sh, sw, ph, pw = dims
    P, Q = conv_out_dim(H, R, sh, ph), conv_out_dim(W, S, sw, pw)
    y = np.empty((Nb, P, Q, Kout), np.float64)
    lib().oracle_conv2d_direct(*dims, _ptr(x), _ptr(w), _ptr(y))
    return y


def conv2d_direct_at(x: np.ndarray, w: np.ndarray, pixels, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """O6 at listed output pixels m=(n*P+p)*Q+q; returns len(pixels) x Kout float64."""
    x, w, dims = _conv_shapes(x, w, stride, pad)
    pix = np.ascontiguousarray(pixels, np.int64)
    y = np.empty((pix.size, dims[4]), np.float64)
    lib().oracle_conv2d_direct_at(*dims, _ptr(x), _ptr(w), _ptr(pix), pix.size, _ptr(y))
    return y


def im2col_f16(x: np.ndarray, R: int, S: int, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.float16
    Nb, H, W, C = x.shape
    sh, sw = stride
    ph, pw = pad
    P, Q = conv_out_dim(H, R, sh, ph), conv_out_dim(W, S, sw, pw)
    col = np.empty((Nb * P * Q, R * S * C), np.float16)
    lib().oracle_im2col_f16(Nb, H, W, C, R, S, sh, sw, ph, pw, _ptr(x), _ptr(col))
    return col


def conv2d_im2col(x: np.ndarray, w: np.ndarray, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """O7: explicit im2col followed by the O1 GEMM."""
    x, w, dims = _conv_shapes(x, w, stride, pad)
    Nb, H, W, C, Kout, R, S, sh, sw, ph, pw = dims
    P, Q = conv_out_dim(H, R, sh, ph), conv_out_dim(W, S, sw, pw)
    y = np.empty((Nb, P, Q, Kout), np.float64)
    lib().oracle_conv2d_im2col(*dims, _ptr(x), _ptr(w), _ptr(y))
    return y


def _qconv_shapes(x, w, stride, pad):
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert x.dtype == np.uint8 and w.dtype == np.int8
    Nb, H, W, C = x.shape
    Kout, R, S, C2 = w.shape
    assert C == C2
    sh, sw = stride
    ph, pw = pad
    return x, w, (Nb, H, W, C, Kout, R, S, sh, sw, ph, pw)


def conv2d_u8i8_direct_at(x: np.ndarray, zA: int, w: np.ndarray, zB: int, pixels,
                          stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """O8 at listed output pixels m=(n*P+p)*Q+q: sum over the in-image taps of
    (x - zA)(w - zB), x NHWC uint8, w KRSC int8; returns len(pixels) x Kout int64."""
    x, w, dims = _qconv_shapes(x, w, stride, pad)
    pix = np.ascontiguousarray(pixels, np.int64)
    y = np.empty((pix.size, dims[4]), np.int64)
    lib().oracle_conv2d_u8i8_direct_at(*dims, _ptr(x), int(zA), _ptr(w), int(zB), _ptr(pix), pix.size,
                                       _ptr(y))
    return y


def conv2d_u8i8_direct(x: np.ndarray, zA: int, w: np.ndarray, zB: int, stride=(1, 1),
                       pad=(0, 0)) -> np.ndarray:
    """O8: the whole NHWC int64 output."""
    Nb, H, W, _ = x.shape
    Kout, R, S, _ = w.shape
    P, Q = conv_out_dim(H, R, stride[0], pad[0]), conv_out_dim(W, S, stride[1], pad[1])
    y = conv2d_u8i8_direct_at(x, zA, w, zB, np.arange(Nb * P * Q), stride, pad)
    return y.reshape(Nb, P, Q, Kout)


def im2col_u8(x: np.ndarray, zA: int, R: int, S: int, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """u8 im2col with the padding filled with the zero point zA."""
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint8
    Nb, H, W, C = x.shape
    sh, sw = stride
    ph, pw = pad
    P, Q = conv_out_dim(H, R, sh, ph), conv_out_dim(W, S, sw, pw)
    col = np.empty((Nb * P * Q, R * S * C), np.uint8)
    lib().oracle_im2col_u8(Nb, H, W, C, R, S, sh, sw, ph, pw, _ptr(x), int(zA), _ptr(col))
    return col


def conv2d_nhwcnc_direct(x: np.ndarray, w: np.ndarray, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """O9: direct convolution in the blocked NHWCnc layout (block size 16).
    x fp16 [Nb/16][H][W][C/16][16][16], w fp16 [R][S][C/16][Kout/16][16][16];
    returns float64 [Nb/16][P][Q][Kout/16][16][16]."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert x.ndim == 6 and w.ndim == 6 and x.shape[4:] == (16, 16) and w.shape[4:] == (16, 16)
    NB, H, W, CB = x.shape[:4]
    R, S, CB2, OB = w.shape[:4]
    assert CB == CB2
    P = conv_out_dim(H, R, stride[0], pad[0])
    Q = conv_out_dim(W, S, stride[1], pad[1])
    y = np.empty((NB, P, Q, OB, 16, 16), np.float64)
    xb, wb = x.view(np.uint16), w.view(np.uint16)
    lib().oracle_conv2d_nhwcnc_direct(16 * NB, H, W, 16 * CB, 16 * OB, R, S, stride[0], stride[1], pad[0], pad[1],
                                      _ptr(xb), _ptr(wb), _ptr(y))
    return y
