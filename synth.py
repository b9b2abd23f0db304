"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers.  It holds none of the method's
arithmetic (no products, sums, im2col or epilogue), so the oracle and the HIP
path can both consume its arrays without sharing any computation.

Workloads (numpy ``default_rng(seed)``, PCG64; draw order A, B, scale, bias).
"B" is always handed over as ``Bt`` = N rows of K (B column-major), the
convolution weight as KRSC.  fp16 values are drawn in float64 and rounded once
to binary16 (round to nearest even).

  c1  fp16 GEMM 256^3,   A, B ~ U[-1, 1]
  c2  u8 x i8 GEMM 1024^3, A ~ U{0..255}, B ~ U{-127..127}, zA=128, zB=3,
      per-tensor scales sA=0.02, sB=0.01 (int32 + dequantized fp32 out)
  c3  fp16 GEMM 4096^3,  A, B ~ N(0, 1)
  c4  fp16 conv2d NHWC 256x14x14x256, KRSC 512x3x3x256, stride 1, pad 1,
      x ~ N(0, 1), w ~ N(0, 0.05^2)
  c5  u8 x i8 GEMM 8192^3, A ~ U{0..255} (zA=128), B ~ U{-127..127} (zB=0),
      per-channel scale ~ U[0.001, 0.01], bias ~ N(0, 1), int8 requantized out

and one more, the quantized convolution (seed 104):

  q4  u8 x i8 conv2d with the shape of c4 (NHWC 256x14x14x256, KRSC
      512x3x3x256, stride 1, pad 1), x ~ U{0..255} (zA=100), w ~ U{-127..127}
      (zB=0), per-channel scale ~ U[0.001, 0.01], bias ~ N(0, 1), int8 out
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f16_uniform(rng: np.random.Generator, shape, lo=-1.0, hi=1.0) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float16)


def f16_normal(rng: np.random.Generator, shape, std=1.0) -> np.ndarray:
    if std == 1.0:
        return rng.standard_normal(size=shape).astype(np.float16)
    return (std * rng.standard_normal(size=shape)).astype(np.float16)


def f16_small_ints(rng: np.random.Generator, shape, lo=-8, hi=8) -> np.ndarray:
    """Integer-valued fp16 operands (exactly representable)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16)


def u8_uniform(rng: np.random.Generator, shape, lo=0, hi=255) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def i8_uniform(rng: np.random.Generator, shape, lo=-127, hi=127) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int8)


@dataclass
class Workload:
    name: str
    kind: str  # "gemm_f16", "gemm_u8i8", "conv_f16", "conv_u8i8"
    dims: dict
    arrays: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)

    def ops(self) -> float:
        """Algorithmic operation count 2*M*N*K (one multiply-add = 2 ops)."""
        d = self.dims
        return 2.0 * d["M"] * d["N"] * d["K"]


DESCRIPTIONS = {
    "c1": "gemm_f16f32 M=N=K=256, A row-major, B column-major, U[-1,1] fp16, fp32 out",
    "c2": "gemm_u8i8_zp M=N=K=1024, zA=128 zB=3, int32 out + fp32 dequant (sA=0.02, sB=0.01)",
    "c3": "gemm_f16f32 M=N=K=4096, A row-major, B column-major, N(0,1) fp16, fp32 out",
    "c4": "conv2d_implicit_gemm NHWC 256x14x14x256 * KRSC 512x3x3x256, s1 p1, fp16 in, fp32 out "
          "(GEMM M=50176 N=512 K=2304)",
    "c5": "gemm_u8i8_zp M=N=K=8192, zA=128 zB=0, per-channel scale+bias, RNE int8 requant",
    "q4": "conv2d_u8i8_zp NHWC 256x14x14x256 u8 (zA=100) * KRSC 512x3x3x256 i8 (zB=0), s1 p1, "
          "per-channel scale+bias, RNE int8 requant (GEMM M=50176 N=512 K=2304); the weights' column sums "
          "formed once (u8i8_colsum, static weights) and passed as colsum_B",
    "b4": "conv2d_implicit_gemm_nhwcnc blocked NHWCnc x (16,14,14,16,16,16) * w (3,3,16,32,16,16), s1 p1, "
          "fp16 in, fp32 out (the 256x14x14 conv in the tutorial's layout; GEMM M=50176 N=512 K=2304)",
}


def workload(name: str, *, scale_down: int = 1) -> Workload:
    """The five workloads, regenerated from their seeds.

    ``scale_down`` > 1 shrinks every GEMM dimension (or the conv batch) by that
    factor while keeping the distribution; it is used only by tests that need
    a small member of the same family.
    """
    seed = int(name[1:]) + {"c": 0, "q": 100, "b": 200}[name[0]]
    rng = np.random.default_rng(seed)
    if name == "c1":
        n = 256 // scale_down
        A = f16_uniform(rng, (n, n))
        Bt = f16_uniform(rng, (n, n))
        return Workload(name, "gemm_f16", dict(M=n, N=n, K=n), dict(A=A, Bt=Bt))
    if name == "c2":
        n = 1024 // scale_down
        A = u8_uniform(rng, (n, n))
        Bt = i8_uniform(rng, (n, n))
        return Workload(name, "gemm_u8i8", dict(M=n, N=n, K=n), dict(A=A, Bt=Bt),
                        dict(zA=128, zB=3, sA=0.02, sB=0.01, outputs=("C_i32", "D_f32")))
    if name == "c3":
        n = 4096 // scale_down
        A = f16_normal(rng, (n, n))
        Bt = f16_normal(rng, (n, n))
        return Workload(name, "gemm_f16", dict(M=n, N=n, K=n), dict(A=A, Bt=Bt))
    if name == "c4":
        nb = 256 // scale_down
        x = f16_normal(rng, (nb, 14, 14, 256))
        w = f16_normal(rng, (512, 3, 3, 256), std=0.05)
        conv = dict(Nb=nb, H=14, W=14, C=256, Kout=512, R=3, S=3,
                    stride_h=1, stride_w=1, pad_h=1, pad_w=1)
        dims = dict(M=nb * 14 * 14, N=512, K=9 * 256, **conv)
        return Workload(name, "conv_f16", dims, dict(x=x, w=w))
    if name == "c5":
        n = 8192 // scale_down
        A = u8_uniform(rng, (n, n))
        Bt = i8_uniform(rng, (n, n))
        scale = rng.uniform(0.001, 0.01, size=n).astype(np.float32)
        bias = rng.standard_normal(size=n).astype(np.float32)
        return Workload(name, "gemm_u8i8", dict(M=n, N=n, K=n), dict(A=A, Bt=Bt, scale=scale, bias=bias),
                        dict(zA=128, zB=0, outputs=("Q_i8",)))
    if name == "q4":
        nb = 256 // scale_down
        x = u8_uniform(rng, (nb, 14, 14, 256))
        w = i8_uniform(rng, (512, 3, 3, 256))
        scale = rng.uniform(0.001, 0.01, size=512).astype(np.float32)
        bias = rng.standard_normal(size=512).astype(np.float32)
        conv = dict(Nb=nb, H=14, W=14, C=256, Kout=512, R=3, S=3,
                    stride_h=1, stride_w=1, pad_h=1, pad_w=1)
        dims = dict(M=nb * 14 * 14, N=512, K=9 * 256, **conv)
        return Workload(name, "conv_u8i8", dims, dict(x=x, w=w, scale=scale, bias=bias),
                        dict(zA=100, zB=0, outputs=("Q_i8",)))
    if name == "b4":
        # c4's problem and distributions, drawn directly in the blocked NHWCnc
        # layout of the conv tutorial (block size 16): x [N/16][H][W][C/16][16n][16c],
        # w [R][S][C/16][K/16][16c][16k]
        nb = 256 // scale_down
        assert nb % 16 == 0
        x = f16_normal(rng, (nb // 16, 14, 14, 16, 16, 16))
        w = f16_normal(rng, (3, 3, 16, 32, 16, 16), std=0.05)
        conv = dict(Nb=nb, H=14, W=14, C=256, Kout=512, R=3, S=3,
                    stride_h=1, stride_w=1, pad_h=1, pad_w=1)
        dims = dict(M=nb * 14 * 14, N=512, K=9 * 256, **conv)
        return Workload(name, "conv_f16_blk", dims, dict(x=x, w=w))
    raise KeyError(name)


WORKLOADS = ("c1", "c2", "c3", "c4", "c5", "q4", "b4")
