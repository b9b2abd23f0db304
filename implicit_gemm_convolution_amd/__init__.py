"""MI355X-native tiled GEMM and implicit-GEMM convolution.

The compute lives in ``libigc.so`` (hand-written HIP for gfx950, C ABI in
``include/igc.h``); this package only builds it and marshals arguments to it.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    IGC_EHIP,
    IGC_EINVAL,
    IGC_ENODEV,
    IGC_EOVERFLOW,
    IGC_EUNSUPPORTED,
    IGC_OK,
    LIB_PATH,
    Epilogue,
    IGCError,
    conv2d_implicit_gemm,
    conv2d_implicit_gemm_nhwcnc,
    conv2d_implicit_gemm_nhwcnc_workspace_size,
    conv2d_implicit_gemm_workspace_size,
    conv2d_u8i8_zp,
    conv2d_u8i8_zp_workspace_size,
    device_check,
    gemm_f16f32,
    gemm_f16f32_noalloc,
    gemm_f16f32_workspace_size,
    gemm_u8i8_zp,
    gemm_u8i8_zp_workspace_size,
    last_error,
    load,
    set_tuning,
    status_string,
    u8i8_colsum,
)
