"""FP8 (e4m3) block-scaled GEMM (NT, and NN/TN/TT with K-major operands), with
M-grouped MoE forms, the K-grouped TN form and an FP8 x FP4 GEMM, for AMD
MI355X (gfx950).  The kernels live in libdg.so behind the C ABI of
include/dg.h; this package is its Python binding."""
from ._lib import (  # noqa: F401
    DGError,
    EXPORTED,
    LIB_PATH,
    dg_bind_stream_workspace,
    dg_check_grouped_layout,
    dg_choose_config,
    dg_fp8_fp4_gemm_nt,
    dg_fp8_gemm_nn,
    dg_fp8_gemm_nt,
    dg_fp8_gemm_nt_noalloc,
    dg_fp8_gemm_tn,
    dg_fp8_gemm_tt,
    dg_init,
    dg_k_grouped_fp8_gemm_tn_contiguous,
    dg_m_grouped_fp8_fp4_gemm_nt_contiguous,
    dg_m_grouped_fp8_fp4_gemm_nt_masked,
    dg_m_grouped_fp8_gemm_nt_contiguous,
    dg_m_grouped_fp8_gemm_nt_masked,
    dg_version,
    load,
)
