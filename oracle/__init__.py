"""CPU oracle for the FP8 block-scaled GEMM (NT and the nn/tn/tt storages), its
M-grouped MoE forms, the K-grouped TN form and the FP8 x FP4 GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library's GPU path
never calls it and shares no code with it.

The oracle is plain numpy in fp64.  See ``fp8_gemm`` for the definitions and
the passages of the DeepGEMM pages each step follows.
"""
from .fp8_gemm import (  # noqa: F401
    E4M3_VALUES,
    decode_e4m3,
    bf16_bits_to_f64,
    round_f64_to_bf16_bits,
    gemm_nt_acc,
    gemm_nt,
    gemm_layout,
    m_grouped_contiguous,
    m_grouped_masked,
    k_grouped_tn_acc,
    k_grouped_tn,
)
from .fp8_fp4 import (  # noqa: F401
    E2M1_VALUES,
    decode_e2m1_packed,
    gemm_fp8_fp4_nt_acc,
    gemm_fp8_fp4_nt,
    m_grouped_fp8_fp4_contiguous,
    m_grouped_fp8_fp4_masked,
)
