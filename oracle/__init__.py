"""fp64 CPU oracle for the ternary-weight FP16 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The library in
``bit_mixed_precision_amd`` never imports it and shares no code with it.
"""

from .tq_oracle import (  # noqa: F401
    BLOCK,
    ternarize_ref,
    fp16_bits_ref,
    pack_tq2_ref,
    unpack_tq2_ref,
    tq1_ldq_ref,
    tq1_encode_group_ref,
    tq1_decode_division_ref,
    tq1_decode_multiply_ref,
    pack_tq1_ref,
    unpack_tq1_ref,
    dequantize_ref,
    gemm_ref,
    gemm_bruteforce_ref,
    silu_ref,
    swiglu_ref,
    gemm_bwd_x_ref,
    ste_grad_w_ref,
)
