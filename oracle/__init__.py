"""fp64 CPU oracle for the q4_0 decode hot path (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the HIP library and its Python binding never do.
"""
from .q4_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    codes_from_nibbles,
    dequant,
    f16_bits_to_f64,
    ffn_down_input_bits,
    first_argmax,
    GELU_SLOPE_MAX,
    gelu_mul,
    gelu_mul_tolerance,
    gelu_tanh_f32,
    gelu_tanh_f64,
    gemm,
    gemv,
    gemv_tolerance,
    lmhead,
    nibbles_from_codes,
    ple_gather,
    q4_quantize,
    rowq_gelu_mul,
    rowq_gather,
    rowq_lmhead,
    rowq_gemv,
    rowq_pack,
    rowq_unpack,
    QUANT_ABSMAX7,
    QUANT_Q4_0,
    softcap,
    top2_margin,
)
