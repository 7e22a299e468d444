"""CPU oracle for the W8A8 int8-dynamic linear layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never calls it, and the two share no code; both take
their inputs from the seeded generators in ``synth_inputs``.

Every function follows a passage of the pages; see ``oracle.w8a8_oracle``.
"""
from .w8a8_oracle import (  # noqa: F401
    K_MAX,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    f16_bits_to_f32,
    f32_to_f16_bits,
    to_f32,
    from_f32,
    quant_rows,
    quant_act,
    quantize_weights,
    gemm_exact,
    gemm_int64_rows,
    epilogue_f32,
    epilogue,
    linear,
    dequant_reference,
    float_reference,
    noise_model_rel_l2,
    rel_l2,
    unpack_pack_quantized,
    scale_to_f32,
    w8a16_acc,
    w8a16_abs_sum,
    w8a16_err_bound,
    w8a16_linear,
    f64_to_bf16_bits,
    layernorm_modulate,
    gelu,
    producer_quant,
    layernorm_modulate_quant,
    gelu_quant,
    layernorm_modulate_err_bound,
    gelu_err_bound,
    bf16_within,
)
