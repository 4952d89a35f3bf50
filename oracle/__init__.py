"""f64 CPU oracle for paged, folded causal attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the attention library never does.  It shares no code
with the GPU path.
"""

from .oracle import (  # noqa: F401
    HostView,
    attend,
    B1_MAX_OUTLIERS,
    block_f32,
    build,
    decode_1bit,
    dequant_f32,
    encode_1bit,
    entry_class,
    f16_bits,
    hot_bits,
    fp8_e4m3_encode,
    fp8_e4m3_value,
    int2_codes,
    int4_codes,
    logical_kv,
    merge_splits,
    pack_int2,
    pack_int4,
    quantize_block,
    quantize_block_fp8,
    reference,
    rope,
    round_bf16,
    regen_values,
    row_info,
    splitmix64,
    widen,
    widen_bits,
)
