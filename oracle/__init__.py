"""fp64 CPU oracle for rotate-then-quantize int4 (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  The product library never imports, links or calls it.
"""
from .rtq_oracle import (  # noqa: F401
    FP16_MAX, INT4_MAX, INT4_MIN, MASK64, SPLITMIX64_GAMMA,
    CODE_BITS, attn_decode, cache_rows, dequant_inv, dequant_inv_ext, dequant_rows, forward_detail_ext, pack_bits,
    quant_fwd_ext, quantize_groups_bits, unpack_bits, fp16_scale_bits, dequantize_groups, forward_detail, fp16_scale_from_absmax,
    int4_roundtrip_blocks, pack_nibbles, quant_fwd, quantize_groups,
    quantize_with_scale, rotate_fwd, rotate_inv, rotation_matrix, row_seed,
    sign_matrix, sign_vector, splitmix64_stream, srft_matrix, srht_matrix, window_schedule,
    unpack_nibbles,
)
