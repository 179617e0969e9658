"""CPU fp64 oracle for paged GQA attention -- test infrastructure only.

Imported by tests/, the smoke check and the benchmark's CPU-baseline leg;
never by the library.
"""
from .pkv_oracle import (  # noqa: F401
    BLOCK_SIZE, append_ref, attend_one, bf16_to_f64, decode_ref, decode_weights_ref,
    default_scale, gather_ref, kv_bytes, kv_bytes_per_token, kv_head_of, prefill_ref,
    slot_ref, softmax_weights,
)
