"""CPU oracle (TEST INFRASTRUCTURE): only tests, smoke() and bench.py's cpu_baseline use it."""
from .paged_oracle import (kv_cache_bytes, bf16_to_f64, e4m3_values, e4m3_to_f64, e4m3_encode,
                           e4m3_quantize, int8_quantize, to_f64, write_kv, slot_mapping, copy_blocks, decode, paged_attention, decode_partials, merge_partials,
                           ELEM_BYTES, E4M3_MAX, LOG2E)
