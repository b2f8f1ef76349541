"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This package draws random numbers and builds the integer bookkeeping a paged-KV
caller owns (block allocation, block tables, slot mappings, context lengths).  It
holds none of the attention arithmetic and none of the pool write: those live in
the HIP library and, independently, in the CPU oracle.
"""
from .allocator import BlockPool, BlockManager, slot_mapping_for, build_step_tensors
from .lengths import p2_length_pairs, p2_context_lens
from .values import (standard_normal_f32, f32_to_bf16_bits, bf16_bits_to_f32_exact,
                     BF16_NAN_BITS, E4M3_NAN_CODE)
from .configs import (DecodeWorkload, make_config, CONFIG_NAMES, deal_tables,
                      shared_prefix_tables, make_mq_config, MQ_CONFIG_NAMES)

__all__ = [
    "BlockPool", "BlockManager", "slot_mapping_for", "build_step_tensors",
    "p2_length_pairs", "p2_context_lens",
    "standard_normal_f32", "f32_to_bf16_bits", "bf16_bits_to_f32_exact",
    "BF16_NAN_BITS", "E4M3_NAN_CODE",
    "DecodeWorkload", "make_config", "CONFIG_NAMES", "deal_tables", "shared_prefix_tables",
    "make_mq_config", "MQ_CONFIG_NAMES",
]
