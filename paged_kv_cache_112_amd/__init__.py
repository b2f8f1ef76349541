"""MI355X (gfx950) paged-KV hot path: slot-mapping K/V write and paged decode attention.

The computation lives in the HIP library ``libpa.so`` (C ABI: ``include/pa.h``);
this package is its ctypes binding.  Nothing here computes attention.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, PA_BF16, PA_ERR_DTYPE, PA_ERR_HIP, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED,
    PA_ERR_SCRATCH, PA_ERR_WORKSPACE, PA_F32, PA_FP8_E4M3, PA_INT8, PA_KERNEL_AUTO, PA_KERNEL_MFMA, PA_KERNEL_VALU, PA_OK, PaError,
    PaKvCache, cache_desc, check, check_decode_inputs, check_slots, copy_blocks, decode, decode_append, decode_partition, decode_partition_append,
    paged_attention, slot_mapping, decode_workspace_bytes, dtype_code, lib, merge,
    pa_copy_blocks, pa_copy_blocks_layers, pa_paged_attention, pa_slot_mapping, pa_decode, pa_decode_append, pa_decode_noalloc,
    pa_decode_partition, pa_decode_partition_append, pa_decode_workspace_bytes, pa_default_partition_tokens, pa_merge, pa_partition_tokens_for,
    pa_write_kv, status_str, workspace_views, write_kv, new_workspace)
