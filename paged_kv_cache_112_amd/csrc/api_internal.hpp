// Host-side entry shared by the C ABI's translation units (not exported).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// pa_decode with the split-K pieces in [scratch, scratch + scratch_bytes) (the layout of
// pa_decode_workspace_bytes); PA_ERR_SCRATCH when the shape needs more.
pa_status decode_in_scratch(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float scale, void* out, int32_t partition_tokens,
                            int32_t kernel, uint8_t* scratch, size_t scratch_bytes, void* stream);

// The checked build's device error word on the current device (nullptr in a release
// build, or when it cannot be found).
uint32_t* checked_error_word();

}  // namespace pa
