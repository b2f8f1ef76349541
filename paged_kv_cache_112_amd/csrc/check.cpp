// Host-side contract checks: the integer inputs of a decode or a write, inspected on the
// host before they are handed to the GPU (tests, debugging, untrusted schedulers).  The
// release kernels trust these contracts; these checks name the first entry that breaks
// one, so a caller can refuse the batch instead of reading or writing outside the pools.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/pa.h"

extern "C" {

pa_status pa_check_decode_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                 int64_t num_blocks, int32_t block_size, int64_t* bad_index) {
  if (bad_index) *bad_index = -1;
  if (!block_tables || !context_lens) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || max_context_len < 0 || num_blocks < 1 || block_size < 1)
    return PA_ERR_SHAPE;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t ctx = context_lens[b];
    if (ctx < 0 || ctx > max_context_len || ctx > cap) {
      if (bad_index) *bad_index = b;
      return PA_ERR_SHAPE;
    }
  }
  for (int32_t b = 0; b < num_seqs; ++b) {
    // only the entries a decode reads: logical blocks 0 .. ceil(ctx / bs) - 1
    const int64_t used = ((int64_t)context_lens[b] + block_size - 1) / block_size;
    const int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < used; ++j) {
      if (row[j] < 0 || row[j] >= num_blocks) {
        if (bad_index) *bad_index = (int64_t)b * max_blocks_per_seq + j;
        return PA_ERR_SHAPE;
      }
    }
  }
  return PA_OK;
}

pa_status pa_check_slots(const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks, int32_t block_size,
                         int64_t* bad_index) {
  if (bad_index) *bad_index = -1;
  if (!slot_mapping) return PA_ERR_NULL;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1) return PA_ERR_SHAPE;
  const int64_t slots = num_blocks * block_size;
  std::vector<std::pair<int32_t, int32_t>> seen;   // (slot, token) of every written token
  seen.reserve((size_t)num_tokens);
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t s = slot_mapping[i];
    if (s < 0) continue;                            // padding: skipped by the write
    if (s >= slots) {
      if (bad_index) *bad_index = i;
      return PA_ERR_SHAPE;
    }
    seen.emplace_back(s, i);
  }
  std::sort(seen.begin(), seen.end());
  int64_t first_dup = -1;
  for (size_t k = 1; k < seen.size(); ++k)
    if (seen[k].first == seen[k - 1].first && (first_dup < 0 || seen[k].second < first_dup)) first_dup = seen[k].second;
  if (first_dup >= 0) {
    if (bad_index) *bad_index = first_dup;
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

}  // extern "C"
