// pa_slot_mapping: this step's slot mapping computed on the device from the block
// tables and context lengths, so a decode loop needs no host work between steps
// and can be captured once in a HIP graph and replayed.
//
// New token j of sequence b sits at position p = seq_lens[b] - n_b + j and is stored
// at slot = table[b][p / block_size] * block_size + p % block_size (LLM stack book
// 4.6, "From Python bookkeeping to the tensors the kernel actually takes": the slot
// mapping the engine rebuilds each step; ai-infra-handbooks "Paged KV cache",
// section "Block tables and slot mapping").  With `advance`, seq_lens[b] first grows
// by n_b: the lengths then count this step's tokens, as pa_decode expects.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

__global__ __launch_bounds__(256) void slot_mapping_kernel(const SlotArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.num_seqs) return;
  int r0, n;
  if (a.query_start_loc) {
    r0 = a.query_start_loc[b];
    n = a.query_start_loc[b + 1] - r0;
  } else {
    r0 = b;
    n = 1;
  }
  int S = a.seq_lens[b];
  if (a.advance) {
    S += n;
    a.seq_lens[b] = S;
  }
  const int32_t* row = a.block_tables + (int64_t)b * a.bt_stride;
  for (int j = 0; j < n; ++j) {
    const int r = r0 + j;
    if (r < 0 || r >= a.num_tokens) continue;
    const int p = S - n + j;
    const int lb = p >> a.log2_bs;
    // a position outside the table (or before the sequence) gets the padding slot -1
    a.slot_mapping[r] = (p < 0 || lb >= a.bt_stride) ? -1
                                                     : row[lb] * a.block_size + (p & (a.block_size - 1));
  }
}

hipError_t launch_slot_mapping(const SlotArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)((a.num_seqs + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
