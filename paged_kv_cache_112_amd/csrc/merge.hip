// Split-K merge: combine the per-partition softmax pieces into the output.
//
// Partition j of a sequence left, per query head, m_j = max of its base-2
// logits, l_j = sum 2^(x - m_j) and o_j = sum 2^(x - m_j) V.  With M = max_j m_j,
//     out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j
// (LLM stack book 4.6, "Performance considerations": long sequences are split
// over the sequence dimension and the pieces reduced afterwards; the rescaling
// is the running-max correction of its online softmax).  Sequences that fit in
// one partition were finished by the partition kernel and are skipped here.
// One wave per (query head, sequence); lanes own head_dim / 64 output columns.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

template <int D, int OF>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
  constexpr int DPL = D / kWave;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int ctx = a.context_lens[b];
  const int n = (ctx + a.partition_tokens - 1) / a.partition_tokens;
  if (n <= 1) return;
  const int64_t base = ((int64_t)b * a.num_q_heads + h) * a.max_parts;
  const float* ms = a.ws_m + base;
  const float* ls = a.ws_l + base;
  const float* os = a.ws_o + base * D + lane * DPL;

  float M = -INFINITY;
  for (int j = lane; j < n; j += kWave) M = fmaxf(M, ms[j]);
  M = wave_max(M);
  float L = 0.f;
  for (int j = lane; j < n; j += kWave) L += ls[j] * __builtin_amdgcn_exp2f(ms[j] - M);
  L = wave_sum(L);

  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int j = 0; j < n; ++j) {
    const float w = __builtin_amdgcn_exp2f(ms[j] - M);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, os[(int64_t)j * D + i], acc[i]);
  }
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)b * a.num_q_heads + h) * D + lane * DPL;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const float y = acc[i] * inv;
    if constexpr (OF == kF32) static_cast<float*>(a.out)[o + i] = y;
    else static_cast<uint16_t*>(a.out)[o + i] = __builtin_bit_cast(uint16_t, (__bf16)y);
  }
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.max_parts <= 1 || a.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  const dim3 block(kWave);
  if (a.head_dim == 128) {
    if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_kernel<128, kF32>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128, kBf16>), grid, block, 0, s, a);
  } else {
    if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_kernel<64, kF32>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<64, kBf16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
