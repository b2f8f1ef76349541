// Split-K merge: combine the per-partition softmax pieces into the output.
//
// Partition j of a sequence left, per query head, m_j = max of its base-2
// logits, l_j = sum 2^(x - m_j) and o_j = sum 2^(x - m_j) V.  With M = max_j m_j,
//     out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j
// (LLM stack book 4.6, "Performance considerations": long sequences are split
// over the sequence dimension and the pieces reduced afterwards; the rescaling
// is the running-max correction of its online softmax).  Sequences that fit in
// one partition were finished by the partition kernel and are skipped here.
//
// Two schedules, chosen by the launch's partition count J (max_parts):
//   * J <= kRowMergeMaxParts: merge_rows_kernel, one wave per (sequence, four query
//     heads), one 16-lane row per head (merge_rows.hpp).
//   * longer: merge_kernel, one wave per (query head, sequence): four groups of 16
//     lanes each take every fourth partition, each lane owning head_dim / 16
//     columns; the groups are summed with cross-lane adds at the end.
// A sequence longer than the launch's J partitions (a context beyond
// max_context_len, which the caller must not pass) is merged over its first J.
#include "common.hpp"
#include "launch.hpp"
#include "merge_rows.hpp"

namespace pa {

template <int D, int OF>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
  // lane = (partition slot pg in 0..3, column group dl in 0..15); each lane owns D/16 columns
  constexpr int DPL = D / 16;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int pg = lane >> 4;
  const int d0 = (lane & 15) * DPL;
  const int ctx = a.context_lens[b];
  const int n = min((ctx + a.partition_tokens - 1) / a.partition_tokens, a.max_parts);
  if (n <= 1) return;
  // pieces are partition-major: partition j of this (sequence, head) is row piece_row(b, j, h)
  const int64_t r0 = piece_row(b, 0, h, a.max_parts, a.num_q_heads);
  const int64_t H = a.num_q_heads;
  const float* ms = a.ws_m + r0;            // ms[j * H]
  const float* ls = a.ws_l + r0;
  const float* os = a.ws_o + r0 * D + d0;   // os[j * H * D]

  // Every load of the first round (16 partitions, all of them for n <= 16) is issued
  // before the maxima are formed: the pieces do not depend on them, so the wave waits
  // for one memory round trip.  Lane j holds m_j and l_j (n <= 64; beyond, the
  // weights are read again from memory).
  f32x4 ov[4][DPL / 4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jc = min(4 * u + pg, n - 1);
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c) ov[u][c] = __builtin_bit_cast(f32x4, ld16(os + jc * H * D + 4 * c));
  }
  const float m_lane = lane < n ? ms[lane * H] : -INFINITY;
  const float l_lane = lane < n ? ls[lane * H] : 0.f;
  float M = m_lane;
  for (int j = lane + kWave; j < n; j += kWave) M = fmaxf(M, ms[j * H]);
  M = wave_max(M);
  float L = lane < n ? l_lane * __builtin_amdgcn_exp2f(m_lane - M) : 0.f;
  for (int j = lane + kWave; j < n; j += kWave) L += ls[j * H] * __builtin_amdgcn_exp2f(ms[j * H] - M);
  L = wave_sum(L);
  auto weight = [&](int j) -> float {   // 2^(m_j - M), 0 past the last partition
    const int jc = min(j, n - 1);
    const float mj = n <= kWave ? __shfl(m_lane, jc) : ms[jc * H];   // every lane takes part
    return j < n ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
  };

  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int j0 = 0;;) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wv = weight(j0 + 4 * u + pg);
#pragma unroll
      for (int c = 0; c < DPL / 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * c + e] = fmaf(wv, ov[u][c][e], acc[4 * c + e]);
    }
    j0 += 16;
    if (j0 >= n) break;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jc = min(j0 + 4 * u + pg, n - 1);
#pragma unroll
      for (int c = 0; c < DPL / 4; ++c) ov[u][c] = __builtin_bit_cast(f32x4, ld16(os + jc * H * D + 4 * c));
    }
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    acc[i] += __shfl_xor(acc[i], 16);
    acc[i] += __shfl_xor(acc[i], 32);
  }
  if (pg != 0) return;
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)b * a.num_q_heads + h) * D + d0;
  if constexpr (OF == kF32) {
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c)
      st16(static_cast<float*>(a.out) + o + 4 * c,
           __builtin_bit_cast(u32x4, f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]} * inv));
  } else {
    uint32_t wds[DPL / 2];
#pragma unroll
    for (int c = 0; c < DPL / 2; ++c) wds[c] = pack_bf16(acc[2 * c] * inv, acc[2 * c + 1] * inv);
    uint16_t* dst = static_cast<uint16_t*>(a.out) + o;
    if constexpr (DPL == 8) st16(dst, u32x4{wds[0], wds[1], wds[2], wds[3]});
    else st8(dst, u32x2{wds[0], wds[1]});
  }
}

template <int D, int OF>
__global__ __launch_bounds__(64) void merge_rows_kernel(const MergeArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int h = 4 * blockIdx.x + (lane >> 4);
  const int ctx = a.context_lens[b];
  const int n = min((ctx + a.partition_tokens - 1) / a.partition_tokens, a.max_parts);
  if (n <= 1 || h >= a.num_q_heads) return;     // uniform per 16-lane row
  merge_head_row<D, OF>(a.ws_m, a.ws_l, a.ws_o, a.max_parts, a.num_q_heads, b, h, n, lane & 15, a.out);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.max_parts <= 1 || a.num_seqs == 0) return hipSuccess;
  const dim3 block(kWave);
  if (a.max_parts <= kRowMergeMaxParts) {
    const dim3 grid((unsigned)((a.num_q_heads + 3) / 4), (unsigned)a.num_seqs);
    if (a.head_dim == 128) {
      if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_rows_kernel<128, kF32>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((merge_rows_kernel<128, kBf16>), grid, block, 0, s, a);
    } else {
      if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_rows_kernel<64, kF32>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((merge_rows_kernel<64, kBf16>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
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
