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
//   * longer: merge_kernel, four waves per (query head, sequence): sixteen groups of
//     16 lanes each take every sixteenth partition, 2, 4 or 8 partitions' pieces (by J)
//     requested at once and the first batch before anything waits, each lane owning
//     head_dim / 16 columns; the maximum and the sum are folded in one pass over the
//     partitions, and the groups are summed with cross-lane adds and through LDS.
// A sequence longer than the launch's J partitions (a context beyond
// max_context_len, which the caller must not pass) is merged over its first J.
#include "common.hpp"
#include "launch.hpp"
#include "merge_rows.hpp"

namespace pa {

template <int D, int OF, int CH>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  // Four waves per (query head, sequence).  Lane (wave, pg, dl) belongs to partition group
  // grp = 4 * wave + pg (16 groups; group grp takes partitions grp, grp + 16, ...) and
  // owns columns dl * DPL .. + DPL - 1.  CH partitions per group have their pieces
  // requested together (the launch picks CH from its partition count).
  constexpr int DPL = D / 16;
  constexpr int NG = 16;        // partition groups
  __shared__ float red[2][4];
  __shared__ f32x4 part[3][16][DPL / 4];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, pg = lane >> 4, dl = lane & 15;
  const int grp = 4 * wave + pg;
  const int ctx = a.context_lens[b];
  const int n = min((ctx + a.partition_tokens - 1) / a.partition_tokens, a.max_parts);
  if (n <= 1) return;                                   // uniform over the workgroup
  // pieces are partition-major: partition j of this (sequence, head) is row piece_row(b, j, h)
  const int64_t r0 = piece_row(b, 0, h, a.max_parts, a.num_q_heads);
  const int64_t H = a.num_q_heads;
  const float* ms = a.ws_m + r0;            // ms[j * H]
  const float* ls = a.ws_l + r0;
  const float* os = a.ws_o + r0 * D + dl * DPL;

  // this group's first CH partitions' pieces, requested before anything waits (indices
  // past the last clamp to it and get weight 0 below)
  f32x4 x[CH][DPL / 4];
  float mj[CH];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int jc = min(grp + NG * (i0 + c), n - 1);
      mj[c] = ms[jc * H];
#pragma unroll
      for (int k = 0; k < DPL / 4; ++k) x[c][k] = __builtin_bit_cast(f32x4, ld16(os + jc * H * D + 4 * k));
    }
  };
  load_batch(0);

  // M = max_j m_j and L = sum_j 2^(m_j - M) l_j: each thread folds partitions t, t + 256,
  // ... in one pass (every partition that exists has a finite m), then the workgroup
  // combines the (max, sum) pairs
  float mt = -INFINITY, lt = 0.f;
  for (int j = t; j < n; j += 256) {
    const float mj = ms[j * H], lj = ls[j * H];
    const float mn = fmaxf(mt, mj);
    lt = lt * __builtin_amdgcn_exp2f(mt - mn) + lj * __builtin_amdgcn_exp2f(mj - mn);
    mt = mn;
  }
  float M = wave_max(mt);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float L = wave_sum(mt == -INFINITY ? 0.f : lt * __builtin_amdgcn_exp2f(mt - M));
  if (lane == 0) red[1][wave] = L;

  // sum_j 2^(m_j - M) o_j over this group's partitions, a batch of CH at a time
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int i0 = 0;;) {                                  // uniform over the workgroup
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float w = grp + NG * (i0 + c) < n ? __builtin_amdgcn_exp2f(mj[c] - M) : 0.f;
#pragma unroll
      for (int k = 0; k < DPL / 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * k + e] = fmaf(w, x[c][k][e], acc[4 * k + e]);
    }
    i0 += CH;
    if (NG * i0 >= n) break;
    load_batch(i0);
  }
  // the four groups of a wave, then the four waves
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    acc[i] += __shfl_xor(acc[i], 16);
    acc[i] += __shfl_xor(acc[i], 32);
  }
  if (wave > 0 && pg == 0) {
#pragma unroll
    for (int k = 0; k < DPL / 4; ++k) part[wave - 1][dl][k] = f32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
  }
  __syncthreads();
  if (wave > 0 || pg != 0) return;
  L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
#pragma unroll
  for (int v = 0; v < 3; ++v)
#pragma unroll
    for (int k = 0; k < DPL / 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * k + e] += part[v][dl][k][e];
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)b * a.num_q_heads + h) * D + dl * DPL;
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

template <int CH>
static hipError_t launch_merge_wide(const MergeArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(4 * kWave);
  if (a.head_dim == 128) {
    if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_kernel<128, kF32, CH>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128, kBf16, CH>), grid, block, 0, s, a);
  } else {
    if (a.out_fmt == kF32) hipLaunchKernelGGL((merge_kernel<64, kF32, CH>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<64, kBf16, CH>), grid, block, 0, s, a);
  }
  return hipGetLastError();
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
  if (a.max_parts <= 32) return launch_merge_wide<2>(a, grid, s);
  if (a.max_parts <= 64) return launch_merge_wide<4>(a, grid, s);
  return launch_merge_wide<8>(a, grid, s);
}

}  // namespace pa
