// Split-K merge of one query head's partition pieces by one 16-lane row of a wave.
//
// Partition j of a sequence left, per query head, m_j = max of its base-2 logits,
// l_j = sum 2^(x - m_j) and o_j = sum 2^(x - m_j) V.  With M = max_j m_j,
//     out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j
// (LLM stack book 4.6, "Performance considerations": long sequences are split over
// the sequence dimension and the pieces reduced afterwards; the rescaling is the
// running-max correction of its online softmax).
//
// The 16 lanes of a DPP row share one head; lane dl owns columns dl*C .. dl*C+C-1
// (C = head_dim / 16) and walks the partitions in order, eight at a time with all of
// their loads issued together.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace pa {

// partitions whose pieces one row loads at once
constexpr int kMergeChunk = 8;

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 8));
  return x;
}

__device__ __forceinline__ float row_sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Merge the n >= 1 pieces of query head h of sequence b into out[b, h, :] (q's format OF).
// Every lane of the row must call it with the same (b, h, n); dl = lane & 15.
template <int D, int OF>
__device__ __forceinline__ void merge_head_row(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
                                               const float* __restrict__ ws_o, int max_parts, int num_q_heads,
                                               int b, int h, int n, int dl, void* out) {
  constexpr int C = D / 16;
  const int64_t H = num_q_heads;
  const int64_t r0 = piece_row(b, 0, h, max_parts, num_q_heads);
  const float* ms = ws_m + r0;               // ms[j * H]
  const float* ls = ws_l + r0;
  const float* os = ws_o + r0 * D + dl * C;  // os[j * H * D]

  // this lane's (m, l) of partition dl and the first chunk's pieces, requested together
  const float m_own = dl < n ? ms[dl * H] : -INFINITY;
  const float l_own = dl < n ? ls[dl * H] : 0.f;
  f32x4 x[kMergeChunk][C / 4];
  float mj[kMergeChunk];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int jc = min(c + u, n - 1);
      mj[u] = ms[jc * H];
#pragma unroll
      for (int k = 0; k < C / 4; ++k) x[u][k] = __builtin_bit_cast(f32x4, ld16(os + jc * H * D + 4 * k));
    }
  };
  load_chunk(0);
  float M = m_own;
  for (int j = dl + 16; j < n; j += 16) M = fmaxf(M, ms[j * H]);
  M = row_max16(M);
  float L = dl < n ? l_own * __builtin_amdgcn_exp2f(m_own - M) : 0.f;
  for (int j = dl + 16; j < n; j += 16) L += ls[j * H] * __builtin_amdgcn_exp2f(ms[j * H] - M);
  L = row_sum16(L);

  float acc[C];
#pragma unroll
  for (int e = 0; e < C; ++e) acc[e] = 0.f;
  for (int c = 0;;) {
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float wv = c + u < n ? __builtin_amdgcn_exp2f(mj[u] - M) : 0.f;
#pragma unroll
      for (int k = 0; k < C / 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * k + e] = fmaf(wv, x[u][k][e], acc[4 * k + e]);
    }
    c += kMergeChunk;
    if (c >= n) break;
    load_chunk(c);
  }
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)b * num_q_heads + h) * D + dl * C;
  if constexpr (OF == kF32) {
#pragma unroll
    for (int k = 0; k < C / 4; ++k)
      st16(static_cast<float*>(out) + o + 4 * k,
           __builtin_bit_cast(u32x4, f32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]} * inv));
  } else {
    uint32_t wds[C / 2];
#pragma unroll
    for (int k = 0; k < C / 2; ++k) wds[k] = pack_bf16(acc[2 * k] * inv, acc[2 * k + 1] * inv);
    uint16_t* dst = static_cast<uint16_t*>(out) + o;
    if constexpr (C == 8) st16(dst, u32x4{wds[0], wds[1], wds[2], wds[3]});
    else st8(dst, u32x2{wds[0], wds[1]});
  }
}

}  // namespace pa
