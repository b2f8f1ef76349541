// Pieces shared by the multi-query paged-attention kernels (attention_mfma.hip,
// attention_lds.hip): uniform loads, a column maximum across the four lane rows of an
// MFMA output, and the longest-first order of requests.
#pragma once

#include "common.hpp"

namespace pa {

__device__ __forceinline__ int32_t attn_load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Maximum over the four lanes n, n+16, n+32, n+48 (gfx950 permlane swaps).
__device__ __forceinline__ float col_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Requests are taken longest context first (ties by index), so the workgroups of the
// longest run first and shorter ones fill the tail.  Up to 64 requests are ranked in
// the kernel, one per lane; beyond that they are taken in index order.  Returns the
// request of rank r (uniform).
__device__ __forceinline__ int request_of_rank(const int32_t* seq_lens, int B, int r) {
  if (B > kWave) return r;
  const int lane = threadIdx.x & 63;
  const int mine = lane < B ? seq_lens[lane] : 0;
  int rank = 0;
  for (int j = 0; j < B; ++j) {
    const int other = __builtin_amdgcn_readlane(mine, j);
    rank += (other > mine || (other == mine && j < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == r);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
}

}  // namespace pa
