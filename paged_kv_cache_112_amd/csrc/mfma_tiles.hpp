// Register tiles and matrix-core steps shared by the paged-decode kernels (gfx950).
//
// A tile is 16 logical tokens of one KV head.  Lane l of a wave is (n = l & 15,
// q4 = l >> 4).
//   K tile: lane (n, q4) holds 16-byte slices of token n's K row: the A operand
//           of v_mfma_f32_16x16x32_bf16 (row m = token, k = head dimension).
//   V tile: lane (n, q4) holds head-dimension columns VEC*n .. VEC*n+VEC-1 of the
//           four tokens 4*q4 .. 4*q4+3 (VEC = D / 16).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace pa {

template <bool FP8, int D>
struct KTile {
  static constexpr int N = FP8 ? D / 64 : D / 32;   // 16-byte loads per lane
  u32x4 w[N];
};

template <bool FP8, int D>
struct VTile {
  // bytes per lane per row: VEC elements, VEC = D / 16
  static constexpr int BYTES = (D / 16) * (FP8 ? 1 : 2);
  typedef typename std::conditional<BYTES == 16, u32x4, typename std::conditional<BYTES == 8, u32x2, uint32_t>::type>::type W;
  W w[4];
};

template <bool FP8, int D>
__device__ __forceinline__ int q_col(int kk, int q4) {
  if constexpr (FP8) {
    if constexpr (D == 128) return 64 * (kk >> 1) + 16 * q4 + 8 * (kk & 1);
    else return 16 * q4 + 8 * kk;
  } else {
    return 32 * kk + 8 * q4;
  }
}

// Eight E4M3 bytes (two words) to a bf16x8 MFMA operand, element order preserved.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = e4m3x2_to_bf16x2(e4m3x2_lo(w0));
  r[1] = e4m3x2_to_bf16x2(e4m3x2_hi(w0));
  r[2] = e4m3x2_to_bf16x2(e4m3x2_lo(w1));
  r[3] = e4m3x2_to_bf16x2(e4m3x2_hi(w1));
  return __builtin_bit_cast(bf16x8, r);
}

// Raw q.K^T of one tile: lane (g = n, q4) gets dot(q_g, K_t) for tokens t = 4*q4 + r in
// register r (the C layout of the 16x16 product with m = token, n = query head).
template <bool FP8, int D>
__device__ __forceinline__ f32x4 qk_tile(const KTile<FP8, D>& k, const bf16x8 (&qB)[D / 32]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!FP8) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.w[kk]), qB[kk], s, 0, 0, 0);
  } else {
#pragma unroll
    for (int h = 0; h < KTile<FP8, D>::N; ++h) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(k.w[h][0], k.w[h][1]), qB[2 * h], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(k.w[h][2], k.w[h][3]), qB[2 * h + 1], s, 0, 0, 0);
    }
  }
  return s;
}

// O += P.V for one tile.  (p01, p23) are the bf16 probabilities of tokens
// 4*q4 .. 4*q4+3 for query head g = n: exactly the A operand (m = g, k = token)
// of v_mfma_f32_16x16x16_bf16.  The V rows are re-paired into token-major B
// operands (k = token, n = column), one product per column offset e < VEC;
// O[e] then holds O[g = 4*q4' + r][VEC*n + e] in lane (n, q4'), register r.
template <bool FP8, int D>
__device__ __forceinline__ void pv_tile(const VTile<FP8, D>& v, uint32_t p01, uint32_t p23, f32x4 (&O)[D / 16]) {
  constexpr int VEC = D / 16;
  const bf16x4 A = __builtin_bit_cast(bf16x4, u32x2{p01, p23});
  uint32_t rw[4][VEC / 2];                  // per token row: bf16 pairs (columns 2c, 2c+1)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (!FP8) {
#pragma unroll
      for (int c = 0; c < VEC / 2; ++c) rw[j][c] = v.w[j][c];
    } else if constexpr (VEC == 8) {
      rw[j][0] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j][0]));
      rw[j][1] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j][0]));
      rw[j][2] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j][1]));
      rw[j][3] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j][1]));
    } else {
      rw[j][0] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j]));
      rw[j][1] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j]));
    }
  }
#pragma unroll
  for (int c = 0; c < VEC / 2; ++c) {
    const u32x2 even = {pack_lo_halves(rw[0][c], rw[1][c]), pack_lo_halves(rw[2][c], rw[3][c])};
    const u32x2 odd = {pack_hi_halves(rw[0][c], rw[1][c]), pack_hi_halves(rw[2][c], rw[3][c])};
    O[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4, even), O[2 * c], 0, 0, 0);
    O[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4, odd), O[2 * c + 1], 0, 0, 0);
  }
}

// O^T += V^T . P^T for one tile, the transposed form of pv_tile: A = V^T (row m =
// head-dimension index, k = token) and B = the probabilities exactly as q.K^T left
// them (k = token, column n = query head).  Lane (n, q4) supplies row n of block e as
// column VEC*n + e of its four V rows.  Afterwards lane (n', q4') register r of O[e]
// holds O[head n'][d = VEC*(4*q4' + r) + e]: every lane keeps its own head's values,
// so a per-head rescale is a lane-local multiply.
template <bool FP8, int D>
__device__ __forceinline__ void pvt_tile(const VTile<FP8, D>& v, uint32_t p01, uint32_t p23, f32x4 (&O)[D / 16]) {
  constexpr int VEC = D / 16;
  const bf16x4 B = __builtin_bit_cast(bf16x4, u32x2{p01, p23});
  uint32_t rw[4][VEC / 2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (!FP8) {
#pragma unroll
      for (int c = 0; c < VEC / 2; ++c) rw[j][c] = v.w[j][c];
    } else if constexpr (VEC == 8) {
      rw[j][0] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j][0]));
      rw[j][1] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j][0]));
      rw[j][2] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j][1]));
      rw[j][3] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j][1]));
    } else {
      rw[j][0] = e4m3x2_to_bf16x2(e4m3x2_lo(v.w[j]));
      rw[j][1] = e4m3x2_to_bf16x2(e4m3x2_hi(v.w[j]));
    }
  }
#pragma unroll
  for (int c = 0; c < VEC / 2; ++c) {
    const u32x2 even = {pack_lo_halves(rw[0][c], rw[1][c]), pack_lo_halves(rw[2][c], rw[3][c])};
    const u32x2 odd = {pack_hi_halves(rw[0][c], rw[1][c]), pack_hi_halves(rw[2][c], rw[3][c])};
    O[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, even), B, O[2 * c], 0, 0, 0);
    O[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, odd), B, O[2 * c + 1], 0, 0, 0);
  }
}

}  // namespace pa
