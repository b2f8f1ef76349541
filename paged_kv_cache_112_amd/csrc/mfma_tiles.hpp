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

// Pool element formats on the matrix-core path (numbered as pa_dtype): bf16 rows go to
// the matrix cores as they are; one-byte formats (e4m3, int8) are widened to bf16 in
// registers, exactly (every e4m3 value and every int8 value is a bf16 value).
constexpr int kFmtBf16 = 1, kFmtE4m3 = 2, kFmtInt8 = 3;
constexpr bool byte_fmt(int KF) { return KF != kFmtBf16; }

// Two signed bytes of w (bytes 0, 1, or with HI bytes 2, 3) to a bf16 pair: each byte is
// sign-extended and converted to f32 exactly (one SDWA convert), and the pair is packed
// by one convert; |x| <= 128 has at most 8 significant bits, so the bf16 is exact.
template <bool HI>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w) {
  const int s = (int)w;
  const float a = HI ? (float)(int8_t)(s >> 16) : (float)(int8_t)s;
  const float b = HI ? (float)(s >> 24) : (float)(int8_t)(s >> 8);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Two E4M3 bytes to a bf16 pair: gfx950's packed fp8 -> f32 convert, then the upper
// halves (every E4M3 value is a bf16 value, so the f32's upper half is exact).  Measured
// faster than the scaled fp8 -> bf16 convert, which does it in one instruction.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const f32x2 v = HI ? e4m3x2_hi(w) : e4m3x2_lo(w);
  return pack_hi_halves(__float_as_uint(v.x), __float_as_uint(v.y));
}

template <int KF, bool HI>
__device__ __forceinline__ uint32_t bytes2_to_bf16x2(uint32_t w) {
  if constexpr (KF == kFmtInt8) return i8x2_to_bf16x2<HI>(w);
  else return e4m3x2_to_bf16x2<HI>(w);
}

template <int KF, int D>
struct KTile {
  static constexpr int N = byte_fmt(KF) ? D / 64 : D / 32;   // 16-byte loads per lane
  u32x4 w[N];
};

template <int KF, int D>
struct VTile {
  // bytes per lane per row: VEC elements, VEC = D / 16
  static constexpr int BYTES = (D / 16) * (byte_fmt(KF) ? 1 : 2);
  typedef typename std::conditional<BYTES == 16, u32x4, typename std::conditional<BYTES == 8, u32x2, uint32_t>::type>::type W;
  W w[4];
};

template <int KF, int D>
__device__ __forceinline__ int q_col(int kk, int q4) {
  if constexpr (byte_fmt(KF)) {
    if constexpr (D == 128) return 64 * (kk >> 1) + 16 * q4 + 8 * (kk & 1);
    else return 16 * q4 + 8 * kk;
  } else {
    return 32 * kk + 8 * q4;
  }
}

// Eight one-byte elements (two words) to a bf16x8 MFMA operand, element order preserved.
template <int KF>
__device__ __forceinline__ bf16x8 bytes8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = bytes2_to_bf16x2<KF, false>(w0);
  r[1] = bytes2_to_bf16x2<KF, true>(w0);
  r[2] = bytes2_to_bf16x2<KF, false>(w1);
  r[3] = bytes2_to_bf16x2<KF, true>(w1);
  return __builtin_bit_cast(bf16x8, r);
}

// Raw q.K^T of one tile: lane (g = n, q4) gets dot(q_g, K_t) for tokens t = 4*q4 + r in
// register r (the C layout of the 16x16 product with m = token, n = query head).
template <int KF, int D>
__device__ __forceinline__ f32x4 qk_tile(const KTile<KF, D>& k, const bf16x8 (&qB)[D / 32]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!byte_fmt(KF)) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.w[kk]), qB[kk], s, 0, 0, 0);
  } else {
#pragma unroll
    for (int h = 0; h < KTile<KF, D>::N; ++h) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bytes8_to_bf16x8<KF>(k.w[h][0], k.w[h][1]), qB[2 * h], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bytes8_to_bf16x8<KF>(k.w[h][2], k.w[h][3]), qB[2 * h + 1], s, 0, 0, 0);
    }
  }
  return s;
}

// O += P.V for one tile.  (p01, p23) are the bf16 probabilities of tokens
// 4*q4 .. 4*q4+3 for query head g = n: exactly the A operand (m = g, k = token)
// of v_mfma_f32_16x16x16_bf16.  The V rows are re-paired into token-major B
// operands (k = token, n = column), one product per column offset e < VEC;
// O[e] then holds O[g = 4*q4' + r][VEC*n + e] in lane (n, q4'), register r.
template <int KF, int D>
__device__ __forceinline__ void pv_tile(const VTile<KF, D>& v, uint32_t p01, uint32_t p23, f32x4 (&O)[D / 16]) {
  constexpr int VEC = D / 16;
  const bf16x4 A = __builtin_bit_cast(bf16x4, u32x2{p01, p23});
  uint32_t rw[4][VEC / 2];                  // per token row: bf16 pairs (columns 2c, 2c+1)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (!byte_fmt(KF)) {
#pragma unroll
      for (int c = 0; c < VEC / 2; ++c) rw[j][c] = v.w[j][c];
    } else if constexpr (VEC == 8) {
      rw[j][0] = bytes2_to_bf16x2<KF, false>(v.w[j][0]);
      rw[j][1] = bytes2_to_bf16x2<KF, true>(v.w[j][0]);
      rw[j][2] = bytes2_to_bf16x2<KF, false>(v.w[j][1]);
      rw[j][3] = bytes2_to_bf16x2<KF, true>(v.w[j][1]);
    } else {
      rw[j][0] = bytes2_to_bf16x2<KF, false>(v.w[j]);
      rw[j][1] = bytes2_to_bf16x2<KF, true>(v.w[j]);
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
template <int KF, int D>
__device__ __forceinline__ void pvt_tile(const VTile<KF, D>& v, uint32_t p01, uint32_t p23, f32x4 (&O)[D / 16]) {
  constexpr int VEC = D / 16;
  const bf16x4 B = __builtin_bit_cast(bf16x4, u32x2{p01, p23});
  uint32_t rw[4][VEC / 2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (!byte_fmt(KF)) {
#pragma unroll
      for (int c = 0; c < VEC / 2; ++c) rw[j][c] = v.w[j][c];
    } else if constexpr (VEC == 8) {
      rw[j][0] = bytes2_to_bf16x2<KF, false>(v.w[j][0]);
      rw[j][1] = bytes2_to_bf16x2<KF, true>(v.w[j][0]);
      rw[j][2] = bytes2_to_bf16x2<KF, false>(v.w[j][1]);
      rw[j][3] = bytes2_to_bf16x2<KF, true>(v.w[j][1]);
    } else {
      rw[j][0] = bytes2_to_bf16x2<KF, false>(v.w[j]);
      rw[j][1] = bytes2_to_bf16x2<KF, true>(v.w[j]);
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
