// Device helpers shared by the paged-KV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace pa {

// Checked build: record a broken contract in the device error word (a vector atomic OR).
__device__ __forceinline__ void flag_error(uint32_t* err, uint32_t bit) {
  if constexpr (kChecked) {
    if (err != nullptr) atomicOr(err, bit);
  }
}

// Checked build: a block id outside [0, num_blocks) is reported and replaced by block 0.
__device__ __forceinline__ int32_t checked_block(int32_t blk, int64_t num_blocks, uint32_t* err) {
  if constexpr (kChecked) {
    if (blk < 0 || (int64_t)blk >= num_blocks) {
      flag_error(err, kErrBlock);
      return 0;
    }
  }
  return blk;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// -- raw loads / stores ------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
// the same with the non-temporal hint, for bytes that one kernel touches once
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
__device__ __forceinline__ void st8_nt(void* p, u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p)); }

// -- bf16 -------------------------------------------------------------------
// A bf16 value is the upper half of a float32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even, two floats to one packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// The same rounding with gfx950's packed convert (one instruction for the pair).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Byte permute: result = (hi.half(sel) << 16) | lo.half(sel) for 16-bit halves.
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// -- OCP E4M3FN -------------------------------------------------------------
// gfx950's packed fp8 -> f32 convert (OCP E4M3FN): bytes 0,1 (word 0) or 2,3 (word 1).
__device__ __forceinline__ f32x2 e4m3x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }
__device__ __forceinline__ f32x2 e4m3x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, true); }


// Round a float to E4M3FN: nearest, ties to even, saturating to +-448; NaN keeps its sign.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;         // >= 448 (and infinity): saturate
  if (a < 0x3c800000u) {                             // below 2^-6: spacing 2^-9
    const float t = __uint_as_float(a) * 512.0f;     // exact: scaling by a power of two
    return sign | (uint32_t)__builtin_rintf(t);      // 0..8; 8 is the smallest normal
  }
  // keep 3 mantissa bits of the float, round to nearest even on bit 20
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  uint32_t code = r - (120u << 3);                   // float exponent bias 127 -> 7
  code = code > 0x7eu ? 0x7eu : code;
  return sign | code;
}

// -- symmetric int8 -----------------------------------------------------------
// Round to a symmetric int8 code: nearest, ties to even, saturating to +-127; NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_i8(float y) {
  if (y != y) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xffu;
}

// -- wave reductions ---------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
// row_half_mirror (lane i <-> 7-i in each 8), row_mirror (i <-> 15-i in each 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N in 1,2,4,...,64); every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);
  if constexpr (N >= 4) x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// -- dense numbering of (sequence, partition) pairs -------------------------------
// Sequence b has F_b = floor(ctx_b / P) full partitions and, when P does not divide
// ctx_b (or ctx_b is 0), one shorter last partition.  Pairs are numbered longest
// first: every full partition (sequence by sequence), then every shorter one, so the
// last workgroups handed out are the short ones.  Every lane of the wave gets pair
// x's sequence, partition and context length; returns false when x is past the last
// pair.  A sequence contributes at most max_parts pairs (the grid holds max_parts per
// sequence), so a context beyond the launch's max_context_len only loses its own later
// partitions.  All context lengths are loaded at once (up to kDenseMaxSeqs sequences).
constexpr int kDenseMaxSeqs = 1024;

// Inclusive prefix sum over the wave, on DPP: shifts right by 1, 2, 4 and 8 lanes
// within each 16-lane row (lanes shifted in from outside the row add 0), then
// row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31
// adds lane 31 to rows 2 and 3.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_scan(int v) {
  v += dpp_or_zero<0x111>(v);        // row_shr:1
  v += dpp_or_zero<0x112>(v);        // row_shr:2
  v += dpp_or_zero<0x114>(v);        // row_shr:4
  v += dpp_or_zero<0x118>(v);        // row_shr:8
  v += dpp_or_zero<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ bool locate_partition(const int32_t* __restrict__ context_lens, int B, int P,
                                                 int max_parts, int x, int& b_out, int& part_out, int& ctx_out) {
  constexpr int NC = kDenseMaxSeqs / 64;
  const int lane = threadIdx.x & 63;
  const int log2p = __builtin_ctz((unsigned)P);   // P is a power of two
  int cx[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int i = 64 * k + lane;
    cx[k] = -1;
    if (64 * k < B && i < B) cx[k] = context_lens[i];
  }
  // pass 0: full partitions; pass 1: the shorter last partitions
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    int base = 0;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (64 * k >= B) break;
      const int c = cx[k];
      // at most max_parts partitions per sequence: a context beyond the launch's bound
      // (a broken caller contract) loses its later partitions, never another sequence's
      const int n = c < 0 ? 0
                    : pass == 0 ? min(c >> log2p, max_parts)
                                : (((c & (P - 1)) != 0 || c == 0) && (c >> log2p) < max_parts ? 1 : 0);
      const int incl = wave_scan(n) + base;
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (x < tot) {
        const unsigned long long m = __ballot(incl > x);
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)m) - 1);
        const int b = 64 * k + l;
        const int cl = __builtin_amdgcn_readlane(c, l);
        // a pair always belongs to a real sequence with 0 <= ctx; anything else is refused
        if (l < 0 || b >= B || cl < 0) return false;
        b_out = b;
        part_out = pass == 0 ? x - __builtin_amdgcn_readlane(incl - n, l) : cl >> log2p;
        ctx_out = cl;
        return true;
      }
      base = tot;
    }
    x -= base;
  }
  return false;
}

}  // namespace pa
