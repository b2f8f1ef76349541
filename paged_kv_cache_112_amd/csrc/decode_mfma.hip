// Paged decode, partition stage, matrix-core path (bf16 or e4m3 pools, bf16 q).
//
// What is computed: for one sequence, one KV head and one partition of P
// logical tokens, the base-2 softmax pieces of
//     out[h] = softmax_t(scale * q[h] . K_t) V_t
// for the G query heads that share the KV head (LLM stack book 4.6, "The
// PagedAttention Kernel": the usual attention, with each token's K/V row found
// through the block table; GQA head h reads KV head h // G).  Token t lives in
// physical block table[t // bs] at offset t % bs (mohdvasim.com "PagedAttention
// - Explained", "The Custom CUDA Kernel Overview").  Long contexts are split into
// partitions whose pieces a second kernel merges (LLM stack book, "Performance
// considerations", split-K over the sequence).
//
// How, on gfx950: one wave per (sequence, KV head, partition); a workgroup holds
// up to four waves (four KV heads) of the same sequence and partition and
// stages that partition's block-table entries in LDS once.  A tile is 16
// logical tokens.
//   * q.K^T: v_mfma_f32_16x16x32_bf16 with A = the K tile (row m = token) and
//     B = q^T (column n = query head of the group).  Lane (m, k-group) of A is
//     exactly a 16-byte slice of one K row, so K goes from HBM to the matrix
//     core with no shuffles.  The sum over d may visit d in any order as long as
//     q is read in the same order; the e4m3 path uses that freedom to load 16
//     contiguous bytes per lane.
//   * The result leaves lane (g, k-group) holding the logits of query head g for
//     tokens 4*k-group .. +3, which is exactly the A-operand layout of
//     v_mfma_f32_16x16x16_bf16 for P.V with k = token, so the probabilities feed
//     the second product in place.  V rows arrive as 16-byte row slices and are
//     re-paired (v_perm_b32) into token-major B operands.
//   * Softmax is two-pass within the partition: all logits first (kept in
//     registers), then one max and one sum, then P.V.  Reduction order depends
//     only on logical token positions, so results are bitwise identical under
//     any block size or physical placement.
// Tokens past the context are clamped to the last valid row for addressing (no
// stray or out-of-range reads, never a table entry past the context) and given
// probability 0.
#include "launch.hpp"
#include "mfma_tiles.hpp"

#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 3   // K or V tiles in flight per wave
#endif
#ifndef PA_NT_LOADS
#define PA_NT_LOADS 0     // 1: K/V tiles loaded with the non-temporal hint (read-once data)
#endif
#ifndef PA_MIN_WAVES_PER_EU
#define PA_MIN_WAVES_PER_EU 1
#endif
#ifndef PA_WG_THREADS
#define PA_WG_THREADS 256
#endif

namespace pa {

template <bool FP8, int D, int PT>
__global__ __launch_bounds__(PA_WG_THREADS) __attribute__((amdgpu_waves_per_eu(PA_MIN_WAVES_PER_EU, 8)))
void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int P = 16 * PT;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int VEC = D / 16;
  constexpr int NKK = D / 32;
  constexpr int DEPTH = PA_MFMA_DEPTH;
  constexpr int KD = PT < DEPTH ? PT : DEPTH;
  __shared__ int32_t tbl[P];

  const int hg = blockIdx.x % a.head_groups;
  int b, part, ctx;
  if (a.dense) {
    // workgroup x / head_groups is the x-th existing (sequence, partition) pair;
    // the grid's surplus workgroups come last and leave at once
    if (!locate_partition(a.context_lens, a.num_seqs, P, blockIdx.x / a.head_groups, b, part, ctx)) return;
  } else {
    b = blockIdx.y;
    part = blockIdx.x / a.head_groups;
    ctx = a.context_lens[b];
    if (part * P >= ctx && !(part == 0 && ctx == 0)) return;
  }
  const int t0 = part * P;          // same for the whole workgroup

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kvh = hg * a.heads_per_wg + wave;
  const int G = a.group;
  const int hq0 = kvh * G;
  const int n = lane & 15;
  const int q4 = lane >> 4;
  uint16_t* out = static_cast<uint16_t*>(a.out);

  if (ctx == 0) {                                                // empty context: zeros
    uint16_t* o = out + ((int64_t)b * a.num_q_heads + hq0) * D;
    for (int i = lane; i < G * D / 8; i += kWave) st16(o + 8 * i, u32x4{0u, 0u, 0u, 0u});
    return;
  }

  const int n_tok = min(P, ctx - t0);
  const int lb0 = t0 >> a.log2_bs;
  const int n_ent = ((t0 + n_tok - 1) >> a.log2_bs) - lb0 + 1;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.bt_stride + lb0;
  for (int i = threadIdx.x; i < n_ent; i += blockDim.x) tbl[i] = bt_row[i];
  __syncthreads();

  const int64_t head_off = (int64_t)kvh * D * ESZ;
  const uint8_t* kbase = a.k_cache + head_off;
  const uint8_t* vbase = a.v_cache + head_off;
  const int bs_mask = a.block_size - 1;
  const int log2bs = a.log2_bs;
  const int64_t block_bytes = a.block_bytes, row_bytes = a.row_bytes;
  auto row_off = [&](int t) -> int64_t {
    const int tc = min(t, ctx - 1);
    const int blk = tbl[(tc >> log2bs) - lb0];
    return (int64_t)blk * block_bytes + (int64_t)(tc & bs_mask) * row_bytes;
  };

  // q^T as the B operand of q.K^T: lane (n = query head in group, q4) holds 8 d's per MFMA
  bf16x8 qB[NKK];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + hq0 + n) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (n < G) w = ld16(qrow + q_col<FP8, D>(kk, q4));
      qB[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  auto load_k = [&](int i) {
    KTile<FP8, D> t;
    const uint8_t* p = kbase + row_off(t0 + 16 * i + n) + 16 * q4;
#pragma unroll
    for (int j = 0; j < KTile<FP8, D>::N; ++j) {
      if constexpr (PA_NT_LOADS) t.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 64 * j));
      else t.w[j] = ld16(p + 64 * j);
    }
    return t;
  };
  auto load_v = [&](int i) {
    VTile<FP8, D> t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* p = vbase + row_off(t0 + 16 * i + 4 * q4 + j) + n * VEC * ESZ;
      if constexpr (PA_NT_LOADS) t.w[j] = __builtin_nontemporal_load(reinterpret_cast<const typename VTile<FP8, D>::W*>(p));
      else t.w[j] = *reinterpret_cast<const typename VTile<FP8, D>::W*>(p);
    }
    return t;
  };

  // ---- phase 1: logits of all tiles (base 2, masked) ----------------------------
  float S[PT][4];
  KTile<FP8, D> kt[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) kt[i] = load_k(i);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const KTile<FP8, D> cur = kt[i % KD];
    if (i + KD < PT) kt[i % KD] = load_k(i + KD);
    const f32x4 s = qk_tile<FP8, D>(cur, qB);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = t0 + 16 * i + 4 * q4 + r;
      S[i][r] = tok < ctx ? s[r] * a.qk_scale : -INFINITY;
    }
  }

  // first V tiles in flight while the softmax runs
  VTile<FP8, D> vt[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) vt[i] = load_v(i);

  // ---- softmax over the partition --------------------------------------------
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[i][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  uint32_t Pk[PT][2];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // probabilities enter P.V as bf16; the denominator sums the same rounded values
      p[r] = (float)(__bf16)__builtin_amdgcn_exp2f(S[i][r] - mx);
      lsum += p[r];
    }
    Pk[i][0] = pack_bf16(p[0], p[1]);
    Pk[i][1] = pack_bf16(p[2], p[3]);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // ---- phase 2: P.V -------------------------------------------------------------
  f32x4 O[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) O[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const VTile<FP8, D> cur = vt[i % KD];
    if (i + KD < PT) vt[i % KD] = load_v(i + KD);
    pv_tile<FP8, D>(cur, Pk[i][0], Pk[i][1], O);
  }

  // ---- write: lane (n, q4) register r holds O[g = 4*q4 + r][d = VEC*n + e] --------
  const bool single = ctx <= P;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * q4 + r;
    const float lg = __shfl(lsum, g & 15);
    if (g < G) {
      const int64_t hrow = (int64_t)b * a.num_q_heads + hq0 + g;
      if (single) {
        const float inv = a.v_scale / lg;
        uint32_t w[VEC / 2];
#pragma unroll
        for (int c = 0; c < VEC / 2; ++c) w[c] = pack_bf16(O[2 * c][r] * inv, O[2 * c + 1][r] * inv);
        uint16_t* o = out + hrow * D + n * VEC;
        if constexpr (VEC == 8) st16(o, u32x4{w[0], w[1], w[2], w[3]});
        else st8(o, u32x2{w[0], w[1]});
      } else {
        float* o = a.ws_o + (hrow * a.max_parts + part) * D + n * VEC;
        if constexpr (VEC == 8) {
          st16(o, __builtin_bit_cast(u32x4, f32x4{O[0][r], O[1][r], O[2][r], O[3][r]} * a.v_scale));
          st16(o + 4, __builtin_bit_cast(u32x4, f32x4{O[4][r], O[5][r], O[6][r], O[7][r]} * a.v_scale));
        } else {
          st16(o, __builtin_bit_cast(u32x4, f32x4{O[0][r], O[1][r], O[2][r], O[3][r]} * a.v_scale));
        }
      }
    }
  }
  if (!single && q4 == 0 && n < G) {
    const int64_t idx = ((int64_t)b * a.num_q_heads + hq0 + n) * a.max_parts + part;
    a.ws_m[idx] = mx;
    a.ws_l[idx] = lsum;
  }
}

template <bool FP8, int D>
static hipError_t launch_pt(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  switch (a.partition_tokens) {
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<FP8, D, 1>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_mfma_kernel<FP8, D, 2>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((decode_mfma_kernel<FP8, D, 4>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((decode_mfma_kernel<FP8, D, 8>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((decode_mfma_kernel<FP8, D, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = a.dense ? dim3((unsigned)(a.max_parts * a.head_groups * a.num_seqs), 1u)
                           : dim3((unsigned)(a.max_parts * a.head_groups), (unsigned)a.num_seqs);
  const dim3 block((unsigned)(kWave * a.heads_per_wg));
  const bool fp8 = a.kv_fmt == kE4m3;
  if (a.head_dim == 128) return fp8 ? launch_pt<true, 128>(a, grid, block, s) : launch_pt<false, 128>(a, grid, block, s);
  return fp8 ? launch_pt<true, 64>(a, grid, block, s) : launch_pt<false, 64>(a, grid, block, s);
}

}  // namespace pa
