// Multi-query paged attention (chunked prefill, or several new tokens per sequence),
// matrix-core path with the K/V tiles shared through LDS: bf16 q on a bf16, e4m3 or
// int8 pool, head_dim 128, blocks of 16 tokens or more.
//
// What is computed is what attention_mfma.hip computes: request i's n_i new tokens are
// the last positions of its context of S_i tokens, new token j attends causally to
// positions 0 .. S_i - n_i + j, out = softmax(scale * q . K^T + causal mask) V with K
// and V gathered through the block table and query head h reading KV head h / G
// (ai-infra-handbooks "Paged KV cache", section "Paged attention").
//
// How, on gfx950: a workgroup of eight waves, two per SIMD, takes one (request, KV
// head) and 8 * NQ query groups of it (a group is 16 / G new tokens with all G query
// heads of the KV head: the 16 columns of one MFMA operand).  Keys advance 32 per step.
// Each step's K and V rows (2 x 8 KiB) are fetched once for the workgroup: every
// thread loads one 16-byte segment of K and one of V two steps ahead into registers
// (two staging sets, even and odd steps) and stores them to a ring of four LDS tiles;
// the waves compute two steps between barriers and store the next two at the end of
// the pair, so a wave holds no K or V beyond the operands of one product, two waves fit
// on each SIMD, and the workgroup meets once per 64 keys.
// One-byte pools (e4m3, int8) are widened to bf16 exactly as the rows go to LDS (every
// e4m3 and int8 value is a bf16 value; the pool's scales are applied to the scores and
// the output), so each element is widened once per workgroup and everything after the
// store is the bf16 kernel.
//   * q.K^T: v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 head dimensions read from LDS
//     (ds_read_b128; a row's 16-byte segments are XOR-swizzled with the row so the 16
//     rows of an operand hit distinct banks), B = q^T held in registers.
//   * P.V: O^T = V^T P^T on the same instruction over the step's 32 keys, A = V^T.
//     gfx950's transposing LDS read (ds_read_b64_tr_b16) gives each lane four keys of
//     one head dimension from four row-major V rows, which is exactly the A operand:
//     within 16 lanes, lane l receives element l % 4 of the rows addressed by lanes
//     l / 4 + 4j, j = 0..3.  Lane (m, q4) gets keys 4*q4 .. 4*q4 + 3 of each 16-key
//     tile at head dimension 16e + m, the k-slots in which q.K^T left the
//     probabilities (8*q4 + j: tile a for j < 4, tile b beyond), so they feed the
//     product without moving.  V rows are swizzled in 32-byte chunks.
//   * Softmax as in attention_mfma.hip: online, base 2, with a lazy reference raised
//     only when a score passes it by 2^kRescaleLog2; steps wholly below every
//     column's causal limit skip the mask.
// Rows past the context are clamped to the last valid row for addressing.
#include "attention_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace pa {

constexpr int kLdsWaves = 8;            // waves per workgroup (two per SIMD)
constexpr float kLdsRescaleLog2 = 8.0f;

// ds_read_b64_tr_b16 at byte offset `off` of an LDS array.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* lds, uint32_t off) {
  const auto p = (__attribute__((address_space(3))) bf16x4*)(const_cast<uint8_t*>(lds) + off);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p));
}

template <int KF, int NQ>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_lds_kernel(const AttnArgs a) {
  constexpr int D = 128;
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;   // pool bytes per element
  constexpr int NKK = D / 32;        // 32-dimension slices of q.K^T
  constexpr int NE = D / 16;         // 16-dimension blocks of P.V
  constexpr int ROWB = D * 2;        // bytes of one key row of one KV head
  constexpr int TILEB = 32 * ROWB;   // one step's K (or V) rows
  __shared__ __attribute__((aligned(16))) uint8_t lk[4][TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t lv[4][TILEB];

  const int kvh = blockIdx.x % a.num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = request_of_rank(a.seq_lens, a.num_seqs, blockIdx.y);
  const int q0 = attn_load_uniform(a.query_start_loc + i);
  const int nq = attn_load_uniform(a.query_start_loc + i + 1) - q0;
  const int S = attn_load_uniform(a.seq_lens + i);
  const int T = 16 >> a.log2_group;                 // query tokens per group
  const int per_wg = kLdsWaves * NQ * T;
  const int t0w = (blockIdx.x / a.num_kv_heads) * per_wg;
  // past this request's queries, or inconsistent lengths: uniform over the workgroup
  if (t0w >= nq || nq > S || q0 < 0 || q0 + nq > a.num_tokens) return;
  if constexpr (kChecked) {                // a context past its table: reported, the request skipped
    if ((int64_t)S > (int64_t)a.bt_stride * a.block_size) {
      flag_error(a.err, kErrLength);
      return;
    }
  }

  const int lane = threadIdx.x & 63;
  const int G = 1 << a.log2_group;
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int g = n & (G - 1);
  const int tn = n >> a.log2_group;
  const int base = S - nq;                           // context position of new token 0
  const int t0 = t0w + wave * NQ * T;                // this wave's first new token
  const int nst_wg = (base + min(t0w + per_wg, nq) + 31) >> 5;
  const float sc = a.qk_scale == 0.f ? 1.f : fabsf(a.qk_scale);
  const uint32_t qflip = a.qk_scale < 0.f ? 0x80008000u : 0u;
  const bool qzero = a.qk_scale == 0.f;

  int qpos[NQ];
  bf16x8 qreg[NQ][NKK];
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const int tq = t0 + c * T + tn;
    qpos[c] = base + tq;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + min(tq, nq - 1)) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (tq < nq && !qzero) w = ld16(qrow + 32 * kk + 8 * q4) ^ qflip;
      qreg[c][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- cooperative staging: thread (key, segment) of the step's 32 rows ----------
  const int32_t* bt_row = a.block_tables + (int64_t)i * a.bt_stride;
  const uint8_t* kbase = a.k_cache + (int64_t)kvh * D * ESZ;
  const uint8_t* vbase = a.v_cache + (int64_t)kvh * D * ESZ;
  const int bs_mask = a.block_size - 1;
  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  const int skey = threadIdx.x >> 4, sseg = threadIdx.x & 15;
  const uint32_t k_st = skey * ROWB + ((sseg ^ (skey & 15)) << 4);
  const uint32_t v_st = skey * ROWB + ((((sseg >> 1) ^ (skey & 7)) << 5) | ((sseg & 1) << 4));
  // ---- per-wave state ----------------------------------------------------------
  f32x4 O[NQ][NE];
  f32x4 L[NQ];
  float m[NQ], thr[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
#pragma unroll
    for (int e = 0; e < NE; ++e) O[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    L[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = -INFINITY;
    thr[c] = -INFINITY;
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const float inv_sc = 1.f / sc;
  const int trk = 4 * q4 + (n >> 2);        // key of this lane's transposing-read row
  const bool active = t0 < nq;               // uniform per wave
  const int nst = active ? (base + min(t0 + NQ * T, nq) + 31) >> 5 : 0;   // this wave's steps
  const int nfull = active ? (base + t0 + 1) >> 5 : 0;   // steps every column of the wave sees whole
  // One step for every query group of the wave: q.K^T (K from LDS tile `buf`), the causal
  // mask on the steps that reach past a column's position, the online softmax and
  // O += P.V (V from the same tile).  Masked and unmasked steps share this one body, the
  // mask being a uniform branch around the comparisons alone: with a copy of the body per
  // case the compiler moved the accumulators to other registers on one path and copied
  // them back at every step.
  auto compute = [&](int st, int buf) {
    const uint8_t* kt = lk[buf];
    const uint8_t* vt = lv[buf];
    bf16x8 kop[2][NKK];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kop[h][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + (16 * h + n) * ROWB + (((4 * kk + q4) ^ n) << 4)));
    bf16x8 pB[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][kk], qreg[c][kk], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][kk], qreg[c][kk], s[1], 0, 0, 0);
      }
      if (st >= nfull) {                          // uniform: a step on the causal diagonal
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (32 * st + 16 * h + 4 * q4 + r > qpos[c]) s[h][r] = -INFINITY;
      }
      bool grow = false;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) grow |= s[h][r] > thr[c];
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {   // uniform, rare
        const float v = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                              fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        const float mn = fmaxf(m[c], col_max(v) * sc);
        const float mref = mn == -INFINITY ? 0.f : mn;   // a column with no visible key yet
        const float alpha = __builtin_amdgcn_exp2f(m[c] - mref);
        m[c] = mref;
        thr[c] = (mref + kLdsRescaleLog2) * inv_sc;
        L[c] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) O[c][e] *= alpha;
      }
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[h][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][r], sc, -m[c]));
      pB[c] = __builtin_bit_cast(bf16x8, u32x4{cvt_bf16x2(p[0][0], p[0][1]), cvt_bf16x2(p[0][2], p[0][3]),
                                               cvt_bf16x2(p[1][0], p[1][1]), cvt_bf16x2(p[1][2], p[1][3])});
      L[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pB[c], L[c], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      u32x2 x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 16 * h + trk;
        x[h] = lds_read_tr16(vt, key * ROWB + ((e ^ (key & 7)) << 5) + ((n & 3) << 3));
      }
      const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{x[0][0], x[0][1], x[1][0], x[1][1]});
#pragma unroll
      for (int c = 0; c < NQ; ++c) O[c][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pB[c], O[c][e], 0, 0, 0);
    }
  };
  // ---- staging ----------------------------------------------------------------
  // Set 0 holds the even steps' segments, set 1 the odd ones'.  idn: block ids of the
  // next step to request.  Each 16-key tile lies in one block; a tile past the context
  // takes the block of its last row, and rows clamp to the context.
  // a segment is 8 elements of one row: 16 bytes of a bf16 pool, 8 of a one-byte pool
  typedef typename std::conditional<byte_fmt(KF), u32x2, u32x4>::type Seg;
  Seg rk0, rv0, rk1, rv1;
  int32_t idn[2];
  auto load_ids = [&](int st, int32_t (&id)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      id[h] = checked_block(attn_load_uniform(bt_row + (min(32 * st + 16 * h, S - 1) >> a.log2_bs)), a.num_blocks, a.err);
  };
  auto fetch2 = [&](int st, const int32_t (&id)[2], Seg& xk, Seg& xv) {
    const int tc = min(32 * st + skey, S - 1);
    const int32_t blk = (skey >> 4) ? id[1] : id[0];
    constexpr uint32_t SEGB = sizeof(Seg);
    const int64_t off = (int64_t)blk * a.block_bytes + (int64_t)((uint32_t)(tc & bs_mask) * row_bytes + SEGB * sseg);
    xk = *reinterpret_cast<const Seg*>(kbase + off);
    xv = *reinterpret_cast<const Seg*>(vbase + off);
  };
  // 8 elements as bf16 (one-byte formats widened exactly)
  auto widen = [&](const Seg& x) -> u32x4 {
    if constexpr (!byte_fmt(KF)) {
      return x;
    } else {
      return u32x4{bytes2_to_bf16x2<KF, false>(x[0]), bytes2_to_bf16x2<KF, true>(x[0]),
                   bytes2_to_bf16x2<KF, false>(x[1]), bytes2_to_bf16x2<KF, true>(x[1])};
    }
  };
  auto put2 = [&](int buf, const Seg& xk, const Seg& xv) {
    *reinterpret_cast<u32x4*>(&lk[buf][k_st]) = widen(xk);
    *reinterpret_cast<u32x4*>(&lv[buf][v_st]) = widen(xv);
  };
  {
    int32_t id[2];
    load_ids(0, id);
    fetch2(0, id, rk0, rv0);
    load_ids(1, id);
    fetch2(1, id, rk1, rv1);
    __builtin_amdgcn_sched_barrier(0);
    put2(0, rk0, rv0);
    load_ids(2, id);
    fetch2(2, id, rk0, rv0);
    // each set's loads stay in the order the loop keeps, so that a store waits only for
    // its own set
    __builtin_amdgcn_sched_barrier(0);
    put2(1, rk1, rv1);
    load_ids(3, id);
    fetch2(3, id, rk1, rv1);
    load_ids(4, idn);
  }
  __syncthreads();
  // Steps st and st + 1 compute from LDS tiles st % 4 and (st + 1) % 4 with no barrier
  // between them; then steps st + 2 and st + 3 go from the staging sets to the other two
  // tiles (last read before the previous barrier), the sets are refilled with steps st + 4
  // and st + 5, and the workgroup meets once.  The staging is unconditional, also for the
  // (at most seven) steps past the last: a fixed count of loads in flight lets each store
  // wait only for its own set.  The loop is unrolled by two pairs so that every tile index
  // is a constant.
  auto run = [&](int st, int buf) {
    if (st < nst) compute(st, buf);
  };
  for (int st = 0; st < nst_wg; st += 4) {
    run(st, 0);
    run(st + 1, 1);
    put2(2, rk0, rv0);
    fetch2(st + 4, idn, rk0, rv0);
    load_ids(st + 5, idn);
    put2(3, rk1, rv1);
    fetch2(st + 5, idn, rk1, rv1);
    load_ids(st + 6, idn);
    __syncthreads();
    run(st + 2, 2);
    run(st + 3, 3);
    put2(0, rk0, rv0);
    fetch2(st + 6, idn, rk0, rv0);
    load_ids(st + 7, idn);
    put2(1, rk1, rv1);
    fetch2(st + 7, idn, rk1, rv1);
    load_ids(st + 8, idn);
    __syncthreads();
  }
  if (!active) return;

  // lane (n, q4) register r of O[c][e] holds group c column n at dimension 16e + 4*q4 + r
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const int tq = t0 + c * T + tn;
    if (tq < nq) {
      const float inv = a.v_scale / L[c][0];
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + tq) * a.num_q_heads + kvh * G + g) * D + 4 * q4;
#pragma unroll
      for (int e = 0; e < NE; ++e)
        st8(o + 16 * e, u32x2{cvt_bf16x2(O[c][e][0] * inv, O[c][e][1] * inv), cvt_bf16x2(O[c][e][2] * inv, O[c][e][3] * inv)});
    }
  }
}

#ifndef PA_ATTN_LDS_NQ
#define PA_ATTN_LDS_NQ 2
#endif
constexpr int kLdsNq = PA_ATTN_LDS_NQ;

bool attention_lds_supported(const AttnArgs& a) {
  return (a.kv_fmt == kBf16 || a.kv_fmt == kE4m3 || a.kv_fmt == kInt8) && a.head_dim == 128 && a.block_size >= 16;
}

int attention_lds_tokens_per_workgroup(int log2_group) { return kLdsWaves * kLdsNq * (16 >> log2_group); }

hipError_t launch_attention_lds(const AttnArgs& a, hipStream_t s) {
  if (!attention_lds_supported(a)) return hipErrorInvalidValue;
  const int per_wg = attention_lds_tokens_per_workgroup(a.log2_group);
  const int wgs = (a.max_query_len + per_wg - 1) / per_wg;
  const dim3 grid((unsigned)(wgs * a.num_kv_heads), (unsigned)a.num_seqs);
  const dim3 block(kWave * kLdsWaves);
  switch (a.kv_fmt) {
    case kBf16: hipLaunchKernelGGL((attention_lds_kernel<kFmtBf16, kLdsNq>), grid, block, 0, s, a); break;
    case kE4m3: hipLaunchKernelGGL((attention_lds_kernel<kFmtE4m3, kLdsNq>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attention_lds_kernel<kFmtInt8, kLdsNq>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace pa
