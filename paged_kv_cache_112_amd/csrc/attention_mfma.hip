// Multi-query paged attention (chunked prefill, or several new tokens per sequence),
// matrix-core path with K/V tiles held in registers: bf16 q with a bf16, e4m3 or int8
// pool.  It serves the shapes the LDS-sharing kernel (attention_lds.hip) does not:
// head_dim 64, and blocks of fewer than 16 tokens.
//
// What is computed: request i's new tokens are q[qsl[i] .. qsl[i+1]), the last
// n_i = qsl[i+1] - qsl[i] positions of its context of S_i = seq_lens[i] tokens; new
// token j sits at position S_i - n_i + j and attends causally to positions 0 .. that
// position:  out = softmax(scale * q . K^T + causal mask) V, with K and V gathered
// through the request's block table and GQA query head h reading KV head h / G
// (ai-infra-handbooks "Paged KV cache", section "Paged attention": the inputs
// block_tables, seq_lens and query_start_loc, the lower-triangular mask offset by
// S - n, and the statement that the math equals contiguous attention).
//
// How, on gfx950: one wave per (request, KV head, run of NQ query groups), requests
// taken longest first.  A query
// group is T = 16 / G new tokens with all G query heads of the KV head: the 16
// columns of one MFMA operand, (token, head) pairs, so the product is dense.  Each
// K/V tile a wave loads (and, for one-byte pools, widens) serves all NQ groups.  The
// four waves of a workgroup take consecutive runs of the same KV head, so a tile one
// of them fetches is found in the CU's cache by the others.
//   * Keys advance 32 per step, as two 16-key tiles a and b.
//   * q.K^T: v_mfma_f32_16x16x32_bf16 with A = a 16-key tile (row = key), B = q^T.
//   * P.V is the transposed product O^T = V^T P^T, on v_mfma_f32_16x16x32_bf16 over
//     the step's 32 keys: k-slot 8*q4 + j is key 4*q4 + j of tile a (j < 4) or key
//     4*q4 + j - 4 of tile b, which is where q.K^T left each lane's probabilities, so
//     they become the B operand without moving between lanes.  The output keeps each
//     column's values in that column's own lanes, so rescaling is lane-local.
//   * Softmax runs online in base 2 with a lazy reference: a column's running max m
//     is raised only when a step's max exceeds it by more than kRescaleLog2, so the
//     probabilities exp2(x - m) stay below 2^kRescaleLog2 and the output and sum are
//     rescaled only on those (rare, wave-uniform) steps.  Numerator and denominator
//     use the same reference, so the quotient is the softmax.
//   * Steps wholly below the causal limit of every column of the wave skip the mask.
// Rows past the context are clamped to the last valid row for addressing.
#include "attention_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace pa {

constexpr int kAttnWaves = 4;          // query runs (waves) per workgroup
constexpr float kRescaleLog2 = 8.0f;   // lazy-rescale threshold, in log2 units

// Element e (0 .. 2*NW-1) of a row of NW packed bf16 pairs, for rows lo and hi, packed
// into one pair.
template <int NW>
__device__ __forceinline__ uint32_t pair_of(const uint32_t (&lo)[NW], const uint32_t (&hi)[NW], int e) {
  return (e & 1) ? pack_hi_halves(lo[e >> 1], hi[e >> 1]) : pack_lo_halves(lo[e >> 1], hi[e >> 1]);
}

template <int KF, int D, bool BIGBS, int NQ>
__global__ __launch_bounds__(256) void attention_mfma_kernel(const AttnArgs a) {
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;
  constexpr int VEC = D / 16;
  constexpr int NKK = D / 32;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = request_of_rank(a.seq_lens, a.num_seqs, blockIdx.y);
  const int q0 = attn_load_uniform(a.query_start_loc + i);
  const int nq = attn_load_uniform(a.query_start_loc + i + 1) - q0;
  const int S = attn_load_uniform(a.seq_lens + i);
  const int T = 16 >> a.log2_group;                 // query tokens per group
  const int t0 = ((blockIdx.x / a.num_kv_heads) * kAttnWaves + wave) * (NQ * T);
  // past this request's queries, or inconsistent lengths (uniform per wave; no barrier follows)
  if (t0 >= nq || nq > S || q0 < 0 || q0 + nq > a.num_tokens) return;
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
  const int tn = n >> a.log2_group;                 // token offset within a group
  const int base = S - nq;                          // context position of new token 0
  const int kend = base + min(t0 + NQ * T, nq);     // keys [0, kend) cover every column
  const int nst = (kend + 31) >> 5;
  const int nfull = (base + t0 + 1) >> 5;           // steps every column sees whole
  // The scale enters as sc > 0: a negative scale is a sign flip of q (exact) and a zero
  // scale is q = 0 with sc = 1 (every score 0), so maxima of raw scores order the
  // scaled ones and a masked score of -inf gives exactly 0.
  const float sc = a.qk_scale == 0.f ? 1.f : fabsf(a.qk_scale);
  const uint32_t qflip = a.qk_scale < 0.f ? 0x80008000u : 0u;
  const bool qzero = a.qk_scale == 0.f;

  // q^T as B operands, kept in registers: group c, lane (n, q4) holds 8 d's of (token
  // t0 + c*T + tn, head g)
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
      if (tq < nq && !qzero) w = ld16(qrow + q_col<KF, D>(kk, q4)) ^ qflip;
      qreg[c][kk] = __builtin_bit_cast(bf16x8, w);
      // q is only ever a matrix-core operand, which may come from the accumulation
      // registers: kept there, it leaves the ordinary registers to the V tiles, which the
      // vector unit re-pairs (otherwise they land in accumulation registers and are copied
      // back at every step).  4-9 % faster.
      asm volatile("" : "+a"(qreg[c][kk]));
    }
  }

  const int32_t* bt_row = a.block_tables + (int64_t)i * a.bt_stride;
  const int64_t head_off = (int64_t)kvh * D * ESZ;
  const uint8_t* kbase = a.k_cache + head_off;
  const uint8_t* vbase = a.v_cache + head_off;
  const int bs_mask = a.block_size - 1;
  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  // per-lane byte offsets within a 16-key tile: K row n; V rows 4*q4 + j
  const uint32_t k_lane = (uint32_t)n * row_bytes + 16 * q4;
  uint32_t v_lane[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v_lane[j] = (uint32_t)(4 * q4 + j) * row_bytes + n * VEC * ESZ;

  // Address of tile `tile`'s key 16*tile + r plus `lane_bytes`, key clamped to the context.
  auto row_ptr = [&](const uint8_t* base, int r, int tile, uint32_t lane_bytes) -> const uint8_t* {
    const int tc = min(16 * tile + r, S - 1);
    if constexpr (BIGBS) {
      const int32_t blk = checked_block(attn_load_uniform(bt_row + (min(16 * tile, S - 1) >> a.log2_bs)), a.num_blocks, a.err);
      return base + (int64_t)blk * a.block_bytes + (size_t)((uint32_t)(tc & bs_mask) * row_bytes + lane_bytes);
    } else {
      const int32_t blk = checked_block(bt_row[tc >> a.log2_bs], a.num_blocks, a.err);
      return base + (int64_t)blk * a.block_bytes + (size_t)((uint32_t)(tc & bs_mask) * row_bytes + lane_bytes);
    }
  };
  // K or V tiles of step st (keys 32*st .. 32*st + 31).  With blocks of 16 tokens or
  // more, a step inside the context has each of its two tiles in one block at a uniform
  // offset, the same for K and V: scalar base plus the per-lane constant offsets.
  // The block ids of a step are read one step before its addresses are formed (at the
  // end of the step before that), so the scalar loads are not waited on.
  struct StepAddr {
    int64_t off[2];
    bool fast;
  };
  auto step_fast = [&](int st) { return __builtin_expect(BIGBS && 32 * st + 32 <= S, 1); };
  auto load_ids = [&](int st, int32_t (&id)[2]) {
    if (step_fast(st)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        id[h] = checked_block(attn_load_uniform(bt_row + ((32 * st + 16 * h) >> a.log2_bs)), a.num_blocks, a.err);
    }
  };
  auto step_addr = [&](int st, const int32_t (&id)[2]) {
    StepAddr t;
    t.fast = step_fast(st);
    if (t.fast) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        t.off[h] = (int64_t)id[h] * a.block_bytes + (int64_t)((uint32_t)((32 * st + 16 * h) & bs_mask) * row_bytes);
    }
    return t;
  };
  auto load_k = [&](KTile<KF, D> (&k)[2], int st, const StepAddr& t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tile = 2 * st + h;
      const uint8_t* pk = t.fast ? kbase + t.off[h] + k_lane : row_ptr(kbase, n, tile, 16 * q4);
#pragma unroll
      for (int j = 0; j < KTile<KF, D>::N; ++j) k[h].w[j] = ld16(pk + 64 * j);
    }
  };
  auto load_v = [&](VTile<KF, D> (&v)[2], int st, const StepAddr& t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tile = 2 * st + h;
      if (t.fast) {
        const uint8_t* vb = vbase + t.off[h];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[h].w[j] = *reinterpret_cast<const typename VTile<KF, D>::W*>(vb + v_lane[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint8_t* pv = row_ptr(vbase, 4 * q4 + j, tile, n * VEC * ESZ);
          v[h].w[j] = *reinterpret_cast<const typename VTile<KF, D>::W*>(pv);
        }
      }
    }
  };

  f32x4 O[NQ][VEC];
  f32x4 L[NQ];        // column sums of the probabilities (every register the same)
  float m[NQ];        // reference max per column, scaled log2 domain
  float thr[NQ];      // raw score above which the reference must be raised
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    L[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = -INFINITY;
    thr[c] = -INFINITY;
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const float inv_sc = 1.f / sc;
  // q.K^T and the softmax of step st for every group: the probabilities as B operands
  auto scores = [&](auto masked_tag, const KTile<KF, D> (&kt)[2], int st, bf16x8 (&pB)[NQ]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // K operands, widened once for every group
    bf16x8 kop[2][NKK];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (!byte_fmt(KF)) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kop[h][kk] = __builtin_bit_cast(bf16x8, kt[h].w[kk]);
      } else {
#pragma unroll
        for (int j = 0; j < KTile<KF, D>::N; ++j) {
          kop[h][2 * j] = bytes8_to_bf16x8<KF>(kt[h].w[j][0], kt[h].w[j][1]);
          kop[h][2 * j + 1] = bytes8_to_bf16x8<KF>(kt[h].w[j][2], kt[h].w[j][3]);
        }
      }
    }
    // q.K^T of group c: s[h] register r = score of key 32*st + 16*h + 4*q4 + r, column n
    auto qk = [&](int c, f32x4 (&s)[2]) {
      s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 qb = qreg[c][kk];
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][kk], qb, s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][kk], qb, s[1], 0, 0, 0);
      }
    };
    // group by group: the next group's q.K^T is issued before this group's softmax, so
    // the matrix core works while the vector unit does the softmax
    f32x4 sn[2];
    qk(0, sn);
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      f32x4 s[2] = {sn[0], sn[1]};
      if (c + 1 < NQ) qk(c + 1, sn);
      if constexpr (MASKED) {
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
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {   // uniform, rare: raise the references
        const float v = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                              fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        const float mn = fmaxf(m[c], col_max(v) * sc);
        const float mref = mn == -INFINITY ? 0.f : mn;   // a column with no visible key yet
        const float alpha = __builtin_amdgcn_exp2f(m[c] - mref);
        m[c] = mref;
        thr[c] = (mref + kRescaleLog2) * inv_sc;
        L[c] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) O[c][e] *= alpha;
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
  };
  // O += P.V of one step for every group
  auto accumulate = [&](const VTile<KF, D> (&vt)[2], const bf16x8 (&pB)[NQ]) {
    // V rows as bf16 pairs: rw[h][j][w] = columns 2w, 2w+1 of row 4*q4 + j of tile h
    constexpr int NW = VEC / 2;
    uint32_t rw[2][4][NW];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (!byte_fmt(KF)) {
#pragma unroll
          for (int w = 0; w < NW; ++w) rw[h][j][w] = vt[h].w[j][w];
        } else if constexpr (VEC == 8) {
          rw[h][j][0] = bytes2_to_bf16x2<KF, false>(vt[h].w[j][0]);
          rw[h][j][1] = bytes2_to_bf16x2<KF, true>(vt[h].w[j][0]);
          rw[h][j][2] = bytes2_to_bf16x2<KF, false>(vt[h].w[j][1]);
          rw[h][j][3] = bytes2_to_bf16x2<KF, true>(vt[h].w[j][1]);
        } else {
          rw[h][j][0] = bytes2_to_bf16x2<KF, false>(vt[h].w[j]);
          rw[h][j][1] = bytes2_to_bf16x2<KF, true>(vt[h].w[j]);
        }
      }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      // A = V^T block e: row m = head-dimension index VEC*m + e, k-slots as pB
      const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{pair_of<NW>(rw[0][0], rw[0][1], e), pair_of<NW>(rw[0][2], rw[0][3], e),
                                                        pair_of<NW>(rw[1][0], rw[1][1], e), pair_of<NW>(rw[1][2], rw[1][3], e)});
#pragma unroll
      for (int c = 0; c < NQ; ++c) O[c][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pB[c], O[c][e], 0, 0, 0);
    }
  };

  // One K and one V buffer: the next step's K is requested as soon as q.K^T has read
  // the current one, and its V as soon as P.V has; the step after the last loads
  // clamped rows.  Steps that every column sees whole run without the mask.
  KTile<KF, D> k[2];
  VTile<KF, D> v[2];
  int32_t ids[2] = {0, 0};   // block ids of the tiles of the next step
  auto step = [&](auto masked_tag, int st) {
    const StepAddr next = step_addr(st + 1, ids);
    bf16x8 pB[NQ];
    scores(masked_tag, k, st, pB);
    load_k(k, st + 1, next);
    accumulate(v, pB);
    load_v(v, st + 1, next);
    load_ids(st + 2, ids);
  };
  {
    int32_t id0[2] = {0, 0};
    load_ids(0, id0);
    const StepAddr first = step_addr(0, id0);
    load_k(k, 0, first);
    load_v(v, 0, first);
    load_ids(1, ids);
  }
  int st = 0;
  for (; st < nfull; ++st) step(std::false_type{}, st);
  for (; st < nst; ++st) step(std::true_type{}, st);

  // lane (n, q4) register r of O[c][e] holds group c column n at d = VEC*(4*q4 + r) + e
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const int tq = t0 + c * T + tn;
    if (tq < nq) {
      const float inv = a.v_scale / L[c][0];
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + tq) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t w[VEC / 2];
#pragma unroll
        for (int x = 0; x < VEC / 2; ++x) w[x] = cvt_bf16x2(O[c][2 * x][r] * inv, O[c][2 * x + 1][r] * inv);
        uint16_t* dst = o + VEC * (4 * q4 + r);
        if constexpr (VEC == 8) st16(dst, u32x4{w[0], w[1], w[2], w[3]});
        else st8(dst, u32x2{w[0], w[1]});
      }
    }
  }
}

// query groups per wave
#ifndef PA_ATTN_NQ
#define PA_ATTN_NQ 4
#endif
constexpr int kAttnNq = PA_ATTN_NQ;

template <int KF, int D>
static void launch_d(const AttnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.block_size >= 16) hipLaunchKernelGGL((attention_mfma_kernel<KF, D, true, kAttnNq>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attention_mfma_kernel<KF, D, false, kAttnNq>), grid, block, 0, s, a);
}

int attention_tokens_per_workgroup(int log2_group) { return kAttnWaves * kAttnNq * (16 >> log2_group); }

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s) {
  const int per_wg = attention_tokens_per_workgroup(a.log2_group);
  const int wgs = (a.max_query_len + per_wg - 1) / per_wg;
  const dim3 grid((unsigned)(wgs * a.num_kv_heads), (unsigned)a.num_seqs);
  const dim3 block((unsigned)(kWave * kAttnWaves));
  const bool d128 = a.head_dim == 128;
  switch (a.kv_fmt) {
    case kBf16: d128 ? launch_d<kFmtBf16, 128>(a, grid, block, s) : launch_d<kFmtBf16, 64>(a, grid, block, s); break;
    case kE4m3: d128 ? launch_d<kFmtE4m3, 128>(a, grid, block, s) : launch_d<kFmtE4m3, 64>(a, grid, block, s); break;
    case kInt8: d128 ? launch_d<kFmtInt8, 128>(a, grid, block, s) : launch_d<kFmtInt8, 64>(a, grid, block, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
