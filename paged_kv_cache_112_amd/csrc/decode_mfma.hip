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
// How, on gfx950: a partition of P tokens belongs to W waves per KV head (W = 1 up
// to 256 tokens, P / 256 beyond), each taking every W-th 16-token tile; a
// workgroup holds up to four waves (KV heads x W) of one sequence and partition.
// With blocks of 16 tokens or more every tile lies in one block, whose id is a
// uniform scalar load; smaller blocks stage the partition's table entries in LDS.
//   * q.K^T: v_mfma_f32_16x16x32_bf16 with A = the K tile (row m = token) and
//     B = q^T (column n = a query head of the group).  Lane (m, k-group) of A is
//     exactly a 16-byte slice of one K row, so K goes from HBM to the matrix
//     core with no shuffles.  The sum over d may visit d in any order as long as
//     q is read in the same order; the e4m3 path uses that freedom to load 16
//     contiguous bytes per lane.
//   * The result leaves lane (column, k-group) holding that head's logits for
//     tokens 4*k-group .. +3, which is exactly the A-operand layout of
//     v_mfma_f32_16x16x16_bf16 for P.V with k = token, so the probabilities feed
//     the second product in place.  V rows arrive as 16-byte row slices and are
//     re-paired (v_perm_b32) into token-major B operands.
//   * Softmax is two-pass within a wave's tiles: all logits first (kept in
//     registers), then one max and one sum, then P.V.  The W waves of a head are
//     combined through LDS.  Reduction order depends only on logical token
//     positions, so results are bitwise identical under any block size or
//     physical placement.
// Tokens past the context are clamped to the last valid row for addressing (no
// stray or out-of-range reads, never a table entry past the context) and given
// probability 0.
// The appending instantiation (pa_decode_append) also stores this step's token: the
// workgroup whose partition holds position ctx - 1 writes the rows there first.
#include "launch.hpp"
#include "mfma_tiles.hpp"

// K or V tiles in flight per wave (bf16 and e4m3 pools; 6 measured best for both).
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 6
#endif
// The appending kernel (bf16 pools) keeps one tile less in flight: at 6 its register
// demand spills.
#ifndef PA_APPEND_DEPTH
#define PA_APPEND_DEPTH 5
#endif
#ifndef PA_MFMA_DEPTH_FP8
#define PA_MFMA_DEPTH_FP8 6
#endif
// Cache hints for the read-once K and V streams.  A V load instruction covers whole
// 128-byte lines (four rows x 256 bytes), so V is loaded non-temporally and does not
// push the partition pieces (written back later) out of the L2.  A K load
// instruction covers half of each line of 16 rows; the other half comes with the
// next instruction, so K keeps the default policy and the line stays for it.
#ifndef PA_NT_K
#define PA_NT_K 0
#endif
#ifndef PA_NT_V
#define PA_NT_V 1
#endif
#ifndef PA_MAX_WAVES_PER_EU
#define PA_MAX_WAVES_PER_EU 8
#endif
#ifndef PA_MIN_WAVES_PER_EU
#define PA_MIN_WAVES_PER_EU 1
#endif
#ifndef PA_WG_THREADS
#define PA_WG_THREADS 512
#endif

namespace pa {

// A uniform load through the scalar data cache (read only).
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// The appended token's K and V rows of KV head kvh, written at position pos in the
// pool's format: bf16 copied, e4m3 / int8 quantized exactly as pa_write_kv does (one
// fp32 multiply by 1/scale, then the rounding).  Lanes 0 .. D/8 - 1 take 8-element
// chunks of K, the next D/8 lanes those of V.
template <int KF, int D>
__device__ __forceinline__ void append_token(const DecodeArgs& a, int b, int kvh, int pos, int lane) {
  constexpr int CH = D / 8;
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;
  if (lane >= 2 * CH) return;
  const bool is_v = lane >= CH;
  const int c = is_v ? lane - CH : lane;
  const int32_t blk = checked_block(a.block_tables[(int64_t)b * a.bt_stride + (pos >> a.log2_bs)], a.num_blocks, a.err);
  const int64_t row = (int64_t)blk * a.block_size + (pos & (a.block_size - 1));
  const u32x4 x = ld16((is_v ? a.v_new : a.k_new) + ((int64_t)b * a.num_kv_heads + kvh) * D + 8 * c);
  uint8_t* dst = (is_v ? a.v_cache_w : a.k_cache_w) + row * a.row_bytes + (int64_t)(kvh * D + 8 * c) * ESZ;
  if constexpr (!byte_fmt(KF)) {
    st16(dst, x);
  } else {
    const float inv = is_v ? a.inv_v : a.inv_k;
    u32x2 o = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = ((i & 1) ? bf16hi(x[i >> 1]) : bf16lo(x[i >> 1])) * inv;
      const uint32_t code = KF == kFmtE4m3 ? f32_to_e4m3(y) : f32_to_i8(y);
      o[i >> 2] |= code << (8 * (i & 3));
    }
    st8(dst, o);
  }
}

// Query head g of the group sits in MFMA column n = 4 * (g % 4) + g / 4, so that
// after P.V lane (n, q4) register r holds head 4 * r + q4: with G <= 4 every lane
// of the wave holds one head's output in register 0.
__device__ __forceinline__ int head_of_column(int n) { return 4 * (n & 3) + (n >> 2); }

template <int KF, int D, int PT, bool BIGBS, bool APPEND>
__global__ __launch_bounds__(PA_WG_THREADS) __attribute__((amdgpu_waves_per_eu(PA_MIN_WAVES_PER_EU, PA_MAX_WAVES_PER_EU)))
void decode_mfma_kernel(const DecodeArgs a) {
  // A partition of P = 16 * PT * W tokens is shared by W waves per KV head: wave w
  // takes tiles w, w + W, w + 2W, ... (PT of them), and the W partial softmax pieces
  // are combined through LDS before anything is written.
  const int W = a.waves_per_head;
  const int P = 16 * PT * W;
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;
  constexpr int VEC = D / 16;
  constexpr int NKK = D / 32;
  constexpr int DEPTH = byte_fmt(KF) ? PA_MFMA_DEPTH_FP8 : (APPEND ? PA_APPEND_DEPTH : PA_MFMA_DEPTH);
  constexpr int KD = PT < DEPTH ? PT : DEPTH;
  __shared__ int32_t tbl[BIGBS ? 1 : kMaxPartitionTokens];
  extern __shared__ float xs[];     // combine area, W > 1 only

  const int hg = blockIdx.x % a.head_groups;
  int b, part, ctx;
  if (a.dense) {
    // workgroup x / head_groups is the x-th existing (sequence, partition) pair;
    // the grid's surplus workgroups come last and leave at once
    if (!locate_partition(a.context_lens, a.num_seqs, P, a.max_parts, blockIdx.x / a.head_groups, b, part, ctx)) return;
  } else {
    b = blockIdx.y;
    part = blockIdx.x / a.head_groups;
    ctx = a.context_lens[b];
    if (part * P >= ctx && !(part == 0 && ctx == 0)) return;
  }
  const int t0 = part * P;          // same for the whole workgroup
  if constexpr (kChecked) {
    // a context past its table would read entries beyond the row: reported and clipped
    if ((int64_t)ctx > (int64_t)a.max_parts * P) flag_error(a.err, kErrLength);
    const int64_t cap = (int64_t)a.bt_stride * a.block_size;
    if ((int64_t)ctx > cap) {
      flag_error(a.err, kErrLength);
      ctx = (int)cap;
      if (t0 >= ctx) return;                                     // uniform over the workgroup
    }
  }

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = wave % a.heads_per_wg;     // KV head within the workgroup
  const int w = wave / a.heads_per_wg;      // this wave's share of the partition
  const int kvh = hg * a.heads_per_wg + hl;
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

  // A token appended in this launch (position ctx - 1, at pa_write_kv's slot through
  // the block table) is stored by the workgroup whose partition holds it before any of
  // the partition's rows are read: the first wave of each KV head writes that head's
  // rows, every store completes, and the workgroup meets at a barrier.
  if constexpr (APPEND) {
    if (ctx <= t0 + P) {
      if (w == 0) append_token<KF, D>(a, b, kvh, ctx - 1, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  const int lb0 = t0 >> a.log2_bs;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.bt_stride + lb0;
  if constexpr (!BIGBS) {
    // blocks shorter than a tile: stage the partition's table entries in LDS
    const int n_tok = min(P, ctx - t0);
    const int n_ent = ((t0 + n_tok - 1) >> a.log2_bs) - lb0 + 1;
    for (int i = threadIdx.x; i < n_ent; i += blockDim.x) tbl[i] = checked_block(bt_row[i], a.num_blocks, a.err);
    __syncthreads();
  }

  const int64_t head_off = (int64_t)kvh * D * ESZ;
  const uint8_t* kbase = a.k_cache + head_off;
  const uint8_t* vbase = a.v_cache + head_off;
  const int bs_mask = a.block_size - 1;
  const int log2bs = a.log2_bs;
  const int64_t block_bytes = a.block_bytes, row_bytes = a.row_bytes;
  // Byte offset of token t (clamped to the last valid one) within the pool.  With
  // blocks of 16 tokens or more a tile lies in one block (tiles are 16-aligned), so
  // its block id is uniform and comes from the scalar cache; tiles past the context
  // clamp to the block of token ctx - 1.
  int32_t tile_blk[BIGBS ? PT : 1];
  if constexpr (BIGBS) {
#pragma unroll
    for (int i = 0; i < PT; ++i)
      tile_blk[i] = checked_block(load_uniform(bt_row + ((min(t0 + 16 * (i * W + w), ctx - 1) >> log2bs) - lb0)),
                                  a.num_blocks, a.err);
  }
  auto tile_block = [&](int i) -> int64_t { return (int64_t)tile_blk[i] * block_bytes; };
  auto row_off = [&](int t) -> int64_t {
    const int tc = min(t, ctx - 1);
    const int blk = tbl[(tc >> log2bs) - lb0];
    return (int64_t)blk * block_bytes + (int64_t)(tc & bs_mask) * row_bytes;
  };
  auto lane_row = [&](int t) -> int64_t { return (int64_t)(min(t, ctx - 1) & bs_mask) * row_bytes; };

  // q^T as the B operand of q.K^T: lane (n, q4) holds 8 d's of head head_of_column(n)
  bf16x8 qB[NKK];
  {
    const int g = head_of_column(n);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + hq0 + min(g, G - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (g < G) w = ld16(qrow + q_col<KF, D>(kk, q4));
      qB[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Wave w of a KV head takes the partition's tiles w, w + W, w + 2W, ... (PT of them).
  auto load_k = [&](int i) {
    KTile<KF, D> t;
    const int tok = t0 + 16 * (i * W + w) + n;
    const uint8_t* p;
    if constexpr (BIGBS) p = kbase + tile_block(i) + lane_row(tok) + 16 * q4;
    else p = kbase + row_off(tok) + 16 * q4;
#pragma unroll
    for (int j = 0; j < KTile<KF, D>::N; ++j) {
      if constexpr (PA_NT_K) t.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 64 * j));
      else t.w[j] = ld16(p + 64 * j);
    }
    return t;
  };
  auto load_v = [&](int i) {
    VTile<KF, D> t;
    int64_t tb = 0;
    if constexpr (BIGBS) tb = tile_block(i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = t0 + 16 * (i * W + w) + 4 * q4 + j;
      const uint8_t* p;
      if constexpr (BIGBS) p = vbase + tb + lane_row(tok) + n * VEC * ESZ;
      else p = vbase + row_off(tok) + n * VEC * ESZ;
      if constexpr (PA_NT_V) t.w[j] = __builtin_nontemporal_load(reinterpret_cast<const typename VTile<KF, D>::W*>(p));
      else t.w[j] = *reinterpret_cast<const typename VTile<KF, D>::W*>(p);
    }
    return t;
  };

  // ---- phase 1: logits of all tiles (base 2, masked) ----------------------------
  // The ring runs on into V: as the last K tiles are consumed, the first V tiles
  // are already requested, so the stream of loads does not pause between phases.
  float S[PT][4];
  KTile<KF, D> kt[KD];
  VTile<KF, D> vt[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) kt[i] = load_k(i);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const KTile<KF, D> cur = kt[i % KD];
    if (i + KD < PT) kt[i % KD] = load_k(i + KD);
    else vt[i + KD - PT] = load_v(i + KD - PT);
    const f32x4 s = qk_tile<KF, D>(cur, qB);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = t0 + 16 * (i * W + w) + 4 * q4 + r;
      S[i][r] = tok < ctx ? s[r] * a.qk_scale : -INFINITY;
    }
  }

  // ---- softmax over the partition (per column n, i.e. per query head) -----------
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[i][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // a wave whose tiles all lie past the context (W > 1) has no valid token
  const float mref = mx == -INFINITY ? 0.f : mx;
  uint32_t Pk[PT][2];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // probabilities enter P.V as bf16; the denominator sums the same rounded values
      p[r] = (float)(__bf16)__builtin_amdgcn_exp2f(S[i][r] - mref);
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
    const VTile<KF, D> cur = vt[i % KD];
    if (i + KD < PT) vt[i % KD] = load_v(i + KD);
    pv_tile<KF, D>(cur, Pk[i][0], Pk[i][1], O);
  }

  // ---- combine the W waves of each KV head (W > 1) --------------------------------
  // Per column n (query head head_of_column(n)): M = max_w m_w, L = sum_w 2^(m_w - M) l_w,
  // and O = sum_w 2^(m_w - M) O_w.  Lane (n, q4) register r of O holds head 4r + q4,
  // whose column is 4 * q4 + r.  lg[r] is that head's L; (Mn, Ln) are column n's.
  const int R = (G + 3) >> 2;                  // registers r in use
  float lg[4], Mn = mx, Ln = lsum;
  if (W == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[r] = __shfl(lsum, 4 * q4 + r);
  } else {
    // this head's area: (m, l) of every wave, then the O registers of waves 1 .. W-1
    float* base = xs + (int64_t)hl * combine_floats(W);
    auto ml = [&](int v) { return base + 32 * v; };
    auto oslot = [&](int v) { return base + 32 * W + (v - 1) * kCombineO; };
    if (w > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r >= R) break;
        float* x = oslot(w) + (r * kWave + lane) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) *reinterpret_cast<f32x4*>(x + e) = f32x4{O[e][r], O[e + 1][r], O[e + 2][r], O[e + 3][r]};
      }
    }
    if (q4 == 0) {
      ml(w)[n] = mx;
      ml(w)[16 + n] = lsum;
    }
    __syncthreads();
    if (w > 0) return;
    auto col_stats = [&](int c, float& Mc, float& Lc, float* aw) {
      Mc = -INFINITY;
      for (int v = 0; v < W; ++v) Mc = fmaxf(Mc, ml(v)[c]);
      Lc = 0.f;
      for (int v = 0; v < W; ++v) {
        const float m = ml(v)[c];
        const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - Mc);
        if (aw) aw[v] = f;
        Lc += f * ml(v)[16 + c];
      }
    };
    col_stats(n, Mn, Ln, nullptr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[r] = 1.f;
      if (r >= R) continue;
      float aw[kMaxWavesPerHead];
      float Mc;
      col_stats(4 * q4 + r, Mc, lg[r], aw);
#pragma unroll
      for (int e = 0; e < VEC; ++e) O[e][r] *= aw[0];
      for (int v = 1; v < W; ++v) {
        const float* x = oslot(v) + (r * kWave + lane) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const f32x4 y = *reinterpret_cast<const f32x4*>(x + e);
          O[e][r] += aw[v] * y[0];
          O[e + 1][r] += aw[v] * y[1];
          O[e + 2][r] += aw[v] * y[2];
          O[e + 3][r] += aw[v] * y[3];
        }
      }
    }
  }

  // ---- write: lane (n, q4) register r holds O[head 4*r + q4][d = VEC*n + e] ----------
  const bool single = ctx <= P;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= R) break;
    const int g = 4 * r + q4;
    if (g < G) {
      const int64_t hrow = (int64_t)b * a.num_q_heads + hq0 + g;
      if (single) {
        const float inv = a.v_scale / lg[r];
        uint32_t wv[VEC / 2];
#pragma unroll
        for (int c = 0; c < VEC / 2; ++c) wv[c] = pack_bf16(O[2 * c][r] * inv, O[2 * c + 1][r] * inv);
        uint16_t* o = out + hrow * D + n * VEC;
        if constexpr (VEC == 8) st16(o, u32x4{wv[0], wv[1], wv[2], wv[3]});
        else st8(o, u32x2{wv[0], wv[1]});
      } else {
        float* o = a.ws_o + piece_row(b, part, hq0 + g, a.max_parts, a.num_q_heads) * D + n * VEC;
        if constexpr (VEC == 8) {
          st16(o, __builtin_bit_cast(u32x4, f32x4{O[0][r], O[1][r], O[2][r], O[3][r]} * a.v_scale));
          st16(o + 4, __builtin_bit_cast(u32x4, f32x4{O[4][r], O[5][r], O[6][r], O[7][r]} * a.v_scale));
        } else {
          st16(o, __builtin_bit_cast(u32x4, f32x4{O[0][r], O[1][r], O[2][r], O[3][r]} * a.v_scale));
        }
      }
    }
  }
  if (!single && q4 == 0 && head_of_column(n) < G) {
    const int64_t idx = piece_row(b, part, hq0 + head_of_column(n), a.max_parts, a.num_q_heads);
    a.ws_m[idx] = Mn;
    a.ws_l[idx] = Ln;
  }
}

template <int KF, int D, bool BIGBS>
static hipError_t launch_pt(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  const size_t lds = a.waves_per_head > 1 ? sizeof(float) * combine_floats(a.waves_per_head) * a.heads_per_wg : 0;
  if (a.k_new != nullptr) {
    // the appending kernel exists for 256-token tiles per wave (partitions of 256, 512, 1024)
    if (a.partition_tokens / a.waves_per_head != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 16, BIGBS, true>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  switch (a.partition_tokens / a.waves_per_head) {
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 1, BIGBS, false>), grid, block, lds, s, a); break;
    case 32: hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 2, BIGBS, false>), grid, block, lds, s, a); break;
    case 64: hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 4, BIGBS, false>), grid, block, lds, s, a); break;
    case 128: hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 8, BIGBS, false>), grid, block, lds, s, a); break;
    case 256: hipLaunchKernelGGL((decode_mfma_kernel<KF, D, 16, BIGBS, false>), grid, block, lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KF, int D>
static hipError_t launch_bs(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  return a.block_size >= 16 ? launch_pt<KF, D, true>(a, grid, block, s) : launch_pt<KF, D, false>(a, grid, block, s);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = a.dense ? dim3((unsigned)(a.max_parts * a.head_groups * a.num_seqs), 1u)
                           : dim3((unsigned)(a.max_parts * a.head_groups), (unsigned)a.num_seqs);
  const dim3 block((unsigned)(kWave * a.heads_per_wg * a.waves_per_head));
  const bool d128 = a.head_dim == 128;
  switch (a.kv_fmt) {
    case kBf16: return d128 ? launch_bs<kFmtBf16, 128>(a, grid, block, s) : launch_bs<kFmtBf16, 64>(a, grid, block, s);
    case kE4m3: return d128 ? launch_bs<kFmtE4m3, 128>(a, grid, block, s) : launch_bs<kFmtE4m3, 64>(a, grid, block, s);
    case kInt8: return d128 ? launch_bs<kFmtInt8, 128>(a, grid, block, s) : launch_bs<kFmtInt8, 64>(a, grid, block, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
