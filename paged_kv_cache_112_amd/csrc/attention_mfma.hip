// Multi-query paged attention (chunked prefill, or several new tokens per sequence),
// matrix-core path: bf16 q with a bf16 or e4m3 pool.
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
// How, on gfx950: one wave per (request, KV head, query tile).  A query tile is
// T = 16 / G new tokens with all G query heads of the KV head, so the 16 columns of
// the MFMA B operand are (token, head) pairs and the product is dense.  The four
// waves of a workgroup take four consecutive query tiles of the same KV head, so a
// K/V tile fetched by one of them is found in the CU's cache by the others.
//   * q.K^T: v_mfma_f32_16x16x32_bf16 with A = a 16-key tile (row = key), B = q^T
//     (column n = token n / G, head n % G), as in the decode kernel.
//   * Softmax runs online over the key tiles in base 2, per column: a running max m,
//     and whenever m grows the running sum and output are scaled by 2^(m_old - m_new).
//   * P.V is the transposed product O^T = V^T P^T (v_mfma_f32_16x16x16_bf16), whose
//     output keeps each column's values in that column's own lanes, so the rescale is
//     a lane-local multiply.
// Keys past the causal limit of a column get probability 0; the key loop stops at
// the last tile any column of the tile can see.  Rows past the context are clamped
// to the last valid row for addressing.
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace pa {

constexpr int kAttnWaves = 4;   // query tiles (waves) per workgroup

__device__ __forceinline__ int32_t attn_load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

template <int KF, int D, bool BIGBS>
__global__ __launch_bounds__(256) void attention_mfma_kernel(const AttnArgs a) {
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;
  constexpr int VEC = D / 16;
  constexpr int NKK = D / 32;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = (blockIdx.x / a.num_kv_heads) * kAttnWaves + wave;
  const int i = blockIdx.y;
  const int q0 = a.query_start_loc[i];
  const int nq = a.query_start_loc[i + 1] - q0;
  const int S = a.seq_lens[i];
  const int T = 16 >> a.log2_group;                 // query tokens per tile
  const int t0 = qt * T;
  // whole workgroup (uniform): past this request's queries, or inconsistent lengths
  if (t0 >= nq || nq > S || q0 < 0 || q0 + nq > a.num_tokens) return;   // per wave: no barrier follows

  const int lane = threadIdx.x & 63;
  const int G = 1 << a.log2_group;
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int tq = t0 + (n >> a.log2_group);          // this column's query token (request-local)
  const int g = n & (G - 1);
  const bool qvalid = tq < nq;
  const int qpos = S - nq + tq;                     // its position in the context
  const int tlast = min(t0 + T, nq) - 1;
  const int kmax = S - nq + tlast;                  // last key any column of the tile sees
  const int nkt = (kmax >> 4) + 1;

  // q^T as the B operand: lane (n, q4) holds 8 d's of (token tq, head g)
  bf16x8 qB[NKK];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + min(tq, nq - 1)) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) w = ld16(qrow + q_col<KF, D>(kk, q4));
      qB[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int32_t* bt_row = a.block_tables + (int64_t)i * a.bt_stride;
  const int64_t head_off = (int64_t)kvh * D * ESZ;
  const uint8_t* kbase = a.k_cache + head_off;
  const uint8_t* vbase = a.v_cache + head_off;
  const int bs_mask = a.block_size - 1;
  // byte offset of key t (clamped to the context) within the pool
  auto row_off = [&](int t, int tile) -> int64_t {
    const int tc = min(t, S - 1);
    int32_t blk;
    if constexpr (BIGBS) blk = attn_load_uniform(bt_row + (min(16 * tile, S - 1) >> a.log2_bs));
    else blk = bt_row[tc >> a.log2_bs];
    return (int64_t)blk * a.block_bytes + (int64_t)(tc & bs_mask) * a.row_bytes;
  };
  auto load_k = [&](int kt) {
    KTile<KF, D> t;
    const uint8_t* p = kbase + row_off(16 * kt + n, kt) + 16 * q4;
#pragma unroll
    for (int j = 0; j < KTile<KF, D>::N; ++j) t.w[j] = ld16(p + 64 * j);
    return t;
  };
  auto load_v = [&](int kt) {
    VTile<KF, D> t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* p = vbase + row_off(16 * kt + 4 * q4 + j, kt) + n * VEC * ESZ;
      t.w[j] = *reinterpret_cast<const typename VTile<KF, D>::W*>(p);
    }
    return t;
  };

  f32x4 O[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) O[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  KTile<KF, D> kc = load_k(0);
  VTile<KF, D> vc = load_v(0);
  for (int kt = 0; kt < nkt; ++kt) {
    KTile<KF, D> kn;
    VTile<KF, D> vn;
    if (kt + 1 < nkt) {                             // next tile in flight while this one computes
      kn = load_k(kt + 1);
      vn = load_v(kt + 1);
    }
    const f32x4 s = qk_tile<KF, D>(kc, qB);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * q4 + r;
      x[r] = (qvalid && key <= qpos) ? s[r] * a.qk_scale : -INFINITY;
    }
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float mref = m_new == -INFINITY ? 0.f : m_new;     // a column with no visible key yet
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mref);
    m = m_new;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // probabilities enter P.V as bf16; the denominator sums the same rounded values
      p[r] = (float)(__bf16)__builtin_amdgcn_exp2f(x[r] - mref);
    }
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] *= alpha;
    pvt_tile<KF, D>(vc, pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), O);
    if (kt + 1 < nkt) {
      kc = kn;
      vc = vn;
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // lane (n, q4) register r of O[e] holds column n's output at d = VEC*(4*q4 + r) + e
  if (qvalid) {
    const float inv = a.v_scale / lsum;
    uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + tq) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t w[VEC / 2];
#pragma unroll
      for (int c = 0; c < VEC / 2; ++c) w[c] = pack_bf16(O[2 * c][r] * inv, O[2 * c + 1][r] * inv);
      uint16_t* dst = o + VEC * (4 * q4 + r);
      if constexpr (VEC == 8) st16(dst, u32x4{w[0], w[1], w[2], w[3]});
      else st8(dst, u32x2{w[0], w[1]});
    }
  }
}

template <int KF, int D>
static void launch_d(const AttnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.block_size >= 16) hipLaunchKernelGGL((attention_mfma_kernel<KF, D, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attention_mfma_kernel<KF, D, false>), grid, block, 0, s, a);
}

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s) {
  const int T = 16 >> a.log2_group;
  const int tiles = (a.max_query_len + T - 1) / T;
  const dim3 grid((unsigned)(((tiles + kAttnWaves - 1) / kAttnWaves) * a.num_kv_heads), (unsigned)a.num_seqs);
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
