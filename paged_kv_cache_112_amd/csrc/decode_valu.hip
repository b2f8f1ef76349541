// Paged decode, partition stage, vector-ALU path: any pool format (f32, bf16,
// e4m3) with f32 or bf16 q.  It serves the fp32 pools and gives a second,
// independently written GPU path for the others.
//
// Same quantity and partition pieces as the matrix-core path (LLM stack book 4.6,
// "The PagedAttention Kernel"; split-K per "Performance considerations").
// Layout: one wave per (sequence, KV head, partition).  A row of one KV head is
// covered by LPR lanes, each loading 16 bytes (8 for e4m3), so one wave load
// covers RPI = 64 / LPR token rows.  Dot products are reduced across the LPR
// lanes of a row with DPP; logits go to LDS, the wave takes one max and one sum
// per query head, and P.V accumulates per lane before a final cross-row
// reduction.  Addressing clamps tokens past the context to the last valid row.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

template <int KVF>
struct Row;  // one lane's slice of a K or V row, widened to float

template <>
struct Row<kF32> {
  static constexpr int E = 4, BYTES = 16;
  __device__ static void load(const uint8_t* p, float* x) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
};
template <>
struct Row<kBf16> {
  static constexpr int E = 8, BYTES = 16;
  __device__ static void load(const uint8_t* p, float* x) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16lo(w[i]); x[2 * i + 1] = bf16hi(w[i]); }
  }
};
template <>
struct Row<kE4m3> {
  static constexpr int E = 8, BYTES = 8;
  __device__ static void load(const uint8_t* p, float* x) {
    const u32x2 w = ld8(p);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 lo = e4m3x2_lo(w[i]), hi = e4m3x2_hi(w[i]);
      x[4 * i] = lo.x; x[4 * i + 1] = lo.y; x[4 * i + 2] = hi.x; x[4 * i + 3] = hi.y;
    }
  }
};

template <>
struct Row<kInt8> {
  static constexpr int E = 8, BYTES = 8;
  __device__ static void load(const uint8_t* p, float* x) {
    const u32x2 w = ld8(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
};

template <int KVF, int QF, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_valu_kernel(const DecodeArgs a) {
  constexpr int ESZ = KVF == kF32 ? 4 : KVF == kBf16 ? 2 : 1;
  constexpr int E = Row<KVF>::E;
  constexpr int LPR = D / E;            // lanes per row
  constexpr int RPI = kWave / LPR;      // rows per wave load
  constexpr int PMAX = 256;
  __shared__ float sS[4][GMAX][PMAX];
  __shared__ int32_t tbl[PMAX];

  const int P = a.partition_tokens;
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
  const int t0 = part * P;
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

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kvh = hg * a.heads_per_wg + wave;
  const int G = a.group;
  const int hq0 = kvh * G;
  const int rg = lane / LPR;            // row within one load
  const int cl = lane % LPR;            // column slice
  const int d0 = cl * E;

  if (ctx == 0) {
    for (int i = lane; i < G * D; i += kWave) {
      const int64_t idx = ((int64_t)b * a.num_q_heads + hq0) * D + i;
      if (QF == kF32) static_cast<float*>(a.out)[idx] = 0.f;
      else static_cast<uint16_t*>(a.out)[idx] = 0;
    }
    return;
  }

  const int n_tok = min(P, ctx - t0);
  const int n_rows = (n_tok + RPI - 1) / RPI * RPI;
  const int lb0 = t0 >> a.log2_bs;
  const int n_ent = ((t0 + n_tok - 1) >> a.log2_bs) - lb0 + 1;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.bt_stride + lb0;
  for (int i = threadIdx.x; i < n_ent; i += blockDim.x) tbl[i] = checked_block(bt_row[i], a.num_blocks, a.err);
  __syncthreads();

  const int64_t head_off = (int64_t)kvh * D * ESZ + (int64_t)d0 * ESZ;
  const uint8_t* kbase = a.k_cache + head_off;
  const uint8_t* vbase = a.v_cache + head_off;
  auto row_off = [&](int t) -> int64_t {
    const int tc = min(t, ctx - 1);
    const int blk = tbl[(tc >> a.log2_bs) - lb0];
    return (int64_t)blk * a.block_bytes + (int64_t)(tc & (a.block_size - 1)) * a.row_bytes;
  };

  float qv[GMAX][E];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    const int64_t qoff = ((int64_t)b * a.num_q_heads + hq0 + min(g, G - 1)) * D + d0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x;
      if constexpr (QF == kF32) x = static_cast<const float*>(a.q)[qoff + e];
      else x = __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.q)[qoff + e] << 16);
      qv[g][e] = g < G ? x : 0.f;
    }
  }

  // ---- phase 1: logits -> LDS -------------------------------------------------
  float* S = &sS[wave][0][0];
  for (int r0 = 0; r0 < n_rows; r0 += RPI) {
    const int t = t0 + r0 + rg;
    float kf[E];
    Row<KVF>::load(kbase + row_off(t), kf);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float part_dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part_dot = fmaf(qv[g][e], kf[e], part_dot);
      const float dot = group_sum<LPR>(part_dot);
      if (g < G && cl == 0) S[g * PMAX + r0 + rg] = t < ctx ? dot * a.qk_scale : -INFINITY;
    }
  }
  __syncthreads();

  // ---- softmax per query head ---------------------------------------------------
  float lg[GMAX], mg[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    float m = -INFINITY;
    for (int i = lane; i < n_rows; i += kWave) m = fmaxf(m, S[g * PMAX + i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < n_rows; i += kWave) {
      const float p = __builtin_amdgcn_exp2f(S[g * PMAX + i] - m);
      S[g * PMAX + i] = p;
      l += p;
    }
    lg[g] = wave_sum(l);
    mg[g] = m;
  }
  __syncthreads();

  // ---- phase 2: P.V ---------------------------------------------------------------
  float acc[GMAX][E];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  for (int r0 = 0; r0 < n_rows; r0 += RPI) {
    const int t = t0 + r0 + rg;
    float vf[E];
    Row<KVF>::load(vbase + row_off(t), vf);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const float p = S[g * PMAX + r0 + rg];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  }
#pragma unroll
  for (int s = LPR; s < kWave; s *= 2)
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] += __shfl_xor(acc[g][e], s);

  // ---- write ------------------------------------------------------------------------
  const bool single = ctx <= P;
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      const int64_t hrow = (int64_t)b * a.num_q_heads + hq0 + g;
      if (single) {
        const float inv = a.v_scale / lg[g];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float y = acc[g][e] * inv;
          if constexpr (QF == kF32) static_cast<float*>(a.out)[hrow * D + d0 + e] = y;
          else static_cast<uint16_t*>(a.out)[hrow * D + d0 + e] = __builtin_bit_cast(uint16_t, (__bf16)y);
        }
      } else {
        const int64_t prow = piece_row(b, part, hq0 + g, a.max_parts, a.num_q_heads);
        float* o = a.ws_o + prow * D + d0;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = acc[g][e] * a.v_scale;
        if (cl == 0) {
          a.ws_m[prow] = mg[g];
          a.ws_l[prow] = lg[g];
        }
      }
    }
  }
}

template <int KVF, int QF, int D>
static hipError_t launch_g(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.group <= 1) hipLaunchKernelGGL((decode_valu_kernel<KVF, QF, D, 1>), grid, block, 0, s, a);
  else if (a.group <= 2) hipLaunchKernelGGL((decode_valu_kernel<KVF, QF, D, 2>), grid, block, 0, s, a);
  else if (a.group <= 4) hipLaunchKernelGGL((decode_valu_kernel<KVF, QF, D, 4>), grid, block, 0, s, a);
  else if (a.group <= 8) hipLaunchKernelGGL((decode_valu_kernel<KVF, QF, D, 8>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int KVF, int QF>
static hipError_t launch_d(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  return a.head_dim == 128 ? launch_g<KVF, QF, 128>(a, grid, block, s) : launch_g<KVF, QF, 64>(a, grid, block, s);
}

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = a.dense ? dim3((unsigned)(a.max_parts * a.head_groups * a.num_seqs), 1u)
                           : dim3((unsigned)(a.max_parts * a.head_groups), (unsigned)a.num_seqs);
  const dim3 block((unsigned)(kWave * a.heads_per_wg));
  if (a.kv_fmt == kF32 && a.q_fmt == kF32) return launch_d<kF32, kF32>(a, grid, block, s);
  if (a.kv_fmt == kBf16 && a.q_fmt == kBf16) return launch_d<kBf16, kBf16>(a, grid, block, s);
  if (a.kv_fmt == kE4m3 && a.q_fmt == kBf16) return launch_d<kE4m3, kBf16>(a, grid, block, s);
  if (a.kv_fmt == kInt8 && a.q_fmt == kBf16) return launch_d<kInt8, kBf16>(a, grid, block, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
