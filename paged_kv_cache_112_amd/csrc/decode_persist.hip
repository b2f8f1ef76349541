// Paged decode, partition stage, persistent matrix-core path (bf16 or e4m3 pools, bf16 q).
//
// Same quantity and partition pieces as the one-workgroup-per-partition kernel
// (LLM stack book 4.6, "The PagedAttention Kernel"; split-K over the sequence per
// "Performance considerations"), scheduled differently for HBM streaming:
//
//   * A fixed grid that fills the GPU once.  The work units (sequence b, partition
//     p, KV head h) are split into one contiguous range of equal count per
//     workgroup; the workgroup's waves take the next unit of their range from a
//     counter in LDS, so they stay busy until the range is empty.  No global
//     atomics: a device-wide counter would serialize the waves of all CUs.
//   * Units are numbered densely: partitions per sequence are max(1, ceil(ctx/P))
//     and their running total (computed per workgroup from context_lens) maps a
//     unit number to (b, p) by binary search; h varies fastest, so the waves that
//     take consecutive units read the same token rows of different heads.
//   * One ring of K/V tile loads flows through a wave across unit boundaries: the
//     next unit is taken one unit ahead, its block-table slice, q rows and context
//     length are loaded while the current unit runs, and its first K tiles are in
//     flight before the current unit's last V tiles are consumed.
//   * Within a unit the arithmetic is that of the one-shot kernel: logits of all
//     tiles, one max and one sum, then P.V, in logical token order.
#include "launch.hpp"
#include "mfma_tiles.hpp"

#ifndef PA_PERSIST_DEPTH
#define PA_PERSIST_DEPTH 4   // tiles in flight per wave; divides 2 * tiles per unit
#endif
#ifndef PA_PERSIST_DEPTH_BYTE
#define PA_PERSIST_DEPTH_BYTE 8   // one-byte pools: tiles are half the bytes, so twice as many
#endif

namespace pa {

template <int KF, int D, int PT, bool BIGBS>
__global__ __launch_bounds__(256) void decode_persist_kernel(const DecodeArgs a) {
  constexpr int P = 16 * PT;
  constexpr int ESZ = byte_fmt(KF) ? 1 : 2;
  constexpr int VEC = D / 16;
  constexpr int NKK = D / 32;
  constexpr int NSTEP = 2 * PT;
  constexpr int RING = byte_fmt(KF) ? PA_PERSIST_DEPTH_BYTE : PA_PERSIST_DEPTH;
  constexpr int DEPTH = NSTEP < RING ? NSTEP : RING;
  static_assert(NSTEP % DEPTH == 0, "ring depth must divide the steps of a unit");
  constexpr int NR = BIGBS ? 1 : (P + 63) / 64;   // block-table registers per lane
  using KT = KTile<KF, D>;
  using VT = VTile<KF, D>;
  static_assert(sizeof(KT) == sizeof(VT), "K and V tiles share ring slots");
  struct Slot { uint32_t w[sizeof(KT) / 4]; };

  __shared__ int32_t s_pre[kPersistMaxSeqs];
  __shared__ uint32_t s_next;

  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int log2bs = a.log2_bs;
  const int bs_mask = a.block_size - 1;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int64_t row_bytes = a.row_bytes, block_bytes = a.block_bytes;

  // ---- running total of partitions per sequence --------------------------------------
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
      const int i = c0 + lane;
      int x = 0;
      if (i < B) {
        const int cx = a.context_lens[i];
        x = cx > P ? (cx + P - 1) / P : 1;
      }
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      x += carry;
      if (i < B) s_pre[i] = x;
      carry = __shfl(x, 63);
    }
  }
  __syncthreads();
  const uint32_t units = (uint32_t)__builtin_amdgcn_readfirstlane(s_pre[B - 1]) * (uint32_t)Hkv;
  // this workgroup's range of units
  const uint32_t lo = (uint32_t)(((uint64_t)blockIdx.x * units) / gridDim.x);
  const uint32_t total = (uint32_t)(((uint64_t)(blockIdx.x + 1) * units) / gridDim.x);
  if (threadIdx.x == 0) s_next = lo;
  __syncthreads();

  struct Unit {
    int b, part, kvh, ctx, np;
  };
  auto describe = [&](uint32_t u) {
    Unit r;
    const int x = (int)(u / (uint32_t)Hkv);
    r.kvh = (int)(u - (uint32_t)x * (uint32_t)Hkv);
    int lo = 0, hi = B - 1;                         // first b with s_pre[b] > x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_pre[mid]) > x) hi = mid;
      else lo = mid + 1;
    }
    const int before = lo > 0 ? __builtin_amdgcn_readfirstlane(s_pre[lo - 1]) : 0;
    r.b = lo;
    r.part = x - before;
    r.np = __builtin_amdgcn_readfirstlane(s_pre[lo]) - before;
    r.ctx = a.context_lens[lo];
    return r;
  };
  // Take the next unit of the workgroup's range (an LDS atomic: it waits only on LDS
  // traffic, never on the wave's HBM loads).  The old value lands in lane 0.
  auto grab = [&]() -> uint32_t {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&s_next, 1u);
    return v;
  };
  auto read_unit = [&](uint32_t v) -> uint32_t { return __builtin_amdgcn_readfirstlane(v); };
  // table entries lb0 + lane + 64k of sequence b (clamped to the row: padding is never used)
  auto load_table = [&](const Unit& r, int32_t (&tb)[NR]) {
    const int lb0 = (r.part * P) >> log2bs;
    const int32_t* row = a.block_tables + (int64_t)r.b * a.bt_stride;
#pragma unroll
    for (int k = 0; k < NR; ++k) tb[k] = row[min(lb0 + lane + 64 * k, a.bt_stride - 1)];
  };
  auto load_q = [&](const Unit& r, bf16x8 (&qv)[NKK]) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)r.b * a.num_q_heads + r.kvh * G + min(n, G - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = ld16(qrow + q_col<KF, D>(kk, q4));
      if (n >= G) w = u32x4{0u, 0u, 0u, 0u};
      qv[kk] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // byte offset of the row of token t (clamped to the context) for unit r
  auto row_offset = [&](const Unit& r, const int32_t (&tb)[NR], int t) -> int64_t {
    if (r.ctx <= 0) return 0;                      // nothing to read: block 0, row 0 stands in
    const int tc = min(t, r.ctx - 1);
    const int lb0 = (r.part * P) >> log2bs;
    const int e = (tc >> log2bs) - lb0;
    int blk;
    if constexpr (NR == 1) {
      blk = __builtin_amdgcn_ds_bpermute(e << 2, tb[0]);
    } else {
      blk = 0;
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int v = __builtin_amdgcn_ds_bpermute((e & 63) << 2, tb[k]);
        blk = (e >> 6) == k ? v : blk;
      }
    }
    return (int64_t)blk * block_bytes + (int64_t)(tc & bs_mask) * row_bytes;
  };
  // block of a whole 16-token tile (block size >= 16: one block per tile, uniform)
  auto tile_base = [&](const Unit& r, const int32_t (&tb)[NR], int tile_first) -> int64_t {
    if (r.ctx <= 0) return 0;
    const int tc = min(tile_first, r.ctx - 1);
    const int e = (tc >> log2bs) - ((r.part * P) >> log2bs);
    const int blk = __builtin_amdgcn_readlane(tb[0], e);
    return (int64_t)blk * block_bytes;
  };
  // issue the loads of step t of unit r (t < PT: K tile t, else V tile t - PT)
  auto issue = [&](int t, const Unit& r, const int32_t (&tb)[NR]) -> Slot {
    const uint8_t* head = (t < PT ? a.k_cache : a.v_cache) + (int64_t)r.kvh * D * ESZ;
    const int i = t < PT ? t : t - PT;
    const int first = r.part * P + 16 * i;
    const int last = max(r.ctx - 1, 0);
    Slot s;
    if (t < PT) {
      int64_t off;
      if constexpr (BIGBS) off = tile_base(r, tb, first) + (int64_t)(min(first + n, last) & bs_mask) * row_bytes;
      else off = row_offset(r, tb, first + n);
      const uint8_t* p = head + off + 16 * q4;
      KT k;
#pragma unroll
      for (int j = 0; j < KT::N; ++j) k.w[j] = ld16(p + 64 * j);
      s = __builtin_bit_cast(Slot, k);
    } else {
      VT v;
      int64_t base = 0;
      if constexpr (BIGBS) base = tile_base(r, tb, first);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = first + 4 * q4 + j;
        int64_t off;
        if constexpr (BIGBS) off = base + (int64_t)(min(tok, last) & bs_mask) * row_bytes;
        else off = row_offset(r, tb, tok);
        v.w[j] = *reinterpret_cast<const typename VT::W*>(head + off + n * VEC * ESZ);
      }
      s = __builtin_bit_cast(Slot, v);
    }
    return s;
  };

  uint16_t* out = static_cast<uint16_t*>(a.out);
  auto finalize = [&](const Unit& r, const f32x4 (&O)[VEC], float mx, float lsum) {
    const int hq0 = r.kvh * G;
    const bool single = r.np == 1;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int g = 4 * q4 + rr;
      const float lg = __shfl(lsum, g & 15);
      if (g < G) {
        const int64_t hrow = (int64_t)r.b * a.num_q_heads + hq0 + g;
        if (single) {
          const float inv = a.v_scale / lg;
          uint32_t w[VEC / 2];
#pragma unroll
          for (int c = 0; c < VEC / 2; ++c)
            w[c] = r.ctx > 0 ? pack_bf16(O[2 * c][rr] * inv, O[2 * c + 1][rr] * inv) : 0u;   // empty: zeros
          uint16_t* o = out + hrow * D + n * VEC;
          if constexpr (VEC == 8) st16(o, u32x4{w[0], w[1], w[2], w[3]});
          else st8(o, u32x2{w[0], w[1]});
        } else {
          float* o = a.ws_o + piece_row(r.b, r.part, hq0 + g, a.max_parts, a.num_q_heads) * D + n * VEC;
          st16(o, __builtin_bit_cast(u32x4, f32x4{O[0][rr], O[1][rr], O[2][rr], O[3][rr]} * a.v_scale));
          if constexpr (VEC == 8)
            st16(o + 4, __builtin_bit_cast(u32x4, f32x4{O[4][rr], O[5][rr], O[6][rr], O[7][rr]} * a.v_scale));
        }
      }
    }
    if (!single && q4 == 0 && n < G) {
      const int64_t idx = piece_row(r.b, r.part, hq0 + n, a.max_parts, a.num_q_heads);
      a.ws_m[idx] = mx;
      a.ws_l[idx] = lsum;
    }
  };

  // ---- the wave's stream of units --------------------------------------------------
  const uint32_t u = read_unit(grab());
  if (u < total) {
    Unit cur = describe(u);
    int32_t tb[NR];
    bf16x8 qB[NKK];
    load_table(cur, tb);
    load_q(cur, qB);
    const uint32_t u1 = read_unit(grab());
    bool has_next = u1 < total;
    Unit nxt = has_next ? describe(u1) : cur;     // without a next unit, loads repeat this one's
    Slot ring[DEPTH];
#pragma unroll
    for (int t = 0; t < DEPTH; ++t) ring[t] = issue(t, cur, tb);

    while (true) {
      const uint32_t u_after = grab();               // read at the end of this unit
      int32_t tb_n[NR];
      bf16x8 qB_n[NKK];
      load_table(nxt, tb_n);
      load_q(nxt, qB_n);

      const int t0 = cur.part * P;
      float S[PT][4];
      uint32_t Pk[PT][2];
      float mx = 0.f, lsum = 0.f;
      f32x4 O[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) O[e] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const Slot data = ring[s % DEPTH];
        const int t = s + DEPTH;
        ring[s % DEPTH] = t < NSTEP ? issue(t, cur, tb) : issue(t - NSTEP, nxt, tb_n);

        if (s < PT) {                                    // logits of tile s, base 2, masked
          const f32x4 sc = qk_tile<KF, D>(__builtin_bit_cast(KT, data), qB);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = t0 + 16 * s + 4 * q4 + r;
            S[s][r] = tok < cur.ctx ? sc[r] * a.qk_scale : -INFINITY;
          }
        }
        if (s == PT - 1) {                               // softmax over the partition
          mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < PT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[i][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          if (mx == -INFINITY) mx = 0.f;                 // empty context: every probability is 0
#pragma unroll
          for (int i = 0; i < PT; ++i) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              p[r] = (float)(__bf16)__builtin_amdgcn_exp2f(S[i][r] - mx);
              lsum += p[r];
            }
            Pk[i][0] = pack_bf16(p[0], p[1]);
            Pk[i][1] = pack_bf16(p[2], p[3]);
          }
          lsum += __shfl_xor(lsum, 16);
          lsum += __shfl_xor(lsum, 32);
        }
        if (s >= PT) pv_tile<KF, D>(__builtin_bit_cast(VT, data), Pk[s - PT][0], Pk[s - PT][1], O);
      }

      finalize(cur, O, mx, lsum);
      if (!has_next) break;
      cur = nxt;
#pragma unroll
      for (int k = 0; k < NR; ++k) tb[k] = tb_n[k];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qB[kk] = qB_n[kk];
      const uint32_t un = read_unit(u_after);
      has_next = un < total;
      nxt = has_next ? describe(un) : cur;
    }
  }

}

template <int KF, int D, int PT>
static hipError_t launch_bs(const DecodeArgs& a, hipStream_t s) {
  const void* fn = a.block_size >= 16 ? reinterpret_cast<const void*>(&decode_persist_kernel<KF, D, PT, true>)
                                      : reinterpret_cast<const void*>(&decode_persist_kernel<KF, D, PT, false>);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
  if (e != hipSuccess) return e;
  const int grid = max(1, cus * max(1, per_cu));
  if (a.block_size >= 16)
    hipLaunchKernelGGL((decode_persist_kernel<KF, D, PT, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_persist_kernel<KF, D, PT, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KF, int D>
static hipError_t launch_pt(const DecodeArgs& a, hipStream_t s) {
  switch (a.partition_tokens) {
    case 16: return launch_bs<KF, D, 1>(a, s);
    case 32: return launch_bs<KF, D, 2>(a, s);
    case 64: return launch_bs<KF, D, 4>(a, s);
    case 128: return launch_bs<KF, D, 8>(a, s);
    case 256: return launch_bs<KF, D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_persist(const DecodeArgs& a, hipStream_t s) {
  const bool d128 = a.head_dim == 128;
  switch (a.kv_fmt) {
    case kBf16: return d128 ? launch_pt<kFmtBf16, 128>(a, s) : launch_pt<kFmtBf16, 64>(a, s);
    case kE4m3: return d128 ? launch_pt<kFmtE4m3, 128>(a, s) : launch_pt<kFmtE4m3, 64>(a, s);
    case kInt8: return d128 ? launch_pt<kFmtInt8, 128>(a, s) : launch_pt<kFmtInt8, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
