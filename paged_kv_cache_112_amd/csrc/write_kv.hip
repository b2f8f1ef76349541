// pa_write_kv kernels: scatter new tokens' K and V rows into the block pools.
//
// The pool [num_blocks, block_size, H_kv, d_h] seen as [num_blocks * block_size,
// H_kv * d_h] is slot-major, so token i's whole row (all KV heads) is one
// contiguous run of bytes at slot_mapping[i] (LLM stack book 4.6, "From Python
// bookkeeping to the tensors the kernel actually takes": the write is one
// indexed copy over the flattened pool).  Each thread moves one 8-element
// chunk of a row for K and the same chunk for V: loads and stores of
// neighbouring threads are contiguous, 16 bytes wide for bf16.  Every byte is
// read or written once, so all of them carry the non-temporal hint (3 % faster
// on a 121k-token bf16 prefill write, no change on a decode step's few rows).
#include "common.hpp"
#include "launch.hpp"

namespace pa {

enum class WriteMode { kCopy16, kCopy32, kBf16ToE4m3, kF32ToE4m3, kBf16ToInt8, kF32ToInt8 };

template <WriteMode M>
__global__ __launch_bounds__(128) void write_kv_kernel(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                       const int32_t* __restrict__ slots, uint8_t* __restrict__ kc,
                                                       uint8_t* __restrict__ vc, int64_t total_chunks,
                                                       int32_t chunks_per_row, float inv_k, float inv_v,
                                                       int64_t num_slots, uint32_t* err) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= total_chunks) return;
  const int64_t tok = item / chunks_per_row;
  const int32_t c = (int32_t)(item - tok * chunks_per_row);
  const int32_t slot = slots[tok];
  if constexpr (kChecked) {                  // a slot past the pool: reported, the token skipped
    if (slot >= num_slots) {
      if (c == 0) flag_error(err, kErrSlot);
      return;
    }
  }
  const int64_t src_elem = item * 8;                                   // == tok * row + c * 8
  const int64_t dst_elem = (int64_t)slot * chunks_per_row * 8 + (int64_t)c * 8;
  if constexpr (M == WriteMode::kCopy16) {                             // bf16 -> bf16
    // the row loads are issued with the slot load (the empty asm keeps them ahead of
    // the slot test), so the thread waits for one memory round trip, not two
    const u32x4 k0 = ld16_nt(k + src_elem * 2), v0 = ld16_nt(v + src_elem * 2);
    asm volatile("" ::"v"(k0), "v"(v0));
    if (slot < 0) return;
    st16_nt(kc + dst_elem * 2, k0);
    st16_nt(vc + dst_elem * 2, v0);
  } else if constexpr (M == WriteMode::kCopy32) {                      // f32 -> f32
    if (slot < 0) return;
    const u32x4 k0 = ld16_nt(k + src_elem * 4), k1 = ld16_nt(k + src_elem * 4 + 16);
    const u32x4 v0 = ld16_nt(v + src_elem * 4), v1 = ld16_nt(v + src_elem * 4 + 16);
    st16_nt(kc + dst_elem * 4, k0);
    st16_nt(kc + dst_elem * 4 + 16, k1);
    st16_nt(vc + dst_elem * 4, v0);
    st16_nt(vc + dst_elem * 4 + 16, v1);
  } else {
    float xk[8], xv[8];
    if constexpr (M == WriteMode::kBf16ToE4m3 || M == WriteMode::kBf16ToInt8) {
      const u32x4 a = ld16_nt(k + src_elem * 2), b = ld16_nt(v + src_elem * 2);
      asm volatile("" ::"v"(a), "v"(b));
      if (slot < 0) return;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xk[2 * i] = bf16lo(a[i]); xk[2 * i + 1] = bf16hi(a[i]);
        xv[2 * i] = bf16lo(b[i]); xv[2 * i + 1] = bf16hi(b[i]);
      }
    } else {
      if (slot < 0) return;
      const u32x4 a0 = ld16_nt(k + src_elem * 4), a1 = ld16_nt(k + src_elem * 4 + 16);
      const u32x4 b0 = ld16_nt(v + src_elem * 4), b1 = ld16_nt(v + src_elem * 4 + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xk[i] = __uint_as_float(a0[i]); xk[4 + i] = __uint_as_float(a1[i]);
        xv[i] = __uint_as_float(b0[i]); xv[4 + i] = __uint_as_float(b1[i]);
      }
    }
    u32x2 ok = {0u, 0u}, ov = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // one fp32 multiply, then round to the one-byte code (no fused multiply-add is possible here)
      if constexpr (M == WriteMode::kBf16ToE4m3 || M == WriteMode::kF32ToE4m3) {
        ok[i >> 2] |= f32_to_e4m3(xk[i] * inv_k) << (8 * (i & 3));
        ov[i >> 2] |= f32_to_e4m3(xv[i] * inv_v) << (8 * (i & 3));
      } else {
        ok[i >> 2] |= f32_to_i8(xk[i] * inv_k) << (8 * (i & 3));
        ov[i >> 2] |= f32_to_i8(xv[i] * inv_v) << (8 * (i & 3));
      }
    }
    st8_nt(kc + dst_elem, ok);
    st8_nt(vc + dst_elem, ov);
  }
}

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream) {
  const int32_t cpr = a.row_elems / 8;
  const int64_t total = (int64_t)a.num_tokens * cpr;
  if (total == 0) return hipSuccess;
  // 128-thread workgroups: 2 % faster than 256 on prefill-sized writes, the same at decode sizes
  const dim3 block(128);
  const dim3 grid((unsigned)((total + 127) / 128));
  const uint8_t* k = static_cast<const uint8_t*>(a.k);
  const uint8_t* v = static_cast<const uint8_t*>(a.v);
  uint8_t* kc = static_cast<uint8_t*>(a.k_cache);
  uint8_t* vc = static_cast<uint8_t*>(a.v_cache);
  switch (a.mode) {
    case 0: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kCopy16>, grid, block, 0, stream, k, v, a.slots, kc, vc,
                               total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
    case 1: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kCopy32>, grid, block, 0, stream, k, v, a.slots, kc, vc,
                               total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
    case 2: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kBf16ToE4m3>, grid, block, 0, stream, k, v, a.slots, kc,
                               vc, total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
    case 3: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kF32ToE4m3>, grid, block, 0, stream, k, v, a.slots, kc,
                               vc, total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
    case 4: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kBf16ToInt8>, grid, block, 0, stream, k, v, a.slots, kc,
                               vc, total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
    default: hipLaunchKernelGGL(write_kv_kernel<WriteMode::kF32ToInt8>, grid, block, 0, stream, k, v, a.slots, kc,
                                vc, total, cpr, a.inv_k, a.inv_v, a.num_slots, a.err); break;
  }
  return hipGetLastError();
}

}  // namespace pa
