// pa_copy_blocks: the device half of copy-on-write.  When a sequence must append
// into a block that other sequences still reference, the allocator gives it a
// fresh block and the contents of the shared one are copied there before the
// write (LLM stack book 4.6, "Copy-on-write for shared prefixes"; ai-infra-
// handbooks "Paged KV cache", exercise 2 on copy-on-write).  One copy moves a
// whole physical block -- every row and every KV head -- of the K pool and of the
// V pool; the bytes are copied as they are, whatever the pool format.
//
// Layers: a multi-layer pool is one allocation of num_layers equal pools, so a
// copy-on-write copy moves the block in every layer; blockIdx.z is the layer.
//
// Workgroup (x, pair): pair = blockIdx.y, and each thread moves U 16-byte chunks
// of K and the same chunks of V, all loads issued before the stores.  Small calls
// (a decode step's few copies) use U = 1 to spread over more workgroups.  Loads and
// stores both carry the non-temporal hint: no byte is touched twice within a call, and
// streaming the stores past the caches was 4 % faster on a 1.1 GB copy than plain
// stores.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

constexpr int kCopyThreads = 256;

template <int U>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyArgs a) {
  const int32_t s = a.src[blockIdx.y];
  const int32_t d = a.dst[blockIdx.y];
  // ids outside the pool (negative padding included) are skipped
  if (s < 0 || d < 0 || (int64_t)s >= a.num_blocks || (int64_t)d >= a.num_blocks) {
    // negative ids are padding; an id past the pool is reported in the checked build
    if ((int64_t)s >= a.num_blocks || (int64_t)d >= a.num_blocks)
      if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.z == 0) flag_error(a.err, kErrPair);
    return;
  }
  const int64_t layer_off = (int64_t)blockIdx.z * a.layer_bytes;
  const int64_t src_off = layer_off + (int64_t)s * a.block_bytes;
  const int64_t dst_off = layer_off + (int64_t)d * a.block_bytes;
  const int64_t c0 = (int64_t)blockIdx.x * kCopyThreads * U + threadIdx.x;
  u32x4 kx[U], vx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + (int64_t)u * kCopyThreads;
    if (c < a.chunks) {
      kx[u] = ld16_nt(reinterpret_cast<const u32x4*>(a.k_cache + src_off) + c);
      vx[u] = ld16_nt(reinterpret_cast<const u32x4*>(a.v_cache + src_off) + c);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + (int64_t)u * kCopyThreads;
    if (c < a.chunks) {
      st16_nt(reinterpret_cast<u32x4*>(a.k_cache + dst_off) + c, kx[u]);
      st16_nt(reinterpret_cast<u32x4*>(a.v_cache + dst_off) + c, vx[u]);
    }
  }
}

template <int U>
static void launch_u(const CopyArgs& a, hipStream_t stream) {
  const int64_t per_wg = (int64_t)kCopyThreads * U;
  const dim3 grid((unsigned)((a.chunks + per_wg - 1) / per_wg), (unsigned)a.num_pairs, (unsigned)a.num_layers);
  hipLaunchKernelGGL(copy_blocks_kernel<U>, grid, dim3(kCopyThreads), 0, stream, a);
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  // enough chunks to fill the chip several times over: unroll; otherwise one chunk per thread
  if ((int64_t)a.num_pairs * a.num_layers * a.chunks >= (int64_t)256 * kCopyThreads * 4 * 8) launch_u<4>(a, stream);
  else launch_u<1>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
