// pa_decode_noalloc: pa_decode with its scratch in a static device array, for callers
// that cannot allocate (graph capture, serving loops, harnesses that forbid it).
//
// `scratch` below is a host-side stand-in for the array in host code: the device
// address of each GPU's copy comes from hipGetSymbolAddress with that device current,
// is looked up once per device, and is the only handle the kernels ever receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"
#include "api_internal.hpp"

namespace {

constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

// The split-K pieces of pa_decode_noalloc: every call writes the pieces it then reads, so
// nothing has to start at zero and nothing one call leaves behind reaches the next.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_mutex;
uint8_t* g_scratch[kMaxDevices];

// The current device's copy of the array (looked up on the first call on that device).
pa_status device_scratch(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PA_ERR_HIP;
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                       const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len, float scale,
                                       void* out, int32_t partition_tokens, int32_t kernel, void* stream) {
  uint8_t* base = nullptr;
  if (const pa_status s = device_scratch(&base); s != PA_OK) return s;
  return pa::decode_in_scratch(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                               max_blocks_per_seq, context_lens, max_context_len, scale, out, partition_tokens,
                               kernel, base, kScratchBytes, stream);
}
