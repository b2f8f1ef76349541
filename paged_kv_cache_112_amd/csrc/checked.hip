// The device error word of the checked build (-DPA_CHECKED=1) and its host access.
//
// Kernels of a checked build report a broken caller contract (a slot or block id
// outside the pool, a context past its table or past max_context_len, a copy id past
// the pool) by OR-ing a bit into this word and carry on with a safe value.  In a release
// build the word does not exist and the kernels compile no checks.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"
#include "api_internal.hpp"
#include "launch.hpp"

#if PA_CHECKED
// `err_word` below is a host-side stand-in for the device word in host code: its device
// address comes from hipGetSymbolAddress with the device current, once per device.
static __device__ uint32_t err_word;   // zero at load

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
uint32_t* g_word[kMaxDevices];
}  // namespace

uint32_t* pa::checked_error_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_word[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(err_word)) != hipSuccess) return nullptr;
    g_word[dev] = static_cast<uint32_t*>(ptr);
  }
  return g_word[dev];
}
#else
uint32_t* pa::checked_error_word() { return nullptr; }
#endif

extern "C" int32_t pa_checked_build(void) { return PA_CHECKED ? 1 : 0; }

extern "C" pa_status pa_checked_errors(uint32_t* flags) {
  if (flags == nullptr) return PA_ERR_NULL;
  *flags = 0;
  if (!PA_CHECKED) return PA_ERR_UNSUPPORTED;
  uint32_t* word = pa::checked_error_word();
  if (word == nullptr) return PA_ERR_HIP;
  // every launch on the device so far has ended; read the word, then clear it
  if (hipDeviceSynchronize() != hipSuccess) return PA_ERR_HIP;
  if (hipMemcpy(flags, word, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return PA_ERR_HIP;
  const uint32_t zero = 0;
  if (hipMemcpy(word, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}
