// Contract-check words of the checked build (see decode_attn_checks in
// decode_attn.h): one pair [flag bits, observation count] per device, in a
// file-scope device array each GPU holds its own copy of.
#include <atomic>

#include "common.h"

#ifdef DA_CHECKED

namespace {

__device__ __attribute__((aligned(16))) unsigned long long g_check_words[2];

constexpr int kMaxDevices = 64;
std::atomic<unsigned long long*> g_words[kMaxDevices];

}  // namespace

unsigned long long* da_host::check_words() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  unsigned long long* p = g_words[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;  // this device's copy of the array
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(g_check_words)) != hipSuccess) return nullptr;
    p = static_cast<unsigned long long*>(addr);
    g_words[dev].store(p, std::memory_order_release);
  }
  return p;
}

extern "C" int32_t decode_attn_checks(uint32_t* flags, uint64_t* count, int32_t reset) {
  unsigned long long* p = da_host::check_words();
  if (!p) return DA_ERR_LAUNCH;
  unsigned long long h[2] = {0, 0};
  if (hipDeviceSynchronize() != hipSuccess) return DA_ERR_LAUNCH;
  if (hipMemcpy(h, p, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return DA_ERR_LAUNCH;
  if (flags) *flags = (uint32_t)h[0];
  if (count) *count = (uint64_t)h[1];
  if (reset) {
    const unsigned long long zero[2] = {0, 0};
    if (hipMemcpy(p, zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return DA_ERR_LAUNCH;
  }
  return DA_OK;
}

#else

unsigned long long* da_host::check_words() { return nullptr; }

extern "C" int32_t decode_attn_checks(uint32_t* flags, uint64_t* count, int32_t reset) {
  (void)flags; (void)count; (void)reset;
  return DA_ERR_UNSUPPORTED;
}

#endif
