// Scratch memory of the allocation-free prefill (kda_chunk_fwd_noalloc): a
// file-scope device array, one copy per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: the address
// on each device comes from hipGetSymbolAddress, looked up once per device with
// that device current, and is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {

namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;   // 64 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** p) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
