// Fixed device scratch for the entry point that allocates nothing
// (global_pooled_attn_fwd_noalloc): one static array per device, its address
// resolved once per device and kept.
#include <mutex>
#include <vector>

#include "internal.h"

// 128 MiB: pooled K and V of the 4K latent at 8 x 8 pooling (2 x 65.8 MB,
// bf16, 24 heads) fit.  Every GPU the library runs on holds its own copy of
// this array from the first use of the library's device code on that GPU
// until the process ends.  Host code never passes the array's name to a
// kernel: in host code it is a host-side stand-in, not a device address.
static __device__ __align__(256) unsigned char scratch[vdsa::STATIC_SCRATCH_BYTES];

namespace vdsa {
namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device ordinal, nullptr until resolved
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[(size_t)dev] == nullptr) {
    // with `dev` current: this device's copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (uintptr_t)p % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[(size_t)dev] = p;
  }
  *ptr = g_scratch_ptr[(size_t)dev];
  return hipSuccess;
}

}  // namespace vdsa
