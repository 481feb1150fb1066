// Fixed device scratch for the no-allocation attention entry point
// (msa_sparse_attn_fwd_noalloc): callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation) run the attention call with this array as its workspace.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, from module load until the process
// ends.  In host code its name is only a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and cached; launches get that address, never the name.
// Every call on one GPU shares the array and it keeps the last call's
// contents: the kernels that use it clear what must start at zero themselves,
// and calls that overlap in time on one GPU (two streams) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace msa {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace msa
