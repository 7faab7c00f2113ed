// Device scratch of the allocation-free reduce-scatter
// (tide_reduce_scatter_local_noalloc), for callers that cannot allocate
// device memory: a fixed array in device memory that holds the tables of the
// latest such call on a device, and the put kernel that writes them there.
//
// The tables (chunk table, segment headers, source and destination pointers;
// the same tables the reduce-scatter kernels read from plan-owned memory in
// the allocating entry point) travel as kernel arguments of put launches, so
// a call needs no staging buffer and stays asynchronous on its stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "tide_internal.h"

// The array exists once per device for the life of the process.  In host code
// its name is only a stand-in for the symbol, not a device address: host code
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[tide::kScratchBytes];

namespace {

// Words carried by one put launch, in its kernel arguments (at most 4 KiB).
struct ScratchPut {
  uint64_t* dst;
  uint32_t nwords;
  uint32_t unused;
  uint64_t words[tide::kPutWords];
};
static_assert(sizeof(ScratchPut) <= 4096, "kernel arguments of a put launch");

__global__ __launch_bounds__(tide::kThreads) void scratch_put_kernel(ScratchPut a) {
  for (uint32_t i = threadIdx.x; i < a.nwords; i += tide::kThreads) {
    __attribute__((address_space(1))) uint64_t* d = (__attribute__((address_space(1))) uint64_t*)(a.dst + i);
    *d = a.words[i];
  }
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[tide::kMaxDevices] = {};

}  // namespace

namespace tide {

int scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return int(hipSuccess);
}

int launch_scratch_put(void* dst, const uint64_t* words, uint32_t nwords, void* stream) {
  ScratchPut a;
  a.dst = static_cast<uint64_t*>(dst);
  a.nwords = nwords;
  a.unused = 0;
  for (uint32_t i = 0; i < nwords; ++i) a.words[i] = words[i];
  hipLaunchKernelGGL(scratch_put_kernel, dim3(1), dim3(unsigned(kThreads)), 0, static_cast<hipStream_t>(stream), a);
  return int(hipGetLastError());
}

}  // namespace tide
