// Instruments of the interference measurements on one MI355X (gfx950), after
// "The Endgame of FSDP Communication" (Wang et al.), Section 2.2 (SM wave
// quantization, Equation 4), Figure 3, Table 4 (victim slowdown) and Table 5
// (SM-id probe):
//   hw_probe_kernel  the analog of the pages' SM-id probe: every workgroup
//                    records where it ran (the hardware-ID and XCC-ID
//                    registers) and when it entered and left (the constant-
//                    rate wall clock), holding its CU for a given time with as
//                    much LDS as asked, so that one probe workgroup can fill a
//                    CU the way one GEMM CTA fills an SM;
//   axpb_kernel      the memory-bound elementwise victim (y = a * x + b);
// and CU-masked streams, the hard counterpart of a grid-limited CU budget.
// Host code of their C ABI is at the end of this file.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "tide_internal.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeWords = 8;  // uint32 words per probe record
constexpr int kAxpbThreads = 256;

// The workgroup's dynamic LDS (its size is the launch's): the probe claims
// it so that nothing else that needs LDS fits beside it on its CU.
extern __shared__ uint32_t s_probe[];

__device__ __forceinline__ uint32_t hw_id_register() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
  return v;
}

__device__ __forceinline__ uint32_t xcc_id_register() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

// Record of workgroup b at rec[8b ..]: b, HW_ID, XCC_ID, 0, entry time (lo,
// hi), exit time (lo, hi), times in wall-clock ticks.  The hold loop ends once
// the wall clock, which only moves forward, has advanced hold_ticks.
__global__ __launch_bounds__(kProbeThreads) void hw_probe_kernel(uint32_t* __restrict__ rec, int64_t hold_ticks,
                                                                 int32_t touch_lds) {
  const uint64_t t0 = wall_clock64();
  const uint32_t hw = hw_id_register();
  const uint32_t xcc = xcc_id_register();
  if (touch_lds && threadIdx.x == 0) s_probe[0] = hw;
  uint64_t t = t0;
  while (int64_t(t - t0) < hold_ticks) t = wall_clock64();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* r = rec + size_t(blockIdx.x) * kProbeWords;
    r[0] = blockIdx.x;
    r[1] = hw;
    r[2] = xcc;
    r[3] = touch_lds ? s_probe[0] ^ hw : 0u;  // 0: the LDS word read back intact
    r[4] = uint32_t(t0);
    r[5] = uint32_t(t0 >> 32);
    r[6] = uint32_t(t);
    r[7] = uint32_t(t >> 32);
  }
}

// y = a * x + b: one binary32 product, then one binary32 sum (the library is
// built without contraction).  Each thread takes one group of four elements
// (16-byte accesses) when VEC, else one element.
template <bool VEC>
__global__ __launch_bounds__(kAxpbThreads) void axpb_kernel(const float* __restrict__ x, float* __restrict__ y,
                                                            int64_t n, float a, float b) {
  const int64_t i = int64_t(blockIdx.x) * kAxpbThreads + threadIdx.x;
  if constexpr (VEC) {
    if (4 * i < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(x + 4 * i);
      f32x4 p;
      p.x = a * v.x;
      p.y = a * v.y;
      p.z = a * v.z;
      p.w = a * v.w;
      *reinterpret_cast<f32x4*>(y + 4 * i) = f32x4{p.x + b, p.y + b, p.z + b, p.w + b};
    }
  } else {
    if (i < n) {
      const float p = a * x[i];
      y[i] = p + b;
    }
  }
}

tide_status hip_error(hipError_t e, const char* what) {
  return tide::set_error(TIDE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

tide_status current_attribute(hipDeviceAttribute_t attr, int32_t* out, const char* what) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e, "hipGetDevice");
  int v = 0;
  e = hipDeviceGetAttribute(&v, attr, dev);
  if (e != hipSuccess) return hip_error(e, what);
  *out = v;
  return TIDE_OK;
}

}  // namespace

extern "C" {

tide_status tide_device_info(int32_t* cu_count, int32_t* max_lds_per_workgroup, int32_t* lds_per_cu,
                             int32_t* wall_clock_khz) {
  return tide::guarded([&]() -> tide_status {
    tide::clear_error();
    tide_status st;
    if (lds_per_cu &&
        (st = current_attribute(hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, lds_per_cu,
                                "hipDeviceGetAttribute")) != TIDE_OK)
      return st;
    if (cu_count &&
        (st = current_attribute(hipDeviceAttributeMultiprocessorCount, cu_count, "hipDeviceGetAttribute")) != TIDE_OK)
      return st;
    if (max_lds_per_workgroup &&
        (st = current_attribute(hipDeviceAttributeMaxSharedMemoryPerBlock, max_lds_per_workgroup,
                                "hipDeviceGetAttribute")) != TIDE_OK)
      return st;
    if (wall_clock_khz &&
        (st = current_attribute(hipDeviceAttributeWallClockRate, wall_clock_khz, "hipDeviceGetAttribute")) != TIDE_OK)
      return st;
    return TIDE_OK;
  });
}

tide_status tide_probe_launch(uint32_t* records, int32_t grid, int32_t lds_bytes, int64_t hold_ns, void* stream) {
  return tide::guarded([&]() -> tide_status {
    tide::clear_error();
    if (records == nullptr) return tide::set_error(TIDE_ERR_INVALID, "records must not be NULL");
    if (reinterpret_cast<uintptr_t>(records) & 3)
      return tide::set_error(TIDE_ERR_ALIGN, "records is not 4-byte aligned");
    if (grid < 1 || grid > 65536) return tide::set_error(TIDE_ERR_INVALID, "grid must be in [1, 65536]");
    if (hold_ns < 0 || hold_ns > 1000000000) return tide::set_error(TIDE_ERR_INVALID, "hold_ns must be in [0, 1e9]");
    int32_t max_lds = 0, khz = 0;
    tide_status st = tide_device_info(nullptr, &max_lds, nullptr, &khz);
    if (st != TIDE_OK) return st;
    if (lds_bytes < 0 || lds_bytes > max_lds)
      return tide::set_error(TIDE_ERR_INVALID, "lds_bytes must be in [0, " + std::to_string(max_lds) + "]");
    if (lds_bytes > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&hw_probe_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
      if (e != hipSuccess) return hip_error(e, "hipFuncSetAttribute");
    }
    const int64_t ticks = hold_ns * int64_t(khz) / 1000000;
    hipLaunchKernelGGL(hw_probe_kernel, dim3(unsigned(grid)), dim3(unsigned(kProbeThreads)), size_t(lds_bytes),
                       static_cast<hipStream_t>(stream), records, ticks, int32_t(lds_bytes >= 4));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "hw_probe_kernel launch");
    return TIDE_OK;
  });
}

tide_status tide_victim_axpb(const float* x, float* y, int64_t n, float a, float b, void* stream) {
  return tide::guarded([&]() -> tide_status {
    tide::clear_error();
    if (n < 0) return tide::set_error(TIDE_ERR_INVALID, "n must be >= 0");
    if (n == 0) return TIDE_OK;
    if (x == nullptr || y == nullptr) return tide::set_error(TIDE_ERR_INVALID, "x and y must not be NULL");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 3)
      return tide::set_error(TIDE_ERR_ALIGN, "x and y must be 4-byte aligned");
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0 && n % 4 == 0;
    const int64_t items = vec ? n / 4 : n;
    const int64_t grid = (items + kAxpbThreads - 1) / kAxpbThreads;
    if (grid > INT32_MAX) return tide::set_error(TIDE_ERR_RANGE, "n is too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vec) {
      hipLaunchKernelGGL(axpb_kernel<true>, dim3(unsigned(grid)), dim3(unsigned(kAxpbThreads)), 0, s, x, y, n, a, b);
    } else {
      hipLaunchKernelGGL(axpb_kernel<false>, dim3(unsigned(grid)), dim3(unsigned(kAxpbThreads)), 0, s, x, y, n, a, b);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "axpb_kernel launch");
    return TIDE_OK;
  });
}

tide_status tide_stream_create(const uint32_t* cu_mask, int32_t mask_words, void** out_stream) {
  return tide::guarded([&]() -> tide_status {
    tide::clear_error();
    if (out_stream == nullptr) return tide::set_error(TIDE_ERR_INVALID, "out_stream must not be NULL");
    *out_stream = nullptr;
    hipStream_t s = nullptr;
    hipError_t e;
    if (cu_mask == nullptr) {
      e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    } else {
      int32_t cus = 0;
      tide_status st = tide_device_info(&cus, nullptr, nullptr, nullptr);
      if (st != TIDE_OK) return st;
      if (mask_words < 1 || int64_t(mask_words) * 32 < cus)
        return tide::set_error(TIDE_ERR_INVALID, "cu_mask must have at least ceil(cu_count / 32) = " +
                                                     std::to_string((cus + 31) / 32) + " words");
      bool any = false;
      for (int32_t i = 0; i < cus; ++i) any = any || ((cu_mask[i / 32] >> (i % 32)) & 1u);
      if (!any) return tide::set_error(TIDE_ERR_INVALID, "cu_mask selects no CU");
      e = hipExtStreamCreateWithCUMask(&s, uint32_t(mask_words), cu_mask);
    }
    if (e != hipSuccess) return hip_error(e, cu_mask ? "hipExtStreamCreateWithCUMask" : "hipStreamCreateWithFlags");
    *out_stream = s;
    return TIDE_OK;
  });
}

tide_status tide_stream_destroy(void* stream) {
  return tide::guarded([&]() -> tide_status {
    tide::clear_error();
    if (stream == nullptr) return TIDE_OK;
    hipError_t e = hipStreamDestroy(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_error(e, "hipStreamDestroy");
    return TIDE_OK;
  });
}

}  // extern "C"
