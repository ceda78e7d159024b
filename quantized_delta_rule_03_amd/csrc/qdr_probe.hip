// qdr_probe.hip -- measurement helpers of libqdr (not part of the decode path).
//
//  - k_probe_copy: a streaming HBM copy (16-byte loads and stores, grid-stride, 4
//    work-groups per CU), the achievable read+write bandwidth that the decode kernels are
//    measured against next to the nominal 8 TB/s.
//  - k_probe_clock: every work-group runs a long dependent chain of fp32 fmas (the VALU
//    busy, as in the decode step) and one lane records the shader cycle counter and the
//    constant-rate counter before and after; their ratio is the engine clock the chip
//    sustained under that load.
//  - k_probe_clock_trace: one lane samples both counters every `period` constant-rate
//    ticks (sleeping in between), so that it can run beside other kernels on another
//    stream and give the engine clock they ran at, interval by interval. It holds one
//    wave and a few registers, and ends after n_sample samples whatever else runs.
#include <stdio.h>

#include "../../include/qdr.h"
#include "qdr_internal.h"

namespace qdr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_probe_copy(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, size_t n) {
  // grid-stride, one 16-byte load and store per thread and iteration (of the variants
  // measured -- 1, 4 or 8 loads in flight per thread, non-temporal hints, contiguous
  // per-group chunks, 4 to 64 groups per CU -- this with 4 groups per CU moved the most)
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(256) k_probe_clock(unsigned long long* out, int iters,
                                                     float seed) {
  unsigned long long c0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    c0 = __builtin_readcyclecounter();
    w0 = __builtin_amdgcn_s_memrealtime();
  }
  float x = seed + (float)threadIdx.x, y = 1.0f - seed;
  for (int i = 0; i < iters; ++i) {
    x = fmaf(x, 0.999999f, y);
    y = fmaf(y, 0.999999f, x);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long c1 = __builtin_readcyclecounter();
    const unsigned long long w1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* o = out + (size_t)blockIdx.x * 4;
    o[0] = c1 - c0;
    o[1] = w1 - w0;
    o[2] = (unsigned long long)(x + y != 12345.0f);  // keeps the chain live
    o[3] = 0;
  }
}

__global__ void __launch_bounds__(64) k_probe_clock_trace(unsigned long long* out,
                                                          int n_sample, int period) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < n_sample; ++i) {
    const unsigned long long due = r0 + (unsigned long long)i * (unsigned)period;
    unsigned long long r = __builtin_amdgcn_s_memrealtime();
    while (r < due) {  // the counter only moves forward: every wait ends
      __builtin_amdgcn_s_sleep(4);
      r = __builtin_amdgcn_s_memrealtime();
    }
    out[2 * (size_t)i] = __builtin_readcyclecounter();
    out[2 * (size_t)i + 1] = r;
  }
}

}  // namespace
}  // namespace qdr

namespace {
thread_local char g_probe_err[256];
}

extern "C" {

int qdr_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || (bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_copy: null, unaligned or odd size");
    return QDR_EINVAL;
  }
  const size_t n = bytes / 16;
  if (n == 0) return QDR_OK;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  size_t blocks = (size_t)(cus > 0 ? cus : 256) * 4;
  const size_t need = (n + 255) / 256;
  if (need < blocks) blocks = need;
  hipLaunchKernelGGL(qdr::k_probe_copy, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const qdr::u32x4*>(src), static_cast<qdr::u32x4*>(dst), n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_copy: %s", hipGetErrorString(e));
    return QDR_EHIP;
  }
  return QDR_OK;
}

int qdr_probe_clock(unsigned long long* out, int32_t n_block, int32_t iters, void* stream) {
  if (!out || n_block < 1 || iters < 1) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_clock: bad arguments");
    return QDR_EINVAL;
  }
  hipLaunchKernelGGL(qdr::k_probe_clock, dim3((unsigned)n_block), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters, 0.5f);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_clock: %s", hipGetErrorString(e));
    return QDR_EHIP;
  }
  return QDR_OK;
}

int qdr_probe_clock_trace(unsigned long long* out, int32_t n_sample, int32_t period,
                          void* stream) {
  if (!out || n_sample < 1 || n_sample > (1 << 20) || period < 1 || period > (1 << 24)) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_clock_trace: bad arguments");
    return QDR_EINVAL;
  }
  hipLaunchKernelGGL(qdr::k_probe_clock_trace, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out, n_sample, period);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_clock_trace: %s",
             hipGetErrorString(e));
    return QDR_EHIP;
  }
  return QDR_OK;
}

int qdr_probe_wall_rate(double* hz) {
  int dev = 0, khz = 0;
  if (!hz) return QDR_EINVAL;
  (void)hipGetDevice(&dev);
  const hipError_t e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess || khz <= 0) {
    snprintf(g_probe_err, sizeof(g_probe_err), "qdr_probe_wall_rate: no wall clock rate");
    return QDR_EHIP;
  }
  *hz = 1e3 * (double)khz;
  return QDR_OK;
}

const char* qdr_probe_last_error(void) { return g_probe_err; }

}  // extern "C"
