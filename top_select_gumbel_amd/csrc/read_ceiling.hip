// read_ceiling.hip -- diagnostic: a plain streaming read of a device array, launched with the
// same shape as the sampling stream kernel (256-thread workgroups, eight non-temporal 16-byte
// loads per thread, all issued before any is consumed), so that its bandwidth is the ceiling
// the stream kernel's is compared against. Each wave writes the fp32 sum of the elements it
// read to its own slot (no atomics), which keeps the loads; the partials sum to the total.
#include <stdint.h>

#include "topselect.h"
#include "ts_device.hpp"
#include "ts_host.hpp"

namespace {

constexpr int kRT1 = 256;
constexpr int kRS = 8;

__global__ __launch_bounds__(kRT1) void ts_read_kernel(const float* x, int64_t n, float* out) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t n4 = n >> 2;
  const int64_t base = (int64_t)blockIdx.x * kRT1 * kRS + threadIdx.x;
  float acc = 0.0f;
  u32x4 v[kRS];
#pragma unroll
  for (int s = 0; s < kRS; ++s) {
    const int64_t q = base + (int64_t)s * kRT1;
    v[s] = q < n4 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + q) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int s = 0; s < kRS; ++s)
    acc += (__uint_as_float(v[s].x) + __uint_as_float(v[s].y)) + (__uint_as_float(v[s].z) + __uint_as_float(v[s].w));
  if (blockIdx.x == 0) {   // the scalar tail past the last whole float4
    for (int64_t i = 4 * n4 + threadIdx.x; i < n; i += kRT1) acc += x[i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (tsd::lane() == 0) out[(int64_t)blockIdx.x * (kRT1 / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

extern "C" int ts_read_ceiling(const float* x, int64_t n, float* out, void* stream) {
  using tsh::fail;
  if (n < 0) return fail(TS_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n == 0) return TS_OK;
  if (!x || !out) return fail(TS_ERR_INVALID_ARG, "x and out are required");
  if (((uintptr_t)x & 15u) != 0) return fail(TS_ERR_INVALID_ARG, "x must be 16-byte aligned");
  const int64_t per = (int64_t)kRT1 * kRS * 4;   // floats per workgroup
  const int64_t blocks = (n + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return fail(TS_ERR_INVALID_ARG, "n too large");
  int dev;
  const int rc = tsh::check_device(&dev);
  if (rc != TS_OK) return rc;
  hipLaunchKernelGGL(ts_read_kernel, dim3((unsigned)blocks), dim3(kRT1), 0, (hipStream_t)stream, x, n, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "read launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}
