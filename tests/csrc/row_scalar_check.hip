// Checks the row kernel's short reciprocal and square-root sequences against
// the IEEE ones hipcc emits for '/' and __builtin_sqrtf, over every positive
// normal fp32 input (2^31 - 2^24 values), on the GPU. Prints per-range counts
// of differences. Uses the library's own device helpers.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include "rnq_device.h"

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s\n", hipGetErrorString(e_)); return 1; } } while (0)

constexpr uint32_t PER = 256;  // inputs per thread

__global__ void check(uint32_t base, uint32_t n_threads, uint32_t* __restrict__ bad) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_threads) return;
  uint32_t b_rcp = 0, b_sqrt = 0;
  for (uint32_t i = 0; i < PER; ++i) {
    const float s = __uint_as_float(base + t * PER + i);
    b_rcp += __float_as_uint(rnq::rcp_rn_fast(s)) != __float_as_uint(1.0f / s);
    b_sqrt += __float_as_uint(rnq::sqrt_rn_fast(s)) != __float_as_uint(__builtin_sqrtf(s));
  }
  bad[2 * t] = b_rcp;
  bad[2 * t + 1] = b_sqrt;
}

int main() {
  const uint32_t chunk = 1u << 24, nt = chunk / PER;
  uint32_t* d = nullptr;
  CK(hipMalloc(&d, (size_t)nt * 2 * sizeof(uint32_t)));
  uint32_t* h = (uint32_t*)malloc((size_t)nt * 2 * sizeof(uint32_t));
  // reciprocal: claimed exact for s in [2^-126, 2^126); square root: for v >= 2^-105
  unsigned long long rcp_in = 0, rcp_out = 0, sq_in = 0, sq_out = 0;
  for (uint32_t base = 0x00800000u; base < 0x7f800000u; base += chunk) {
    hipLaunchKernelGGL(check, dim3(nt / 256), dim3(256), 0, 0, base, nt, d);
    CK(hipGetLastError());
    CK(hipMemcpy(h, d, (size_t)nt * 2 * sizeof(uint32_t), hipMemcpyDeviceToHost));
    unsigned long long r = 0, q = 0;
    for (uint32_t i = 0; i < nt; ++i) { r += h[2 * i]; q += h[2 * i + 1]; }
    const int e0 = (int)(base >> 23) - 127;  // inputs of this chunk lie in [2^e0, 2^(e0+2))
    if (e0 + 2 <= 126) rcp_in += r; else rcp_out += r;
    if (e0 >= -105) sq_in += q; else sq_out += q;
  }
  printf("rcp_mismatch_in_range %llu\nrcp_mismatch_outside %llu\nsqrt_mismatch_in_range %llu\nsqrt_mismatch_outside %llu\n",
         rcp_in, rcp_out, sq_in, sq_out);
  free(h);
  CK(hipFree(d));
  return 0;
}
