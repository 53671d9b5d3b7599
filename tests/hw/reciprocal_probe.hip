// Test fixture, not part of the library: reciprocal_rn (the library's
// device.h) against the correctly rounded division 1.0f / s, for every fp32
// bit pattern s in [lo, hi] (positive, normal).  Counts the patterns that
// differ and keeps up to 16 of them.
#include "device.h"

__global__ __launch_bounds__(256) void reciprocal_probe(uint32_t lo, uint32_t hi,
                                                        unsigned long long* bad, uint32_t* kept) {
  const uint32_t stride = gridDim.x * blockDim.x;
  unsigned long long n = 0;
  for (uint64_t u = (uint64_t)lo + blockIdx.x * blockDim.x + threadIdx.x; u <= hi; u += stride) {
    const float s = __uint_as_float((uint32_t)u);
    if (__float_as_uint(fp8kv::reciprocal_rn(s)) != __float_as_uint(1.0f / s)) {
      ++n;
      const uint32_t slot = atomicAdd(&kept[0], 1u);
      if (slot < 16) kept[1 + slot] = (uint32_t)u;
    }
  }
  if (n) atomicAdd(bad, n);
}

// bad: one zeroed 64-bit word; kept: 17 zeroed words.
extern "C" int reciprocal_probe_launch(uint32_t lo, uint32_t hi, unsigned long long* bad,
                                       uint32_t* kept, void* stream) {
  if (!bad || !kept || lo > hi) return -1;
  hipLaunchKernelGGL(reciprocal_probe, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     lo, hi, bad, kept);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
