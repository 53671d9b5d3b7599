// Test fixture, not part of the library: exposes the fp8 matrix instruction
// the narrow-QK decode path uses (v_mfma_scale_f32_16x16x128_f8f6f4 with unit
// block scales, accumulator starting at zero) on caller-given e4m3 codes, so
// a test can measure how far its sum of the 128 exact code products lies
// from the exact sum ("FP8 KV attention: hardware paths and tile
// preparation", section "AMD CDNA 3": FP8 operands, FP32 accumulation).
//
// One wave per 16x16 tile: out[tile][i][j] = sum over k of
// value(a[tile][i][k]) * value(b[tile][j][k]), k < 128.  Lane l supplies
// row / column l % 16 and the 32 bytes 32 * (l / 16) .. + 31 of that row in
// both operands; the instruction pairs byte p of lane l in A with byte p of
// lane l in B, so the same (lane group, byte) -> k assignment on both sides
// gives the full 128-term dot product whatever that assignment is.  The
// result holds rows 4 * (l / 16) .. + 3 of column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void fp8_mfma_tiles(const uint8_t* __restrict__ a,
                                                     const uint8_t* __restrict__ b,
                                                     float* __restrict__ out) {
  const int tile = blockIdx.x;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const size_t base = (size_t)tile * 16 * 128 + (size_t)r * 128 + 32 * g;
  const i32x8_t av = *reinterpret_cast<const i32x8_t*>(a + base);
  const i32x8_t bv = *reinterpret_cast<const i32x8_t*>(b + base);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  float* o = out + (size_t)tile * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[(4 * g + i) * 16 + r] = acc[i];
}

extern "C" int fp8_mfma_probe(const uint8_t* a, const uint8_t* b, float* out, int n_tiles,
                              void* stream) {
  if (n_tiles <= 0 || !a || !b || !out) return -1;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) % 32 != 0) return -1;
  hipLaunchKernelGGL(fp8_mfma_tiles, dim3(n_tiles), dim3(64), 0,
                     static_cast<hipStream_t>(stream), a, b, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
