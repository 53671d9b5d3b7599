// Benchmark fixture, not part of the library: a plain streaming read of n
// bytes (16-byte loads, grid-stride), for the HBM read floor a single
// launch of a given size reaches on this device.  Each work-group folds
// what it read into one word (xor) and writes it, so the loads cannot be
// dropped; the writes are 4 bytes per work-group.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read(const u32x4_t* __restrict__ src, uint64_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

// n_bytes a multiple of 16, src 16-byte aligned, sink holds n_blocks words.
extern "C" int stream_read_launch(const void* src, uint64_t n_bytes, uint32_t* sink,
                                  int n_blocks, void* stream) {
  if (!src || !sink || n_bytes % 16 != 0 || n_blocks <= 0) return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return -1;
  hipLaunchKernelGGL(stream_read, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), n_bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
