// Dequantisation of a stored cache into a bf16 cache of the same geometry:
// the unfused control, which converts the cache before attention instead of
// converting only the active tile on chip ("Fused KV-cache quantization";
// the dtype controls of "FP8 KV attention: hardware paths and tile
// preparation", "Collect the profiler evidence").
//
// Each element of an e4m3 side becomes bf16(fp32(value(code) * scale)): the
// packed convert gives the exact fp32 value, one fp32 multiply rounds the
// product, v_cvt_pk_bf16_f32 rounds it to nearest even.  A bf16 side is
// copied.  Rows are read and written D/16 lanes at a time (16 elements per
// lane: one 16-byte load of codes, two 16-byte stores), K and V rows of one
// (slot, head) interleaved.
#include "device.h"
#include "launch.h"

namespace fp8kv {

struct DequantArgs {
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  uint16_t* dk;
  uint16_t* dv;
  int64_t n_rows;  // 2 * cache rows (K and V)
};

template <int MODE, int D>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  constexpr int kLanesPerRow = D / 16;  // 16 elements per lane: one 16-byte load of codes
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row_id = gtid / kLanesPerRow;
  const int sub = (int)(gtid % kLanesPerRow);
  if (row_id >= a.n_rows) return;
  const bool is_v = (row_id & 1) != 0;
  const int64_t row = row_id >> 1;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>((is_v ? a.dv : a.dk) + row * D + 16 * sub);
  const bool e4m3 = is_v ? v_is_e4m3(MODE) : k_is_e4m3(MODE);
  if (e4m3) {
    const u32x4_t codes = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(is_v ? a.v : a.k) + row * D)[sub];
    // source and destination share the layout, so row r is the same
    // (token, head) in both, and its scale is element r
    const float s = (is_v ? a.vs : a.ks)[row];
    uint32_t out[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], true);
      out[2 * w] = f32x2_to_bf16x2(lo[0] * s, lo[1] * s);
      out[2 * w + 1] = f32x2_to_bf16x2(hi[0] * s, hi[1] * s);
    }
    dst[0] = u32x4_t{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4_t{out[4], out[5], out[6], out[7]};
  } else {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint16_t*>(is_v ? a.v : a.k) + row * D + 16 * sub);
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

template <int MODE>
static hipError_t dequant_for_d(int d, const DequantArgs& a, hipStream_t stream) {
  const int64_t threads = a.n_rows * (d / 16);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0xFFFFFFFFll) return hipErrorInvalidValue;
  if (d == 128)
    hipLaunchKernelGGL((dequantize_kernel<MODE, 128>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((dequantize_kernel<MODE, 64>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const CacheView& src, const CacheView& dst, hipStream_t stream) {
  DequantArgs a{src.k, src.v, src.ks, src.vs, static_cast<uint16_t*>(dst.k),
                static_cast<uint16_t*>(dst.v),
                2 * (int64_t)src.num_blocks * src.bs * src.hkv};
  switch (src.mode) {
    case kK8V8: return dequant_for_d<kK8V8>(src.d, a, stream);
    case kK16V8: return dequant_for_d<kK16V8>(src.d, a, stream);
    case kK8V16: return dequant_for_d<kK8V16>(src.d, a, stream);
    case kBF16: return dequant_for_d<kBF16>(src.d, a, stream);
    default: return hipErrorInvalidValue;  // block-scaled K: rejected by the caller
  }
}

}  // namespace fp8kv
