// Append: quantise new K/V rows and write them once into the paged cache.
//
// Storage rule ("kadirnar/kernel-agent/fp8-kv-cache", section "Storage"):
// one fp32 scale per (token, KV head) row, scale = amax(|row|) / 448 over the
// head dimension, codes in e4m3, written at append and never re-quantised.
//
// Mapping: a row of D fp32 values is read by D/4 lanes with one 16-byte load
// each (32 lanes for D = 128, 16 for D = 64), so a wave covers the K row and
// the V row of one or two (token, head) pairs and every HBM access is a full,
// coalesced 16-byte-per-lane transaction.  The row maximum is a butterfly
// over those lanes.  The quotient x / scale uses the correctly rounded fp32
// division (no reciprocal, no fast-math) so the codes are bit-exact with the
// definition; v_cvt_pk_fp8_f32 rounds to nearest even onto OCP e4m3fn, and
// the explicit clamp to +-448 makes rows whose scale is an fp32 subnormal
// saturate instead of overflowing.
#include "device.h"
#include "launch.h"

namespace fp8kv {

struct AppendArgs {
  const float* k_new;
  const float* v_new;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* table;
  void* k;
  void* v;
  float* ks;
  float* vs;
  int64_t n_rows;  // 2 * n_tok * hkv: K and V rows interleaved per (token, head)
  int hkv;
  int bs;
  int mbps;
  int num_seqs;
  int num_blocks;
};

template <int MODE, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int kLanesPerRow = D / 4;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row_id = gtid / kLanesPerRow;
  const int sub = (int)(gtid % kLanesPerRow);
  // All lanes of one row leave together, so the butterfly below never reads
  // an inactive lane.
  if (row_id >= a.n_rows) return;
  const int is_v = (int)(row_id & 1);
  const int64_t pair = row_id >> 1;
  const int64_t tok = pair / a.hkv;
  const int h = (int)(pair % a.hkv);
  const int seq = a.seq_idx[tok];
  const int p = a.pos[tok];
  // Out-of-range device data is skipped, never followed (uniform per row).
  if (seq < 0 || seq >= a.num_seqs || p < 0 || p >= a.mbps * a.bs) return;
  const int blk = a.table[(int64_t)seq * a.mbps + p / a.bs];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int64_t row = ((int64_t)blk * a.bs + p % a.bs) * a.hkv + h;

  const float* src = (is_v ? a.v_new : a.k_new) + pair * D + 4 * sub;
  const float4 x = *reinterpret_cast<const float4*>(src);

  const bool quantise = (MODE == kK8V8) || (MODE == kK16V8 && is_v);
  if (quantise) {
    float amax = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
#pragma unroll
    for (int o = kLanesPerRow / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax / kE4M3Max;  // correctly rounded fp32 division
    uint32_t codes = 0;
    if (scale != 0.0f) {
      const float y0 = fminf(fmaxf(x.x / scale, -kE4M3Max), kE4M3Max);
      const float y1 = fminf(fmaxf(x.y / scale, -kE4M3Max), kE4M3Max);
      const float y2 = fminf(fmaxf(x.z / scale, -kE4M3Max), kE4M3Max);
      const float y3 = fminf(fmaxf(x.w / scale, -kE4M3Max), kE4M3Max);
      codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)codes, true);
    }
    uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v : a.k) + row * D + 4 * sub;
    *reinterpret_cast<uint32_t*>(dst) = codes;
    if (sub == 0) (is_v ? a.vs : a.ks)[row] = scale;
  } else {
    u32x2_t w;
    w[0] = f32x2_to_bf16x2(x.x, x.y);
    w[1] = f32x2_to_bf16x2(x.z, x.w);
    uint16_t* dst = static_cast<uint16_t*>(is_v ? a.v : a.k) + row * D + 4 * sub;
    *reinterpret_cast<u32x2_t*>(dst) = w;
  }
}

template <int MODE>
static hipError_t append_for_d(const CacheView& c, const AppendArgs& a, hipStream_t stream) {
  const int lanes = c.d / 4;
  const int64_t threads = a.n_rows * lanes;
  const int64_t blocks = (threads + 255) / 256;
  if (c.d == 128)
    hipLaunchKernelGGL((append_kernel<MODE, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((append_kernel<MODE, 64>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& c, const float* k_new, const float* v_new,
                         const int32_t* seq_idx, const int32_t* pos, int n_tok,
                         hipStream_t stream) {
  AppendArgs a{k_new, v_new, seq_idx, pos, c.table, c.k, c.v, c.ks, c.vs,
               2 * (int64_t)n_tok * c.hkv, c.hkv, c.bs, c.mbps, c.num_seqs, c.num_blocks};
  switch (c.mode) {
    case kK8V8: return append_for_d<kK8V8>(c, a, stream);
    case kK16V8: return append_for_d<kK16V8>(c, a, stream);
    default: return append_for_d<kBF16>(c, a, stream);
  }
}

}  // namespace fp8kv
