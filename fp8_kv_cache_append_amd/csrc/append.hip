// Append: quantise new K/V rows and write them once into the paged cache.
//
// Storage rule ("kadirnar/kernel-agent/fp8-kv-cache", section "Storage"):
// one fp32 scale per (token, KV head) row, scale = amax(|row|) / 448 over the
// head dimension, codes in e4m3, written at append and never re-quantised.
//
// Mapping: a row of D fp32 values is read by D/4 lanes with one 16-byte load
// each (32 lanes for D = 128, 16 for D = 64), so a wave covers the K row and
// the V row of one or two (token, head) pairs and every HBM access is a full,
// coalesced 16-byte-per-lane transaction.  The arithmetic (row_amax,
// e4m3_codes4, bf16x4 in device.h) is shared with the fused append of the
// split-KV decode, so both write the same bytes.
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
  uint8_t* kexp;   // kMXK8V8: E8M0 byte per 32-value K block
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

  const bool quantise = is_v ? v_is_e4m3(MODE) : k_is_e4m3(MODE);
  if (k_is_mx(MODE) && !is_v) {
    // block-scaled K: eight lanes hold a block of 32 values
    const int e = mx_exponent(row_amax<8>(x));
    uint8_t* dst = static_cast<uint8_t*>(a.k) + row * D + 4 * sub;
    *reinterpret_cast<uint32_t*>(dst) = e4m3_codes4(x, e8m0_value((uint32_t)(e + 127)));
    if ((sub & 7) == 0) a.kexp[row * (D / 32) + sub / 8] = (uint8_t)(e + 127);
  } else if (quantise) {
    const float scale = row_amax<kLanesPerRow>(x) / kE4M3Max;  // correctly rounded
    uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v : a.k) + row * D + 4 * sub;
    *reinterpret_cast<uint32_t*>(dst) = e4m3_codes4(x, scale);
    if (sub == 0) (is_v ? a.vs : a.ks)[row] = scale;
  } else {
    uint16_t* dst = static_cast<uint16_t*>(is_v ? a.v : a.k) + row * D + 4 * sub;
    *reinterpret_cast<u32x2_t*>(dst) = bf16x4(x);
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
  AppendArgs a{k_new, v_new, seq_idx, pos, c.table, c.k, c.v, c.ks, c.vs, c.kexp,
               2 * (int64_t)n_tok * c.hkv, c.hkv, c.bs, c.mbps, c.num_seqs, c.num_blocks};
  switch (c.mode) {
    case kK8V8: return append_for_d<kK8V8>(c, a, stream);
    case kK16V8: return append_for_d<kK16V8>(c, a, stream);
    case kK8V16: return append_for_d<kK8V16>(c, a, stream);
    case kMXK8V8: return append_for_d<kMXK8V8>(c, a, stream);
    default: return append_for_d<kBF16>(c, a, stream);
  }
}

}  // namespace fp8kv
