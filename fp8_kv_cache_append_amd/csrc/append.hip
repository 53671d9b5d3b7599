// Append: quantise new K/V rows and write them once into the paged cache.
//
// Storage rule ("kadirnar/kernel-agent/fp8-kv-cache", section "Storage"):
// one fp32 scale per (token, KV head) row, scale = amax(|row|) / 448 over the
// head dimension, codes in e4m3, written at append and never re-quantised.
// A row (one (token, KV head) pair) of a block sits at the index the cache's
// layout gives it (cache_row: token-major [slot][head] or head-major
// [head][slot]); its codes, scale and K exponents all use that index.
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
  int n_rows;      // 2 * n_tok * hkv (< 2^31): K and V rows interleaved per (token, head)
  int hkv;
  int bs;
  int mbps;
  int num_seqs;
  int num_blocks;
  int layout;
  FastDiv div_hkv;  // by hkv: the token of a (token, head) pair
  FastDiv div_bs;   // by bs: the block of a position
};

// Rows per thread: for a bulk append each thread handles R = 4 rows one
// grid-sized stride apart and issues all their loads (the fp32 values, then
// the token's sequence and position) before it uses any, so a wave keeps
// 4 KB of input in flight instead of waiting on one dependent chain
// (indices, block id, values) per kilobyte.  An append too small to fill the
// GPU (a decode step's rows) takes R = 1: there the per-row vector work, not
// the memory, sets the time, and it is better spread over more threads.
constexpr int kBulkRowsPerThread = 4;
constexpr int64_t kBulkThreads = 256 * 2048;  // threads the compute units hold at once
constexpr int kAppendThreads = 256;           // threads per work-group

// ROW32: the cache has fewer than 2^31 rows (checked on the host), so a row
// index is computed in 32 bits and its address is one multiply-add onto the
// lane's base.
template <int MODE, int D, int R, bool ROW32>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int kLanesPerRow = D / 4;
  // Row indices fit in 32 bits (checked on the host), so the per-row
  // divisions by the head count and the block size are 32-bit.
  const uint32_t gtid = blockIdx.x * kAppendThreads + threadIdx.x;
  // rows per sweep: even (a work-group holds 8 or 16 rows), so every row of
  // a thread is a K row or every one a V row, as its first row is
  const uint32_t slots = gridDim.x * (kAppendThreads / kLanesPerRow);
  const uint32_t r0 = gtid / kLanesPerRow;
  const int sub = (int)(gtid % kLanesPerRow);
  const bool is_v = (r0 & 1u) != 0;
  const bool quantise = is_v ? v_is_e4m3(MODE) : k_is_e4m3(MODE);
  const int elem = quantise ? 1 : 2;  // bytes per stored value: e4m3 or bf16
  // this lane's bytes of row 0 of the cache (its four values) and the scales
  uint8_t* const lane_dst = static_cast<uint8_t*>(is_v ? a.v : a.k) + 4 * sub * elem;
  float* const scales = is_v ? a.vs : a.ks;

  // Every row's state is uniform over its kLanesPerRow lanes, so the lane
  // moves of the row maximum, which stay inside a row's lane group and run
  // under a per-row condition, never read a lane of another row or an
  // inactive one.
  uint32_t pair[R];
  bool in[R];
  float4 x[R];
  int seq[R], p[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t row_id = r0 + k * slots;
    in[k] = row_id < (uint32_t)a.n_rows;
    const uint32_t rid = in[k] ? row_id : 0u;  // (a row that does not exist reads row 0)
    pair[k] = rid >> 1;
    const float* src = (is_v ? a.v_new : a.k_new) + (uint64_t)pair[k] * D + 4 * sub;
    x[k] = *reinterpret_cast<const float4*>(src);
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t tok = (uint32_t)a.div_hkv.div((int)pair[k]);  // pair < 2^30
    seq[k] = a.seq_idx[tok];
    p[k] = a.pos[tok];
  }
  // Out-of-range device data is skipped, never followed (uniform per row).
  int blk[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    in[k] = in[k] && seq[k] >= 0 && seq[k] < a.num_seqs && p[k] >= 0 && p[k] < a.mbps * a.bs;
    const int64_t ti = in[k] ? (int64_t)seq[k] * a.mbps + a.div_bs.div(p[k]) : 0;
    blk[k] = a.table ? a.table[ti] : (int)ti;  // no table: contiguous
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (!in[k] || blk[k] < 0 || blk[k] >= a.num_blocks) continue;
    const int h = a.div_hkv.mod((int)pair[k]);
    const int slot = a.div_bs.mod(p[k]);  // 0 <= p < mbps * bs < 2^31
    int64_t row;
    if constexpr (ROW32) {
      const uint32_t b = (uint32_t)blk[k];
      row = a.layout == kHeadMajor ? (b * a.hkv + h) * a.bs + slot : (b * a.bs + slot) * a.hkv + h;
    } else {
      row = cache_row(a.layout, blk[k], slot, h, a.bs, a.hkv);
    }
    uint8_t* dst = lane_dst + (uint64_t)row * (D * elem);
    if (k_is_mx(MODE) && !is_v) {
      // block-scaled K: eight lanes hold a block of 32 values
      const int e = mx_exponent(row_amax<8>(x[k]));
      *reinterpret_cast<uint32_t*>(dst) = e4m3_codes4(x[k], e8m0_value((uint32_t)(e + 127)));
      if ((sub & 7) == 0) a.kexp[row * (D / 32) + sub / 8] = (uint8_t)(e + 127);
    } else if (quantise) {
      const float scale = storage_scale(row_amax<kLanesPerRow>(x[k]));  // RN(amax / 448)
      *reinterpret_cast<uint32_t*>(dst) = e4m3_codes4(x[k], scale);
      if (sub == 0) scales[row] = scale;
    } else {
      *reinterpret_cast<u32x2_t*>(dst) = bf16x4(x[k]);
    }
  }
}

template <int MODE, int R, bool ROW32>
static hipError_t append_for_rows(const CacheView& c, const AppendArgs& a, hipStream_t stream) {
  const int lanes = c.d / 4;
  const int64_t threads = ((int64_t)a.n_rows + R - 1) / R * lanes;
  const int64_t blocks = (threads + kAppendThreads - 1) / kAppendThreads;
  // gtid and the row indices of the last sweep stay below 2^32
  if (blocks * kAppendThreads > UINT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kAppendThreads);
  if (c.d == 128)
    hipLaunchKernelGGL((append_kernel<MODE, 128, R, ROW32>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((append_kernel<MODE, 64, R, ROW32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int MODE, int R>
static hipError_t append_for_d(const CacheView& c, const AppendArgs& a, hipStream_t stream) {
  if ((int64_t)c.num_blocks * c.bs * c.hkv <= INT32_MAX)
    return append_for_rows<MODE, R, true>(c, a, stream);
  return append_for_rows<MODE, R, false>(c, a, stream);
}

template <int MODE>
static hipError_t append_mode(const CacheView& c, const AppendArgs& a, hipStream_t stream) {
  if ((int64_t)a.n_rows * (c.d / 4) >= kBulkThreads)
    return append_for_d<MODE, kBulkRowsPerThread>(c, a, stream);
  return append_for_d<MODE, 1>(c, a, stream);
}

hipError_t launch_append(const CacheView& c, const float* k_new, const float* v_new,
                         const int32_t* seq_idx, const int32_t* pos, int n_tok,
                         hipStream_t stream) {
  const int64_t n_rows = 2 * (int64_t)n_tok * c.hkv;
  if (n_rows > INT32_MAX) return hipErrorInvalidValue;
  AppendArgs a{k_new, v_new, seq_idx, pos, c.table, c.k, c.v, c.ks, c.vs, c.kexp,
               (int)n_rows, c.hkv, c.bs, c.mbps, c.num_seqs, c.num_blocks, c.layout,
               FastDiv::of(c.hkv), FastDiv::of(c.bs)};
  switch (c.mode) {
    case kK8V8: return append_mode<kK8V8>(c, a, stream);
    case kK16V8: return append_mode<kK16V8>(c, a, stream);
    case kK8V16: return append_mode<kK8V16>(c, a, stream);
    case kMXK8V8: return append_mode<kMXK8V8>(c, a, stream);
    default: return append_mode<kBF16>(c, a, stream);
  }
}

}  // namespace fp8kv
