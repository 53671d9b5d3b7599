// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

// Cache formats: which side holds e4m3 codes + an fp32 scale per (token,
// KV head); the other side, if any, holds bf16.
// kMXK8V8: K as e4m3 codes with one power-of-two (E8M0) scale per 32
// consecutive values of a row (block-scaled, MXFP8), V as in kK8V8.
enum { kK8V8 = 0, kK16V8 = 1, kBF16 = 2, kK8V16 = 3, kMXK8V8 = 4 };
constexpr bool k_is_e4m3(int mode) { return mode == kK8V8 || mode == kK8V16 || mode == kMXK8V8; }
constexpr bool v_is_e4m3(int mode) { return mode == kK8V8 || mode == kK16V8 || mode == kMXK8V8; }
constexpr bool k_is_mx(int mode) { return mode == kMXK8V8; }
// an fp32 scale per (token, KV head) on the K side
constexpr bool k_has_row_scale(int mode) { return k_is_e4m3(mode) && !k_is_mx(mode); }

// Row order inside a block: token-major [slot][head] or head-major
// [head][slot]; codes, scales and K exponents of row r sit at r * D, r and
// r * D / 32 of their arrays.
enum { kTokenMajor = 0, kHeadMajor = 1 };

__host__ __device__ inline int64_t cache_row(int layout, int64_t blk, int slot, int h, int bs,
                                             int hkv) {
  return layout == kHeadMajor ? (blk * hkv + h) * bs + slot : (blk * bs + slot) * hkv + h;
}

// Rows from one slot of a head to the next slot of the same head.
__host__ __device__ inline int slot_stride(int layout, int hkv) {
  return layout == kHeadMajor ? 1 : hkv;
}

// Division by a divisor fixed for a launch (head count, block size, split
// count) as a multiply-high, an add and a shift instead of the ~20
// instructions of a general integer division: the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994), section 4.  With l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1 (below 2^32 for every d >= 1),
// floor(n / d) = (mulhi(m, n) + n) >> l for every n < 2^32; the sum needs a
// 33rd bit only for n >= 2^31, so dividends are kept below 2^31.
struct FastDiv {
  uint32_t m;
  uint32_t l;
  int d;
  static FastDiv of(int d) {  // d >= 1
    uint32_t l = 0;
    while ((uint64_t(1) << l) < (uint64_t)d) ++l;
    const uint64_t m = (((uint64_t(1) << l) - (uint64_t)d) << 32) / (uint64_t)d + 1;
    return FastDiv{(uint32_t)m, l, d};
  }
  __device__ __forceinline__ int div(int n) const {  // 0 <= n < 2^31
    return (int)((__umulhi(m, (uint32_t)n) + (uint32_t)n) >> l);
  }
  __device__ __forceinline__ int mod(int n) const { return n - div(n) * d; }
};

struct CacheView {
  int mode;   // kK8V8 / kK16V8 / kBF16 / kK8V16 / kMXK8V8
  int bs;     // tokens per block (multiple of 16)
  int hkv;    // KV heads
  int d;      // head_dim, 64 or 128
  int mbps;   // block-table row length
  int num_seqs;    // block-table rows
  int num_blocks;  // blocks in the cache
  void* k;
  void* v;
  float* ks;
  float* vs;
  const int32_t* table;
  const float* kbias;  // exact K bias [hkv][d] of a pre-bias residual cache, or null
  uint8_t* kexp;       // kMXK8V8: E8M0 byte per 32-value K block [row][d/32]
  int layout;          // kTokenMajor / kHeadMajor
};

// Work-groups of the split kernel one compute unit holds at once (one
// register buffer per wave): three where a lane's registers fit in 168 (the
// e4m3 K and V tiles of K8V8 and MXK8V8, and every D = 64 tile), else two
// (a bf16 side at D = 128 needs up to 240): the kernel's launch bounds.
constexpr int split_wgs_per_cu(int mode, int d) {
  return (mode == kK8V8 || mode == kMXK8V8 || d == 64) ? 3 : 2;
}
constexpr int kComputeUnits = 256;  // MI355X

// Bytes of the library-owned scratch (one copy per device) that
// fp8kv_decode_noalloc keeps the split partials in, and its device address
// on the current device (resolved on the first call per device, then kept).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void** ptr);

hipError_t launch_append(const CacheView& c, const float* k_new, const float* v_new,
                         const int32_t* seq_idx, const int32_t* pos, int n_tok,
                         hipStream_t stream);

// Split kernel: one work-group per (sequence, KV head, split).  c_scale is
// sm_scale * log2(e) rounded to fp32.  With k_new / v_new (fp32
// [batch][hkv][D]) the kernel first appends each sequence's new token at
// position seq_lens[b] - 1 (fused append); null pointers: plain decode.
// q8: narrow QK (Q quantised to e4m3 in the kernel; e4m3 K modes only).
// out (only where direct_output_ok): the output rows, written by the split
// kernel as the merge kernel would write them; null: partials.
hipError_t launch_decode_partial(const CacheView& c, const uint16_t* q, int group,
                                 const int32_t* seq_lens, int batch, float c_scale,
                                 int chunk, int n_splits, float* part_acc,
                                 float* part_ml, const float* k_new, const float* v_new,
                                 float* out, bool q8, hipStream_t stream);

// A plan whose splits the split kernel can finish itself: one split of at
// most one tile per wave (256 keys), no K bias, per-row K scales (bf16 or
// narrow QK).
inline bool direct_output_ok(const CacheView& c, int chunk, int n_splits) {
  return n_splits == 1 && chunk <= 256 && !c.kbias && !k_is_mx(c.mode);
}

hipError_t launch_decode_merge(int batch, int hkv, int group, int d, int n_splits,
                               const float* part_acc, const float* part_ml, float* out,
                               hipStream_t stream);

// Every row of src into dst (BF16 mode, same geometry).
hipError_t launch_dequantize(const CacheView& src, const CacheView& dst, hipStream_t stream);

hipError_t launch_prefill(const CacheView& c, const uint16_t* q, int group,
                          const int32_t* cu_q, const int32_t* q_pos0,
                          const int32_t* seq_lens, int batch, int total_q, int max_q_len,
                          float c_scale, float* out, hipStream_t stream);

}  // namespace fp8kv
