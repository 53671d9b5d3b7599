// C ABI of the fp8kv library: argument validation, split planning, dispatch.
// Every check here runs on the host before anything is enqueued, so a bad
// argument never reaches a kernel.  Semantics of each call: include/fp8kv.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "fp8kv.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 128;
constexpr int kMaxGroup = 16;
constexpr double kLog2e = 1.4426950408889634073599246810018921;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FP8KV_ERR_UNSUPPORTED;
  }
  int v = g_arch[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FP8KV_ERR_UNSUPPORTED;
    }
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? FP8KV_OK : FP8KV_ERR_UNSUPPORTED;
}

int validate_cache(const fp8kv_cache* c) {
  if (!c) return FP8KV_ERR_INVALID;
  if (c->mode != FP8KV_K8V8 && c->mode != FP8KV_K16V8 && c->mode != FP8KV_BF16 &&
      c->mode != FP8KV_K8V16 && c->mode != FP8KV_MXK8V8)
    return FP8KV_ERR_INVALID;
  if (c->layout != FP8KV_TOKEN_MAJOR && c->layout != FP8KV_HEAD_MAJOR) return FP8KV_ERR_INVALID;
  if (c->head_dim != 64 && c->head_dim != 128) return FP8KV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->max_blocks_per_seq <= 0 ||
      c->num_seqs <= 0)
    return FP8KV_ERR_INVALID;
  if ((int64_t)c->max_blocks_per_seq * c->block_size > INT32_MAX) return FP8KV_ERR_INVALID;
  if (c->block_size <= 0 || c->block_size % 16 != 0) return FP8KV_ERR_INVALID;
  if (!c->k || !c->v) return FP8KV_ERR_INVALID;
  if (!aligned(c->k, 16) || !aligned(c->v, 16) || !aligned(c->block_table, 4))
    return FP8KV_ERR_INVALID;
  // no table: block e of sequence b is block b * max_blocks_per_seq + e, an int32
  if (!c->block_table && (int64_t)c->num_seqs * c->max_blocks_per_seq > INT32_MAX)
    return FP8KV_ERR_INVALID;
  // ... and every such id must be a block of the cache: a smaller allocation
  // would make the kernels drop keys and skip appends without an error
  if (!c->block_table && (int64_t)c->num_seqs * c->max_blocks_per_seq > c->num_blocks)
    return FP8KV_ERR_INVALID;
  const bool need_ks = fp8kv::k_has_row_scale(c->mode);
  const bool need_vs = fp8kv::v_is_e4m3(c->mode);
  const bool need_kx = fp8kv::k_is_mx(c->mode);
  // A scale pointer must be present exactly when the mode stores that scale:
  // a mismatch means the caller and the cache disagree about the format.
  if (need_ks != (c->k_scale != nullptr)) return FP8KV_ERR_INVALID;
  if (need_vs != (c->v_scale != nullptr)) return FP8KV_ERR_INVALID;
  if (c->k_scale && !aligned(c->k_scale, 4)) return FP8KV_ERR_INVALID;
  if (c->v_scale && !aligned(c->v_scale, 4)) return FP8KV_ERR_INVALID;
  if (c->k_bias && !aligned(c->k_bias, 16)) return FP8KV_ERR_INVALID;
  if (need_kx != (c->k_exp != nullptr)) return FP8KV_ERR_INVALID;
  if (c->k_exp && !aligned(c->k_exp, 4)) return FP8KV_ERR_INVALID;
  if (need_kx && c->k_bias) return FP8KV_ERR_UNSUPPORTED;  // no bias on block-scaled K
  return FP8KV_OK;
}

fp8kv::CacheView view_of(const fp8kv_cache* c) {
  return fp8kv::CacheView{c->mode, c->block_size, c->num_kv_heads, c->head_dim,
                          c->max_blocks_per_seq, c->num_seqs, c->num_blocks, c->k, c->v,
                          c->k_scale, c->v_scale, c->block_table, c->k_bias, c->k_exp,
                          c->layout};
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return FP8KV_OK;
  (void)hipGetLastError();  // read and clear, so the stream is not poisoned
  return FP8KV_ERR_LAUNCH;
}

float log2_scale(float sm_scale) { return (float)((double)sm_scale * kLog2e); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The split kernel reads the block ids of a split with one load per lane of
// a 64-lane wave, so a split may touch at most 64 blocks.  Splits start at
// multiples of chunk, hence at offsets into a block that are multiples of
// g = gcd(chunk, block_size), the largest being block_size - g; the last
// 16-key sub-block of the split then lies (block_size - g + chunk - 16) /
// block_size blocks after the first.
bool split_fits_table_window(int64_t chunk, int64_t bs) {
  int64_t g = chunk, r = bs;
  while (r != 0) {
    const int64_t t = g % r;
    g = r;
    r = t;
  }
  return (bs - g + chunk - 16) / bs <= 63;
}

int plan(const fp8kv_cache* c, int32_t batch, int32_t max_seq_len, int32_t* chunk,
         int32_t* n_splits) {
  // Splits of 256 keys (one 64-key tile per wave of a 4-wave work-group),
  // doubled (up to 1024) while the grid still gives every compute unit a
  // work-group: a wave then streams several tiles, half by half, and fewer
  // splits make the merge cheaper.  When 256-key splits leave compute units
  // without a work-group, 128-key splits (half a tile per wave) double the
  // work-groups, as long as the merge takes the splits in one batch (32).
  const int64_t pairs = (int64_t)batch * c->num_kv_heads;
  int64_t ch = 256;
  if (pairs * ceil_div(max_seq_len, 256) < fp8kv::kComputeUnits &&
      ceil_div(max_seq_len, 128) <= 32) {
    ch = 128;
  } else {
    while (ch < 1024 && pairs * ceil_div(max_seq_len, 2 * ch) >= fp8kv::kComputeUnits) ch *= 2;
  }
  *chunk = (int32_t)ch;
  *n_splits = max_seq_len > 0 ? (int32_t)ceil_div(max_seq_len, ch) : 0;
  return FP8KV_OK;
}

int validate_decode_common(const fp8kv_cache* c, int32_t gqa, int32_t batch,
                           int32_t max_seq_len) {
  int st = validate_cache(c);
  if (st != FP8KV_OK) return st;
  if (gqa < 1) return FP8KV_ERR_INVALID;
  if (gqa > kMaxGroup) return FP8KV_ERR_UNSUPPORTED;
  if (batch < 0 || max_seq_len < 0 || batch > c->num_seqs) return FP8KV_ERR_INVALID;
  if ((int64_t)max_seq_len > (int64_t)c->max_blocks_per_seq * c->block_size)
    return FP8KV_ERR_INVALID;
  return FP8KV_OK;
}

}  // namespace

extern "C" {

const char* fp8kv_strerror(int status) {
  switch (status) {
    case FP8KV_OK: return "ok";
    case FP8KV_ERR_INVALID: return "invalid argument";
    case FP8KV_ERR_WORKSPACE: return "workspace too small";
    case FP8KV_ERR_LAUNCH: return "kernel launch failed";
    case FP8KV_ERR_UNSUPPORTED: return "unsupported device or shape";
    case FP8KV_ERR_TOO_LARGE: return "request exceeds the library's 64 MiB device scratch";
    default: return "unknown status";
  }
}

int fp8kv_append(const fp8kv_cache* cache, const float* k_new, const float* v_new,
                 const int32_t* seq_idx, const int32_t* pos, int32_t n_tok, void* stream) {
  int st = validate_cache(cache);
  if (st != FP8KV_OK) return st;
  if (n_tok < 0) return FP8KV_ERR_INVALID;
  if (n_tok == 0) return FP8KV_OK;
  if (!k_new || !v_new || !seq_idx || !pos) return FP8KV_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(seq_idx, 4) || !aligned(pos, 4))
    return FP8KV_ERR_INVALID;
  // K and V rows of every (token, KV head): the kernel indexes them in 32 bits
  if (2 * (int64_t)n_tok * cache->num_kv_heads > INT32_MAX) return FP8KV_ERR_INVALID;
  if ((st = check_device()) != FP8KV_OK) return st;
  return launch_status(fp8kv::launch_append(view_of(cache), k_new, v_new, seq_idx, pos, n_tok,
                                            static_cast<hipStream_t>(stream)));
}

int fp8kv_decode_plan(const fp8kv_cache* cache, int32_t batch, int32_t gqa_group,
                      int32_t max_seq_len, int32_t* chunk_tokens, int32_t* n_splits) {
  int st = validate_decode_common(cache, gqa_group, batch, max_seq_len);
  if (st != FP8KV_OK) return st;
  if (!chunk_tokens || !n_splits) return FP8KV_ERR_INVALID;
  return plan(cache, batch, max_seq_len, chunk_tokens, n_splits);
}

size_t fp8kv_decode_workspace_bytes(const fp8kv_cache* cache, int32_t batch,
                                    int32_t gqa_group, int32_t max_seq_len) {
  int32_t chunk = 0, splits = 0;
  if (fp8kv_decode_plan(cache, batch, gqa_group, max_seq_len, &chunk, &splits) != FP8KV_OK)
    return 0;
  return (size_t)batch * cache->num_kv_heads * splits * gqa_group * (cache->head_dim + 2) *
         sizeof(float);
}

namespace {

int decode_partial_impl(const fp8kv_cache* cache, const float* k_new, const float* v_new,
                        const uint16_t* q, int32_t gqa_group, const int32_t* seq_lens,
                        int32_t batch, int32_t max_seq_len, float sm_scale, int32_t chunk_tokens,
                        int32_t n_splits, float* part_acc, float* part_ml, bool q8,
                        void* stream, float* out = nullptr) {
  int st = validate_decode_common(cache, gqa_group, batch, max_seq_len);
  if (st != FP8KV_OK) return st;
  if (q8 && (!fp8kv::k_is_e4m3(cache->mode) || cache->k_bias))
    return FP8KV_ERR_UNSUPPORTED;  // narrow QK takes the K codes as they are, no bias
  if (k_new && fp8kv::k_is_mx(cache->mode))
    return FP8KV_ERR_UNSUPPORTED;  // no fused append into block-scaled K
  if (chunk_tokens <= 0 || chunk_tokens % 64 != 0 || n_splits < 0) return FP8KV_ERR_INVALID;
  if (!split_fits_table_window(chunk_tokens, cache->block_size)) return FP8KV_ERR_INVALID;
  if ((int64_t)n_splits * chunk_tokens < max_seq_len) return FP8KV_ERR_INVALID;
  // The kernel computes split * chunk_tokens (and that plus chunk_tokens) in
  // 32 bits; a split that starts at or past the block-table capacity holds
  // no key, so more splits than the capacity needs are rejected, which also
  // keeps those values inside an int32.
  const int64_t capacity = (int64_t)cache->max_blocks_per_seq * cache->block_size;
  if ((int64_t)n_splits * chunk_tokens > capacity + chunk_tokens - 1 ||
      (int64_t)n_splits * chunk_tokens > INT32_MAX)
    return FP8KV_ERR_INVALID;
  const int64_t n_wg = (int64_t)batch * cache->num_kv_heads * n_splits;
  if (n_wg > INT32_MAX) return FP8KV_ERR_INVALID;
  if (n_wg == 0) return FP8KV_OK;
  if (!q || !seq_lens || !part_acc || !part_ml) return FP8KV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(seq_lens, 4) || !aligned(part_acc, 16) ||
      !aligned(part_ml, 8))
    return FP8KV_ERR_INVALID;
  if ((k_new == nullptr) != (v_new == nullptr)) return FP8KV_ERR_INVALID;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return FP8KV_ERR_INVALID;
  if ((st = check_device()) != FP8KV_OK) return st;
  return launch_status(fp8kv::launch_decode_partial(
      view_of(cache), q, gqa_group, seq_lens, batch, log2_scale(sm_scale), chunk_tokens,
      n_splits, part_acc, part_ml, k_new, v_new, out, q8, static_cast<hipStream_t>(stream)));
}

}  // namespace

int fp8kv_decode_partial(const fp8kv_cache* cache, const uint16_t* q, int32_t gqa_group,
                         const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                         float sm_scale, int32_t chunk_tokens, int32_t n_splits,
                         float* part_acc, float* part_ml, void* stream) {
  return decode_partial_impl(cache, nullptr, nullptr, q, gqa_group, seq_lens, batch,
                             max_seq_len, sm_scale, chunk_tokens, n_splits, part_acc, part_ml,
                             false, stream);
}

int fp8kv_decode_append_partial(const fp8kv_cache* cache, const float* k_new,
                                const float* v_new, const uint16_t* q, int32_t gqa_group,
                                const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                float sm_scale, int32_t chunk_tokens, int32_t n_splits,
                                float* part_acc, float* part_ml, void* stream) {
  if (batch > 0 && n_splits > 0 && (!k_new || !v_new)) return FP8KV_ERR_INVALID;
  return decode_partial_impl(cache, k_new, v_new, q, gqa_group, seq_lens, batch, max_seq_len,
                             sm_scale, chunk_tokens, n_splits, part_acc, part_ml, false, stream);
}

int fp8kv_decode_merge(int32_t batch, int32_t num_kv_heads, int32_t gqa_group,
                       int32_t head_dim, int32_t n_splits, const float* part_acc,
                       const float* part_ml, float* out, void* stream) {
  if (batch < 0 || num_kv_heads <= 0 || gqa_group < 1 || n_splits < 0) return FP8KV_ERR_INVALID;
  if (gqa_group > kMaxGroup || (head_dim != 64 && head_dim != 128)) return FP8KV_ERR_UNSUPPORTED;
  if ((int64_t)batch * num_kv_heads * gqa_group > INT32_MAX) return FP8KV_ERR_INVALID;
  if (batch == 0) return FP8KV_OK;
  if (!out || !aligned(out, 16)) return FP8KV_ERR_INVALID;
  if (n_splits > 0 && (!part_acc || !part_ml || !aligned(part_acc, 16) || !aligned(part_ml, 8)))
    return FP8KV_ERR_INVALID;
  int st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_status(fp8kv::launch_decode_merge(batch, num_kv_heads, gqa_group, head_dim,
                                                  n_splits, part_acc, part_ml, out,
                                                  static_cast<hipStream_t>(stream)));
}

namespace {

int decode_impl(const fp8kv_cache* cache, const float* k_new, const float* v_new,
                const uint16_t* q, int32_t gqa_group, const int32_t* seq_lens, int32_t batch,
                int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                size_t workspace_bytes, bool q8, void* stream) {
  int32_t chunk = 0, splits = 0;
  int st = fp8kv_decode_plan(cache, batch, gqa_group, max_seq_len, &chunk, &splits);
  if (st != FP8KV_OK) return st;
  if (q8 && (!fp8kv::k_is_e4m3(cache->mode) || cache->k_bias)) return FP8KV_ERR_UNSUPPORTED;
  if (k_new && fp8kv::k_is_mx(cache->mode)) return FP8KV_ERR_UNSUPPORTED;
  if (batch == 0) return FP8KV_OK;
  const size_t acc_floats = (size_t)batch * cache->num_kv_heads * splits * gqa_group *
                            cache->head_dim;
  const size_t need = fp8kv_decode_workspace_bytes(cache, batch, gqa_group, max_seq_len);
  if (splits > 0 && (!workspace || workspace_bytes < need)) return FP8KV_ERR_WORKSPACE;
  if (splits > 0 && !aligned(workspace, 16)) return FP8KV_ERR_INVALID;
  float* part_acc = static_cast<float*>(workspace);
  float* part_ml = splits > 0 ? part_acc + acc_floats : nullptr;
  if (!out || !aligned(out, 16)) return FP8KV_ERR_INVALID;
  if (splits > 0 && (!q || !seq_lens || !aligned(q, 16) || !aligned(seq_lens, 4)))
    return FP8KV_ERR_INVALID;
  // A plan of one split (of at most 256 keys, no K bias, per-row K scales):
  // the split kernel writes the output rows itself, since the merge of one
  // split is a division by its row sum, and no merge kernel follows.
  const bool direct = fp8kv::direct_output_ok(view_of(cache), chunk, splits);
  st = decode_partial_impl(cache, k_new, v_new, q, gqa_group, seq_lens, batch, max_seq_len,
                           sm_scale, chunk, splits, part_acc, part_ml, q8, stream,
                           direct ? out : nullptr);
  if (st != FP8KV_OK || direct) return st;
  return fp8kv_decode_merge(batch, cache->num_kv_heads, gqa_group, cache->head_dim, splits,
                            part_acc, part_ml, out, stream);
}

}  // namespace

int fp8kv_decode(const fp8kv_cache* cache, const uint16_t* q, int32_t gqa_group,
                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                 float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cache, nullptr, nullptr, q, gqa_group, seq_lens, batch, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, false, stream);
}

int fp8kv_decode_q8(const fp8kv_cache* cache, const uint16_t* q, int32_t gqa_group,
                    const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                    float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cache, nullptr, nullptr, q, gqa_group, seq_lens, batch, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, true, stream);
}

int fp8kv_decode_append(const fp8kv_cache* cache, const float* k_new, const float* v_new,
                        const uint16_t* q, int32_t gqa_group, const int32_t* seq_lens,
                        int32_t batch, int32_t max_seq_len, float sm_scale, float* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && max_seq_len > 0 && (!k_new || !v_new)) return FP8KV_ERR_INVALID;
  return decode_impl(cache, k_new, v_new, q, gqa_group, seq_lens, batch, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, false, stream);
}

int fp8kv_decode_append_q8(const fp8kv_cache* cache, const float* k_new, const float* v_new,
                           const uint16_t* q, int32_t gqa_group, const int32_t* seq_lens,
                           int32_t batch, int32_t max_seq_len, float sm_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && max_seq_len > 0 && (!k_new || !v_new)) return FP8KV_ERR_INVALID;
  return decode_impl(cache, k_new, v_new, q, gqa_group, seq_lens, batch, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, true, stream);
}

int fp8kv_decode_noalloc(const fp8kv_cache* cache, const uint16_t* q, int32_t gqa_group,
                         const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                         float sm_scale, float* out, void* stream) {
  int32_t chunk = 0, splits = 0;
  int st = fp8kv_decode_plan(cache, batch, gqa_group, max_seq_len, &chunk, &splits);
  if (st != FP8KV_OK) return st;
  const size_t need = fp8kv_decode_workspace_bytes(cache, batch, gqa_group, max_seq_len);
  if (need > fp8kv::kScratchBytes) return FP8KV_ERR_TOO_LARGE;
  if (batch == 0) return FP8KV_OK;
  if ((st = check_device()) != FP8KV_OK) return st;
  void* ws = nullptr;
  if (fp8kv::scratch_address(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return FP8KV_ERR_LAUNCH;
  }
  // the same two kernels as fp8kv_decode, with the partials in the scratch
  return decode_impl(cache, nullptr, nullptr, q, gqa_group, seq_lens, batch, max_seq_len,
                     sm_scale, out, ws, fp8kv::kScratchBytes, false, stream);
}

int fp8kv_dequantize(const fp8kv_cache* src, const fp8kv_cache* dst, void* stream) {
  int st = validate_cache(src);
  if (st != FP8KV_OK) return st;
  if ((st = validate_cache(dst)) != FP8KV_OK) return st;
  if (dst->mode != FP8KV_BF16 || dst->num_blocks != src->num_blocks ||
      dst->block_size != src->block_size || dst->num_kv_heads != src->num_kv_heads ||
      dst->head_dim != src->head_dim || dst->layout != src->layout)
    return FP8KV_ERR_INVALID;
  if (dst->k == src->k || dst->v == src->v) return FP8KV_ERR_INVALID;  // no in-place
  if (fp8kv::k_is_mx(src->mode)) return FP8KV_ERR_UNSUPPORTED;
  if ((st = check_device()) != FP8KV_OK) return st;
  return launch_status(
      fp8kv::launch_dequantize(view_of(src), view_of(dst), static_cast<hipStream_t>(stream)));
}

int fp8kv_prefill(const fp8kv_cache* cache, const uint16_t* q, int32_t gqa_group,
                  const int32_t* cu_q, const int32_t* q_pos0, const int32_t* seq_lens,
                  int32_t batch, int32_t total_q, int32_t max_q_len, float sm_scale, float* out,
                  void* stream) {
  int st = validate_cache(cache);
  if (st != FP8KV_OK) return st;
  if (gqa_group < 1 || batch < 0 || max_q_len < 0 || total_q < 0 || batch > cache->num_seqs)
    return FP8KV_ERR_INVALID;
  if (gqa_group > kMaxGroup) return FP8KV_ERR_UNSUPPORTED;
  if (cache->k_bias || fp8kv::k_is_mx(cache->mode))
    return FP8KV_ERR_UNSUPPORTED;  // pre-bias and block-scaled caches: decode only
  if (batch == 0 || max_q_len == 0 || total_q == 0) return FP8KV_OK;
  if (!q || !cu_q || !q_pos0 || !seq_lens || !out) return FP8KV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(cu_q, 4) || !aligned(q_pos0, 4) ||
      !aligned(seq_lens, 4))
    return FP8KV_ERR_INVALID;
  if ((st = check_device()) != FP8KV_OK) return st;
  return launch_status(fp8kv::launch_prefill(view_of(cache), q, gqa_group, cu_q, q_pos0,
                                             seq_lens, batch, total_q, max_q_len,
                                             log2_scale(sm_scale), out,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
