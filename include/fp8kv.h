/*
 * fp8kv: attention over an FP8 (OCP e4m3fn) KV cache on MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named as "device" is HIP device memory; the
 * caller owns every buffer.  The library allocates no device memory, keeps
 * no state between calls apart from a per-device architecture check (and,
 * for fp8kv_decode_noalloc, the address of its per-device scratch), and
 * never synchronises: each call validates its arguments on the host, enqueues
 * its kernels on `stream` (a hipStream_t; NULL is the default stream) and
 * returns.  Calls are HIP-graph capturable (no allocation, no memset).
 *
 * Status codes: FP8KV_OK (0) or a negative fp8kv_status.  INVALID,
 * WORKSPACE and UNSUPPORTED mean nothing was enqueued.  LAUNCH means the HIP
 * runtime reported a launch failure; the error has been read (and so
 * cleared) before returning, so it does not leak into later calls on the
 * stream.
 *
 * Device-side data (positions, sequence indices, lengths, block-table
 * entries) cannot be checked on the host without a synchronisation.  The
 * kernels therefore guard every index they read: an append row whose
 * sequence index, position or block id is out of range is not written, a
 * length is clamped to the block-table capacity, and a key whose block id is
 * out of range is not read (it does not take part in the attention).  The
 * results for such inputs are unspecified but no access leaves the buffers
 * the descriptor describes.  Inputs must be finite.
 *
 * Sources (page titles as published):
 *   [SKILL] "kadirnar/kernel-agent/fp8-kv-cache": sections "Storage"
 *           (e4m3 + one fp32 scale per (token, KV head), amax/448, written
 *           once at append), "Math" (K scale folded into the scores, V scale
 *           folded into P rounded to bf16) and "Speed" (split the cache over
 *           programs; fp32 partials merged by a second kernel).
 *   [HW]    "FP8 KV attention: hardware paths and tile preparation":
 *           "Operating model" (reconstruct only the active tile, online
 *           softmax tile by tile; path 2, quantise Q and use FP8 QK),
 *           "NVIDIA Hopper" path 3 (K16/V8, the no-K-transform control),
 *           "AMD CDNA 3" (FP8-by-FP8 matrix instruction, a per-row scale
 *           applied outside the dot product), "Use a native narrow QK path"
 *           (quantise Q once per decode step), "Collect the profiler
 *           evidence" (dtype controls including K16/V16).
 *   [FQ]    "Fused KV-cache quantization": "Latency analysis" (the
 *           separate cache-write kernel is one part of the decode gap),
 *           "Bias-aware symmetric FP8" (pre-bias residual, exact bias).
 *   [FA]    "03 . 8n - FA-style tiled prefill attention": sections 2.1
 *           (online softmax), 3.1 (64-token query tiles, GQA slicing,
 *           positions are data, causal mask) and 3.2/3.3 (a row with no
 *           visible key outputs 0; a fully masked tile keeps the state).
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element formats ([SKILL] Storage; [HW] Hopper path 3, "Account for
 * V preparation" and the dtype controls of "Collect the profiler evidence").
 *   FP8KV_K8V8   K and V: uint8 e4m3 codes + fp32 scale per (token, KV head)
 *   FP8KV_K16V8  K: bf16; V: e4m3 codes + fp32 scale (no K preparation)
 *   FP8KV_BF16   K and V: bf16 (no scales)
 *   FP8KV_K8V16  K: e4m3 codes + fp32 scale; V: bf16 (no V preparation)
 *   FP8KV_MXK8V8 K: block-scaled e4m3 (MXFP8, [HW] "Measure block-scaled
 *                QK"): one power-of-two scale 2^E per 32 consecutive values
 *                of a row, E = ceil(log2(fp32(amax / 448))) clamped to
 *                [-126, 127], codes e4m3(x / 2^E); V as in K8V8 */
typedef enum {
  FP8KV_K8V8 = 0,
  FP8KV_K16V8 = 1,
  FP8KV_BF16 = 2,
  FP8KV_K8V16 = 3,
  FP8KV_MXK8V8 = 4
} fp8kv_mode;

typedef enum {
  FP8KV_OK = 0,
  FP8KV_ERR_INVALID = -1,     /* bad argument: null pointer, shape, alignment */
  FP8KV_ERR_WORKSPACE = -2,   /* workspace smaller than the size query says  */
  FP8KV_ERR_LAUNCH = -3,      /* the HIP runtime rejected a launch           */
  FP8KV_ERR_UNSUPPORTED = -4, /* device is not gfx950, or head_dim/G unsupported */
  FP8KV_ERR_TOO_LARGE = -5    /* fp8kv_decode_noalloc: partials exceed its scratch */
} fp8kv_status;

/* Order of the rows of a block (one row = one (token, KV head) pair):
 *   FP8KV_TOKEN_MAJOR  [block][slot][head]: a contiguous cache is
 *                      [B][T][Hkv][D] with scales [B][T][Hkv]
 *   FP8KV_HEAD_MAJOR   [block][head][slot]: one KV head's rows of a block
 *                      are contiguous (codes and scales), the order the
 *                      decode tile reads ([HW] "Store the preferred cache
 *                      layout once": align pages and scale blocks with the
 *                      decode tile) */
typedef enum { FP8KV_TOKEN_MAJOR = 0, FP8KV_HEAD_MAJOR = 1 } fp8kv_layout;

/*
 * Paged KV cache descriptor (all pointers device memory, owned by the
 * caller).  With R the rows of a block in the order `layout` names
 * ([slot][head] or [head][slot]):
 *   k, v            [num_blocks][R][head_dim]
 *                   K8V8: uint8 codes for both; K16V8: k bf16, v uint8;
 *                   BF16: bf16 for both; K8V16: k uint8, v bf16
 *   k_scale         [num_blocks][R] fp32, K8V8 and K8V16 (NULL otherwise)
 *   k_exp           MXK8V8 only (NULL otherwise): uint8
 *                   [num_blocks][R][head_dim / 32], the
 *                   byte E + 127 of each 32-value K block, 4-byte aligned.
 *                   Decode reads it with bf16 Q (codes converted by their
 *                   block's scale) or with block-scaled Q through the q8
 *                   entries (the matrix instruction applies both operands'
 *                   block scales); the fused append, prefill, dequantize and
 *                   a K bias give FP8KV_ERR_UNSUPPORTED for such a cache.
 *   v_scale         [num_blocks][R] fp32, K8V8 and K16V8 (NULL otherwise)
 *   block_table     int32 [num_seqs][max_blocks_per_seq]; token t of sequence
 *                   b is slot t % block_size of block
 *                   block_table[b * max_blocks_per_seq + t / block_size].
 *                   NULL: a contiguous cache, where that block is
 *                   b * max_blocks_per_seq + t / block_size (no table is
 *                   read, so the first K/V loads need not wait for one;
 *                   num_seqs * max_blocks_per_seq must fit an int32 and
 *                   be at most num_blocks, else FP8KV_ERR_INVALID).
 * A contiguous cache ([B][T][Hkv][D] token-major, [B][Hkv][T][D] head-major)
 * is block_size = T, max_blocks_per_seq = 1 and block_table NULL (or
 * block_table[b] = b).
 *   layout          fp8kv_layout of every array above; any other value is
 *                   FP8KV_ERR_INVALID.
 *   k_bias          NULL, or fp32 [num_kv_heads][head_dim], 16-byte aligned:
 *                   a pre-bias residual cache ([HW] "Treat numerical safety
 *                   and kernel speed as separate gates"; [FQ] "Bias-aware
 *                   symmetric FP8").  The stored K rows are the residual r
 *                   (the caller appends r, e.g. the key projection before its
 *                   bias); the key is r + b with b kept exact, and decode
 *                   applies the equivalent score correction: the score of
 *                   query row q gains (q . b) * sm_scale * log2(e).
 *                   fp8kv_decode, fp8kv_decode_append and their partials
 *                   support it; narrow QK and prefill give
 *                   FP8KV_ERR_UNSUPPORTED for such a cache.
 * Requirements: head_dim 64 or 128; block_size a multiple of 16; k, v 16-byte
 * aligned; k_scale, v_scale, block_table 4-byte aligned.
 * Slots at or past a sequence's length (and slots of blocks it does not
 * hold) may contain any bytes, NaN codes included: attention reads whole
 * 16-token sub-blocks but no such key reaches an output.
 */
typedef struct fp8kv_cache {
  int32_t mode;                /* fp8kv_mode */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;            /* rows of block_table */
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  const int32_t* block_table;
  const float* k_bias;         /* exact fixed K bias, or NULL (see above) */
  uint8_t* k_exp;              /* FP8KV_MXK8V8: K block exponents (see above) */
  int32_t layout;              /* fp8kv_layout */
} fp8kv_cache;

/*
 * Append (quantise and store) n_tok new tokens, all KV heads.  [SKILL]
 * Storage: per (token, KV head) row of head_dim values
 *   amax = max |x|,  scale = fp32(amax / 448) (correctly rounded),
 *   code = e4m3 round-to-nearest-even of fp32(x / scale), saturated at 448,
 *   a row whose scale is 0 stores all-zero codes.
 * K16V8 stores K as bf16 (round-to-nearest-even); BF16 stores K and V as bf16.
 *   k_new, v_new   device fp32 [n_tok][num_kv_heads][head_dim]
 *   seq_idx, pos   device int32 [n_tok]: token i goes to sequence seq_idx[i]
 *                  at position pos[i]
 * Each (token, head) row is written exactly once per call; two tokens of one
 * call must not target the same slot.  n_tok == 0 is a no-op; a call with
 * 2 * n_tok * num_kv_heads >= 2^31 rows gives FP8KV_ERR_INVALID (split it).
 */
int fp8kv_append(const fp8kv_cache* cache, const float* k_new,
                 const float* v_new, const int32_t* seq_idx,
                 const int32_t* pos, int32_t n_tok, void* stream);

/*
 * Split plan for decode: keys of each (sequence, KV head) are cut into
 * splits of *chunk_tokens keys (a multiple of 64); *n_splits =
 * ceil(max_seq_len / chunk_tokens).  The chunk is 256, 512 or 1024 keys:
 * the largest whose grid (batch * num_kv_heads * n_splits work-groups)
 * still gives each of MI355X's 256 compute units a work-group, so that the
 * splits feed every unit ([SKILL] Speed) while each wave streams as many
 * tiles as it can and the merge has few splits.  Host-only and
 * deterministic.
 */
int fp8kv_decode_plan(const fp8kv_cache* cache, int32_t batch,
                      int32_t gqa_group, int32_t max_seq_len,
                      int32_t* chunk_tokens, int32_t* n_splits);

/* Bytes of workspace fp8kv_decode needs: the partials of the plan above,
 * batch * num_kv_heads * n_splits * gqa_group * (head_dim + 2) * 4. */
size_t fp8kv_decode_workspace_bytes(const fp8kv_cache* cache, int32_t batch,
                                    int32_t gqa_group, int32_t max_seq_len);

/*
 * Split-KV decode, first kernel.  For every (sequence b, KV head h, split s)
 * the keys t in [s*chunk, min((s+1)*chunk, seq_lens[b])) are attended by the
 * gqa_group query heads h*G .. h*G+G-1 ([FA] 3.1 GQA slicing) and the
 * unnormalised partial is written:
 *   score     s_t = (q . K_t) * k_scale_t * sm_scale * log2(e)   (log2 units)
 *   M         integer reference, >= every s_t of the split (the running
 *             maximum rounded up to an integer, updated tile by tile)
 *   part_l    sum_t 2^(s_t - M)
 *   part_acc  sum_t bf16(2^(s_t - M) * v_scale_t) * V_t
 * ([SKILL] Math; [FA] 2.1).  A split with no key gets M = -inf and l = 0.
 *   q            device bf16 [batch][num_kv_heads * gqa_group][head_dim]
 *   seq_lens     device int32 [batch], 0 <= seq_lens[b] <= max_seq_len
 *   part_acc     device fp32 [batch][num_kv_heads][n_splits][G][head_dim]
 *   part_ml      device fp32 [batch][num_kv_heads][n_splits][G][2] = (M, l)
 * chunk_tokens must be a positive multiple of 64 and a split may span at
 * most 64 blocks: with g = gcd(chunk_tokens, block_size),
 * (block_size - g + chunk_tokens - 16) / block_size <= 63.  This holds for
 * every chunk_tokens <= 64 * block_size that block_size divides or that
 * divides block_size, and for every plan fp8kv_decode_plan returns;
 * otherwise FP8KV_ERR_INVALID.  n_splits >= ceil(max_seq_len / chunk_tokens),
 * and no split may start past the block table: n_splits * chunk_tokens <
 * max_blocks_per_seq * block_size + chunk_tokens (else FP8KV_ERR_INVALID).
 * gqa_group in 1..16.
 */
int fp8kv_decode_partial(const fp8kv_cache* cache, const uint16_t* q,
                         int32_t gqa_group, const int32_t* seq_lens,
                         int32_t batch, int32_t max_seq_len, float sm_scale,
                         int32_t chunk_tokens, int32_t n_splits,
                         float* part_acc, float* part_ml, void* stream);

/*
 * Split-KV decode, second kernel ([SKILL] Speed): merge the fp32 partials of
 * every (sequence, query head):
 *   M* = max_s M_s,  w_s = 2^(M_s - M*) (0 for an empty split),
 *   out = sum_s w_s acc_s / sum_s w_s l_s,  out = 0 when every split is empty.
 *   out   device fp32 [batch][num_kv_heads * gqa_group][head_dim]
 */
int fp8kv_decode_merge(int32_t batch, int32_t num_kv_heads, int32_t gqa_group,
                       int32_t head_dim, int32_t n_splits,
                       const float* part_acc, const float* part_ml, float* out,
                       void* stream);

/*
 * Decode attention: fp8kv_decode_partial with the plan of fp8kv_decode_plan
 * (partials in `workspace`), then fp8kv_decode_merge.  A plan of one split
 * of at most 256 keys (no K bias, per-row K scales; also for the narrow-QK
 * entry points) runs the split kernel alone: it writes the output rows
 * itself, bit-identical to the merge of its one split.  One query token per sequence; seq_lens counts the keys
 * it attends (the appended token included).
 * out: device fp32 [batch][num_kv_heads * gqa_group][head_dim].
 */
int fp8kv_decode(const fp8kv_cache* cache, const uint16_t* q,
                 int32_t gqa_group, const int32_t* seq_lens, int32_t batch,
                 int32_t max_seq_len, float sm_scale, float* out,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step with the append fused in ([SKILL] Storage; [FQ] Latency
 * analysis): for every sequence b with 1 <= seq_lens[b] <= the block-table
 * capacity, the step's new token (k_new[b], v_new[b]) is stored at position
 * seq_lens[b] - 1 exactly as fp8kv_append stores it (same codes, scales and
 * bf16 bytes; not written if that position's block id is out of range), and
 * then attended with the rest of the sequence: the result equals
 * fp8kv_append followed by fp8kv_decode, in the kernels of the split-KV
 * decode (two, or one for a plan of one split) instead of one more.  The slot is written by the work-group whose
 * split holds it, so it must not lie in keys that another sequence of the
 * same call attends (shared blocks must be full).
 *   k_new, v_new  device fp32 [batch][num_kv_heads][head_dim], 16-byte aligned
 * Other arguments and the workspace as for fp8kv_decode.
 */
int fp8kv_decode_append(const fp8kv_cache* cache, const float* k_new,
                        const float* v_new, const uint16_t* q,
                        int32_t gqa_group, const int32_t* seq_lens,
                        int32_t batch, int32_t max_seq_len, float sm_scale,
                        float* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Narrow QK ([HW] "Operating model" path 2, "Use a native narrow QK path",
 * "AMD CDNA 3"): fp8kv_decode and fp8kv_decode_append with the query rows
 * quantised once per call, inside the split kernel, by the cache-row rule
 * (per query row of head_dim values: q_scale = fp32(amax / 448), codes =
 * e4m3 sat-RNE of fp32(q / q_scale)), and QK computed by the fp8 matrix
 * instruction directly on the stored K codes:
 *   s_t = (sum_d value(qc_d) * value(kc_t,d)) * q_scale * k_scale_t
 *         * sm_scale * log2(e)
 * Everything after the score is unchanged.  On an MXK8V8 cache this is
 * block-scaled QK ([HW] "Measure block-scaled QK"): each 32-value block of a
 * query row gets its own power-of-two scale by the MXK8V8 rule, and the
 * matrix instruction applies the Q and K block scales itself:
 *   s_t = sum_blocks 2^(Eq + Ek) (sum_{d in block} value(qc_d) value(kc_t,d))
 *         * sm_scale * log2(e)
 * The Q rounding is an extra error source (a few percent relative L2 against
 * bf16 Q on N(0,1) data), which the caller accepts by choosing these entry
 * points.  Arguments, workspace and guards as for fp8kv_decode /
 * fp8kv_decode_append; caches whose K is not e4m3 (K16V8, BF16), or that
 * carry a K bias, give FP8KV_ERR_UNSUPPORTED.
 */
int fp8kv_decode_q8(const fp8kv_cache* cache, const uint16_t* q,
                    int32_t gqa_group, const int32_t* seq_lens, int32_t batch,
                    int32_t max_seq_len, float sm_scale, float* out,
                    void* workspace, size_t workspace_bytes, void* stream);

int fp8kv_decode_append_q8(const fp8kv_cache* cache, const float* k_new,
                           const float* v_new, const uint16_t* q,
                           int32_t gqa_group, const int32_t* seq_lens,
                           int32_t batch, int32_t max_seq_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The first kernel of fp8kv_decode_append on its own: the fused append and
 * the split partials, arguments as for fp8kv_decode_partial plus k_new and
 * v_new; fp8kv_decode_merge completes the step.
 */
int fp8kv_decode_append_partial(const fp8kv_cache* cache, const float* k_new,
                                const float* v_new, const uint16_t* q,
                                int32_t gqa_group, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len,
                                float sm_scale, int32_t chunk_tokens,
                                int32_t n_splits, float* part_acc,
                                float* part_ml, void* stream);

/*
 * fp8kv_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that
 * forbid allocation).  The same kernels and the same plan as
 * fp8kv_decode, so the output is bit-identical to fp8kv_decode's; the split
 * partials live in a device array the library owns instead of a caller
 * workspace: 64 MiB, one copy per GPU, loaded with the library's code
 * object and held until the process ends.  No call allocates or frees.
 *   Limit: fp8kv_decode_workspace_bytes(cache, batch, gqa_group,
 *   max_seq_len) must be at most 64 MiB (2^26 bytes), else
 *   FP8KV_ERR_TOO_LARGE and nothing is enqueued (e.g. 64 sequences x 8 KV
 *   heads x G 4 x D 128 up to 32768 keys take 32.5 MiB).
 *   Nothing in the array needs clearing between calls: every split writes
 *   its (M, l) before the merge of the same call reads it, and an empty
 *   split's accumulator is never read.
 *   Calls that overlap on one GPU (other streams, other threads) share the
 *   array and race: serialise them.  The array's address is resolved on the
 *   first call on each device (hipGetSymbolAddress), a host-side step that
 *   is best taken before any graph capture.
 * Arguments, guards and other errors as for fp8kv_decode.
 */
int fp8kv_decode_noalloc(const fp8kv_cache* cache, const uint16_t* q,
                         int32_t gqa_group, const int32_t* seq_lens, int32_t batch,
                         int32_t max_seq_len, float sm_scale, float* out,
                         void* stream);

/*
 * Causal prefill attention ([FA] 3.1): queries of sequence b are rows
 * cu_q[b] .. cu_q[b+1]-1 of q; query i of the sequence sits at position
 * q_pos0[b] + i and attends the cached keys t <= q_pos0[b] + i with
 * t < seq_lens[b].  The keys must already be in the cache (fp8kv_append).
 * Per row the result equals decode attention over its visible keys; a row
 * with no visible key outputs 0.
 *   q        device bf16 [total_q][num_kv_heads * gqa_group][head_dim]
 *   cu_q     device int32 [batch + 1], cu_q[0] = 0, non-decreasing, at most
 *            total_q (rows outside [0, total_q) are neither read nor written)
 *   q_pos0, seq_lens  device int32 [batch]
 *   max_q_len  >= every cu_q[b+1] - cu_q[b]
 *   out      device fp32 [total_q][num_kv_heads * gqa_group][head_dim]
 */
int fp8kv_prefill(const fp8kv_cache* cache, const uint16_t* q,
                  int32_t gqa_group, const int32_t* cu_q,
                  const int32_t* q_pos0, const int32_t* seq_lens,
                  int32_t batch, int32_t total_q, int32_t max_q_len,
                  float sm_scale, float* out, void* stream);

/*
 * The unfused control ("Fused KV-cache quantization"; [HW] Collect the
 * profiler evidence): every row of src, in any mode, converted into dst, a
 * BF16-mode cache of the same num_blocks, block_size, num_kv_heads,
 * head_dim and layout (its own buffers; block tables are not read).  An e4m3 element
 * becomes bf16(fp32(value(code) * scale)) -- the fp32 product rounded once,
 * then to the nearest-even bf16; a bf16 element is copied.  Attention on dst
 * with the BF16 kernels is then the pipeline that dequantises the cache in
 * HBM instead of converting only the active tile on chip.
 */
int fp8kv_dequantize(const fp8kv_cache* src, const fp8kv_cache* dst,
                     void* stream);

/* Static description of a status code. */
const char* fp8kv_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* FP8KV_H */
