/*
 * Plain CPU oracle for attention over an e4m3 KV cache with one fp32 scale
 * per (token, KV head).
 *
 * TEST INFRASTRUCTURE ONLY.  This file and oracle.c are the slow, obviously
 * correct statement of what the GPU library computes.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  The
 * GPU library never links, includes or calls it, and it shares no code,
 * header, table or constant with the GPU library.
 *
 * Sources (page titles as published):
 *   [SKILL]  "kadirnar/kernel-agent/fp8-kv-cache", sections "Storage" and
 *            "Math": e4m3 codes plus one fp32 scale per (token, KV head),
 *            scale = amax over the head dimension / 448, written once at
 *            append; scores (q . codes) * k_scale * sm_scale with the products
 *            exact in fp32; the V scale folded into P, which is rounded to
 *            bf16 before the P.V product.
 *   [FA]     "03 . 8n - FA-style tiled prefill attention", section 2.1
 *            (online softmax) and section 3.1 (GQA slicing: query head h
 *            reads KV head h/gqa; causal mask kv <= q position; a row with no
 *            valid key outputs 0).
 *   [HW]     "FP8 KV attention: hardware paths and tile preparation", section
 *            "AMD CDNA 3" (a per-row scale moves outside the dot product).
 *   OCP 8-bit floating point specification (E4M3, bias 7, no infinities,
 *   S.1111.111 is NaN, largest finite 448): the pages only fix the 448.
 *
 * Precision: every sum, product, exponential and quotient of the attention is
 * carried in fp64.  The pages fix three narrower roundings and those are kept
 * exactly: the fp32 scale (a correctly rounded fp32 division amax / 448), the
 * e4m3 code (fp32 division x / scale, then round-to-nearest-even with
 * saturation at 448) and the bf16 rounding of P (after the V scale is
 * folded in).
 *
 * Reading of the pages where they are silent: P is rounded relative to an
 * integer log2-domain reference M = ceil(max_t s_t) where s_t is the score in
 * log2 units.  Any other integer reference gives the same output because
 * scaling by a power of two commutes with bf16 rounding; a running maximum
 * that changes from tile to tile therefore leaves the rounding unchanged.
 */
#ifndef FP8KV_ORACLE_H
#define FP8KV_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache formats: K8V8 (both e4m3 + scale), K16V8 (K bf16, V e4m3 + scale),
 * BF16 (both bf16), K8V16 (K e4m3 + scale, V bf16), MXK8V8 (K block-scaled
 * e4m3, V as in K8V8). */
enum { ORC_K8V8 = 0, ORC_K16V8 = 1, ORC_BF16 = 2, ORC_K8V16 = 3, ORC_MXK8V8 = 4 };

/* Value of an OCP e4m3fn code (NaN for 0x7F / 0xFF). */
double orc_e4m3_value(uint8_t code);

/* Round-to-nearest-even e4m3 code of y after clamping |y| to 448.
 * The sign is kept, so a negative value that rounds to zero gives 0x80. */
uint8_t orc_e4m3_encode(float y);

/* Round-to-nearest-even bf16 of a finite double; returns the bf16 bit
 * pattern.  Used for bf16 cache storage and for P. */
uint16_t orc_bf16_round(double x);

/* Value of a bf16 bit pattern. */
double orc_bf16_value(uint16_t bits);

/* Array helpers over the scalar functions above (n elements). */
void orc_e4m3_encode_array(const float* y, uint8_t* codes, size_t n);
void orc_bf16_round_array_f32(const float* x, uint16_t* bits, size_t n);

/* Quantise n_rows rows of d fp32 values each: per row
 * amax = max |x|, scale = fp32(amax / 448), code = e4m3(fp32(x / scale)).
 * A row whose scale is 0 gets all-zero codes. */
void orc_quantize_rows(const float* x, int64_t n_rows, int d,
                       uint8_t* codes, float* scales);

/* The unfused control's conversion of stored rows to bf16: per element
 * bf16(fp32(value(code) * scale)), the fp32 product rounded to nearest and
 * then to the nearest-even bf16.  Returns bf16 bit patterns. */
void orc_dequantize_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                         int d, uint16_t* out);

/*
 * Attention of n_rows query rows against one KV head's keys.
 *
 *   q      bf16 bits [n_rows][d]
 *   k8/ks  K8V8, K8V16: e4m3 codes [n_keys][d] and fp32 scales [n_keys]
 *   k16    K16V8, BF16: bf16 bits [n_keys][d]
 *   v8/vs  K8V8, K16V8: e4m3 codes [n_keys][d] and fp32 scales [n_keys]
 *   v16    BF16, K8V16: bf16 bits [n_keys][d]
 *   n_valid[r]  keys 0 .. n_valid[r]-1 are visible to row r
 *   round_p     1: P rounded to bf16 (the method); 0: unrounded (for pins)
 *   out    fp64 [n_rows][d]
 *   out_lo, out_hi  optional (both NULL or both set): the smallest and
 *          largest output reachable when every P whose value p * v_scale
 *          lies within fp32 rounding noise of a bf16 rounding midpoint is
 *          rounded either way.  Both roundings are correct results of the
 *          method for such a P (the scores themselves are only defined to
 *          fp32 accuracy), so a GPU result is valid when it lies in
 *          [out_lo, out_hi] up to its fp32 accumulation error.
 *
 * Per row (two-pass form):
 *   s_t  = (sum_d q_d * K_td) * ks_t * sm_scale * log2(e)
 *   M    = ceil(max_t s_t)
 *   p_t  = 2^(s_t - M),   l = sum_t p_t
 *   P_t  = bf16(p_t * vs_t)
 *   o_d  = (sum_t P_t * V_td) / l,  and o = 0 when no key is visible.
 */
void orc_attend_rows(int mode, int d, int n_rows, const uint16_t* q,
                     int n_keys, const uint8_t* k8, const uint16_t* k16,
                     const float* ks, const uint8_t* v8, const uint16_t* v16,
                     const float* vs, const int32_t* n_valid, float sm_scale,
                     int round_p, double* out, double* out_lo, double* out_hi);

/*
 * The same attention in the online form of the FA page, section 2.1: keys
 * are consumed in tiles of `tile` keys, grouped into splits of `split` keys;
 * each split carries (M, l, acc) across its tiles and writes an unnormalised
 * partial; the partials are merged with power-of-two weights.  Used to pin
 * the two-pass form (they must agree to rounding order) and as the reference
 * for the partial/merge entry points.
 *
 *   part_acc [n_splits][n_rows][d], part_l / part_m [n_splits][n_rows]
 *   (may be NULL when only `out` is wanted); part_m is -inf for a split
 *   with no visible key.
 */
void orc_attend_rows_online(int mode, int d, int n_rows, const uint16_t* q,
                            int n_keys, const uint8_t* k8, const uint16_t* k16,
                            const float* ks, const uint8_t* v8,
                            const uint16_t* v16, const float* vs,
                            const int32_t* n_valid, float sm_scale,
                            int round_p, int tile, int split,
                            double* part_acc, double* part_l, double* part_m,
                            double* out);

/*
 * Narrow QK (path 2 of the "Operating model" section of the hardware notes,
 * and its "Use a native narrow QK path" item): the query rows are quantised
 * once per decode step exactly like cache rows (orc_quantize_rows: q_scale =
 * fp32(amax / 448), codes e4m3(fp32(q / q_scale))) and the score takes the
 * code values, with the row's scale outside the dot product (CDNA 3
 * section):
 *   s_t = (sum_d value(qc_d) * K_td) * q_scale * ks_t * sm_scale * log2(e)
 * Everything after the score is as above.  q8: e4m3 codes [n_rows][d];
 * q_scale: fp32 [n_rows].  Other arguments as for the bf16 forms.  The
 * rounding interval (out_lo, out_hi) of the narrow form also allows the
 * fp8 matrix instruction's own sum of the d code products an error of up to
 * 2^-10 of their absolute sum (that sum is not correctly rounded fp32 on the
 * hardware); the nominal output is the exact one.
 */
void orc_attend_rows_q8(int mode, int d, int n_rows, const uint8_t* q8,
                        const float* q_scale, int n_keys, const uint8_t* k8,
                        const uint16_t* k16, const float* ks, const uint8_t* v8,
                        const uint16_t* v16, const float* vs,
                        const int32_t* n_valid, float sm_scale, int round_p,
                        double* out, double* out_lo, double* out_hi);

void orc_attend_rows_online_q8(int mode, int d, int n_rows, const uint8_t* q8,
                               const float* q_scale, int n_keys, const uint8_t* k8,
                               const uint16_t* k16, const float* ks, const uint8_t* v8,
                               const uint16_t* v16, const float* vs,
                               const int32_t* n_valid, float sm_scale, int round_p,
                               int tile, int split, double* part_acc, double* part_l,
                               double* part_m, double* out);

/* Block-scaled (MX) rows, MXFP8 (OCP Microscaling: E4M3 elements, one
 * power-of-two scale per 32 consecutive values; "Measure block-scaled QK" in
 * the hardware notes): per block E = ceil(log2(fp32(amax / 448))) (the
 * smallest power of two not below the storage-rule scale, so nothing
 * clamps; a reading, the pages leave the scale policy open), clamped to
 * [-126, 127]; codes e4m3(x / 2^E) rounded to nearest even, saturated at 448.
 * exps: E + 127 per block, [n_rows][d / 32].  orc_mx_exponent gives E. */
int orc_mx_exponent(float amax);
void orc_quantize_rows_mx(const float* x, int64_t n_rows, int d, uint8_t* codes,
                          uint8_t* exps);

/*
 * Every form above in one entry, with the options together:
 *   q16              bf16 rows, or NULL with
 *   q8 + q_scale     narrow rows with one fp32 scale per row, or
 *   q8 + q_exp       block-scaled rows ([n_rows][d/32] E8M0 bytes, q_scale NULL)
 *   k_bias           optional exact K bias, fp32 [d] (NULL for none).  With a
 *                    bias the stored K rows are the pre-bias residual and the
 *                    key is residual + bias ("Treat numerical safety and
 *                    kernel speed as separate gates" in the hardware notes;
 *                    "Bias-aware symmetric FP8" in the fused-quantisation
 *                    README: quantise the pre-bias residual, keep the fixed
 *                    bias exact, apply the equivalent score-space correction):
 *                    s_t = ((sum_d q_d K_td) ks_t + sum_d q_d b_d) sm_scale log2(e)
 *   mode ORC_MXK8V8  K rows are block-scaled (k8 codes + kx E8M0 bytes
 *                    [n_keys][d/32], ks unused): K_td = value(code) 2^E of
 *                    its block; V as in K8V8.
 */
void orc_attend_rows_ex(int mode, int d, int n_rows, const uint16_t* q16, const uint8_t* q8,
                        const float* q_scale, const uint8_t* q_exp, const float* k_bias,
                        int n_keys, const uint8_t* k8, const uint8_t* kx, const uint16_t* k16,
                        const float* ks, const uint8_t* v8, const uint16_t* v16,
                        const float* vs, const int32_t* n_valid, float sm_scale, int round_p,
                        double* out, double* out_lo, double* out_hi);

void orc_attend_rows_online_ex(int mode, int d, int n_rows, const uint16_t* q16,
                               const uint8_t* q8, const float* q_scale, const uint8_t* q_exp,
                               const float* k_bias, int n_keys, const uint8_t* k8,
                               const uint8_t* kx, const uint16_t* k16, const float* ks,
                               const uint8_t* v8, const uint16_t* v16, const float* vs,
                               const int32_t* n_valid, float sm_scale, int round_p, int tile,
                               int split, double* part_acc, double* part_l, double* part_m,
                               double* out);

#ifdef __cplusplus
}
#endif
#endif
