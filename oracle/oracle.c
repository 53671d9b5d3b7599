/*
 * Plain CPU oracle.  TEST INFRASTRUCTURE ONLY: see oracle.h for the sources
 * followed, the precision rules and who may load this code.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off oracle.c -lm
 * (no fast-math: the fp32 divisions below must be correctly rounded and the
 * fp64 sums must be evaluated as written).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORC_LOG2E 1.4426950408889634073599246810018921 /* log2(e) */

/* ---- number formats --------------------------------------------------- */

/* OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
 * field 0 is the subnormal range m * 2^-9; S.1111.111 is NaN; there are no
 * infinities.  0x7E = 1.75 * 2^8 = 448 is the largest finite value, the
 * maximum the storage section of the fp8-kv-cache page divides by. */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* Round-to-nearest-even onto the e4m3 grid after saturating at 448.
 * In the binade [2^e, 2^(e+1)) (e >= -6) the grid spacing is 2^(e-3); below
 * 2^-6 the subnormals keep the spacing 2^-9.  a / spacing is the integer
 * significand (8 + m, or m for subnormals), so rounding it half-to-even is
 * rounding the code half-to-even. */
uint8_t orc_e4m3_encode(float y) {
  double a = fabs((double)y);
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  int ex, e;
  double spacing, r;
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return sign;
  frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  e = ex - 1;    /* a in [2^e, 2^(e+1)) */
  if (e < -6) e = -6;
  spacing = ldexp(1.0, e - 3);
  r = rint(a / spacing) * spacing; /* default rounding mode: half to even */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) /* subnormal: exponent field 0, m = r / 2^-9 */
    return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
  frexp(r, &ex);
  /* r = (8 + m) * 2^(ex-4), exponent field E = ex + 6 */
  return (uint8_t)(sign | ((ex + 6) << 3) | ((int)ldexp(r, 4 - ex) - 8));
}

/* bf16: 8 significant bits, the exponent range of fp32, subnormals below
 * 2^-126 with spacing 2^-133.  Same grid argument as above. */
uint16_t orc_bf16_round(double x) {
  double a = fabs(x);
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  int ex, e;
  double r;
  float f;
  uint32_t u;
  if (a == 0.0) return sign;
  frexp(a, &ex);
  e = ex - 1;
  if (e < -126) e = -126;
  r = rint(ldexp(a, 7 - e));
  r = ldexp(r, e - 7);
  f = (float)r; /* exact: r has at most 8 significant bits (inf on overflow) */
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void orc_e4m3_encode_array(const float* y, uint8_t* codes, size_t n) {
  size_t i;
  for (i = 0; i < n; ++i) codes[i] = orc_e4m3_encode(y[i]);
}

void orc_bf16_round_array_f32(const float* x, uint16_t* bits, size_t n) {
  size_t i;
  for (i = 0; i < n; ++i) bits[i] = orc_bf16_round((double)x[i]);
}

/* ---- append: per-(token, KV head) row quantisation -------------------- */

/* Storage section of the fp8-kv-cache page: one fp32 scale per row,
 * amax(|row|) / 448 over the head dimension, codes in e4m3. */
void orc_quantize_rows(const float* x, int64_t n_rows, int d, uint8_t* codes,
                       float* scales) {
  int64_t r;
  int j;
  for (r = 0; r < n_rows; ++r) {
    const float* row = x + r * d;
    float amax = 0.0f, scale;
    for (j = 0; j < d; ++j) {
      float a = fabsf(row[j]);
      if (a > amax) amax = a;
    }
    scale = amax / 448.0f; /* fp32 division, correctly rounded */
    scales[r] = scale;
    for (j = 0; j < d; ++j) {
      float y;
      if (scale == 0.0f) {
        codes[r * d + j] = 0x00;
        continue;
      }
      y = row[j] / scale; /* fp32 division, correctly rounded */
      codes[r * d + j] = orc_e4m3_encode(y);
    }
  }
}

/* ---- block-scaled (MX) rows ------------------------------------------- */

/* Block-scaled (MX) rows: MXFP8 (OCP Microscaling formats, E4M3 elements,
 * one power-of-two scale per block of 32 consecutive values) for the
 * block-scaled QK of the hardware notes ("Measure block-scaled QK", which
 * leaves the scale policy to be validated).  Reading: the block scale is the
 * smallest power of two not below the block's storage-rule scale,
 * 2^E with E = ceil(log2(fp32(amax / 448))), so that, as with the per-row
 * rule, no element needs clamping (OCP's floor(log2(amax)) - 8 maps amax
 * into [256, 512) and clamps the block's largest values at 448).  E is
 * clamped to [-126, 127], so every scale is a normal fp32; a block of zeros
 * (or one whose quotient is an fp32 subnormal) takes E = -126.  Elements are
 * e4m3(x / 2^E), rounded to nearest even and saturated at 448.  exps holds
 * E + 127 (the E8M0 byte). */
int orc_mx_exponent(float amax) {
  const float s = amax / 448.0f; /* fp32 division, correctly rounded */
  int ex, e;
  float m;
  if (!(s >= 0x1p-126f)) return -126;
  m = frexpf(s, &ex); /* s = m * 2^ex, m in [0.5, 1) */
  e = (m == 0.5f) ? ex - 1 : ex;
  return e > 127 ? 127 : e;
}

void orc_quantize_rows_mx(const float* x, int64_t n_rows, int d, uint8_t* codes,
                          uint8_t* exps) {
  int64_t r;
  int blk, j;
  for (r = 0; r < n_rows; ++r)
    for (blk = 0; blk < d / 32; ++blk) {
      const float* v = x + r * d + 32 * blk;
      float amax = 0.0f, scale;
      int e;
      for (j = 0; j < 32; ++j)
        if (fabsf(v[j]) > amax) amax = fabsf(v[j]);
      e = orc_mx_exponent(amax);
      exps[r * (d / 32) + blk] = (uint8_t)(e + 127);
      scale = ldexpf(1.0f, e);
      for (j = 0; j < 32; ++j)
        codes[r * d + 32 * blk + j] = orc_e4m3_encode(v[j] / scale); /* exact quotient */
    }
}

void orc_dequantize_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                         int d, uint16_t* out) {
  int64_t r;
  int j;
  for (r = 0; r < n_rows; ++r) {
    for (j = 0; j < d; ++j) {
      /* every e4m3 value is exact in fp32; the product is rounded once */
      const float prod = (float)orc_e4m3_value(codes[r * d + j]) * scales[r];
      out[r * d + j] = orc_bf16_round((double)prod);
    }
  }
}

/* ---- attention -------------------------------------------------------- */

typedef struct {
  int mode, d, n_keys;
  const uint8_t *k8, *v8;
  const uint16_t *k16, *v16;
  const float *ks, *vs;
  const float* kb; /* exact K bias [d] (pre-bias residual cache), or NULL */
  const uint8_t* kx; /* MXK8V8: E8M0 byte of each 32-element K block [n_keys][d/32] */
} kv_view;

/* Which side of the cache holds e4m3 codes with a scale (else bf16). */
static int k_is_e4m3(int mode) {
  return mode == ORC_K8V8 || mode == ORC_K8V16 || mode == ORC_MXK8V8;
}
static int v_is_e4m3(int mode) {
  return mode == ORC_K8V8 || mode == ORC_K16V8 || mode == ORC_MXK8V8;
}

static double k_elem(const kv_view* kv, int t, int j) {
  if (kv->mode == ORC_MXK8V8) /* code value times its block's scale 2^E */
    return orc_e4m3_value(kv->k8[(size_t)t * kv->d + j]) *
           ldexp(1.0, (int)kv->kx[(size_t)t * (kv->d / 32) + j / 32] - 127);
  if (k_is_e4m3(kv->mode)) return orc_e4m3_value(kv->k8[(size_t)t * kv->d + j]);
  return orc_bf16_value(kv->k16[(size_t)t * kv->d + j]);
}

static double v_elem(const kv_view* kv, int t, int j) {
  if (v_is_e4m3(kv->mode)) return orc_e4m3_value(kv->v8[(size_t)t * kv->d + j]);
  return orc_bf16_value(kv->v16[(size_t)t * kv->d + j]);
}

static double k_scale(const kv_view* kv, int t) {
  if (kv->mode == ORC_MXK8V8) return 1.0; /* the block scales are in k_elem */
  return k_is_e4m3(kv->mode) ? (double)kv->ks[t] : 1.0;
}

static double v_scale(const kv_view* kv, int t) {
  return v_is_e4m3(kv->mode) ? (double)kv->vs[t] : 1.0;
}

/* q . b for the exact K bias (0 without one). */
static double bias_dot(const kv_view* kv, const double* qv) {
  double dot = 0.0;
  int j;
  if (!kv->kb) return 0.0;
  for (j = 0; j < kv->d; ++j) dot += qv[j] * (double)kv->kb[j];
  return dot;
}

/* Score in log2 units: (q . K_t) * k_scale_t * sm_scale * log2(e).
 * The K scale sits outside the dot product (CDNA 3 section of the hardware
 * notes; "Math" section of the fp8-kv-cache page).  With an exact K bias the
 * stored rows are the pre-bias residual and the key is residual + bias, so
 * the score gains q . b ("Treat numerical safety and kernel speed as
 * separate gates": keep the fixed bias exact, correct in score space);
 * qb is that dot product for the row. */
static double score(const kv_view* kv, const double* qv, int t, double c, double qb) {
  double dot = 0.0;
  int j;
  for (j = 0; j < kv->d; ++j) dot += qv[j] * k_elem(kv, t, j);
  return (dot * k_scale(kv, t) + qb) * c;
}

/* P with the V scale folded in, rounded to bf16 when round_p is set. */
static double p_folded(const kv_view* kv, double p, int t, int round_p) {
  double w = p * v_scale(kv, t);
  return round_p ? orc_bf16_value(orc_bf16_round(w)) : w;
}

static int clamp_valid(int nv, int n_keys) {
  if (nv < 0) return 0;
  return nv > n_keys ? n_keys : nv;
}

/* Narrow QK: the error allowed to the matrix instruction's own sum of the d
 * exact code products, relative to their absolute sum.  The instruction's
 * sum is not the correctly rounded fp32 one (it rounds, unbiased, at about
 * 2^-13 of that absolute sum: measured worst 2^-12.2 over 32768 dot products
 * of random codes on gfx950); 2^-10 leaves a margin of four. */
#define ORC_NARROW_SUM_ERR 0x1p-10

/* Bound on |fp32 score - exact score| in log2 units for any summation order
 * of the d exact products (the classic (n-1)u sum|x_i| bound, doubled, plus
 * the roundings of the scale products; on the narrow path also the
 * instruction's sum error above), as a relative window on p = 2^(s - M)
 * with 2^-20 added for an fp32 exp2 within a few ulp. */
static double p_window(const kv_view* kv, const double* qv, int t, double c, int narrow) {
  double sabs = 0.0, babs = 0.0;
  int j;
  for (j = 0; j < kv->d; ++j) sabs += fabs(qv[j] * k_elem(kv, t, j));
  if (kv->kb)
    for (j = 0; j < kv->d; ++j) babs += fabs(qv[j] * (double)kv->kb[j]);
  sabs = (sabs * fabs(k_scale(kv, t)) + babs) * fabs(c);
  return 0.6931471805599453 *
             (2.0 * (double)(kv->d + 4) * ldexp(1.0, -24) +
              (narrow ? ORC_NARROW_SUM_ERR : 0.0)) * sabs +
         ldexp(1.0, -20);
}

/* Query row r as fp64 values, and the row's score constant: bf16 rows
 * (q16) are their values with c = sm_scale * log2(e); e4m3 rows (q8) are the
 * code values, and the row's scale joins the constant outside the dot
 * product (CDNA 3 section of the hardware notes). */
static double query_row(int d, int r, const uint16_t* q16, const uint8_t* q8,
                        const float* q_scale, const uint8_t* q_exp, double c, double* qv) {
  int j;
  if (q8 && q_exp) { /* block-scaled (MX) rows: code value times 2^E of its block */
    for (j = 0; j < d; ++j)
      qv[j] = orc_e4m3_value(q8[(size_t)r * d + j]) *
              ldexp(1.0, (int)q_exp[(size_t)r * (d / 32) + j / 32] - 127);
    return c;
  }
  if (q8) {
    for (j = 0; j < d; ++j) qv[j] = orc_e4m3_value(q8[(size_t)r * d + j]);
    return c * (double)q_scale[r];
  }
  for (j = 0; j < d; ++j) qv[j] = orc_bf16_value(q16[(size_t)r * d + j]);
  return c;
}

static void attend_rows(int mode, int d, int n_rows, const uint16_t* q16,
                        const uint8_t* q8, const float* q_scale, const uint8_t* q_exp,
                        const float* k_bias, int n_keys, const uint8_t* k8,
                        const uint8_t* kx, const uint16_t* k16, const float* ks,
                        const uint8_t* v8, const uint16_t* v16, const float* vs,
                        const int32_t* n_valid, float sm_scale, int round_p,
                        double* out, double* out_lo, double* out_hi) {
  kv_view kv = {mode, d, n_keys, k8, v8, k16, v16, ks, vs, k_bias, kx};
  const double c0 = (double)sm_scale * ORC_LOG2E;
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* alo = (double*)malloc(sizeof(double) * (size_t)d);
  double* ahi = (double*)malloc(sizeof(double) * (size_t)d);
  int bounds = out_lo != NULL && out_hi != NULL;
  int r, t, j;
  for (r = 0; r < n_rows; ++r) {
    int nv = clamp_valid(n_valid[r], n_keys);
    double smax = -INFINITY, m, l = 0.0;
    double* o = out + (size_t)r * d;
    const double c = query_row(d, r, q16, q8, q_scale, q_exp, c0, qv);
    const double qb = bias_dot(&kv, qv);
    if (nv == 0) { /* no visible key: the row outputs 0 */
      for (j = 0; j < d; ++j) o[j] = 0.0;
      if (bounds)
        for (j = 0; j < d; ++j) out_lo[(size_t)r * d + j] = out_hi[(size_t)r * d + j] = 0.0;
      continue;
    }
    /* pass 1: scores and their maximum */
    for (t = 0; t < nv; ++t) {
      s[t] = score(&kv, qv, t, c, qb);
      if (s[t] > smax) smax = s[t];
    }
    m = ceil(smax);
    /* pass 2: probabilities, normaliser, P.V */
    for (j = 0; j < d; ++j) acc[j] = alo[j] = ahi[j] = 0.0;
    for (t = 0; t < nv; ++t) {
      double p = exp2(s[t] - m);
      double w = p_folded(&kv, p, t, round_p);
      l += p;
      for (j = 0; j < d; ++j) acc[j] += w * v_elem(&kv, t, j);
      if (bounds) {
        /* Both bf16 neighbours are valid roundings when p * v_scale lies
         * within fp32 noise of a rounding midpoint. */
        double win = round_p ? p_window(&kv, qv, t, c, q8 != NULL) : 0.0;
        double wa = round_p ? p_folded(&kv, p * (1.0 - win), t, 1) : w;
        double wb = round_p ? p_folded(&kv, p * (1.0 + win), t, 1) : w;
        for (j = 0; j < d; ++j) {
          double va = wa * v_elem(&kv, t, j), vb = wb * v_elem(&kv, t, j);
          alo[j] += va < vb ? va : vb;
          ahi[j] += va < vb ? vb : va;
        }
      }
    }
    for (j = 0; j < d; ++j) o[j] = acc[j] / l;
    if (bounds)
      for (j = 0; j < d; ++j) {
        out_lo[(size_t)r * d + j] = alo[j] / l;
        out_hi[(size_t)r * d + j] = ahi[j] / l;
      }
  }
  free(qv);
  free(s);
  free(acc);
  free(alo);
  free(ahi);
}

void orc_attend_rows(int mode, int d, int n_rows, const uint16_t* q,
                     int n_keys, const uint8_t* k8, const uint16_t* k16,
                     const float* ks, const uint8_t* v8, const uint16_t* v16,
                     const float* vs, const int32_t* n_valid, float sm_scale,
                     int round_p, double* out, double* out_lo, double* out_hi) {
  attend_rows(mode, d, n_rows, q, NULL, NULL, NULL, NULL, n_keys, k8, NULL, k16, ks, v8, v16, vs,
              n_valid,
              sm_scale, round_p, out, out_lo, out_hi);
}

void orc_attend_rows_q8(int mode, int d, int n_rows, const uint8_t* q8,
                        const float* q_scale, int n_keys, const uint8_t* k8,
                        const uint16_t* k16, const float* ks, const uint8_t* v8,
                        const uint16_t* v16, const float* vs,
                        const int32_t* n_valid, float sm_scale, int round_p,
                        double* out, double* out_lo, double* out_hi) {
  attend_rows(mode, d, n_rows, NULL, q8, q_scale, NULL, NULL, n_keys, k8, NULL, k16, ks, v8, v16,
              vs, n_valid,
              sm_scale, round_p, out, out_lo, out_hi);
}

static void attend_rows_online(int mode, int d, int n_rows, const uint16_t* q16,
                               const uint8_t* q8, const float* q_scale, const uint8_t* q_exp,
                               const float* k_bias, int n_keys, const uint8_t* k8,
                               const uint8_t* kx, const uint16_t* k16, const float* ks,
                               const uint8_t* v8, const uint16_t* v16, const float* vs,
                               const int32_t* n_valid, float sm_scale, int round_p,
                               int tile, int split, double* part_acc, double* part_l,
                               double* part_m, double* out) {
  kv_view kv = {mode, d, n_keys, k8, v8, k16, v16, ks, vs, k_bias, kx};
  const double c0 = (double)sm_scale * ORC_LOG2E;
  int n_splits = n_keys > 0 ? (n_keys + split - 1) / split : 0;
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)tile);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* sacc = (double*)malloc(sizeof(double) * (size_t)(n_splits > 0 ? n_splits : 1) * d);
  double* sl = (double*)malloc(sizeof(double) * (size_t)(n_splits > 0 ? n_splits : 1));
  double* sm = (double*)malloc(sizeof(double) * (size_t)(n_splits > 0 ? n_splits : 1));
  int r, sp, t0, t, j;
  for (r = 0; r < n_rows; ++r) {
    int nv = clamp_valid(n_valid[r], n_keys);
    double mstar = -INFINITY, lsum = 0.0;
    const double c = query_row(d, r, q16, q8, q_scale, q_exp, c0, qv);
    const double qb = bias_dot(&kv, qv);
    for (sp = 0; sp < n_splits; ++sp) {
      int k_lo = sp * split;
      int k_hi = k_lo + split < n_keys ? k_lo + split : n_keys;
      double m = -INFINITY, l = 0.0;
      for (j = 0; j < d; ++j) acc[j] = 0.0;
      for (t0 = k_lo; t0 < k_hi; t0 += tile) {
        int t1 = t0 + tile < k_hi ? t0 + tile : k_hi;
        double tmax = -INFINITY, m_new, alpha;
        /* scores of the visible keys of this tile */
        for (t = t0; t < t1; ++t) {
          if (t >= nv) break;
          s[t - t0] = score(&kv, qv, t, c, qb);
          if (s[t - t0] > tmax) tmax = s[t - t0];
        }
        if (tmax == -INFINITY) continue; /* fully masked tile: keep state */
        m_new = ceil(tmax) > m ? ceil(tmax) : m;
        alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new); /* power of two */
        l *= alpha;
        for (j = 0; j < d; ++j) acc[j] *= alpha;
        for (t = t0; t < t1 && t < nv; ++t) {
          double p = exp2(s[t - t0] - m_new);
          double w = p_folded(&kv, p, t, round_p);
          l += p;
          for (j = 0; j < d; ++j) acc[j] += w * v_elem(&kv, t, j);
        }
        m = m_new;
      }
      sm[sp] = m;
      sl[sp] = l;
      memcpy(sacc + (size_t)sp * d, acc, sizeof(double) * (size_t)d);
      if (part_acc)
        memcpy(part_acc + ((size_t)sp * n_rows + r) * d, acc, sizeof(double) * (size_t)d);
      if (part_l) part_l[(size_t)sp * n_rows + r] = l;
      if (part_m) part_m[(size_t)sp * n_rows + r] = m;
      if (m > mstar) mstar = m;
    }
    /* merge: weights 2^(M_s - M*), zero for a split with no visible key */
    for (j = 0; j < d; ++j) acc[j] = 0.0;
    for (sp = 0; sp < n_splits; ++sp) {
      double w;
      if (sm[sp] == -INFINITY) continue;
      w = exp2(sm[sp] - mstar);
      lsum += w * sl[sp];
      for (j = 0; j < d; ++j) acc[j] += w * sacc[(size_t)sp * d + j];
    }
    for (j = 0; j < d; ++j)
      out[(size_t)r * d + j] = lsum > 0.0 ? acc[j] / lsum : 0.0;
  }
  free(qv);
  free(s);
  free(acc);
  free(sacc);
  free(sl);
  free(sm);
}

void orc_attend_rows_online(int mode, int d, int n_rows, const uint16_t* q,
                            int n_keys, const uint8_t* k8, const uint16_t* k16,
                            const float* ks, const uint8_t* v8,
                            const uint16_t* v16, const float* vs,
                            const int32_t* n_valid, float sm_scale,
                            int round_p, int tile, int split,
                            double* part_acc, double* part_l, double* part_m,
                            double* out) {
  attend_rows_online(mode, d, n_rows, q, NULL, NULL, NULL, NULL, n_keys, k8, NULL, k16, ks, v8,
                     v16, vs,
                     n_valid, sm_scale, round_p, tile, split, part_acc, part_l, part_m, out);
}

void orc_attend_rows_online_q8(int mode, int d, int n_rows, const uint8_t* q8,
                               const float* q_scale, int n_keys, const uint8_t* k8,
                               const uint16_t* k16, const float* ks, const uint8_t* v8,
                               const uint16_t* v16, const float* vs,
                               const int32_t* n_valid, float sm_scale, int round_p,
                               int tile, int split, double* part_acc, double* part_l,
                               double* part_m, double* out) {
  attend_rows_online(mode, d, n_rows, NULL, q8, q_scale, NULL, NULL, n_keys, k8, NULL, k16, ks,
                     v8, v16, vs,
                     n_valid, sm_scale, round_p, tile, split, part_acc, part_l, part_m, out);
}

void orc_attend_rows_ex(int mode, int d, int n_rows, const uint16_t* q16, const uint8_t* q8,
                        const float* q_scale, const uint8_t* q_exp, const float* k_bias,
                        int n_keys, const uint8_t* k8, const uint8_t* kx, const uint16_t* k16,
                        const float* ks, const uint8_t* v8, const uint16_t* v16,
                        const float* vs, const int32_t* n_valid, float sm_scale, int round_p,
                        double* out, double* out_lo, double* out_hi) {
  attend_rows(mode, d, n_rows, q16, q8, q_scale, q_exp, k_bias, n_keys, k8, kx, k16, ks, v8,
              v16, vs, n_valid, sm_scale, round_p, out, out_lo, out_hi);
}

void orc_attend_rows_online_ex(int mode, int d, int n_rows, const uint16_t* q16,
                               const uint8_t* q8, const float* q_scale, const uint8_t* q_exp,
                               const float* k_bias, int n_keys, const uint8_t* k8,
                               const uint8_t* kx, const uint16_t* k16, const float* ks,
                               const uint8_t* v8, const uint16_t* v16, const float* vs,
                               const int32_t* n_valid, float sm_scale, int round_p, int tile,
                               int split, double* part_acc, double* part_l, double* part_m,
                               double* out) {
  attend_rows_online(mode, d, n_rows, q16, q8, q_scale, q_exp, k_bias, n_keys, k8, kx, k16, ks,
                     v8, v16, vs, n_valid, sm_scale, round_p, tile, split, part_acc, part_l,
                     part_m, out);
}
