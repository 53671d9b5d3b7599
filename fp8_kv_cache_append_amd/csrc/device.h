// Device-side helpers shared by the fp8kv kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));


constexpr float kE4M3Max = 448.0f;
constexpr float kLog2e = 1.4426950408889634f;

// Two e4m3 codes (bytes 2*HI and 2*HI+1 of w) -> two bf16 (low half from the
// lower byte).  Every e4m3 value, subnormals included, is exact in bf16; the
// scale operand 1.0 leaves the value unchanged.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

// Same, with the half chosen by a value the caller's unrolled loop makes
// constant (the instruction encodes the half as an immediate).
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  return hi ? e4m3x2_to_bf16x2<true>(w) : e4m3x2_to_bf16x2<false>(w);
}

// Two fp32 -> two bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Byte select over {src0 (selector values 4..7), src1 (values 0..3)}.
__device__ __forceinline__ uint32_t byte_perm(uint32_t src0, uint32_t src1, uint32_t sel) {
  return __builtin_amdgcn_perm(src0, src1, sel);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds row/column
// l % 16 and the eight k-slots 8*(l/16) .. 8*(l/16)+7 of A and B; the result
// rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3), block scales 2^0 (E8M0
// 127): the plain fp8 product.  Lane l holds row / column l % 16 of A / B
// and 32 of the 128 k-slots (32 bytes); byte p of lane l is the same k-slot
// in A and in B, so any assignment of the contraction index to (lane group,
// byte) that A and B share gives the same result.  Output layout as above:
// rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma_16x16x128_e4m3(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// max / sum over the four lane groups (lanes c, c+16, c+32, c+48) with the
// gfx950 lane swaps: with both operands equal, the two results of a 32-lane
// swap hold x[l] and x[l ^ 32], those of a 16-lane swap x[l] and x[l ^ 16].
__device__ __forceinline__ float max_over_groups(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float sum_over_groups(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Storage rule of a (token, KV head) row ("kadirnar/kernel-agent/fp8-kv-cache",
// section "Storage"), for a row of D values held four per lane by D/4
// consecutive, aligned lanes.
//
// A lane move inside a 16-lane row by a DPP control word (gfx9 encoding:
// quad permutation, row rotation, half-row mirror), every lane enabled.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// row_amax: max |x| over the row (exact).  Each lane takes the maximum of its
// four magnitudes; the lane group is then reduced by lane moves that stay
// inside it: the two quad swaps (lane ^ 1, lane ^ 2), then for 8 lanes the
// half-row mirror (the other quad), for 16 the rotations by 4 and 8 lanes
// (the other three quads), for 32 the 16-lane row swap as well.  The
// magnitudes are compared as their bit patterns: for finite non-negative
// floats the unsigned order of the patterns is the order of the values, and
// an integer maximum takes the lane move as its operand (one instruction a
// step).
template <int LANES_PER_ROW>
__device__ __forceinline__ float row_amax(float4 x) {
  static_assert(LANES_PER_ROW == 8 || LANES_PER_ROW == 16 || LANES_PER_ROW == 32, "lane group");
  uint32_t m = __float_as_uint(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  m = max(m, dpp_move<0xB1>(m));  // quad_perm [1, 0, 3, 2]
  m = max(m, dpp_move<0x4E>(m));  // quad_perm [2, 3, 0, 1]
  if constexpr (LANES_PER_ROW == 8) {
    m = max(m, dpp_move<0x141>(m));  // row_half_mirror
  } else {
    m = max(m, dpp_move<0x124>(m));  // row_ror 4
    m = max(m, dpp_move<0x128>(m));  // row_ror 8
  }
  if constexpr (LANES_PER_ROW == 32) {
    auto q = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    m = max((uint32_t)q[0], (uint32_t)q[1]);
  }
  return __uint_as_float(m);
}

// x / b from y = RN(1 / b): q = RN(x y), the exact remainder r = x - b q (one
// fma), then RN(q + r y).  With y the correctly rounded reciprocal this
// correction step returns the correctly rounded quotient whenever nothing
// underflows (Markstein's theorem on division by an fma-corrected
// reciprocal); the sign is taken from x so that -0 stays -0.
__host__ __device__ __forceinline__ float quotient_rn(float x, float b, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-b, q, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// RN(1 / s) for s in [2^-53, 2^125]: the hardware reciprocal (within an ulp)
// and one Newton step, e = 1 - s y0 (exact, one fma), y0 + e y0.  On gfx950
// this is the correctly rounded reciprocal for every fp32 s in that range
// (tests/test_gpu_reciprocal.py checks all 1.5 G of them on the device; from
// 2^126 on, where 1 / s is subnormal, it is not).
__device__ __forceinline__ float reciprocal_rn(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// The storage rule's scale RN(amax / 448) from the constant RN(1 / 448) and
// quotient_rn: exact for every fp32 amax in [2^-100, FLT_MAX] (checked for
// all of them on the host; tests/test_quotient_cpu.py repeats it on a
// stride); other values (zero, tiny, inf, NaN) divide.
__host__ __device__ __forceinline__ float storage_scale(float amax) {
  if (amax >= 0x1p-100f && amax <= 0x1.fffffep127f)
    return quotient_rn(amax, kE4M3Max, 1.0f / kE4M3Max);
  return amax / kE4M3Max;
}

// Four codes of the row with scale = amax / 448: the correctly rounded fp32
// quotient x / scale (no fast math), clamped to +-448 so that a row whose
// scale is an fp32 subnormal saturates, then rounded to nearest even onto OCP
// e4m3fn by v_cvt_pk_fp8_f32.  A zero scale gives zero codes.
// For a scale in [2^-53, 2^125] (every scale of a finite amax from
// 448 * 2^-53 up: amax / 448 < 2^120) the quotients come from one correctly
// rounded reciprocal per row (reciprocal_rn) and quotient_rn (three
// instructions each instead of a full division).  A quotient of magnitude
// 2^-11 or more is then exactly the correctly rounded one; below that quotient_rn may differ from it in the
// last bits, but both are under 2^-10 with the sign of x, so both round to the
// same signed zero code.  (Checked on the host against division for every
// fp32 x with |x| <= amax at several scales, among them significands of all
// ones and 2^-53; tests/test_quotient_cpu.py repeats the check on samples.)
// Other scales take the division.
__device__ __forceinline__ uint32_t e4m3_codes4(float4 x, float scale) {
  if (scale == 0.0f) return 0u;
  float q0, q1, q2, q3;
  if (scale >= 0x1p-53f && scale <= 0x1p125f) {
    // quotient_rn without its sign step, which is taken after the clamp
    // below: a nonzero quotient already has the sign of x, and the clamp
    // is symmetric, so the codes are those of quotient_rn
    const float y = reciprocal_rn(scale);  // RN(1 / scale)
    const float a0 = x.x * y, a1 = x.y * y, a2 = x.z * y, a3 = x.w * y;
    q0 = __builtin_fmaf(__builtin_fmaf(-scale, a0, x.x), y, a0);
    q1 = __builtin_fmaf(__builtin_fmaf(-scale, a1, x.y), y, a1);
    q2 = __builtin_fmaf(__builtin_fmaf(-scale, a2, x.z), y, a2);
    q3 = __builtin_fmaf(__builtin_fmaf(-scale, a3, x.w), y, a3);
  } else {
    q0 = x.x / scale;
    q1 = x.y / scale;
    q2 = x.z / scale;
    q3 = x.w / scale;
  }
  const float y0 = __builtin_copysignf(__builtin_amdgcn_fmed3f(q0, -kE4M3Max, kE4M3Max), x.x);
  const float y1 = __builtin_copysignf(__builtin_amdgcn_fmed3f(q1, -kE4M3Max, kE4M3Max), x.y);
  const float y2 = __builtin_copysignf(__builtin_amdgcn_fmed3f(q2, -kE4M3Max, kE4M3Max), x.z);
  const float y3 = __builtin_copysignf(__builtin_amdgcn_fmed3f(q3, -kE4M3Max, kE4M3Max), x.w);
  uint32_t codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)codes, true);
}

// Block-scaled (MX) rule for a block of 32 values: the scale is 2^E, the
// smallest power of two not below the storage rule's amax / 448 (so no code
// clamps), E clamped to [-126, 127] (a zero or tiny block takes -126).  The
// fp32 quotient is rounded like the per-row scale; E is read from its bits.
__device__ __forceinline__ int mx_exponent(float amax) {
  const float s = amax / kE4M3Max;  // correctly rounded
  if (!(s >= 0x1p-126f)) return -126;
  const uint32_t bits = __float_as_uint(s);
  const int e = (int)((bits >> 23) & 0xff) - 127;
  return min((bits & 0x7fffffu) ? e + 1 : e, 127);
}

// 2^E as fp32 (normal for E in [-126, 127]) from the E8M0 byte E + 127.
__device__ __forceinline__ float e8m0_value(uint32_t byte) { return __uint_as_float(byte << 23); }

// Two e4m3 codes times a power-of-two scale -> two bf16 (exact while the
// products stay in the normal range).
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2_scaled(uint32_t w, float scale, bool hi) {
  bf16x2_t v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
  return __builtin_bit_cast(uint32_t, v);
}

// D += A * B with per-lane block scales 2^(sa - 127), 2^(sb - 127) (E8M0
// bytes) applied by the instruction to the lane's 32 k-slots.
__device__ __forceinline__ f32x4_t mfma_16x16x128_e4m3_scaled(i32x8_t a, i32x8_t b, f32x4_t c,
                                                              int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Four values rounded to bf16 (nearest even): the K row of the K16V8 control
// and both rows of the BF16 control.
__device__ __forceinline__ u32x2_t bf16x4(float4 x) {
  return u32x2_t{f32x2_to_bf16x2(x.x, x.y), f32x2_to_bf16x2(x.z, x.w)};
}

}  // namespace fp8kv

// Raw buffer resource over the bytes [base, base + n_bytes): a load at an
// offset at or past n_bytes returns zeros and makes no memory access, so
// n_bytes = 0 turns a load into a no-op that still counts as issued.  Word 3
// is the gfx9-family default (data format 32: untyped buffer loads need a
// nonzero format there).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base,
                                                               uint32_t n_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n_bytes,
                                           0x00020000);
}
