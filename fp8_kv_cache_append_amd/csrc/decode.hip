// Split-KV decode attention over the paged e4m3 / bf16 cache.
//
// What is computed ("kadirnar/kernel-agent/fp8-kv-cache", sections "Math" and
// "Speed"; "FP8 KV attention: hardware paths and tile preparation", section
// "Operating model"; "03 . 8n - FA-style tiled prefill attention", section
// 2.1):  each work-group owns one (sequence, KV head, split of the keys).
// It reads the split's K/V codes once from HBM, turns only the active
// 64-token tile into bf16 MFMA operands in registers, folds k_scale into the
// scores after the QK product and v_scale into P before its bf16 rounding,
// and advances the online softmax tile by tile.  The unnormalised partial
// (M, l, acc) goes to HBM; a second kernel merges the splits.
//
// Softmax reference.  M is an integer in log2 units (the running maximum of
// the scores rounded up).  Every rescale 2^(M_old - M_new) is then an exact
// power of two, and since bf16 rounding commutes with power-of-two scaling the
// rounded P does not depend on how the keys are cut into tiles and splits.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, lane l = 16*g4 + c):
//   QK   S^T[t][head] = K[t][:] . Q[head][:]  A = K tile (16 tokens x 32 d),
//        B = Q^T (32 d x 16 heads; heads >= G are zero).  The contraction
//        order over d is free, so lane (g4, r) takes d in
//        [16*g4, 16*g4+16) (+64 for D = 128): its A operand is one or two
//        16-byte loads of token r's row, converted e4m3 -> bf16 in pairs.
//        Result: lane (g4, c) holds head c, tokens 4*g4 + i of the 16-block.
//   PV   O^T[d][head] = sum_t V^T[d][t] * P^T[t][head]   A = V^T, B = P^T.
//        The k-slots of lane group g4 are mapped to the tokens whose P that
//        lane already holds (4*g4 + i of two 16-blocks), so P needs no data
//        movement, and the accumulator rows stay indexed by the head of the
//        softmax state.  A row m of V^T is d = DPR*m + db for MFMA number db:
//        lane (g4, r) loads DPR contiguous codes of each of its 8 tokens and
//        transposes them in registers with byte permutes.
//   Result: lane (g4, c) holds O[head c][d] for d in [4*DPR*g4, 4*DPR*(g4+1)).
//
// No LDS traffic on the K/V path; LDS holds the tile's per-token scales (so
// each lane can read the four it needs) and the work-group merge.
#include "device.h"
#include "launch.h"

namespace fp8kv {

struct DecodeArgs {
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  const int32_t* table;
  const uint16_t* q;
  const int32_t* seq_lens;
  float* part_acc;
  float* part_ml;
  float c_scale;  // sm_scale * log2(e)
  int hkv;
  int group;
  int bs;
  int mbps;
  int chunk;
  int n_splits;
};

constexpr int kWaves = 4;     // waves per work-group; tiles are dealt round-robin
constexpr int kTile = 64;     // tokens per tile
constexpr int kMaxGroup = 16; // query heads per KV head (one MFMA column block)

template <int MODE, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_partial_kernel(DecodeArgs a) {
  constexpr int KP = D / 64;         // 16-element pieces of a lane's d-set
  constexpr int KC = D / 32;         // MFMA k-chunks for QK
  constexpr int DPR = D / 16;        // d values per V^T row group (MFMAs per PV chunk)
  constexpr bool kK8 = (MODE == kK8V8);
  constexpr bool kV8 = (MODE != kBF16);

  __shared__ float s_scale[kWaves][2][kTile];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];
  __shared__ float s_acc[kWaves][kMaxGroup][D];

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4;   // k-slot group of the lane
  const int c = lane & 15;    // row / column of the lane

  const int wg = blockIdx.x;
  const int split = wg % a.n_splits;
  const int bh = wg / a.n_splits;  // b * hkv + h
  const int h = bh % a.hkv;
  const int b = bh / a.hkv;
  const int len = a.seq_lens[b];
  const int t_begin = split * a.chunk;
  const int t_end = min(len, t_begin + a.chunk);
  const int G = a.group;

  float* pacc = a.part_acc + ((int64_t)bh * a.n_splits + split) * G * D;
  float* pml = a.part_ml + ((int64_t)bh * a.n_splits + split) * G * 2;
  if (t_begin >= t_end) {  // no key in this split
    for (int i = threadIdx.x; i < G; i += blockDim.x) {
      pml[2 * i] = -INFINITY;
      pml[2 * i + 1] = 0.0f;
    }
    return;
  }

  // Q^T as the B operand of QK: lane (g4, c) holds head c's d-set.
  u32x4_t qb[KC];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.hkv * G + (int64_t)h * G + c) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
      if (c < G)
        qb[kc] = *reinterpret_cast<const u32x4_t*>(qrow + d0);
      else
        qb[kc] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  float m_run = -INFINITY;  // integer reference (log2 units) of head c
  float l_run = 0.0f;       // this lane's share of the normaliser of head c
  f32x4_t acc[DPR];
#pragma unroll
  for (int j = 0; j < DPR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t tab_row = (int64_t)b * a.mbps;
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;

  for (int tile = wave; tile < n_tiles; tile += kWaves) {
    const int t0 = t_begin + tile * kTile;
    // Block of each 16-token sub-block (bs is a multiple of 16, so a
    // sub-block never straddles two blocks).  Tokens past t_end load the
    // last valid token instead and are masked below.
    int blk[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int tb = min(t0 + 16 * kb, t_end - 1);
      blk[kb] = a.table[tab_row + tb / a.bs];
    }
    auto row_of = [&](int kb, int t) -> int64_t {
      const int tc = min(t, t_end - 1);
      return ((int64_t)blk[kb] * a.bs + tc % a.bs) * a.hkv + h;
    };

    // --- per-token scales of the tile -> LDS (lane l: token t0 + l)
    if (kK8 || kV8) {
      const int64_t r = row_of(lane >> 4, t0 + lane);
      if (kK8) s_scale[wave][0][lane] = a.ks[r];
      if (kV8) s_scale[wave][1][lane] = a.vs[r];
    }

    // --- K tile loads: lane (g4, r = c) reads token 16*kb + c
    u32x4_t kraw[4][kK8 ? KP : 2 * KP];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t r = row_of(kb, t0 + 16 * kb + c);
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        if (kK8) {
          const uint8_t* src = static_cast<const uint8_t*>(a.k) + r * D + 64 * p + 16 * g4;
          kraw[kb][p] = *reinterpret_cast<const u32x4_t*>(src);
        } else {
          const uint16_t* src = static_cast<const uint16_t*>(a.k) + r * D + 64 * p + 16 * g4;
          kraw[kb][2 * p] = *reinterpret_cast<const u32x4_t*>(src);
          kraw[kb][2 * p + 1] = *reinterpret_cast<const u32x4_t*>(src + 8);
        }
      }
    }

    // --- V tile loads: lane (g4, r = c), chunk kp, k-slot j -> token
    //     32*kp + 16*(j/4) + 4*g4 + (j%4); DPR contiguous elements at d = DPR*c
    constexpr int VW = kV8 ? DPR / 4 : DPR / 2;  // dwords per token
    uint32_t vraw[2][8][VW];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = 2 * kp + (j >> 2);
        const int64_t r = row_of(kb, t0 + 16 * kb + 4 * g4 + (j & 3));
        if (kV8) {
          const uint8_t* src = static_cast<const uint8_t*>(a.v) + r * D + DPR * c;
          if constexpr (VW == 2) {
            const u32x2_t w = *reinterpret_cast<const u32x2_t*>(src);
            vraw[kp][j][0] = w[0];
            vraw[kp][j][VW - 1] = w[1];
          } else {
            vraw[kp][j][0] = *reinterpret_cast<const uint32_t*>(src);
          }
        } else {
          const uint16_t* src = static_cast<const uint16_t*>(a.v) + r * D + DPR * c;
          if constexpr (VW == 4) {
            const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
            for (int e = 0; e < VW; ++e) vraw[kp][j][e] = w[e];
          } else {
            const u32x2_t w = *reinterpret_cast<const u32x2_t*>(src);
            vraw[kp][j][0] = w[0];
            vraw[kp][j][VW - 1] = w[1];
          }
        }
      }
    }

    // --- QK on the matrix cores
    f32x4_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4_t av;
        if (kK8) {
          const u32x4_t w = kraw[kb][kc >> 1];
          const uint32_t lo = w[2 * (kc & 1)], hi = w[2 * (kc & 1) + 1];
          av = u32x4_t{e4m3x2_to_bf16x2(lo, false), e4m3x2_to_bf16x2(lo, true),
                       e4m3x2_to_bf16x2(hi, false), e4m3x2_to_bf16x2(hi, true)};
        } else {
          av = kraw[kb][kc];
        }
        s = mfma_16x16x32_bf16(av, qb[kc], s);
      }
      sacc[kb] = s;
    }

    // --- scores in log2 units, K scale folded in after the product
    float ksc[4][4], vsc[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int base = 16 * kb + 4 * g4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ksc[kb][i] = kK8 ? s_scale[wave][0][base + i] : 1.0f;
        vsc[kb][i] = kV8 ? s_scale[wave][1][base + i] : 1.0f;
      }
    }
    float sc[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * kb + 4 * g4 + i;
        float s = kK8 ? (sacc[kb][i] * ksc[kb][i]) * a.c_scale : sacc[kb][i] * a.c_scale;
        s = (t < t_end) ? s : -INFINITY;
        sc[kb][i] = s;
        tmax = fmaxf(tmax, s);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // --- online softmax update with an integer reference
    const float m_new = fmaxf(m_run, ceilf(tmax));
    if (m_new != m_run) {
      const float alpha = (m_run == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(m_run - m_new));
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < DPR; ++j) acc[j] *= alpha;
      m_run = m_new;
    }

    // --- P with the V scale folded in, rounded to bf16: B operand of PV
    u32x4_t pb[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = 2 * kp + (j >> 2), i = j & 3;
        const float p = exp2f(sc[kb][i] - m_run);
        l_run += p;
        pv[j] = p * vsc[kb][i];
      }
      pb[kp] = u32x4_t{f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3]),
                       f32x2_to_bf16x2(pv[4], pv[5]), f32x2_to_bf16x2(pv[6], pv[7])};
    }

    // --- PV on the matrix cores: V^T tile as the A operand
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int db = 0; db < DPR; ++db) {
        u32x4_t av;
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const int j0 = 2 * jp, j1 = 2 * jp + 1;
          if (kV8) {
            // codes of token j0 and j1 at d = DPR*c + db -> bf16 pair
            const int wsel = db >> 2, byte = db & 3;
            const int k2 = byte & 2;  // byte pair (k2, k2+1)
            const uint32_t sel = (uint32_t)(k2 + 4) | ((uint32_t)k2 << 8) |
                                 ((uint32_t)(k2 + 5) << 16) | ((uint32_t)(k2 + 1) << 24);
            const uint32_t x = byte_perm(vraw[kp][j0][wsel], vraw[kp][j1][wsel], sel);
            av[jp] = e4m3x2_to_bf16x2(x, (byte & 1) != 0);
          } else {
            const int e = db >> 1;
            const uint32_t sel = (db & 1) ? 0x03020706u : 0x01000504u;
            av[jp] = byte_perm(vraw[kp][j0][e], vraw[kp][j1][e], sel);
          }
        }
        acc[db] = mfma_16x16x32_bf16(av, pb[kp], acc[db]);
      }
    }
  }

  // --- normaliser of head c: sum the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // --- merge the waves of the work-group (power-of-two weights)
  if (g4 == 0) {
    s_m[wave][c] = m_run;
    s_l[wave][c] = l_run;
  }
  __syncthreads();
  float m_star = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m_star = fmaxf(m_star, s_m[w][c]);
  const float wgt = (m_run == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(m_run - m_star));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4_t lo, hi;
#pragma unroll
    for (int db = 0; db < 4; ++db) lo[db] = acc[db][i] * wgt;
    *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][DPR * (4 * g4 + i)]) = lo;
    if constexpr (DPR == 8) {
#pragma unroll
      for (int db = 0; db < 4; ++db) hi[db] = acc[4 + db][i] * wgt;
      *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][DPR * (4 * g4 + i) + 4]) = hi;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += s_acc[w][g][d];
    pacc[idx] = sum;
  }
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    float lsum = 0.0f;
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, s_m[w][g]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (s_m[w][g] != -INFINITY) lsum += ldexpf(s_l[w][g], (int)(s_m[w][g] - ms));
    pml[2 * g] = ms;
    pml[2 * g + 1] = lsum;
  }
}

// Second kernel: merge the splits of each (sequence, query head).
template <int D>
__global__ __launch_bounds__(512) void decode_merge_kernel(int hkv, int group, int n_splits,
                                                           const float* __restrict__ part_acc,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ out) {
  constexpr int L = D / 4;  // lanes per head, four values each
  const int bh = blockIdx.x;
  const int g = threadIdx.x / L;
  const int d4 = threadIdx.x % L;
  if (g >= group) return;
  const float* ml = part_ml + (int64_t)bh * n_splits * group * 2;
  const float* pa = part_acc + (int64_t)bh * n_splits * group * D;
  float m_star = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m_star = fmaxf(m_star, ml[(s * group + g) * 2]);
  float lsum = 0.0f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (m_star != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float m = ml[(s * group + g) * 2];
      if (m == -INFINITY) continue;
      const float w = ldexpf(1.0f, (int)(m - m_star));
      lsum += w * ml[(s * group + g) * 2 + 1];
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(pa + ((int64_t)s * group + g) * D + 4 * d4);
      acc += w * x;
    }
  }
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  if (lsum > 0.0f) o = acc / lsum;
  // bh = b * hkv + h, output head h * group + g
  *reinterpret_cast<f32x4_t*>(out + ((int64_t)bh * group + g) * D + 4 * d4) = o;
}

template <int MODE>
static void launch_partial_mode(const CacheView& c, const DecodeArgs& a, unsigned n_wg,
                                hipStream_t stream) {
  if (c.d == 128)
    hipLaunchKernelGGL((decode_partial_kernel<MODE, 128>), dim3(n_wg), dim3(64 * kWaves), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((decode_partial_kernel<MODE, 64>), dim3(n_wg), dim3(64 * kWaves), 0,
                       stream, a);
}

hipError_t launch_decode_partial(const CacheView& c, const uint16_t* q, int group,
                                 const int32_t* seq_lens, int batch, float c_scale,
                                 int chunk, int n_splits, float* part_acc,
                                 float* part_ml, hipStream_t stream) {
  DecodeArgs a{c.k, c.v, c.ks, c.vs, c.table, q, seq_lens, part_acc, part_ml,
               c_scale, c.hkv, group, c.bs, c.mbps, chunk, n_splits};
  const unsigned n_wg = (unsigned)((int64_t)batch * c.hkv * n_splits);
  switch (c.mode) {
    case kK8V8: launch_partial_mode<kK8V8>(c, a, n_wg, stream); break;
    case kK16V8: launch_partial_mode<kK16V8>(c, a, n_wg, stream); break;
    default: launch_partial_mode<kBF16>(c, a, n_wg, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(int batch, int hkv, int group, int d, int n_splits,
                               const float* part_acc, const float* part_ml, float* out,
                               hipStream_t stream) {
  const unsigned n_wg = (unsigned)((int64_t)batch * hkv);
  const unsigned threads = (unsigned)(group * (d / 4));
  if (d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(n_wg), dim3(threads), 0, stream, hkv,
                       group, n_splits, part_acc, part_ml, out);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(n_wg), dim3(threads), 0, stream, hkv,
                       group, n_splits, part_acc, part_ml, out);
  return hipGetLastError();
}

}  // namespace fp8kv
