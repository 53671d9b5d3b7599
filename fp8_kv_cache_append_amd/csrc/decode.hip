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

// Raw (still compressed) K/V of one 64-token tile in the registers of one
// lane, plus the scales of the lane's own token (token t0 + lane).
template <int MODE, int D>
struct TileRegs {
  static constexpr bool K8 = (MODE == kK8V8);
  static constexpr bool V8 = (MODE != kBF16);
  static constexpr int KP = D / 64;                      // 16-element pieces
  static constexpr int KRAW = K8 ? KP : 2 * KP;          // 16-byte K loads per sub-block
  static constexpr int DPR = D / 16;
  static constexpr int VW = V8 ? DPR / 4 : DPR / 2;      // dwords of V per token
  u32x4_t k[4][KRAW];
  uint32_t v[2][8][VW];
  float ks, vs;
};

// Issue the loads of the tile starting at token t0.  Tokens at or past t_end
// are not read (their registers are zero).  tab holds, in lane e, the block
// id of block t_begin / bs + e of the sequence; it is indexed with a
// wave-uniform lane, so every block id is a scalar.
template <int MODE, int D>
__device__ __forceinline__ void load_tile(TileRegs<MODE, D>& r, const DecodeArgs& a, int t0,
                                          int t_end, int tab, int e_base, int h, int g4, int c,
                                          int lane) {
  using T = TileRegs<MODE, D>;
  int blk[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    blk[kb] = __builtin_amdgcn_readlane(tab, min((t0 + 16 * kb) / a.bs - e_base, 63));
  auto row_of = [&](int kb, int t) -> int64_t {
    return ((int64_t)blk[kb] * a.bs + t % a.bs) * a.hkv + h;
  };
  {  // scales of token t0 + lane
    const int t = t0 + lane;
    const int kb = lane >> 4;
    const int64_t rr = ((int64_t)(kb == 0 ? blk[0] : kb == 1 ? blk[1] : kb == 2 ? blk[2] : blk[3]) *
                            a.bs + t % a.bs) * a.hkv + h;
    r.ks = (T::K8 && t < t_end) ? a.ks[rr] : 0.0f;
    r.vs = (T::V8 && t < t_end) ? a.vs[rr] : 0.0f;
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {  // K: lane (g4, c) reads token 16*kb + c
    const int t = t0 + 16 * kb + c;
    const bool ok = t < t_end;
    const int64_t rr = row_of(kb, t);
#pragma unroll
    for (int p = 0; p < T::KP; ++p) {
      if (T::K8) {
        const uint8_t* src = static_cast<const uint8_t*>(a.k) + rr * D + 64 * p + 16 * g4;
        r.k[kb][p] = ok ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const uint16_t* src = static_cast<const uint16_t*>(a.k) + rr * D + 64 * p + 16 * g4;
        r.k[kb][2 * p] = ok ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
        r.k[kb][2 * p + 1] =
            ok ? *reinterpret_cast<const u32x4_t*>(src + 8) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {  // V: k-slot j of chunk kp -> token 32kp + 16(j/4) + 4g4 + j%4
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = 2 * kp + (j >> 2);
      const int t = t0 + 16 * kb + 4 * g4 + (j & 3);
      const bool ok = t < t_end;
      const int64_t rr = row_of(kb, t);
      const uint8_t* src = static_cast<const uint8_t*>(a.v) + (rr * D + T::DPR * c) * (T::V8 ? 1 : 2);
      if constexpr (T::VW == 4) {
        const u32x4_t w = ok ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) r.v[kp][j][e] = w[e];
      } else if constexpr (T::VW == 2) {
        const u32x2_t w = ok ? *reinterpret_cast<const u32x2_t*>(src) : u32x2_t{0u, 0u};
        r.v[kp][j][0] = w[0];
        r.v[kp][j][1] = w[1];
      } else {
        r.v[kp][j][0] = ok ? *reinterpret_cast<const uint32_t*>(src) : 0u;
      }
    }
  }
}

template <int MODE, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_partial_kernel(DecodeArgs a) {
  using T = TileRegs<MODE, D>;
  constexpr int KC = D / 32;         // MFMA k-chunks for QK
  constexpr int DPR = T::DPR;        // d values per V^T row group (MFMAs per PV chunk)
  constexpr bool kK8 = T::K8;
  constexpr bool kV8 = T::V8;

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
  const int G = a.group;
  const int t_begin = split * a.chunk;

  // First round trip, all independent: the sequence length, the block ids
  // of this split (lane e: block t_begin / bs + e, index kept inside the
  // table row; ids past the sequence are never used) and Q.
  const int len = a.seq_lens[b];
  const int e_base = t_begin / a.bs;
  const int tab = a.table[(int64_t)b * a.mbps + min(e_base + lane, a.mbps - 1)];
  u32x4_t qb[KC];  // Q^T as the B operand of QK: lane (g4, c) holds head c's d-set
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.hkv * G + (int64_t)h * G + min(c, G - 1)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + d0);
      qb[kc] = (c < G) ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const int t_end = min(len, t_begin + a.chunk);

  float* pacc = a.part_acc + ((int64_t)bh * a.n_splits + split) * G * D;
  float* pml = a.part_ml + ((int64_t)bh * a.n_splits + split) * G * 2;
  if (t_begin >= t_end) {  // no key in this split
    for (int i = threadIdx.x; i < G; i += blockDim.x) {
      pml[2 * i] = -INFINITY;
      pml[2 * i + 1] = 0.0f;
    }
    return;
  }

  float m_run = -INFINITY;  // integer reference (log2 units) of head c
  float l_run = 0.0f;       // this lane's share of the normaliser of head c
  f32x4_t acc[DPR];
#pragma unroll
  for (int j = 0; j < DPR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  // Double buffer: the loads of tile i + kWaves are in flight while tile i
  // is computed.
  T cur, nxt;
  if (wave < n_tiles)
    load_tile<MODE, D>(cur, a, t_begin + wave * kTile, t_end, tab, e_base, h, g4, c, lane);

  for (int tile = wave; tile < n_tiles; tile += kWaves) {
    const int t0 = t_begin + tile * kTile;
    const bool more = tile + kWaves < n_tiles;
    if (more)
      load_tile<MODE, D>(nxt, a, t0 + kWaves * kTile, t_end, tab, e_base, h, g4, c, lane);

    // --- per-token scales of the tile -> LDS, then the four each lane needs.
    // The wave writes and reads its own slice; LDS operations of one wave
    // complete in order, and the previous tile's reads precede these writes
    // in program order.
    if (kK8) s_scale[wave][0][lane] = cur.ks;
    if (kV8) s_scale[wave][1][lane] = cur.vs;
    __builtin_amdgcn_wave_barrier();

    // --- QK on the matrix cores
    f32x4_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4_t av;
        if (kK8) {
          const u32x4_t w = cur.k[kb][kc >> 1];
          const uint32_t lo = w[2 * (kc & 1)], hi = w[2 * (kc & 1) + 1];
          av = u32x4_t{e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                       e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi)};
        } else {
          av = cur.k[kb][kc];
        }
        s = mfma_16x16x32_bf16(av, qb[kc], s);
      }
      sacc[kb] = s;
    }

    // --- scores in log2 units, K scale folded in after the product
    float sc[4][4], vsc[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int base = 16 * kb + 4 * g4;
      f32x4_t ksv = {1.f, 1.f, 1.f, 1.f}, vsv = {1.f, 1.f, 1.f, 1.f};
      if (kK8) ksv = *reinterpret_cast<const f32x4_t*>(&s_scale[wave][0][base]);
      if (kV8) vsv = *reinterpret_cast<const f32x4_t*>(&s_scale[wave][1][base]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + base + i;
        float s = kK8 ? (sacc[kb][i] * ksv[i]) * a.c_scale : sacc[kb][i] * a.c_scale;
        s = (t < t_end) ? s : -INFINITY;
        sc[kb][i] = s;
        vsc[kb][i] = vsv[i];
        tmax = fmaxf(tmax, s);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // --- online softmax update with an integer reference (every tile holds
    //     at least one valid token, so tmax is finite)
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
            const uint32_t x = byte_perm(cur.v[kp][j0][wsel], cur.v[kp][j1][wsel], sel);
            av[jp] = e4m3x2_to_bf16x2(x, (byte & 1) != 0);
          } else {
            const int e = db >> 1;
            const uint32_t sel = (db & 1) ? 0x03020706u : 0x01000504u;
            av[jp] = byte_perm(cur.v[kp][j0][e], cur.v[kp][j1][e], sel);
          }
        }
        acc[db] = mfma_16x16x32_bf16(av, pb[kp], acc[db]);
      }
    }
    if (more) cur = nxt;
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
  for (int idx = 4 * threadIdx.x; idx < G * D; idx += 4 * blockDim.x) {
    const int g = idx / D, d = idx % D;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += *reinterpret_cast<const f32x4_t*>(&s_acc[w][g][d]);
    *reinterpret_cast<f32x4_t*>(pacc + idx) = sum;
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

// Second kernel: merge the splits of each (sequence, query head).  The splits
// are consumed in batches of kMergeBatch whose loads are all issued before
// any is used, and the batches are combined online with power-of-two weights
// (one memory round trip per batch, not per split).
constexpr int kMergeBatch = 8;

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
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_splits; s0 += kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch];
    f32x4_t x[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int s = min(s0 + i, n_splits - 1);
      const f32x2_t v = *reinterpret_cast<const f32x2_t*>(ml + ((int64_t)s * group + g) * 2);
      m[i] = (s0 + i < n_splits) ? v[0] : -INFINITY;
      l[i] = v[1];
      x[i] = *reinterpret_cast<const f32x4_t*>(pa + ((int64_t)s * group + g) * D + 4 * d4);
    }
    float mb = m_run;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) mb = fmaxf(mb, m[i]);
    if (mb == -INFINITY) continue;  // nothing yet
    if (m_run != -INFINITY && mb != m_run) {
      const float alpha = ldexpf(1.0f, (int)(m_run - mb));
      l_run *= alpha;
      acc *= alpha;
    }
    m_run = mb;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (m[i] == -INFINITY) continue;  // empty split: weight 0
      const float w = ldexpf(1.0f, (int)(m[i] - m_run));
      l_run += w * l[i];
      acc += w * x[i];
    }
  }
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  if (l_run > 0.0f) o = acc / l_run;
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
