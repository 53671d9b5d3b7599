// FA-style tiled causal prefill over the paged e4m3 / bf16 cache.
//
// Shape ("03 . 8n - FA-style tiled prefill attention", sections 2.1-3.3):
// one work-group per (64-query tile, query head); query head h reads KV head
// h / G; K/V stream through on-chip memory tile by tile (64 keys), the
// output accumulator stays in registers, the softmax is online, keys past the
// tile's last query position are never read (positions are data), the
// causal mask is kv <= q position, a fully masked tile leaves the state
// untouched and a row with no visible key writes 0.  Scores follow
// "kadirnar/kernel-agent/fp8-kv-cache" ("Math"): k_scale multiplies the
// QK product, v_scale is folded into P before its bf16 rounding.
//
// gfx950 mapping.  Four waves; wave w owns query rows 16w .. 16w+15 of the
// tile.  Each 64-key tile is loaded once per work-group (16-byte global
// loads), converted e4m3 -> bf16 with the packed gfx950 convert and written
// to LDS (rows padded by 16 bytes against bank conflicts), double-buffered so
// the next tile's global loads are in flight during the current tile's
// matrix work.  QK and PV use v_mfma_f32_16x16x32_bf16 in the transposed
// form of the decode kernel: S^T = K Q^T (lane (g4, c) holds query row c,
// keys 4*g4 + i of each 16-key block) and O^T = V^T P^T, so P goes from the
// QK result straight into the PV operand and the accumulator rows share the
// softmax state of their lane.  The integer log2-domain reference makes every
// rescale an exact power of two.
//
// LDS reuse: tile j is written into buffer j & 1 before the barrier of
// iteration j and read after it.  Iteration j + 1 writes buffer (j + 1) & 1,
// which was last read in iteration j - 1; every wave has left iteration j - 1
// once it passes the barrier of iteration j, which precedes that write in
// program order.  One barrier per tile is therefore enough.
#include "device.h"
#include "launch.h"

namespace fp8kv {

struct PrefillArgs {
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  const int32_t* table;
  const uint16_t* q;
  const int32_t* cu_q;
  const int32_t* q_pos0;
  const int32_t* seq_lens;
  float* out;
  float c_scale;
  int hkv;
  int group;
  int bs;
  int mbps;
  int n_qt;  // query tiles per sequence (ceil(max_q_len / 64))
  int total_q;
  int num_blocks;
};

constexpr int kPWaves = 4;
constexpr int kQT = 64;   // queries per tile
constexpr int kKT = 64;   // keys per tile

template <int MODE, int D>
struct PrefillShape {
  static constexpr bool K8 = (MODE == kK8V8);
  static constexpr bool V8 = (MODE != kBF16);
  static constexpr int LD = D + 8;                           // LDS row (bf16), padded
  static constexpr int KBYTES = K8 ? D : 2 * D;              // bytes of one K row in HBM
  static constexpr int VBYTES = V8 ? D : 2 * D;
  static constexpr int KW = KBYTES / 4 / 16;                 // 16-byte loads per thread (K)
  static constexpr int VW = VBYTES / 4 / 16;                 // (V)
};

template <int MODE, int D>
__global__ __launch_bounds__(64 * kPWaves) void prefill_kernel(PrefillArgs a) {
  using S = PrefillShape<MODE, D>;
  constexpr int KC = D / 32;
  constexpr int DPR = D / 16;

  __shared__ __attribute__((aligned(16))) __bf16 s_k[2][kKT][S::LD];
  __shared__ __attribute__((aligned(16))) __bf16 s_v[2][kKT][S::LD];
  __shared__ float s_ks[2][kKT];
  __shared__ float s_vs[2][kKT];
  __shared__ float s_ok[2][kKT];  // 1: the key's block id is valid, 0: key not read

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int c = lane & 15;

  // Largest query tiles first: causal work grows with the tile index.
  const int hq = a.hkv * a.group;
  const int h = blockIdx.x % hq;
  const int rest = blockIdx.x / hq;
  const int qt = a.n_qt - 1 - (rest % a.n_qt);
  const int b = rest / a.n_qt;
  const int hk = h / a.group;

  // Device data is clamped so that no access leaves the buffers: query rows
  // stay inside [0, total_q), lengths inside the block-table capacity.
  const int q_begin = min(max(a.cu_q[b], 0), a.total_q);
  const int q_end = min(max(a.cu_q[b + 1], q_begin), a.total_q);
  const int n_q = min(q_end - q_begin, a.n_qt * kQT);
  if (qt * kQT >= n_q) return;
  const int pos0 = a.q_pos0[b];
  const int seq_len = min(max(a.seq_lens[b], 0), a.mbps * a.bs);
  const int last_q = min(qt * kQT + kQT, n_q) - 1;
  const int kv_end = max(0, min(seq_len, pos0 + last_q + 1));  // keys past the last query: skipped

  // query row of this lane and its position (-1: padding row, sees nothing)
  const int qrow = qt * kQT + 16 * wave + c;
  const int qpos = (qrow < n_q) ? pos0 + qrow : -1;

  // Q^T as the B operand of QK
  u32x4_t qb[KC];
  {
    const uint16_t* qp = a.q + ((int64_t)(q_begin + min(qrow, n_q - 1)) * hq + h) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
      qb[kc] = (qrow < n_q) ? *reinterpret_cast<const u32x4_t*>(qp + d0) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[DPR];
#pragma unroll
  for (int j = 0; j < DPR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int n_kt = (kv_end + kKT - 1) / kKT;
  const int64_t tab_row = (int64_t)b * a.mbps;

  // staging: thread -> (key tid / 4, quarter tid % 4 of the row)
  const int skey = tid >> 2, spart = tid & 3;
  u32x4_t kreg[S::KW], vreg[S::VW];
  float ksreg = 0.0f, vsreg = 0.0f, okreg = 0.0f;
  auto load_tile = [&](int t0) {
    const int t = min(t0 + skey, kv_end - 1);
    const int blk = a.table[tab_row + t / a.bs];
    const bool ok = (unsigned)blk < (unsigned)a.num_blocks;  // else: key not read
    const int64_t row = ((int64_t)(ok ? blk : 0) * a.bs + t % a.bs) * a.hkv + hk;
    const uint8_t* kp = static_cast<const uint8_t*>(a.k) + row * S::KBYTES + spart * (S::KBYTES / 4);
    const uint8_t* vp = static_cast<const uint8_t*>(a.v) + row * S::VBYTES + spart * (S::VBYTES / 4);
#pragma unroll
    for (int i = 0; i < S::KW; ++i)
      kreg[i] = ok ? reinterpret_cast<const u32x4_t*>(kp)[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < S::VW; ++i)
      vreg[i] = ok ? reinterpret_cast<const u32x4_t*>(vp)[i] : u32x4_t{0u, 0u, 0u, 0u};
    if (spart == 0) {
      ksreg = (S::K8 && ok) ? a.ks[row] : 1.0f;
      vsreg = (S::V8 && ok) ? a.vs[row] : 1.0f;
      okreg = ok ? 1.0f : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
    // K: bf16 elements [spart * D/4, (spart+1) * D/4) of row skey
    __bf16* kd = &s_k[buf][skey][spart * (D / 4)];
    __bf16* vd = &s_v[buf][skey][spart * (D / 4)];
    if (S::K8) {
#pragma unroll
      for (int i = 0; i < S::KW; ++i) {
        const u32x4_t w = kreg[i];
        u32x4_t lo = {e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
                      e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
        u32x4_t hi = {e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
                      e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
        reinterpret_cast<u32x4_t*>(kd)[2 * i] = lo;
        reinterpret_cast<u32x4_t*>(kd)[2 * i + 1] = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::KW; ++i) reinterpret_cast<u32x4_t*>(kd)[i] = kreg[i];
    }
    if (S::V8) {
#pragma unroll
      for (int i = 0; i < S::VW; ++i) {
        const u32x4_t w = vreg[i];
        u32x4_t lo = {e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
                      e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
        u32x4_t hi = {e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
                      e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
        reinterpret_cast<u32x4_t*>(vd)[2 * i] = lo;
        reinterpret_cast<u32x4_t*>(vd)[2 * i + 1] = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::VW; ++i) reinterpret_cast<u32x4_t*>(vd)[i] = vreg[i];
    }
    if (spart == 0) {
      s_ks[buf][skey] = ksreg;
      s_vs[buf][skey] = vsreg;
      s_ok[buf][skey] = okreg;
    }
  };

  if (n_kt > 0) load_tile(0);
  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const int t0 = j * kKT;
    store_tile(buf);
    __syncthreads();
    if (j + 1 < n_kt) load_tile(t0 + kKT);

    // --- S^T = K Q^T for 4 blocks of 16 keys
    f32x4_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
      const __bf16* krow = &s_k[buf][16 * kb + c][0];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
        s = mfma_16x16x32_bf16(*reinterpret_cast<const u32x4_t*>(krow + d0), qb[kc], s);
      }
      sacc[kb] = s;
    }

    // --- scores (log2 units), causal and length mask
    float sc[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4_t ksv = *reinterpret_cast<const f32x4_t*>(&s_ks[buf][16 * kb + 4 * g4]);
      const f32x4_t okv = *reinterpret_cast<const f32x4_t*>(&s_ok[buf][16 * kb + 4 * g4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * kb + 4 * g4 + i;
        float s = S::K8 ? (sacc[kb][i] * ksv[i]) * a.c_scale : sacc[kb][i] * a.c_scale;
        s = (t <= qpos && t < kv_end && okv[i] != 0.0f) ? s : -INFINITY;
        sc[kb][i] = s;
        tmax = fmaxf(tmax, s);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // --- online softmax; a fully masked tile (tmax = -inf) keeps the state
    const float m_new = fmaxf(m_run, ceilf(tmax));
    if (m_new != m_run && m_new != -INFINITY) {
      const float alpha = (m_run == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(m_run - m_new));
      l_run *= alpha;
#pragma unroll
      for (int jj = 0; jj < DPR; ++jj) acc[jj] *= alpha;
      m_run = m_new;
    }

    u32x4_t pb[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      float pv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int kb = 2 * kp + (jj >> 2), i = jj & 3;
        const float p = (sc[kb][i] == -INFINITY) ? 0.0f : exp2f(sc[kb][i] - m_run);
        l_run += p;
        pv[jj] = p * s_vs[buf][16 * kb + 4 * g4 + i];
      }
      pb[kp] = u32x4_t{f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3]),
                       f32x2_to_bf16x2(pv[4], pv[5]), f32x2_to_bf16x2(pv[6], pv[7])};
    }

    // --- O^T += V^T P^T: lane (g4, r) reads DPR values at d = DPR*r of its
    //     8 keys and transposes them into the A operands with byte permutes
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      uint32_t vw[8][DPR / 2];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int key = 32 * kp + 16 * (jj >> 2) + 4 * g4 + (jj & 3);
        const __bf16* src = &s_v[buf][key][DPR * c];
        if constexpr (DPR == 8) {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
          for (int e = 0; e < 4; ++e) vw[jj][e] = x[e];
        } else {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(src);
          vw[jj][0] = x[0];
          vw[jj][1] = x[1];
        }
      }
#pragma unroll
      for (int db = 0; db < DPR; ++db) {
        u32x4_t av;
        const uint32_t sel = (db & 1) ? 0x03020706u : 0x01000504u;
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) av[jp] = byte_perm(vw[2 * jp][db >> 1], vw[2 * jp + 1][db >> 1], sel);
        acc[db] = mfma_16x16x32_bf16(av, pb[kp], acc[db]);
      }
    }
  }

  // --- normalise and write: lane (g4, c) holds d = DPR*(4*g4 + i) + db
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qrow < n_q) {
    float* orow = a.out + ((int64_t)(q_begin + qrow) * hq + h) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t lo, hi;
#pragma unroll
      for (int db = 0; db < 4; ++db) lo[db] = (l_run > 0.0f) ? acc[db][i] / l_run : 0.0f;
      *reinterpret_cast<f32x4_t*>(orow + DPR * (4 * g4 + i)) = lo;
      if constexpr (DPR == 8) {
#pragma unroll
        for (int db = 0; db < 4; ++db) hi[db] = (l_run > 0.0f) ? acc[4 + db][i] / l_run : 0.0f;
        *reinterpret_cast<f32x4_t*>(orow + DPR * (4 * g4 + i) + 4) = hi;
      }
    }
  }
}

template <int MODE>
static void launch_prefill_mode(int d, const PrefillArgs& a, unsigned n_wg, hipStream_t stream) {
  if (d == 128)
    hipLaunchKernelGGL((prefill_kernel<MODE, 128>), dim3(n_wg), dim3(64 * kPWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<MODE, 64>), dim3(n_wg), dim3(64 * kPWaves), 0, stream, a);
}

hipError_t launch_prefill(const CacheView& c, const uint16_t* q, int group,
                          const int32_t* cu_q, const int32_t* q_pos0,
                          const int32_t* seq_lens, int batch, int total_q, int max_q_len,
                          float c_scale, float* out, hipStream_t stream) {
  const int n_qt = (max_q_len + kQT - 1) / kQT;
  PrefillArgs a{c.k, c.v, c.ks, c.vs, c.table, q, cu_q, q_pos0, seq_lens, out,
                c_scale, c.hkv, group, c.bs, c.mbps, n_qt, total_q, c.num_blocks};
  const int64_t n_wg = (int64_t)batch * n_qt * c.hkv * group;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  switch (c.mode) {
    case kK8V8: launch_prefill_mode<kK8V8>(c.d, a, (unsigned)n_wg, stream); break;
    case kK16V8: launch_prefill_mode<kK16V8>(c.d, a, (unsigned)n_wg, stream); break;
    default: launch_prefill_mode<kBF16>(c.d, a, (unsigned)n_wg, stream); break;
  }
  return hipGetLastError();
}

}  // namespace fp8kv
