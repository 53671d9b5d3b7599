// FA-style tiled causal prefill over the paged e4m3 / bf16 cache.
//
// Shape ("03 . 8n - FA-style tiled prefill attention", sections 2.1-3.3):
// one work-group per (128-query tile, query head); query head h reads KV head
// h / G; K/V stream through on-chip memory tile by tile (64 keys), the
// output accumulator stays in registers, the softmax is online, keys past the
// tile's last query position are never read (positions are data), the
// causal mask is kv <= q position, a fully masked tile leaves the state
// untouched and a row with no visible key writes 0.  Scores follow
// "kadirnar/kernel-agent/fp8-kv-cache" ("Math"): k_scale multiplies the
// QK product, v_scale is folded into P before its bf16 rounding.
//
// gfx950 mapping.  Four waves; wave w owns query rows 32w .. 32w+31 of the
// tile as two 16-row MFMA column blocks, so every operand read from LDS
// feeds two matrix instructions (LDS bandwidth, not the matrix cores, is
// what limits a one-block-per-wave layout).  Each 64-key tile is loaded once
// per work-group, converted e4m3 -> bf16 with the packed gfx950 convert and
// written to LDS: K row-major (rows padded by 16 bytes), V transposed (V^T,
// keys permuted so each lane's eight PV keys are contiguous), so both MFMA
// A operands are single 16-byte conflict-free LDS reads.  QK and PV use
// v_mfma_f32_16x16x32_bf16 in the transposed form of the decode kernel:
// S^T = K Q^T (lane (g4, c) holds query row c, keys 4*g4 + i of each 16-key
// block) and O^T = V^T P^T, so P goes from the QK result straight into the
// PV operand and the accumulator rows share the softmax state of their
// lane.  The softmax reference is an integer in log2 units moved lazily
// (only when a score exceeds it by more than 8), so every rescale is an
// exact power of two and rare.  Tiles whose keys every row of a wave sees
// skip the masks.
//
// LDS reuse: iteration j computes on buffer j & 1 and meanwhile stages tile
// j + 1 into buffer (j + 1) & 1, which was last read by the compute of
// iteration j - 1; the barrier that ends iteration j - 1 separates that read
// from this write, and the barrier that ends iteration j separates this write
// from the reads of iteration j + 1.  One barrier per tile is therefore
// enough.
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
  int n_qt;  // query tiles per sequence (ceil(max_q_len / 128))
  int total_q;
  int num_blocks;
};

constexpr int kPWaves = 4;
constexpr int kCB = 2;    // MFMA column blocks (16 query rows each) per wave
constexpr int kQT = 16 * kCB * kPWaves;  // queries per tile (128)
constexpr int kKT = 64;   // keys per tile
constexpr float kPLazy = 8.0f;  // log2 units the scores may exceed the reference by

template <int MODE, int D>
struct PrefillShape {
  static constexpr bool K8 = k_is_e4m3(MODE);
  static constexpr bool V8 = v_is_e4m3(MODE);
  static constexpr int LDK = D + 8;                          // LDS K row (bf16), padded
  static constexpr int LDV = kKT + 8;                        // LDS V^T row (bf16), padded
  static constexpr int KBYTES = K8 ? D : 2 * D;              // bytes of one K row in HBM
  static constexpr int KW = KBYTES / 4 / 16;                 // 16-byte K loads per thread
  static constexpr int DG = D / 16;                          // d values per V staging thread
  static constexpr int VE = V8 ? 1 : 2;                      // bytes per V element
  static constexpr int VWORDS = DG * VE / 4;                 // dwords of V per key per thread
};

// Position of key k of a 64-key tile in an LDS V^T row.  Key
// 32*kp + 16*hh + 4*g4 + i goes to 32*kp + 8*g4 + 4*hh + i: the eight keys
// whose P a lane of lane group g4 holds for PV chunk kp (keys 4*g4 + i of the
// chunk's two 16-key blocks) are then contiguous, and the MFMA A operand of
// PV is one 16-byte LDS read.
__device__ __forceinline__ int vt_pos_of_quad(int kq) {  // kq = key / 4
  return 32 * (kq >> 3) + 8 * (kq & 3) + 4 * ((kq >> 2) & 1);
}

// 4 keys x 4 e4m3 codes (one dword per key) -> 4 dwords of 4 codes (one per
// d), by byte permutes: out[j] holds code j of keys 0..3.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t r[4], uint32_t out[4]) {
  const uint32_t p01l = byte_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  const uint32_t p23l = byte_perm(r[3], r[2], 0x05010400u);
  const uint32_t p01h = byte_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  const uint32_t p23h = byte_perm(r[3], r[2], 0x07030602u);
  out[0] = byte_perm(p23l, p01l, 0x05040100u);
  out[1] = byte_perm(p23l, p01l, 0x07060302u);
  out[2] = byte_perm(p23h, p01h, 0x05040100u);
  out[3] = byte_perm(p23h, p01h, 0x07060302u);
}

template <int MODE, int D>
__global__ __launch_bounds__(64 * kPWaves, 2) void prefill_kernel(PrefillArgs a) {
  using S = PrefillShape<MODE, D>;
  constexpr int KC = D / 32;
  constexpr int NDB = D / 16;  // PV MFMAs per 32-key chunk: d in [16 db, 16 db + 16)

  __shared__ __attribute__((aligned(16))) __bf16 s_k[2][kKT][S::LDK];
  __shared__ __attribute__((aligned(16))) __bf16 s_vt[2][D][S::LDV];
  __shared__ __attribute__((aligned(16))) float s_ks[2][kKT];  // k_scale * sm_scale * log2 e
  __shared__ __attribute__((aligned(16))) float s_vs[2][kKT];
  __shared__ __attribute__((aligned(16))) float s_ok[2][kKT];  // 1: block id valid, 0: key not read
  __shared__ uint32_t s_allok[2][kPWaves];                    // per staging wave: all 16 keys valid

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

  // query rows of this lane (one per column block) and their positions
  // (-1: padding row, sees nothing)
  int qrow[kCB], qpos[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    qrow[cb] = qt * kQT + 16 * (kCB * wave + cb) + c;
    qpos[cb] = (qrow[cb] < n_q) ? pos0 + qrow[cb] : -1;
  }
  // every key t <= first_pos is visible to every row of this wave
  const int first_pos = pos0 + qt * kQT + 16 * kCB * wave;

  // Q^T as the B operand of QK, per column block
  u32x4_t qb[kCB][KC];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const uint16_t* qp = a.q + ((int64_t)(q_begin + min(qrow[cb], n_q - 1)) * hq + h) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
      qb[cb][kc] = (qrow[cb] < n_q) ? *reinterpret_cast<const u32x4_t*>(qp + d0)
                                     : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  float m_run[kCB], l_run[kCB];
  f32x4_t acc[kCB][NDB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.0f;
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[cb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int n_kt = (kv_end + kKT - 1) / kKT;
  const int64_t tab_row = (int64_t)b * a.mbps;

  // Staging of one tile by the work-group's 256 threads:
  //   K  thread -> (key tid / 4, quarter tid % 4 of the row), row-major bf16;
  //   V  thread -> (keys 4*kq .. 4*kq+3 with kq = tid % 16, d in
  //      [DG*dq, DG*dq + DG) with dq = tid / 16), written transposed (V^T):
  //      the 16 lanes of one d group fill a whole V^T row, so a write
  //      instruction of 64 lanes touches 4 rows (the 2-way minimum).
  // A 16-key sub-block lies inside one block (block_size is a multiple of
  // 16), so a key quad has one block id.
  const int skey = tid >> 2, spart = tid & 3;
  const int kq = tid & 15, dq = tid >> 4;
  u32x4_t kreg[S::KW];
  uint32_t vreg[4][S::VWORDS];
  float ksreg = 0.0f, vsreg = 0.0f;
  bool okreg = false;
  auto load_tile = [&](int t0) {
    {  // K row and its scale
      const int t = min(t0 + skey, kv_end - 1);
      const int blk = a.table[tab_row + t / a.bs];
      const bool ok = (unsigned)blk < (unsigned)a.num_blocks;  // else: key not read
      const int64_t row = ((int64_t)(ok ? blk : 0) * a.bs + t % a.bs) * a.hkv + hk;
      const uint8_t* kp = static_cast<const uint8_t*>(a.k) + row * S::KBYTES + spart * (S::KBYTES / 4);
#pragma unroll
      for (int i = 0; i < S::KW; ++i)
        kreg[i] = ok ? reinterpret_cast<const u32x4_t*>(kp)[i] : u32x4_t{0u, 0u, 0u, 0u};
      okreg = ok;
      ksreg = (S::K8 && ok) ? a.ks[row] : 1.0f;
      vsreg = (S::V8 && ok) ? a.vs[row] : 1.0f;
    }
    {  // V: four rows of a quad, DG values each
      const int t = min(t0 + 4 * kq, kv_end - 1) & ~3;
      const int blk = a.table[tab_row + t / a.bs];
      const bool ok = (unsigned)blk < (unsigned)a.num_blocks;
      const int64_t row0 = ((int64_t)(ok ? blk : 0) * a.bs + t % a.bs) * a.hkv + hk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint8_t* vp = static_cast<const uint8_t*>(a.v) + (row0 + (int64_t)r * a.hkv) * (D * S::VE) +
                            dq * (S::DG * S::VE);
        if constexpr (S::VWORDS == 4) {
          const u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(vp) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 4; ++e) vreg[r][e] = x[e];
        } else if constexpr (S::VWORDS == 2) {
          const u32x2_t x = ok ? *reinterpret_cast<const u32x2_t*>(vp) : u32x2_t{0u, 0u};
          vreg[r][0] = x[0];
          vreg[r][1] = x[1];
        } else {
          vreg[r][0] = ok ? *reinterpret_cast<const uint32_t*>(vp) : 0u;
        }
      }
    }
  };
  auto store_tile = [&](int buf, int t0) {
    // K: bf16 elements [spart * D/4, (spart+1) * D/4) of row skey
    __bf16* kd = &s_k[buf][skey][spart * (D / 4)];
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
    if (spart == 0) {
      s_ks[buf][skey] = ksreg * a.c_scale;
      s_vs[buf][skey] = vsreg;
      s_ok[buf][skey] = okreg ? 1.0f : 0.0f;
    }
    {  // the 16 keys of this wave all valid (and inside kv_end)?
      const bool good = okreg && (t0 + skey < kv_end);
      const uint64_t m = __builtin_amdgcn_ballot_w64(good);
      if (lane == 0) s_allok[buf][wave] = (m == ~0ull) ? 1u : 0u;
    }
    // V^T: for each of this thread's DG d values, its 4 keys' values as
    // 4 bf16 at the quad's position in the row
    const int pos = vt_pos_of_quad(kq);
#pragma unroll
    for (int w = 0; w < S::VWORDS; ++w) {
      if constexpr (S::V8) {
        uint32_t rr[4] = {vreg[0][w], vreg[1][w], vreg[2][w], vreg[3][w]};
        uint32_t cols[4];
        transpose4x4_bytes(rr, cols);  // cols[j]: code of d = DG*dq + 4w + j, keys 0..3
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2_t bf = {e4m3x2_to_bf16x2<false>(cols[j]), e4m3x2_to_bf16x2<true>(cols[j])};
          *reinterpret_cast<u32x2_t*>(&s_vt[buf][S::DG * dq + 4 * w + j][pos]) = bf;
        }
      } else {
        // dword w holds d = DG*dq + 2w (low half) and + 2w + 1 (high half)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t sel = hf ? 0x07060302u : 0x05040100u;
          const u32x2_t bf = {byte_perm(vreg[1][w], vreg[0][w], sel),
                              byte_perm(vreg[3][w], vreg[2][w], sel)};
          *reinterpret_cast<u32x2_t*>(&s_vt[buf][S::DG * dq + 2 * w + hf][pos]) = bf;
        }
      }
    }
  };

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0, 0);
    load_tile(kKT);
  }
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const int t0 = j * kKT;
    // Stage tile j + 1 into the other buffer (its loads were issued an
    // iteration ago) and issue tile j + 2's loads while tile j is computed.
    // Both are unconditional -- past the last tile they are clamped reloads
    // into a buffer nobody reads -- so they stay in the compute's basic block
    // and the scheduler can interleave them with the matrix instructions.
    store_tile(buf ^ 1, t0 + kKT);
    load_tile(t0 + 2 * kKT);

    // every key of the tile visible to every row of this wave, all inside
    // the sequence and in valid blocks: no mask needed (wave-uniform)
    const bool fast = (t0 + kKT - 1 <= first_pos) && (t0 + kKT <= kv_end) &&
                      (s_allok[buf][0] & s_allok[buf][1] & s_allok[buf][2] & s_allok[buf][3]);

    // --- S^T = K Q^T for 4 blocks of 16 keys and the wave's column blocks:
    //     each K operand read from LDS feeds kCB matrix instructions
    f32x4_t sacc[kCB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) sacc[cb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const __bf16* krow = &s_k[buf][16 * kb + c][0];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(krow + d0);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          sacc[cb][kb] = mfma_16x16x32_bf16(ka, qb[cb][kc], sacc[cb][kb]);
      }
    }

    f32x4_t ksv[4], vsv[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ksv[kb] = f32x4_t{a.c_scale, a.c_scale, a.c_scale, a.c_scale};
      if (S::K8) ksv[kb] = *reinterpret_cast<const f32x4_t*>(&s_ks[buf][16 * kb + 4 * g4]);
      vsv[kb] = f32x4_t{1.f, 1.f, 1.f, 1.f};
      if (S::V8) vsv[kb] = *reinterpret_cast<const f32x4_t*>(&s_vs[buf][16 * kb + 4 * g4]);
    }

    u32x4_t pb[kCB][2];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      // --- scores in log2 units: (q . K) * k_scale * sm_scale * log2 e;
      //     causal, length and block masks only where some key is hidden
      float sc[4][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = sacc[cb][kb][i] * ksv[kb][i];
        if (!fast) {
          const f32x4_t okv = *reinterpret_cast<const f32x4_t*>(&s_ok[buf][16 * kb + 4 * g4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * kb + 4 * g4 + i;
            sc[kb][i] = (t <= qpos[cb] && t < kv_end && okv[i] != 0.0f) ? sc[kb][i] : -INFINITY;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[kb][i]);
      }
      tmax = max_over_groups(tmax);

      // --- online softmax with a lazily moved integer reference; a fully
      //     masked tile (tmax = -inf) keeps the state
      const float t_ref = ceilf(tmax);
      if (m_run[cb] == -INFINITY) {
        m_run[cb] = t_ref;  // l and acc are still zero: nothing to rescale
      } else if (t_ref > m_run[cb] + kPLazy) {
        const float alpha = ldexpf(1.0f, (int)(m_run[cb] - t_ref));
        l_run[cb] *= alpha;
#pragma unroll
        for (int jj = 0; jj < NDB; ++jj) acc[cb][jj] *= alpha;
        m_run[cb] = t_ref;
      }
      const float m_ref = (m_run[cb] == -INFINITY) ? 0.0f : m_run[cb];

#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        float pv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int kb = 2 * kp + (jj >> 2), i = jj & 3;
          const float p = __builtin_amdgcn_exp2f(sc[kb][i] - m_ref);
          l_run[cb] += p;
          pv[jj] = p * vsv[kb][i];
        }
        pb[cb][kp] = u32x4_t{f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3]),
                             f32x2_to_bf16x2(pv[4], pv[5]), f32x2_to_bf16x2(pv[6], pv[7])};
      }
    }

    // --- O^T += V^T P^T: MFMA db covers d in [16 db, 16 db + 16); lane
    //     (g4, r) reads row d = 16 db + r of V^T at its eight keys, once for
    //     all column blocks
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4_t av =
            *reinterpret_cast<const u32x4_t*>(&s_vt[buf][16 * db + c][32 * kp + 8 * g4]);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          acc[cb][db] = mfma_16x16x32_bf16(av, pb[cb][kp], acc[cb][db]);
      }
    }
    __syncthreads();
  }

  // --- normalise and write: lane (g4, c) holds d = 16 db + 4 g4 + i of row c
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float l = l_run[cb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qrow[cb] < n_q) {
      float* orow = a.out + ((int64_t)(q_begin + qrow[cb]) * hq + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (l > 0.0f) ? acc[cb][db][i] / l : 0.0f;
        *reinterpret_cast<f32x4_t*>(orow + 16 * db + 4 * g4) = o;
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
    case kK8V16: launch_prefill_mode<kK8V16>(c.d, a, (unsigned)n_wg, stream); break;
    case kBF16: launch_prefill_mode<kBF16>(c.d, a, (unsigned)n_wg, stream); break;
    default: break;  // block-scaled K: rejected by the caller
  }
  return hipGetLastError();
}

}  // namespace fp8kv
