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
// gfx950 mapping.  Eight waves in two key groups of four.  Group p computes
// the key tiles p, p + 2, p + 4, ... of the work-group's query tile, and
// within a group wave r owns query rows 32r .. 32r+31 as two 16-row MFMA
// column blocks, so every operand read from LDS feeds two matrix
// instructions.  The two groups run the same online softmax on alternate
// tiles and meet once at the end, where group 1's state (integer reference,
// row sum, accumulator) is merged into group 0's with exact power-of-two
// weights.  So the longest work-group of a causal launch (the last query
// tile, which sees every key) walks half as many tiles in sequence, and each
// SIMD holds two waves whose softmax and matrix work interleave.
//
// Each group stages its own tiles: a 64-key tile is loaded once per group,
// converted e4m3 -> bf16 with the packed gfx950 convert and written to LDS:
// K row-major (rows padded by 16 bytes), V transposed (V^T, keys permuted so
// each lane's eight PV keys are contiguous), so both MFMA A operands are
// single 16-byte conflict-free LDS reads.  QK and PV use
// v_mfma_f32_16x16x32_bf16 in the transposed form of the decode kernel:
// S^T = K Q^T (lane (g4, c) holds query row c, keys 4*g4 + i of each 16-key
// block) and O^T = V^T P^T, so P goes from the QK result straight into the
// PV operand and the accumulator rows share the softmax state of their
// lane.  The softmax reference is an integer in log2 units moved lazily
// (only when a score exceeds it by more than 8), so every rescale is an
// exact power of two and rare.  Tiles whose keys every row of a wave sees
// skip the masks.
//
// Memory pipeline, per group: the block ids of tile n + 3 are fetched while
// tile n + 2's codes are loaded, tile n + 1 is staged to LDS and tile n is
// computed.  Every load of a tile that exists is issued, for every lane,
// from an address inside the cache (a key that does not exist reads row 0
// and is neutralised when staged), so the only wait per tile is for loads
// issued a whole tile earlier; past the group's last tile nothing is
// loaded.  Each lane follows one 16-key sub-block through the sequence with
// a (block index, offset) cursor: no division per tile.
//
// LDS reuse: iteration j computes on buffer j & 1 and meanwhile stages tile
// j + 1 into buffer (j + 1) & 1, which was last read by the compute of
// iteration j - 1; the barrier that ends iteration j - 1 separates that read
// from this write, and the barrier that ends iteration j separates this write
// from the reads of iteration j + 1.  One barrier per tile is therefore
// enough.  The final merge reuses the tile buffers after the last barrier.
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
  int layout;  // kTokenMajor / kHeadMajor (cache_row)
  FastDiv div_hq;     // by the query heads hkv * group
  FastDiv div_nqt;    // by n_qt
  FastDiv div_group;  // by group
  FastDiv div_bs;     // by bs
};

constexpr int kPGroups = 2;                   // key groups (alternate tiles)
constexpr int kPRowWaves = 4;                 // waves per key group
constexpr int kPWaves = kPGroups * kPRowWaves;
constexpr int kCB = 2;    // MFMA column blocks (16 query rows each) per wave
constexpr int kQT = 16 * kCB * kPRowWaves;  // queries per tile (128)
constexpr int kKT = 64;   // keys per tile
constexpr float kPLazy = 8.0f;  // log2 units the scores may exceed the reference by
constexpr float kPLazyP = 256.0f;  // 2^kPLazy: the largest p = 2^(s - M) the reference allows

template <int MODE, int D>
struct PrefillShape {
  static constexpr bool K8 = k_is_e4m3(MODE);
  static constexpr bool V8 = v_is_e4m3(MODE);
  // LDS rows: K unpadded, its 16-byte chunks permuted (k_chunk), V^T padded
  // to kKT + 16 bf16 (160 bytes at kKT = 64).  Both make the QK and PV
  // operand reads and the staging writes free of LDS bank conflicts.
  static constexpr int LDK = D;
  static constexpr int KSWZ = (D / 8 - 1) < 15 ? (D / 8 - 1) : 15;
  static constexpr int LDV = kKT + 16;
  static constexpr int KBYTES = K8 ? D : 2 * D;              // bytes of one K row in HBM
  static constexpr int KW = KBYTES / 4 / 16;                 // 16-byte K loads per thread
  static constexpr int DG = D / 16;                          // d values per V staging thread
  static constexpr int VE = V8 ? 1 : 2;                      // bytes per V element
  static constexpr int VWORDS = DG * VE / 4;                 // dwords of V per key per thread
  static constexpr int NDB = D / 16;                         // PV column blocks of 16 d
  static constexpr int MF = 2 * kCB + 4 * kCB * NDB;         // merged floats per lane
};

// Place of 16-byte chunk j of K row r inside the row.  gfx950's LDS serves a
// 16-byte access per lane in lane groups: a K operand read (16 lanes at 16
// rows, one column) is conflict-free when those rows put the column in 16
// different chunks, which j ^ (r % 16) does (a row padding of 16 bytes
// leaves 4 extra cycles per read); a staging write (8 lanes: two rows, four
// chunks 4 apart in each) when the eight land in different 16-byte slots of
// 128 bytes, which the extra flip of bit 1 by bit 3 of j adds.  The map is a
// permutation of each row's chunks.
template <int KSWZ>
__device__ __forceinline__ int k_chunk(int r, int j) {
  return j ^ (r & KSWZ) ^ (((j >> 3) & 1) << 1);
}

// One staged 64-key tile.
template <int MODE, int D>
struct __attribute__((aligned(16))) PrefillTile {
  using S = PrefillShape<MODE, D>;
  __bf16 k[kKT][S::LDK];
  __bf16 vt[D][S::LDV];
  float ks[kKT];   // k_scale * sm_scale * log2 e
  float vs[kKT];
  float ok[kKT];   // 1: key exists (inside the sequence, valid block), 0: masked
  uint32_t allok[kPRowWaves];  // per staging wave: all 16 keys exist
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

// How a key's cache row is found:
//  - kPTable: through the block table in memory;
//  - kPComputed: no table (contiguous cache), block ids computed, so that no
//    wait for a table load joins the paths of the loads;
//  - kPLinear: no table and token-major rows, so key t of the sequence and
//    KV head is row r0 + t * hkv; every K, V and scale load is then a 32-bit
//    offset into a buffer resource over the sequence's rows up to the last
//    key the query tile attends, and a key past it reads zeros (no row
//    arithmetic in 64 bits, no selects for missing keys).  The host picks it
//    when the whole cache's rows fit 31-bit byte offsets.
enum { kPTable = 0, kPComputed = 1, kPLinear = 2 };

template <int MODE, int D, int ADDR>
__global__ __launch_bounds__(64 * kPWaves, 1) void prefill_kernel(PrefillArgs a) {
  constexpr bool TB = ADDR == kPTable;
  constexpr bool LIN = ADDR == kPLinear;
  using S = PrefillShape<MODE, D>;
  using Tile = PrefillTile<MODE, D>;
  constexpr int KC = D / 32;
  constexpr int NDB = S::NDB;  // PV MFMAs per 32-key chunk: d in [16 db, 16 db + 16)

  __shared__ Tile s_t[kPGroups][2];

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int grp = wave / kPRowWaves;   // key group: tiles grp, grp + 2, ...
  const int rw = wave % kPRowWaves;    // row group inside the query tile
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int c = lane & 15;

  // Largest query tiles first: causal work grows with the tile index.
  const int hq = a.div_hq.d;
  const int rest = a.div_hq.div(blockIdx.x);
  const int h = blockIdx.x - rest * hq;
  const int b = a.div_nqt.div(rest);
  const int qt = a.n_qt - 1 - (rest - b * a.n_qt);
  const int hk = a.div_group.div(h);

  // Device data is clamped so that no access leaves the buffers: query rows
  // stay inside [0, total_q), lengths inside the block-table capacity.  The
  // sequence's four values are read together, in one round trip.
  const int cu0 = a.cu_q[b], cu1 = a.cu_q[b + 1];
  const int pos0 = a.q_pos0[b];
  const int seq_len_raw = a.seq_lens[b];
  // (used here, so that the compiler loads them with the query offsets
  // rather than after the test below, a round trip later; likewise the
  // cache's base addresses, read from the kernel arguments with the first)
  asm volatile("" ::"s"(cu0), "s"(cu1), "s"(pos0), "s"(seq_len_raw), "s"(a.k), "s"(a.v),
               "s"(a.ks), "s"(a.vs));
  const int q_begin = min(max(cu0, 0), a.total_q);
  const int q_end = min(max(cu1, q_begin), a.total_q);
  const int n_q = min(q_end - q_begin, a.n_qt * kQT);
  if (qt * kQT >= n_q) return;
  const int seq_len = min(max(seq_len_raw, 0), a.mbps * a.bs);
  const int last_q = min(qt * kQT + kQT, n_q) - 1;
  const int kv_end = max(0, min(seq_len, pos0 + last_q + 1));  // keys past the last query: skipped

  // query rows of this lane (one per column block) and their positions
  // (-1: padding row, sees nothing)
  int qrow[kCB], qpos[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    qrow[cb] = qt * kQT + 16 * (kCB * rw + cb) + c;
    qpos[cb] = (qrow[cb] < n_q) ? pos0 + qrow[cb] : -1;
  }
  // every key t <= first_pos is visible to every row of this wave
  const int first_pos = pos0 + qt * kQT + 16 * kCB * rw;

  // Q^T as the B operand of QK, per column block
  u32x4_t qb[kCB][KC];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const uint16_t* qp = a.q + ((int64_t)(q_begin + min(qrow[cb], n_q - 1)) * hq + h) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      // loaded for every lane (a padding row reads the last row) and zeroed
      // after: a load under a lane condition would join two paths, and the
      // wait where they meet would wait for every load before it
      const int d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1);
      qb[cb][kc] = *reinterpret_cast<const u32x4_t*>(qp + d0);
    }
  }
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      if (qrow[cb] >= n_q) qb[cb][kc] = u32x4_t{0u, 0u, 0u, 0u};

  float m_run[kCB], l_run[kCB];
  f32x4_t acc[kCB][NDB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.0f;
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[cb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int n_kt = (kv_end + kKT - 1) / kKT;   // key tiles of the query tile
  const int n_it = (n_kt + kPGroups - 1) / kPGroups;  // tiles of key group 0
  const int64_t tab_row = (int64_t)b * a.mbps;
  // a key that does not exist reads head hk's slot 0 of block 0 (masked)
  const int64_t row_invalid = cache_row(a.layout, 0, 0, hk, a.bs, a.hkv);
  const int ss = slot_stride(a.layout, a.hkv);

  // Staging of one tile by the group's 256 threads (gt = thread in group):
  //   K  thread -> (key gt / 4, quarter gt % 4 of the row), row-major bf16;
  //      its key lies in 16-key sub-block rw of the tile;
  //   V  thread -> (keys 4*kq .. 4*kq+3 with kq = gt % 16, d in
  //      [DG*dq, DG*dq + DG) with dq = gt / 16), written transposed (V^T):
  //      the 16 lanes of one d group fill a whole V^T row, so a write
  //      instruction of 64 lanes touches 4 rows (the 2-way minimum).
  //      Its keys lie in sub-block sbv = kq / 4.
  // A 16-key sub-block lies inside one block (block_size is a multiple of
  // 16), so it has one block id; lane 4*rw follows sub-block rw, which the
  // wave's K threads read from it.
  const int gt = tid % (64 * kPRowWaves);
  const int spart = gt & 3;
  const int kq = gt & 15, dq = gt >> 4;
  const int sbv = kq >> 2;
  const int kin = lane >> 2;  // K thread's key inside sub-block rw

  // Cursor over this lane's sub-block sbv of the group's tiles: first key,
  // block index in the table row and 16-key offset inside the block.  A
  // group advances by kPGroups tiles = 8 sub-blocks per tile.
  const int nsb = a.bs >> 4;
  const int adv = kPGroups * kKT / 16;
  const int adv_q = adv / nsb, adv_r = adv % nsb;
  int cur_t = grp * kKT + 16 * sbv;
  int cur_b = a.div_bs.div(cur_t);
  int cur_r = (cur_t - cur_b * a.bs) >> 4;

  // kPLinear: buffer resources over the sequence's rows of KV head hk, from
  // key 0 up to kv_end (and never past the end of the arrays); byte steps
  // of one key
  const int lin_step_k = a.hkv * S::KBYTES, lin_step_v = a.hkv * D * S::VE, lin_step_s = a.hkv * 4;
  const int64_t lin_r0 = (int64_t)b * a.mbps * a.bs * a.hkv + hk;  // row of key 0
  auto lin_rsrc = [&](const void* base, int64_t elem_bytes, int step) {
    const int64_t rows = (int64_t)a.num_blocks * a.bs * a.hkv;       // rows in the cache
    const int64_t want = (int64_t)kv_end * step;
    const int64_t have = (rows - lin_r0) * elem_bytes;
    const int64_t n = want < have ? want : have;
    return buffer_rsrc(static_cast<const uint8_t*>(base) + lin_r0 * elem_bytes,
                       n > 0 ? (uint32_t)n : 0u);
  };
  const __amdgpu_buffer_rsrc_t lin_k = lin_rsrc(a.k, S::KBYTES, lin_step_k);
  const __amdgpu_buffer_rsrc_t lin_v = lin_rsrc(a.v, D * S::VE, lin_step_v);
  const __amdgpu_buffer_rsrc_t lin_ks = lin_rsrc(a.ks, 4, lin_step_s);
  const __amdgpu_buffer_rsrc_t lin_vs = lin_rsrc(a.vs, 4, lin_step_s);

  // A tile's block id (this lane's sub-block), its 16-key offset inside the
  // block and its first key, fetched ahead of the tile's loads.
  struct Pend {
    int id, r, t;
  };
  auto fetch_id = [&]() {
    const int64_t ti = tab_row + (cur_t < kv_end ? cur_b : 0);
    Pend pd;
    pd.id = TB ? a.table[ti] : (int)ti;  // no table: contiguous
    pd.r = cur_r;
    pd.t = cur_t;
    cur_t += kPGroups * kKT;
    cur_b += adv_q;
    cur_r += adv_r;
    if (cur_r >= nsb) {
      cur_r -= nsb;
      ++cur_b;
    }
    return pd;
  };

  // One tile's codes and scales in flight to this thread's registers.
  struct StageRegs {
    u32x4_t kreg[S::KW];
    uint32_t vreg[4][S::VWORDS];
    float ksreg = 1.0f, vsreg = 1.0f;
    bool okk = false;
    uint32_t okv = 0;  // bit r: key 4*kq + r of the tile exists
  };
  auto load_tile = [&](StageRegs& R, const Pend& pd) {
    if constexpr (LIN) {
      // K row of key t_k (sub-block rw, from lane 4*rw), its scales, and this
      // lane's four V rows (keys p_t + 4*(kq % 4) + r, r from the scalar
      // offset); keys at or past kv_end read zeros
      const int t_k = __builtin_amdgcn_readlane(pd.t, 4 * rw) + kin;
      R.okk = t_k < kv_end;
      const int ok_off = t_k * lin_step_k + spart * (S::KBYTES / 4);
#pragma unroll
      for (int i = 0; i < S::KW; ++i)
        R.kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(lin_k, ok_off + 16 * i, 0, 0);
      if (S::K8)
        R.ksreg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lin_ks, t_k * lin_step_s, 0, 0));
      if (S::V8)
        R.vsreg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lin_vs, t_k * lin_step_s, 0, 0));
      R.okv = 0xfu;  // a missing key's V is already zero
      const int ov_off = (pd.t + 4 * (kq & 3)) * lin_step_v + dq * (S::DG * S::VE);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int soff = r * lin_step_v;
        if constexpr (S::VWORDS == 4) {
          const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(lin_v, ov_off, soff, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) R.vreg[r][e] = x[e];
        } else if constexpr (S::VWORDS == 2) {
          const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(lin_v, ov_off, soff, 0);
          R.vreg[r][0] = x[0];
          R.vreg[r][1] = x[1];
        } else {
          R.vreg[r][0] = __builtin_amdgcn_raw_buffer_load_b32(lin_v, ov_off, soff, 0);
        }
      }
      return;
    }
    const int p_id = pd.id, p_r = pd.r, p_t = pd.t;
    const bool sb_ok = (p_t < kv_end) && ((unsigned)p_id < (unsigned)a.num_blocks);
    // first row of this lane's V sub-block; its later slots follow every ss rows
    const int64_t row_v = sb_ok ? cache_row(a.layout, p_id, 16 * p_r, hk, a.bs, a.hkv)
                                : row_invalid;
    {  // K row (sub-block rw, from lane 4*rw) and its scales
      const int id_k = __builtin_amdgcn_readlane(p_id, 4 * rw);
      const int r_k = __builtin_amdgcn_readlane(p_r, 4 * rw);
      const int t_k = __builtin_amdgcn_readlane(p_t, 4 * rw) + kin;
      R.okk = (t_k < kv_end) && ((unsigned)id_k < (unsigned)a.num_blocks);
      const int64_t row = R.okk ? cache_row(a.layout, id_k, 16 * r_k + kin, hk, a.bs, a.hkv)
                              : row_invalid;
      const uint8_t* kp = static_cast<const uint8_t*>(a.k) + row * S::KBYTES + spart * (S::KBYTES / 4);
#pragma unroll
      for (int i = 0; i < S::KW; ++i) R.kreg[i] = reinterpret_cast<const u32x4_t*>(kp)[i];
      if (S::K8) R.ksreg = a.ks[row];
      if (S::V8) R.vsreg = a.vs[row];
    }
    R.okv = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // V: four rows of a quad, DG values each
      const int kk = 4 * (kq & 3) + r;
      const bool ok = sb_ok && (p_t + kk < kv_end);
      R.okv |= ok ? (1u << r) : 0u;
      const int64_t row = ok ? row_v + (int64_t)kk * ss : row_invalid;
      const uint8_t* vp = static_cast<const uint8_t*>(a.v) + row * (D * S::VE) + dq * (S::DG * S::VE);
      if constexpr (S::VWORDS == 4) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp);
#pragma unroll
        for (int e = 0; e < 4; ++e) R.vreg[r][e] = x[e];
      } else if constexpr (S::VWORDS == 2) {
        const u32x2_t x = *reinterpret_cast<const u32x2_t*>(vp);
        R.vreg[r][0] = x[0];
        R.vreg[r][1] = x[1];
      } else {
        R.vreg[r][0] = *reinterpret_cast<const uint32_t*>(vp);
      }
    }
  };
  auto store_tile = [&](Tile& T, const StageRegs& R) {
    // K: 16-byte chunks [spart * D/32, (spart+1) * D/32) of row gt / 4, each
    // at its k_chunk place.  A key that does not exist keeps whatever row 0
    // holds: its score is masked.
    u32x4_t* kd = reinterpret_cast<u32x4_t*>(&T.k[gt >> 2][0]);
    constexpr int QCH = D / 32;  // chunks per quarter row
    if (S::K8) {
#pragma unroll
      for (int i = 0; i < S::KW; ++i) {
        const u32x4_t w = R.kreg[i];
        u32x4_t lo = {e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
                      e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
        u32x4_t hi = {e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
                      e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
        kd[k_chunk<S::KSWZ>(gt >> 2, QCH * spart + 2 * i)] = lo;
        kd[k_chunk<S::KSWZ>(gt >> 2, QCH * spart + 2 * i + 1)] = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::KW; ++i) kd[k_chunk<S::KSWZ>(gt >> 2, QCH * spart + i)] = R.kreg[i];
    }
    if (spart == 0) {
      T.ks[gt >> 2] = R.okk ? R.ksreg * a.c_scale : 0.0f;
      T.vs[gt >> 2] = R.okk ? R.vsreg : 0.0f;
      T.ok[gt >> 2] = R.okk ? 1.0f : 0.0f;
    }
    {  // the 16 keys of this wave all exist?
      const uint64_t m = __builtin_amdgcn_ballot_w64(R.okk);
      if (lane == 0) T.allok[rw] = (m == ~0ull) ? 1u : 0u;
    }
    // V^T: for each of this thread's DG d values, its 4 keys' values as
    // 4 bf16 at the quad's position in the row; a key that does not exist
    // contributes zeros (its P is 0, and row 0 may hold any bytes)
    const int pos = vt_pos_of_quad(kq);
#pragma unroll
    for (int w = 0; w < S::VWORDS; ++w) {
      uint32_t rr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rr[r] = ((R.okv >> r) & 1u) ? R.vreg[r][w] : 0u;
      if constexpr (S::V8) {
        uint32_t cols[4];
        transpose4x4_bytes(rr, cols);  // cols[j]: code of d = DG*dq + 4w + j, keys 0..3
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2_t bf = {e4m3x2_to_bf16x2<false>(cols[j]), e4m3x2_to_bf16x2<true>(cols[j])};
          *reinterpret_cast<u32x2_t*>(&T.vt[S::DG * dq + 4 * w + j][pos]) = bf;
        }
      } else {
        // dword w holds d = DG*dq + 2w (low half) and + 2w + 1 (high half)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t sel = hf ? 0x07060302u : 0x05040100u;
          const u32x2_t bf = {byte_perm(rr[1], rr[0], sel), byte_perm(rr[3], rr[2], sel)};
          *reinterpret_cast<u32x2_t*>(&T.vt[S::DG * dq + 2 * w + hf][pos]) = bf;
        }
      }
    }
  };

  // Prologue: tile 0 staged, tile 1's codes and tile 2's block ids in flight
  // (tile 1's loads issued before tile 0 is waited for, into registers of
  // their own, so the two round trips overlap).
  StageRegs R;
  Pend pn{0, 0, 0};  // block id of the next tile to load
  if (n_it > 0) {
    StageRegs R0;
    const Pend p0 = fetch_id();
    const Pend p1 = fetch_id();
    pn = fetch_id();
    load_tile(R0, p0);
    load_tile(R, p1);
    store_tile(s_t[grp][0], R0);
  }
  __syncthreads();
  for (int j = 0; j < n_it; ++j) {
    const int buf = j & 1;
    const int t0 = (kPGroups * j + grp) * kKT;
    // Stage the group's next tile (its loads were issued an iteration ago),
    // issue the codes of the one after and the block ids of the third, so
    // the only wait is for loads a tile old.  Past the group's last tile
    // nothing is loaded (the registers keep stale bytes, staged into a buffer
    // that is never computed), so no load is left in flight when the loop
    // ends.
    const bool more = (kPGroups * (j + 2) + grp) * kKT < kv_end;  // wave-uniform
    auto stage = [&]() __attribute__((always_inline)) {
      store_tile(s_t[grp][buf ^ 1], R);
      if (more) {
        load_tile(R, pn);
        pn = fetch_id();
      }
    };
    auto compute_tile = [&]() __attribute__((always_inline)) {
      if (t0 < kv_end) {
        const Tile& T = s_t[grp][buf];
        // every key of the tile visible to every row of this wave, all inside
        // the sequence and in valid blocks: no mask needed (wave-uniform)
        const bool fast = (t0 + kKT - 1 <= first_pos) && (t0 + kKT <= kv_end) &&
                          (T.allok[0] & T.allok[1] & T.allok[2] & T.allok[3]);

        // The tile is computed in two 32-key halves kp, each QK -> softmax ->
        // PV, so only one half's scores and scales are live at a time; the
        // matrix work of one half can overlap the softmax of the other.
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          // --- S^T = K Q^T for the half's two blocks of 16 keys and the
          //     wave's column blocks: each K operand read from LDS feeds kCB
          //     matrix instructions
          f32x4_t sacc[kCB][2];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) sacc[cb][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const u32x4_t* krow = reinterpret_cast<const u32x4_t*>(&T.k[16 * (2 * kp + hb) + c][0]);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              // d in [d0, d0 + 8), d0 = 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1):
              // chunk d0 / 8 of row 16 * (2 * kp + hb) + c
              const int ch = 8 * (kc >> 1) + 2 * g4 + (kc & 1);
              const u32x4_t ka = krow[k_chunk<S::KSWZ>(c, ch)];
#pragma unroll
              for (int cb = 0; cb < kCB; ++cb)
                sacc[cb][hb] = mfma_16x16x32_bf16(ka, qb[cb][kc], sacc[cb][hb]);
            }
          }

          f32x4_t ksv[2], vsv[2];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            ksv[hb] = *reinterpret_cast<const f32x4_t*>(&T.ks[16 * (2 * kp + hb) + 4 * g4]);
            vsv[hb] = *reinterpret_cast<const f32x4_t*>(&T.vs[16 * (2 * kp + hb) + 4 * g4]);
          }
          // visibility of the lane's eight keys to its rows: causal, length and
          // block masks, only where some key is hidden
          bool vis[kCB][8];
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) vis[cb][jj] = true;
          if (!fast) {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              const int kb = 2 * kp + hb;
              const f32x4_t okf = *reinterpret_cast<const f32x4_t*>(&T.ok[16 * kb + 4 * g4]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * kb + 4 * g4 + i;
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb)
                  vis[cb][4 * hb + i] = t <= qpos[cb] && okf[i] != 0.0f;
              }
            }
          }

          // --- online softmax against the row's integer reference M (log2
          //     units of the score): p = 2^(s - M) with s = (q . K) * k_scale *
          //     sm_scale * log2 e, one fma into the exp2.  M moves (an exact
          //     power-of-two rescale) only when a score exceeds it by more than
          //     kPLazy; such a score makes its p, and so the lane's sum of p,
          //     exceed 2^kPLazy.  Only then, or while the row has no reference,
          //     is the row maximum taken and the step redone with the exact
          //     rule (wave-uniform branch, rare).  Fully masked keys keep the
          //     state.
          float p[kCB][8], psum[kCB];
          bool redo = false;
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) {
            const float off = (m_run[cb] == -INFINITY) ? 0.0f : -m_run[cb];
            psum[cb] = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int hb = jj >> 2, i = jj & 3;
              const float arg = vis[cb][jj] ? __builtin_fmaf(sacc[cb][hb][i], ksv[hb][i], off)
                                            : -INFINITY;
              p[cb][jj] = __builtin_amdgcn_exp2f(arg);
              psum[cb] += p[cb][jj];
            }
            redo = redo || (m_run[cb] == -INFINITY) || !(psum[cb] <= kPLazyP);
          }
          if (__builtin_amdgcn_ballot_w64(redo) != 0) {
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
              float tmax = -INFINITY;
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const int hb = jj >> 2, i = jj & 3;
                tmax = fmaxf(tmax, vis[cb][jj] ? sacc[cb][hb][i] * ksv[hb][i] : -INFINITY);
              }
              const float t_ref = ceilf(max_over_groups(tmax));
              if (m_run[cb] == -INFINITY) {
                m_run[cb] = t_ref;  // l and acc are still zero: nothing to rescale
              } else if (t_ref > m_run[cb] + kPLazy) {
                const float alpha = ldexpf(1.0f, (int)(m_run[cb] - t_ref));
                l_run[cb] *= alpha;
#pragma unroll
                for (int jj = 0; jj < NDB; ++jj) acc[cb][jj] *= alpha;
                m_run[cb] = t_ref;
              }
              // exp2(-inf - M) is 0 for finite M; M is -inf only while every
              // key so far is masked, and then the reference 0 avoids -inf - -inf
              const float off = (m_run[cb] == -INFINITY) ? 0.0f : -m_run[cb];
              psum[cb] = 0.0f;
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const int hb = jj >> 2, i = jj & 3;
                const float arg = vis[cb][jj] ? __builtin_fmaf(sacc[cb][hb][i], ksv[hb][i], off)
                                              : -INFINITY;
                p[cb][jj] = __builtin_amdgcn_exp2f(arg);
                psum[cb] += p[cb][jj];
              }
            }
          }
          u32x4_t pb[kCB];
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) {
            l_run[cb] += psum[cb];
            float pv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) pv[jj] = p[cb][jj] * vsv[jj >> 2][jj & 3];
            pb[cb] = u32x4_t{f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3]),
                             f32x2_to_bf16x2(pv[4], pv[5]), f32x2_to_bf16x2(pv[6], pv[7])};
          }

          // --- O^T += V^T P^T: MFMA db covers d in [16 db, 16 db + 16); lane
          //     (g4, r) reads row d = 16 db + r of V^T at its eight keys of the
          //     half, once for all column blocks
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&T.vt[16 * db + c][32 * kp + 8 * g4]);
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) acc[cb][db] = mfma_16x16x32_bf16(av, pb[cb], acc[cb][db]);
          }
        }
      }
    };
    // The two groups take the iteration's halves in opposite order (group 0
    // stages then computes, group 1 computes then stages), so the two waves
    // that share a SIMD, one of each group, run vector work and matrix work
    // side by side instead of in step.  Both orders are safe: group 1's
    // compute reads buffer buf, staged an iteration ago, and its staging
    // writes buffer buf ^ 1, last read before the previous barrier.
    if (grp == 0) stage();
    compute_tile();
    if (grp != 0) stage();
    __syncthreads();
  }

  // --- merge key group 1 into group 0 through LDS (the tile buffers are free
  //     after the loop's last barrier): exact power-of-two weights 2^(M - M*),
  //     a group that saw no key (M = -inf) weighs 0
  //     Each lane's state is contiguous ([rw][lane][MF]: M and l of both
  //     column blocks, then the accumulators), written and read with 16-byte
  //     LDS operations; the lane stride of MF floats keeps each group of 16
  //     lanes on distinct banks.
  static_assert(kCB == 2 && S::MF == 4 + 4 * kCB * NDB, "merge layout");
  static_assert(sizeof(float) * kPRowWaves * S::MF * 64 <= sizeof(s_t), "merge area");
  f32x4_t* mine = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(&s_t[0][0]) +
                                             (rw * 64 + lane) * S::MF);
  if (grp == 1) {
    mine[0] = f32x4_t{m_run[0], l_run[0], m_run[1], l_run[1]};
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) mine[1 + NDB * cb + db] = acc[cb][db];
  }
  __syncthreads();
  if (grp != 0) return;
  const f32x4_t ml1 = mine[0];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const float m1 = ml1[2 * cb];
    const float l1 = ml1[2 * cb + 1];
    const float ms = fmaxf(m_run[cb], m1);
    const float w0 = (m_run[cb] == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(m_run[cb] - ms));
    const float w1 = (m1 == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(m1 - ms));
    l_run[cb] = l_run[cb] * w0 + l1 * w1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4_t a1 = mine[1 + NDB * cb + db];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[cb][db][i] = acc[cb][db][i] * w0 + a1[i] * w1;
    }
  }

  // --- normalise and write: lane (g4, c) holds d = 16 db + 4 g4 + i of row c
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float l = l_run[cb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qrow[cb] < n_q) {
      float* orow = a.out + ((int64_t)(q_begin + qrow[cb]) * hq + h) * D;
      const float inv_l = (l > 0.0f) ? 1.0f / l : 0.0f;  // a row that sees no key: 0
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc[cb][db][i] * inv_l;
        *reinterpret_cast<f32x4_t*>(orow + 16 * db + 4 * g4) = o;
      }
    }
  }
}

template <int MODE, int D>
static void launch_prefill_d(const PrefillArgs& a, unsigned n_wg, hipStream_t stream) {
  using S = PrefillShape<MODE, D>;
  // kPLinear: every byte offset into the K, V and scale arrays fits 31 bits,
  // also for the keys the staging may address past a sequence's capacity
  // (they read zeros): the first two tiles of each group are loaded whatever
  // the length, so keys below 4 * kKT, later tiles only when they start
  // below the length
  const int64_t rows = (int64_t)a.num_blocks * a.bs * a.hkv + 4 * kKT * a.hkv;
  const int64_t row_bytes = S::KBYTES > D * S::VE ? S::KBYTES : D * S::VE;
  const bool linear = !a.table && a.layout == kTokenMajor && rows * row_bytes < (int64_t(1) << 31);
  if (a.table)
    hipLaunchKernelGGL((prefill_kernel<MODE, D, kPTable>), dim3(n_wg), dim3(64 * kPWaves), 0,
                       stream, a);
  else if (linear)
    hipLaunchKernelGGL((prefill_kernel<MODE, D, kPLinear>), dim3(n_wg), dim3(64 * kPWaves), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<MODE, D, kPComputed>), dim3(n_wg), dim3(64 * kPWaves), 0,
                       stream, a);
}

template <int MODE>
static void launch_prefill_mode(int d, const PrefillArgs& a, unsigned n_wg, hipStream_t stream) {
  if (d == 128)
    launch_prefill_d<MODE, 128>(a, n_wg, stream);
  else
    launch_prefill_d<MODE, 64>(a, n_wg, stream);
}

hipError_t launch_prefill(const CacheView& c, const uint16_t* q, int group,
                          const int32_t* cu_q, const int32_t* q_pos0,
                          const int32_t* seq_lens, int batch, int total_q, int max_q_len,
                          float c_scale, float* out, hipStream_t stream) {
  const int n_qt = (max_q_len + kQT - 1) / kQT;
  const int64_t n_wg = (int64_t)batch * n_qt * c.hkv * group;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  if (n_wg == 0) return hipSuccess;
  PrefillArgs a{c.k, c.v, c.ks, c.vs, c.table, q, cu_q, q_pos0, seq_lens, out,
                c_scale, c.hkv, group, c.bs, c.mbps, n_qt, total_q, c.num_blocks, c.layout,
                FastDiv::of(c.hkv * group), FastDiv::of(n_qt), FastDiv::of(group),
                FastDiv::of(c.bs)};
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
