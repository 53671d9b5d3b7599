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
// Softmax reference.  M is an integer in log2 units.  Every rescale
// 2^(M_old - M_new) is then an exact power of two, and since bf16 rounding
// commutes with power-of-two scaling the rounded P does not depend on which
// integer is used, nor on how the keys are cut into tiles and splits.  The
// reference is set from the first scores seen (rounded up) and moves only
// when a later maximum exceeds it by more than kLazy: p = 2^(s - M) then stays
// below 2^kLazy, and the rescale of the accumulator, which would otherwise
// follow almost every step, becomes rare.
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
#include <type_traits>

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
  const float* k_new;  // fused append: the step's new K/V rows, fp32
  const float* v_new;  //   [batch][hkv][D]; unused by the plain decode
  const float* kbias;  // pre-bias residual cache: exact K bias [hkv][D], else null
  const uint8_t* kexp; // block-scaled K: E8M0 byte per 32-value block [..][hkv][D/32]
  float c_scale;  // sm_scale * log2(e)
  int hkv;
  int group;
  int bs;
  int mbps;
  int chunk;
  int n_splits;
  int num_blocks;
  int layout;  // kTokenMajor / kHeadMajor (cache_row)
  int ss;      // rows from one slot of a head to its next slot (slot_stride)
  uint64_t k_bytes;  // bytes of the K and V arrays (hardware bound of the tile loads)
  uint64_t v_bytes;
  FastDiv div_hkv;     // by hkv
  FastDiv div_bs;      // by bs
  FastDiv div_splits;  // by n_splits
  FastDiv div_pairs;   // by the (sequence, KV head) pairs of the grid
  float* out;          // a plan of one split: the output rows, written here (else null)
};

constexpr int kWaves = 4;     // waves per work-group; tiles are dealt round-robin
constexpr int kTile = 64;     // tokens per tile
enum { kHalf = 0, kOne = 1, kMulti = 2 };  // keys per wave: half a tile, one, several
constexpr int kMaxGroup = 16; // query heads per KV head (one MFMA column block)
constexpr float kLazy = 8.0f; // log2 units the scores may exceed the reference by
constexpr float kLazyP = 256.0f;  // 2^kLazy: the largest p = 2^(s - M) the reference allows

// Raw (still compressed) K/V of one 64-token tile in the registers of one
// lane, the scales of the lane's own token (token t0 + lane) and the
// validity needed to neutralise keys outside the sequence.
template <int MODE, int D>
struct TileRegs {
  static constexpr bool K8 = k_is_e4m3(MODE);
  static constexpr bool V8 = v_is_e4m3(MODE);
  static constexpr bool MX = k_is_mx(MODE);               // block-scaled K
  static constexpr bool KS = k_has_row_scale(MODE);       // fp32 K scale per row
  static constexpr int KP = D / 64;                      // 16-element pieces
  // d of a lane's K bytes: piece p, byte i of lane group g4 holds
  // d = KPIECE * p + KLANE * g4 + i (in the 32-value blocks of block-scaled
  // K: piece p of lane group g4 lies in block 2p + g4 / 2)
  static constexpr int KLANE = 16;
  static constexpr int KPIECE = 64;
  static constexpr int KRAW = K8 ? KP : 2 * KP;          // 16-byte K loads per sub-block
  static constexpr int DPR = D / 16;
  static constexpr int VW = V8 ? DPR / 4 : DPR / 2;      // dwords of V per token
  static constexpr int KE = K8 ? 1 : 2;                  // bytes per K element
  static constexpr int VE = V8 ? 1 : 2;                  // bytes per V element
  u32x4_t k[4][KRAW];
  uint32_t v[2][8][VW];
  uint32_t kxw;  // block-scaled K: the E8M0 bytes of token t0 + lane (like ks)
  float ks, vs;
  bool tok_ok;     // this lane's own token is before t_end in a valid block
  bool blk_ok[4];  // block id of each 16-token sub-block is a valid block
  bool full;       // all 64 tokens are before t_end and in valid blocks
};

// Per-lane byte offsets inside a 16-token sub-block; they do not depend on
// the tile, so they are computed once per kernel.
struct LaneOffsets {
  uint32_t k;        // token c, d-piece of lane group g4
  uint32_t v;        // token 4*g4, d = DPR*c
  uint32_t v_token;  // bytes from one token's row to the next (uniform)
};

// Issue the loads of the tile starting at token t0.  tab holds, in lane e,
// the block id of block t_begin / bs + e of the sequence; it is indexed with
// a wave-uniform lane, so every block id is a scalar.  A 16-token sub-block
// lies inside one block, so its first row (cache_row of the layout) is one
// scalar per sub-block (four scalar divisions per tile), its later slots
// follow every ss rows, and every load is a scalar base plus a per-lane
// offset fixed for the kernel.
//
// Every load is issued unconditionally and stays inside the cache: a
// sub-block whose block id is out of range reads block 0 instead (block_size
// >= 16 keeps the lane offsets inside it), and a token at or past t_end
// reads a slot of its own, valid block.  The values of such keys are
// neutralised where they are used (score -inf, V and v_scale 0).  A fixed
// number of loads in a fixed order lets the compiler wait for exactly the
// loads each step needs instead of for all of them.
//
// The K/V loads are buffer loads on a resource per sub-block whose extent
// ends where the cache ends.  A tile that is not live (no tile left for this
// wave) is issued all the same with an empty extent: its loads return zeros
// without a memory access, but they are counted like the others, so every
// path into a compute step has the same loads outstanding and the waits
// before it stay exact.  (Issued under a branch instead, they would leave
// the compiler two counts to reconcile where the paths join, and it keeps
// the smaller: the wait for the current tile then also waits for the whole
// next one.)  Empty loads are not free (each still passes through the
// load pipeline; measured at about 3 us per launch when every wave of the
// B16, 8192-key step issued two empty tiles), so a wave issues one only when
// it has no tile at all.
//
// PART selects what is issued: 2 the whole tile; 0 the tile's flags, its
// scales and keys 0-31; 1 keys 32-63 only (the flags and scales are left as
// they are).  A wave that streams several tiles issues the next tile's part
// 0 once it has computed the current tile's first half (whose registers it
// overwrites) and part 1 after the second half.  NK: the keys the flags
// cover (64, or 32 for a wave that attends half a tile: part 0 alone).
template <int MODE, int D, int PART = 2, int NK = 64>
__device__ __forceinline__ void load_tile(TileRegs<MODE, D>& r, const DecodeArgs& a,
                                          const LaneOffsets& lo, int t0, int t_end, int tab,
                                          int e_base, int h, int lane, bool live) {
  using T = TileRegs<MODE, D>;
  int64_t row0[4];
  bool blk_ok[4];
  bool all_ok = t0 + NK <= t_end;
  const int64_t row_invalid = cache_row(a.layout, 0, 0, h, a.bs, a.hkv);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int tb = t0 + 16 * kb;
    const int eb = a.div_bs.div(tb);
    const int blk = __builtin_amdgcn_readlane(tab, min(eb - e_base, 63));
    blk_ok[kb] = (unsigned)blk < (unsigned)a.num_blocks;
    if (kb < NK / 16) all_ok = all_ok && blk_ok[kb];
    // the sub-block's first row (its codes at row * D, its scales at row;
    // the next slot of the head is ss rows on)
    row0[kb] = blk_ok[kb] ? cache_row(a.layout, blk, tb - eb * a.bs, h, a.bs, a.hkv)
                          : row_invalid;
  }
  if constexpr (PART != 1) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) r.blk_ok[kb] = blk_ok[kb];
    r.full = all_ok;
  }
  if constexpr (PART != 1) {
    // scales of token t0 + lane.  The sub-block is lane dependent, so its
    // values are picked with selects: indexing the arrays with it would
    // move them to scratch memory.
    const int kb = lane >> 4;
    const int64_t base = kb == 0 ? row0[0] : kb == 1 ? row0[1] : kb == 2 ? row0[2] : row0[3];
    const bool bok = kb == 0 ? blk_ok[0] : kb == 1 ? blk_ok[1] : kb == 2 ? blk_ok[2]
                                                                         : blk_ok[3];
    r.tok_ok = t0 + lane < t_end && bok;
    // (a tile that is not live reads the scales of head h's slot 0 in block 0)
    const int64_t rr = live ? base + (int64_t)((lane & 15) * a.ss) : row_invalid;
    r.ks = T::KS ? a.ks[rr] : 1.0f;
    if constexpr (T::MX)  // the row's E8M0 bytes (D / 32 of them)
      r.kxw = D == 128 ? *reinterpret_cast<const uint32_t*>(a.kexp + rr * 4)
                       : (uint32_t)*reinterpret_cast<const uint16_t*>(a.kexp + rr * 2);
    r.vs = T::V8 ? a.vs[rr] : 1.0f;
  }
  // Loads half by half (K then V of keys 0-31, then of keys 32-63), so the
  // first half can be computed while the second is in flight.
  // A sub-block's resource (scalar: the row bases are uniform) covers the
  // bytes from its first row to the end of the array, saturated to 32 bits.
  auto rsrc = [&](const void* arr, uint64_t arr_bytes, int kb, int elem_bytes)
      __attribute__((always_inline)) {
    const uint64_t off = (uint64_t)row0[kb] * (uint64_t)(D * elem_bytes);
    const uint64_t rem = arr_bytes - off;
    const uint32_t n = (rem >> 32) ? 0xffffffffu : (uint32_t)rem;
    return buffer_rsrc(static_cast<const uint8_t*>(arr) + off, live ? n : 0u);
  };
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    if (PART != 2 && kp != PART) continue;
#pragma unroll
    for (int kb = 2 * kp; kb < 2 * kp + 2; ++kb) {
      const __amdgpu_buffer_rsrc_t krs = rsrc(a.k, a.k_bytes, kb, T::KE);
#pragma unroll
      for (int p = 0; p < T::KP; ++p) {
        const int off = (int)lo.k + T::KPIECE * T::KE * p;
        if (T::K8) {
          r.k[kb][p] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
        } else {
          r.k[kb][2 * p] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
          r.k[kb][2 * p + 1] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0);
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int kb = 2 * kp + hb;
      const __amdgpu_buffer_rsrc_t vrs = rsrc(a.v, a.v_bytes, kb, T::VE);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * hb + jj;
        const int soff = jj * (int)lo.v_token;  // uniform: token row within the 4
        if constexpr (T::VW == 4) {
          const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)lo.v, soff, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) r.v[kp][j][e] = w[e];
        } else if constexpr (T::VW == 2) {
          const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(vrs, (int)lo.v, soff, 0);
          r.v[kp][j][0] = w[0];
          r.v[kp][j][1] = w[1];
        } else {
          r.v[kp][j][0] = __builtin_amdgcn_raw_buffer_load_b32(vrs, (int)lo.v, soff, 0);
        }
      }
    }
  }
}

// KV head of pair index pi (sequence b = pi / hkv): rotated by the
// sequence, h = (pi mod hkv - b mod hkv) mod hkv, so that pairs 8k + x (one
// XCD) cover every head.
__device__ __forceinline__ int rotated_head(int pi, int b, const FastDiv& div_hkv) {
  const int h = (pi - b * div_hkv.d) - div_hkv.mod(b);
  return h < 0 ? h + div_hkv.d : h;
}


// APPEND: the decode step's new token of sequence b (fp32 rows k_new[b],
// v_new[b]) sits at position seq_lens[b] - 1.  The work-group whose split
// holds that position quantises it by the storage rule, writes it to its
// cache slot (the only write of that slot) and substitutes it for the slot's
// previous bytes in the registers of the tile being attended, so the append
// costs no kernel of its own and no extra memory round trip.
//
// Q8 (narrow QK, e4m3 K only): the work-group quantises its G query rows
// once, by the cache-row rule (fp32 scale amax / 448 per row, e4m3 codes),
// and QK runs on the fp8 matrix instruction straight from the K codes as
// loaded, with no conversion; the row's scale multiplies the score ("FP8 KV
// attention: hardware paths and tile preparation", "Operating model" path 2
// and "AMD CDNA 3": a per-row scale moves outside the dot product).
//
// KB (pre-bias residual cache): the stored K rows are residuals r and the
// key is r + b with the bias b exact; every score of query row q gains
// (q . b) * sm_scale * log2(e), computed once per work-group ("Treat
// numerical safety and kernel speed as separate gates": keep the fixed bias
// exact, correct in score space).
//
// SHAPE: kMulti, the split holds more than one tile per wave (chunk > 4
// tiles), so the waves loop over their tiles; kOne, each wave computes at
// most one tile and there is no loop (a function of its own, so that its
// register allocation is not shaped by the loop's); kHalf, each wave
// attends at most half a tile (32 keys; chunk <= 128), so that a short
// context spreads over twice the work-groups and two waves share a SIMD.
//
// TB: the cache has a block table in memory; without one (contiguous cache)
// the block ids are computed, a variant of its own so that no wait for a
// table load sits in front of the first K/V loads.
//
// DIRECT: the plan has one split, so the work-group writes the pair's output
// rows (a.out) as the merge kernel would and no merge kernel follows; an
// instantiation of its own (at most one tile per wave, per-row K scales, no
// bias), so that the other kernels carry none of its code.
template <int MODE, int D, bool APPEND, bool Q8, bool KB, int SHAPE, bool TB, bool DIRECT>
__global__ __launch_bounds__(64 * kWaves, split_wgs_per_cu(MODE, D))
void decode_partial_kernel(DecodeArgs a) {
  static_assert(!Q8 || k_is_e4m3(MODE), "narrow QK needs e4m3 K codes");
  static_assert(!DIRECT || (SHAPE != kMulti && !KB && !k_is_mx(MODE)),
                "one-split output: single-pass shapes, per-row K scales, no bias");
  static_assert(!(Q8 && KB), "narrow QK takes no K bias");
  static_assert(!(k_is_mx(MODE) && (KB || APPEND)), "block-scaled K: no bias, no fused append");
  using T = TileRegs<MODE, D>;
  constexpr int KC = D / 32;         // MFMA k-chunks for QK
  constexpr int DPR = T::DPR;        // d values per V^T row group (MFMAs per PV chunk)
  constexpr bool kK8 = T::K8;
  constexpr bool kV8 = T::V8;
  constexpr bool MULTI = SHAPE == kMulti;
  constexpr bool HALF = SHAPE == kHalf;
  constexpr int kTW = HALF ? kTile / 2 : kTile;  // keys a wave attends per tile
  // the first tile's loads go out before the sequence length is known
  constexpr bool kEarly = !TB && !MULTI;

  __shared__ float s_scale[kWaves][2][kTile];
  __shared__ uint32_t s_kx[k_is_mx(MODE) ? kWaves : 1][kTile];  // block-scaled K: E8M0 words
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][4][kMaxGroup];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][kMaxGroup][D];
  __shared__ u32x4_t s_q[Q8 ? 1 : KC][64];
  // Q8: lane (g4, c)'s 32 code bytes of head c (the d of its K bytes) and
  // the query rows' scales
  __shared__ u32x4_t s_q8[Q8 ? 2 : 1][64];
  __shared__ float s_qs[Q8 ? kMaxGroup : 1];
  // block-scaled Q: E8M0 byte of block b of head c (the instruction takes the
  // scale of block b from lane group b)
  __shared__ uint32_t s_qx[Q8 && k_is_mx(MODE) ? 16 : 1][4];
  // fused append: the new token's K bytes, V bytes (each at most 2D) and
  // scales, in cache layout, for the wave that attends it
  __shared__ __attribute__((aligned(16))) uint32_t s_new[APPEND ? D + 4 : 1];
  //   s_new[D], s_new[D+1]: K and V scale; s_new[D+2], s_new[D+3]: the
  //   slot's cache row (low, high word; high word ~0u: not stored)

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4;   // k-slot group of the lane
  const int c = lane & 15;    // row / column of the lane

  // Work-group -> (sequence, KV head, split).  Consecutive work-groups are
  // dealt round-robin to the eight XCDs (each with its own L2), so
  // work-group wg runs on XCD wg % 8.  When the (sequence, KV head) pairs
  // come in multiples of eight, XCD x gets whole pairs (pair index
  // pi = 8k + x), their splits consecutive in its dispatch order; the KV
  // head is rotated by the sequence (h = (pi - b) mod Hkv), so every XCD
  // gets every head and every sequence once: equal work per XCD however
  // the lengths are spread, Q and block ids reused from one L2, and no XCD
  // confined to one head's rows of the cache.  The merge kernel maps pair
  // pi to the same XCD and finds the partials in that L2.
  const int wg = blockIdx.x;
  const int pairs = a.div_pairs.d;
  int pi, split;
  if ((pairs & 7) == 0) {
    const int q = wg >> 3;
    const int qd = a.div_splits.div(q);
    pi = qd * 8 + (wg & 7);
    split = q - qd * a.n_splits;
  } else {
    split = a.div_pairs.div(wg);
    pi = wg - split * pairs;
  }
  const int b = a.div_hkv.div(pi);
  const int h = rotated_head(pi, b, a.div_hkv);
  const int bh = b * a.hkv + h;
  const int G = a.group;
  const int t_begin = split * a.chunk;

  // First round trip, all independent and issued in this order: the
  // sequence length, the block ids of this split (lane e: block
  // t_begin / bs + e, index kept inside the table row; ids past the
  // sequence are never used), Q, the step's new K/V rows and the K bias.
  // Nothing is written to LDS before the first tile's loads are out: a
  // write of loaded data waits for its load, and the wait would sit in
  // front of them.
  //
  // kEarly: the early tile's base addresses and bounds are read from the
  // kernel arguments with the first ones.  Loaded only where they are used,
  // they would come after the length's scalar load, and the wait for them
  // (scalar loads return out of order: a wait for one is a wait for all)
  // would wait for the length too.  After this statement the length is
  // read with a vector load, whose wait counts in order.
  if constexpr (kEarly)
    asm volatile("" ::"s"(a.k), "s"(a.v), "s"(a.ks), "s"(a.vs), "s"(a.k_bytes), "s"(a.v_bytes));
  int len = a.seq_lens[b];  // clamped below to the block-table capacity
  const int e_base = a.div_bs.div(t_begin);
  const int64_t tab_i = (int64_t)b * a.mbps + min(e_base + lane, a.mbps - 1);
  int tab = (int)tab_i;  // no table: contiguous
  if constexpr (TB) tab = a.table[tab_i];
  // Q^T, the B operand of QK, goes to LDS in operand order: s_q[kc][lane] is
  // lane (g4, c)'s 16 bytes of head c for k-chunk kc; wave kc loads chunk kc.
  static_assert(KC <= kWaves, "one Q k-chunk per wave");
  const uint16_t* qrow = a.q + ((int64_t)b * a.hkv * G + (int64_t)h * G + min(c, G - 1)) * D;
  u32x4_t qx = {0u, 0u, 0u, 0u};
  if constexpr (!Q8) {
    const int kc = min(wave, KC - 1);
    // the d of the K bytes the lane converts for k-chunk kc
    const int d0 = T::KPIECE * (kc >> 1) + T::KLANE * g4 + 8 * (kc & 1);
    qx = *reinterpret_cast<const u32x4_t*>(qrow + d0);
  }
  // Q8 and KB: lane (g4, c) takes head c's values at d = KPIECE p + KLANE g4
  // + i (i < 16), the d of its K bytes (every wave loads them; wave 0
  // quantises them for Q8).
  constexpr int kQW = (Q8 || KB) ? T::KP : 1;
  u32x4_t qw[kQW][2];
  if constexpr (Q8 || KB) {
#pragma unroll
    for (int p = 0; p < T::KP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        qw[p][j] = *reinterpret_cast<const u32x4_t*>(qrow + T::KPIECE * p + T::KLANE * g4 + 8 * j);
  }
  // Fused append: lanes [0, D/4) hold four values of the K row, lanes
  // [D/4, D/2) four of the V row.  Every lane loads (the lanes past D/2
  // repeat the first ones): a load under a lane condition would make the
  // compiler wait for all later loads, tile data included, before the
  // values can be used.
  constexpr int kLR = D / 4;  // lanes per row
  float4 xnew = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (APPEND) {
    const int l2 = lane & (2 * kLR - 1);
    xnew = *reinterpret_cast<const float4*>((l2 < kLR ? a.k_new : a.v_new) +
                                            ((int64_t)b * a.hkv + h) * D + 4 * (l2 % kLR));
  }
  // KB: the bias values at the same d as qw
  constexpr int kBW = KB ? T::KP : 1;
  f32x4_t bw[kBW][2][2];
  if constexpr (KB) {
    const float* brow = a.kbias + (int64_t)h * D;
#pragma unroll
    for (int p = 0; p < T::KP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d0 = T::KPIECE * p + T::KLANE * g4 + 8 * j;
        bw[p][j][0] = *reinterpret_cast<const f32x4_t*>(brow + d0);
        bw[p][j][1] = *reinterpret_cast<const f32x4_t*>(brow + d0 + 4);
      }
  }
  float qb_c = 0.0f;  // KB: (q . b) of head c, in log2 units of the score

  LaneOffsets lo;
  lo.k = (uint32_t)(c * a.ss) * (D * T::KE) + T::KLANE * T::KE * g4;
  lo.v = (uint32_t)(4 * g4 * a.ss) * (D * T::VE) + DPR * T::VE * c;
  lo.v_token = (uint32_t)wave_uniform(a.ss * D * T::VE);

  // kEarly (no block table, one tile per wave): the first tile's addresses
  // depend on nothing in memory, so its loads go out now, with the first
  // round trip, as if the split held every key up to its end or the
  // block-table capacity (t_cap): every row they read lies inside the cache.
  // Once the length is known the tile's flags are narrowed to it, and a
  // wave whose tile turns out to lie past the length does not compute it.
  // A split with no key at all leaves only after the barrier below: a
  // return before it would let the compiler move these loads after the
  // test, behind the length.  Otherwise the loads wait for the length, and
  // with a table for the block ids.  (The split kernel that streams several
  // tiles per wave issues its first tile after the length: with the early
  // tile's registers live from the start it runs out of scalar registers.)
  const int t_cap = min(a.mbps * a.bs, t_begin + a.chunk);
  T buf;
  if constexpr (kEarly) {
    load_tile<MODE, D, HALF ? 0 : 2, kTW>(buf, a, lo, t_begin + wave * kTW, t_cap, tab, e_base,
                                          h, lane, t_begin + wave * kTW < t_cap);
    // (the length, loaded before the tile, is used only from here on: the
    // compiler would otherwise move its wait in front of the tile's loads)
    asm volatile("" : "+v"(len));
    len = __builtin_amdgcn_readfirstlane(len);
  }
  const int t_end = min(max(len, 0), t_cap);

  float* pacc = a.part_acc + ((int64_t)bh * a.n_splits + split) * G * D;
  float* pml = a.part_ml + ((int64_t)bh * a.n_splits + split) * G * 2;
  const bool empty = t_begin >= t_end;  // no key in this split
  // DIRECT: the pair's output rows
  float* const out_rows = DIRECT ? a.out + (int64_t)bh * G * D : nullptr;
  auto leave_empty = [&]() __attribute__((always_inline)) {
    if constexpr (DIRECT) {  // no key: the rows are 0
      for (int idx = 4 * threadIdx.x; idx < G * D; idx += 4 * blockDim.x)
        *reinterpret_cast<f32x4_t*>(out_rows + idx) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      return;
    }
    for (int i = threadIdx.x; i < G; i += blockDim.x) {
      pml[2 * i] = -INFINITY;
      pml[2 * i + 1] = 0.0f;
    }
  };
  if constexpr (!kEarly) {
    // The test reads the block ids too (no block id is INT_MIN, so the
    // second term is always true): without it the compiler sinks the table
    // load below the branch, a whole round trip before the first K/V load.
    if (empty & (__builtin_amdgcn_readfirstlane(tab) != INT_MIN)) {
      leave_empty();
      return;
    }
  }

  // Fused append: the new token (position len - 1, only if it lies inside
  // the block table) belongs to this split's tiles; the wave that attends it
  // quantises and stores it (after issuing its first tile's loads, so the
  // work overlaps their latency) and keeps its bytes in LDS for the
  // substitution.
  int pos_n = -1;  // wave-uniform; -1: this wave does not attend the new token
  if constexpr (APPEND) {
    const int p = len - 1;
    if (len >= 1 && len <= a.mbps * a.bs && p >= t_begin && p < t_end &&
        ((p - t_begin) / kTW) % kWaves == wave)
      pos_n = p;
  }
  pos_n = wave_uniform(pos_n);
  auto append_new = [&]() __attribute__((always_inline)) {
    if constexpr (!APPEND) return;  // (s_new is a placeholder then)
    const int p = pos_n;
    const int pb = a.div_bs.div(p);
    const int blk = __builtin_amdgcn_readlane(tab, pb - e_base);
    const bool is_v = lane >= kLR;
    const bool quantise = is_v ? kV8 : kK8;
    const float scale = storage_scale(row_amax<kLR>(xnew));  // RN(amax / 448), as append
    const int sub = lane % kLR;
    if (lane == 0) {
      const int64_t row = (unsigned)blk < (unsigned)a.num_blocks
                              ? cache_row(a.layout, blk, p - pb * a.bs, h, a.bs, a.hkv)
                              : -1;  // invalid block: not stored, key excluded
      s_new[D + 2] = (uint32_t)row;
      s_new[D + 3] = (uint32_t)((uint64_t)row >> 32);
    }
    if (lane < 2 * kLR) {
      // LDS image: K bytes at dword 0, V bytes at dword D/2, scales at D, D+1
      uint32_t* img = s_new + (is_v ? D / 2 : 0);
      if (quantise) {
        img[sub] = e4m3_codes4(xnew, scale);
        if (sub == 0) s_new[D + (is_v ? 1 : 0)] = __float_as_uint(scale);
      } else {
        *reinterpret_cast<u32x2_t*>(img + 2 * sub) = bf16x4(xnew);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // The fused append's only write of the slot: the bytes of the LDS image
  // (the same as fp8kv_append writes).  Issued after the last tile has been
  // consumed, because on gfx9 stores share the load counter: a store among
  // the tile loads would make every wait for tile data wait for it too.
  auto store_new = [&]() __attribute__((always_inline)) {
    if constexpr (!APPEND) return;
    const int64_t row =
        (int64_t)(((uint64_t)s_new[D + 3] << 32) | (uint64_t)s_new[D + 2]);
    if (row < 0 || lane >= 2 * kLR) return;  // invalid block: key excluded
    const bool is_v = lane >= kLR;
    const bool quantise = is_v ? kV8 : kK8;
    const int sub = lane % kLR;
    const uint32_t* img = s_new + (is_v ? D / 2 : 0);
    if (quantise) {
      uint8_t* dst = static_cast<uint8_t*>(const_cast<void*>(is_v ? a.v : a.k)) + row * D;
      *reinterpret_cast<uint32_t*>(dst + 4 * sub) = img[sub];
      if (sub == 0)
        const_cast<float*>(is_v ? a.vs : a.ks)[row] = __uint_as_float(s_new[D + (is_v ? 1 : 0)]);
    } else {
      uint16_t* dst = static_cast<uint16_t*>(const_cast<void*>(is_v ? a.v : a.k)) + row * D;
      *reinterpret_cast<u32x2_t*>(dst + 4 * sub) = *reinterpret_cast<const u32x2_t*>(img + 2 * sub);
    }
  };

  // Substitute the new token for its slot's previous bytes in a tile
  // (t0 <= pos_n < t0 + 64): K of token c in lanes (*, c), V of token
  // 4*g4 + jj in lanes (g4, *), scales in lane t.  Each half of the tile is
  // patched just before it is used, so the wait for the half's data stays
  // per half.  Every register is written through a select: a store to the
  // one matching element would index the arrays with a runtime value and
  // move them to scratch memory.
  auto patch_scales = [&](T& r, int t0) __attribute__((always_inline)) {
    if constexpr (!APPEND) return;
    const int tn = pos_n - t0;
    if (T::KS) r.ks = (lane == tn) ? __uint_as_float(s_new[D]) : r.ks;
    if (kV8) r.vs = (lane == tn) ? __uint_as_float(s_new[D + 1]) : r.vs;
  };
  auto patch_half = [&](T& r, int t0, int kp) __attribute__((always_inline)) {
    if constexpr (!APPEND) return;
    const int tn = pos_n - t0, kbn = tn >> 4, cn = tn & 15;
    if ((kbn >> 1) != kp) return;  // wave-uniform
    const uint8_t* img = reinterpret_cast<const uint8_t*>(s_new);
    u32x4_t nk[T::KRAW];
#pragma unroll
    for (int p = 0; p < T::KP; ++p) {
      const uint8_t* src = img + (64 * p + 16 * g4) * T::KE;
      if (kK8) {
        nk[p] = *reinterpret_cast<const u32x4_t*>(src);
      } else {
        nk[2 * p] = *reinterpret_cast<const u32x4_t*>(src);
        nk[2 * p + 1] = *reinterpret_cast<const u32x4_t*>(src + 16);
      }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bool sel = (c == cn) && ((kbn & 1) == hb);
#pragma unroll
      for (int q = 0; q < T::KRAW; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r.k[2 * kp + hb][q][e] = sel ? nk[q][e] : r.k[2 * kp + hb][q][e];
    }
    uint32_t nv[T::VW];
    const uint32_t* vimg = s_new + D / 2 + (DPR * T::VE / 4) * c;
#pragma unroll
    for (int e = 0; e < T::VW; ++e) nv[e] = vimg[e];
    const int jn = ((kbn & 1) << 2) | (cn & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool sel = (g4 == (cn >> 2)) && (j == jn);
#pragma unroll
      for (int e = 0; e < T::VW; ++e) r.v[kp][j][e] = sel ? nv[e] : r.v[kp][j][e];
    }
  };

  float q_scale_c = 1.0f;   // Q8: set once s_qs is complete
  int q_exp_c = 127;        // Q8, block-scaled: this lane's Q block E8M0 byte
  float m_run = -INFINITY;  // integer reference (log2 units) of head c
  float l_run = 0.0f;       // this lane's share of the normaliser of head c
  f32x4_t acc[DPR];
#pragma unroll
  for (int j = 0; j < DPR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A tile is computed whole (QK of its four sub-blocks, one online-softmax
  // step, PV) or, in the streaming loop, in two halves of 32 keys (sub-blocks
  // 2kp and 2kp+1, PV chunk kp), so that the second half's data may still be
  // arriving while the first is computed.  Its scales are staged through this
  // wave's slice of LDS first (written and read by the same wave; its LDS
  // operations complete in order, and the previous tile's reads precede these
  // writes in program order).
  auto compute_head = [&](T& cur, int t0) __attribute__((always_inline)) {
    const bool has_new = APPEND && pos_n >= t0 && pos_n < t0 + kTile;  // wave-uniform
    if (has_new) patch_scales(cur, t0);
    // K scale with sm_scale * log2(e) folded in (one product per token),
    // V scale as is.
    if (T::KS) s_scale[wave][0][lane] = cur.ks * a.c_scale;
    if constexpr (T::MX) s_kx[wave][lane] = cur.kxw;
    if (kV8) s_scale[wave][1][lane] = cur.tok_ok ? cur.vs : 0.0f;
    __builtin_amdgcn_wave_barrier();
  };
  // QK of sub-block kb on the matrix cores: S^T for its 16 keys (rows) and
  // the 16 query-head columns.
  auto qk_block = [&](T& cur, int kb) __attribute__((always_inline)) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Q8) {
      // the K codes as loaded: one fp8 instruction per 16 keys
      const u32x4_t k0 = cur.k[kb][0];
      const u32x4_t k1 = T::KP == 2 ? cur.k[kb][T::KP - 1] : u32x4_t{0u, 0u, 0u, 0u};
      const u32x4_t q0 = s_q8[0][lane], q1 = s_q8[1][lane];
      // (built with a shuffle: element-wise construction with the zero
      // half of head_dim 64 sends the operand through scratch memory)
      const i32x8_t av =
          __builtin_bit_cast(i32x8_t, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
      const i32x8_t bq =
          __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (T::MX) {
        // the lane's K block: head_dim 128 block g4, 64 block g4 / 2
        // the instruction takes the scale of K block g4 from lane group g4
        const int kexp = g4 < D / 32 ? (int)((s_kx[wave][16 * kb + c] >> (8 * g4)) & 0xffu) : 127;
        s = mfma_16x16x128_e4m3_scaled(av, bq, s, kexp, q_exp_c);
      } else {
        s = mfma_16x16x128_e4m3(av, bq, s);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4_t av;
        if (T::MX) {
          // codes times the lane's block scale (exact in bf16)
          // piece kc / 2 of lane group g4 lies in block 2 (kc / 2) + g4 / 2
          const float ksc = e8m0_value(
              (s_kx[wave][16 * kb + c] >> (8 * (2 * (kc >> 1) + (g4 >> 1)))) & 0xffu);
          const u32x4_t w = cur.k[kb][kc >> 1];
          const uint32_t lo32 = w[2 * (kc & 1)], hi32 = w[2 * (kc & 1) + 1];
          av = u32x4_t{e4m3x2_to_bf16x2_scaled(lo32, ksc, false),
                       e4m3x2_to_bf16x2_scaled(lo32, ksc, true),
                       e4m3x2_to_bf16x2_scaled(hi32, ksc, false),
                       e4m3x2_to_bf16x2_scaled(hi32, ksc, true)};
        } else if (kK8) {
          const u32x4_t w = cur.k[kb][kc >> 1];
          const uint32_t lo32 = w[2 * (kc & 1)], hi32 = w[2 * (kc & 1) + 1];
          av = u32x4_t{e4m3x2_to_bf16x2<false>(lo32), e4m3x2_to_bf16x2<true>(lo32),
                       e4m3x2_to_bf16x2<false>(hi32), e4m3x2_to_bf16x2<true>(hi32)};
        } else {
          av = cur.k[kb][kc];
        }
        s = mfma_16x16x32_bf16(av, s_q[kc][lane], s);
      }
    }
    return s;
  };

  // One online-softmax step over the NB sub-blocks kb0 .. kb0 + NB - 1 of a
  // tile (NB 2: one 32-key half, NB 4: the whole tile), then their PV chunks
  // kb0 / 2 .. (kb0 + NB) / 2 - 1.  okb[kb]: the block id of sub-block kb is
  // valid; full: every key of the tile is valid.  The flags come in as
  // values, so that the next tile's first part may already have replaced the
  // tile's own while its second half is computed.
  //
  // Scores: s = (q . K) * mult + add in log2 units, mult = k_scale * sm_scale
  // * log2(e) (times the query row's scale on the narrow path), add = (q . b)
  // * sm_scale * log2(e) for a K bias.  p = 2^(s - M) against the integer
  // reference M, computed as one fma into the exp2.  M moves (lazily) only
  // when a score exceeds it by more than kLazy; such a score makes its p
  // exceed 2^kLazy and with it its lane's sum of p, so only then (or while
  // no reference is set) is the row maximum taken and the step redone with
  // the exact rule.  That is the decision of comparing every row maximum
  // with M + kLazy, without the maximum on the common path.
  auto attend = [&](T& cur, int t0, auto nb_c, int kb0, bool full, const bool (&okb)[4])
      __attribute__((always_inline)) {
    constexpr int NB = decltype(nb_c)::value;
    constexpr int NS = 4 * NB;  // scores per lane
    const bool has_new = APPEND && pos_n >= t0 && pos_n < t0 + kTile;  // wave-uniform
    if (has_new) {
#pragma unroll
      for (int kp = kb0 / 2; kp < (kb0 + NB) / 2; ++kp) patch_half(cur, t0, kp);
    }
    f32x4_t sacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sacc[nb] = qk_block(cur, kb0 + nb);

    // per key: mult, v_scale, validity; score j is token
    // 16 * (kb0 + j / 4) + 4 * g4 + j % 4 (k-slot j % 8 of its PV chunk)
    float mult[NS], vsc[NS];
    bool okk[NS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int kb = kb0 + nb;
      const int base = 16 * kb + 4 * g4;
      f32x4_t ksv = {a.c_scale, a.c_scale, a.c_scale, a.c_scale};
      f32x4_t vsv = {1.f, 1.f, 1.f, 1.f};
      if (T::KS) ksv = *reinterpret_cast<const f32x4_t*>(&s_scale[wave][0][base]);
      if (kV8) vsv = *reinterpret_cast<const f32x4_t*>(&s_scale[wave][1][base]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mult[4 * nb + i] = Q8 ? ksv[i] * q_scale_c : ksv[i];
        vsc[4 * nb + i] = vsv[i];
        okk[4 * nb + i] = full || ((t0 + base + i < t_end) && okb[kb]);
      }
    }
    const float add = KB ? qb_c : 0.0f;

    float p[NS];
    float psum = 0.0f;
    {
      const float off = add - (m_run == -INFINITY ? 0.0f : m_run);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float arg = okk[j] ? __builtin_fmaf(sacc[j >> 2][j & 3], mult[j], off) : -INFINITY;
        p[j] = __builtin_amdgcn_exp2f(arg);
        psum += p[j];
      }
    }
    const bool redo = (m_run == -INFINITY) || !(psum <= kLazyP);
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {  // wave-uniform, rare
      float sc[NS];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        sc[j] = okk[j] ? __builtin_fmaf(sacc[j >> 2][j & 3], mult[j], add) : -INFINITY;
        tmax = fmaxf(tmax, sc[j]);
      }
      tmax = max_over_groups(tmax);
      // a step with no valid key (tmax = -inf) leaves the state unchanged
      const float t_ref = ceilf(tmax);
      if (m_run == -INFINITY) {
        m_run = t_ref;  // l and acc are still zero: nothing to rescale
      } else if (t_ref > m_run + kLazy) {
        const float alpha = ldexpf(1.0f, (int)(m_run - t_ref));
        l_run *= alpha;
#pragma unroll
        for (int j = 0; j < DPR; ++j) acc[j] *= alpha;
        m_run = t_ref;
      }
      // exp2(-inf - m) is 0 for finite m; m is -inf only while every score
      // so far is -inf, and then the reference 0 avoids -inf - -inf.
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
      psum = 0.0f;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sc[j] - m_ref);
        psum += p[j];
      }
    }
    l_run += psum;

#pragma unroll
    for (int ch = 0; ch < NB / 2; ++ch) {
      const int kp = kb0 / 2 + ch;
      // --- P with the V scale folded in, rounded to bf16: B operand of PV
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = p[8 * ch + j] * vsc[8 * ch + j];
      const u32x4_t pb = {f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3]),
                          f32x2_to_bf16x2(pv[4], pv[5]), f32x2_to_bf16x2(pv[6], pv[7])};

      // --- V of keys outside the sequence may hold any bits (even NaN
      //     codes): zero them in place so that P = 0 contributes exactly 0
      auto& vv = cur.v[kp];
      if (!full) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = okk[8 * ch + j];
#pragma unroll
          for (int e = 0; e < T::VW; ++e) vv[j][e] = ok ? vv[j][e] : 0u;
        }
      }

      // --- PV on the matrix cores: V^T chunk as the A operand
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
            const uint32_t x = byte_perm(vv[j0][wsel], vv[j1][wsel], sel);
            av[jp] = e4m3x2_to_bf16x2(x, (byte & 1) != 0);
          } else {
            const int e = db >> 1;
            const uint32_t sel = (db & 1) ? 0x03020706u : 0x01000504u;
            av[jp] = byte_perm(vv[j0][e], vv[j1][e], sel);
          }
        }
        acc[db] = mfma_16x16x32_bf16(av, pb, acc[db]);
      }
    }
  };
  using Half = std::integral_constant<int, 2>;
  using Whole = std::integral_constant<int, 4>;
  // Half kp of the tile (the streaming loop).
  auto compute_half = [&](T& cur, int t0, int kp, bool full, const bool (&okb)[4])
      __attribute__((always_inline)) { attend(cur, t0, Half{}, 2 * kp, full, okb); };
  // The whole tile in one step: its four sub-blocks' QK, one online-softmax
  // step, both PV chunks, so the scheduler has four independent chains.
  auto compute = [&](T& cur, int t0) __attribute__((always_inline)) {
    compute_head(cur, t0);
    const bool okb[4] = {cur.blk_ok[0], cur.blk_ok[1], cur.blk_ok[2], cur.blk_ok[3]};
    attend(cur, t0, Whole{}, 0, cur.full, okb);
  };

  // Tiles are dealt round-robin to the waves: wave w takes tiles w, w + 4,
  // ...  The first tile's loads go out before the barrier, so its wait
  // overlaps them.  A wave with several tiles streams them through one
  // register buffer, half by half: the next tile's first half is loaded into
  // the registers of the half just computed while the second half is
  // computed, and its second half after that (one buffer leaves room for
  // three work-groups per compute unit; the other waves on the SIMD cover
  // the rest of the latency).
  // Two alternating buffers were measured slower (8192 keys: split 18.3
  // against 17.9 us; ragged 64-sequence step 431 against 406 us): a wave's
  // loads issue in order, and with the memory pipeline full the issue of the
  // second tile's loads held back the compute of the first until late in the
  // stream.  Every load is issued unconditionally (a tile that does not exist
  // is issued empty, see load_tile), so the waits before each compute step
  // are exact.
  const int n_tiles = (t_end - t_begin + kTW - 1) / kTW;
  if constexpr (!kEarly)
    load_tile<MODE, D, HALF ? 0 : 2, kTW>(buf, a, lo, t_begin + wave * kTW, t_end, tab, e_base,
                                          h, lane, wave < n_tiles);
  // The first round trip's data, now that the tile loads are out: Q to LDS
  // (narrow QK: quantised first), the K bias product.
  if constexpr (!Q8) {
    if (wave < KC) s_q[wave][lane] = (c < G) ? qx : u32x4_t{0u, 0u, 0u, 0u};
  } else if (wave == 0) {
    // Q8: byte i of piece p is the same contraction index in the Q codes
    // and the lane's K bytes.  amax over the row is the max over
    // the four lane groups.
    float4 xq[T::KP][4];
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < T::KP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t w = qw[p][j];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float4 f = make_float4(__uint_as_float(w[2 * e] << 16),
                                       __uint_as_float(w[2 * e] & 0xffff0000u),
                                       __uint_as_float(w[2 * e + 1] << 16),
                                       __uint_as_float(w[2 * e + 1] & 0xffff0000u));
          xq[p][2 * j + e] = f;
          m = fmaxf(m, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
        }
      }
    // per-row rule: the row's scale (max over the four lane groups); block
    // rule: piece p of lane group g4 lies in block 2p + g4 / 2, shared with
    // lane group g4 ^ 1 (a 16-lane swap)
    float q_scale = 0.0f;
    float piece_scale[2] = {0.0f, 0.0f};
    if constexpr (T::MX) {
#pragma unroll
      for (int p = 0; p < T::KP; ++p) {
        float mp = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mp = fmaxf(mp, fmaxf(fmaxf(fabsf(xq[p][e].x), fabsf(xq[p][e].y)),
                               fmaxf(fabsf(xq[p][e].z), fabsf(xq[p][e].w))));
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mp), __float_as_uint(mp),
                                                  false, false);
        const int ep = mx_exponent(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
        piece_scale[p] = e8m0_value((uint32_t)(ep + 127));
        if ((g4 & 1) == 0 && c < G) s_qx[c][2 * p + (g4 >> 1)] = (uint32_t)(ep + 127);
      }
    } else {
      q_scale = max_over_groups(m) / kE4M3Max;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4_t codes = {0u, 0u, 0u, 0u};  // D = 64: the upper 16 k-slots are zero
      if (p < T::KP) {
        const float sc = T::MX ? piece_scale[p < T::KP ? p : 0] : q_scale;
#pragma unroll
        for (int e = 0; e < 4; ++e) codes[e] = e4m3_codes4(xq[p < T::KP ? p : 0][e], sc);
      }
      s_q8[p][lane] = (c < G) ? codes : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (g4 == 0 && c < G) s_qs[c] = T::MX ? 1.0f : q_scale;
  }
  // KB: (q . b) of head c, in log2 units of the score; the lane's products
  // at its d, summed over the four lane groups.
  if constexpr (KB) {
    float part = 0.0f;
#pragma unroll
    for (int p = 0; p < T::KP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4_t& bb = bw[p][j][e >> 1];
          part += __uint_as_float(qw[p][j][e] << 16) * bb[2 * (e & 1)];
          part += __uint_as_float(qw[p][j][e] & 0xffff0000u) * bb[2 * (e & 1) + 1];
        }
    qb_c = sum_over_groups(part) * a.c_scale;
  }
  if constexpr (kEarly) {  // narrow the early tile's flags to the length
    const int t0 = t_begin + wave * kTW;
    buf.full = buf.full && t0 + kTW <= t_end;
    buf.tok_ok = buf.tok_ok && t0 + lane < t_end;
  }
  if (APPEND && pos_n >= 0) append_new();
  __syncthreads();  // s_q complete (after the first tiles' loads are in flight)
  if constexpr (kEarly) {
    if (empty) {
      leave_empty();
      return;
    }
  }
  // Q8: the query row's scale of head c (0 for the padding heads c >= G,
  // whose B columns are zero)
  if constexpr (Q8) q_scale_c = (c < G) ? s_qs[c] : 0.0f;
  // block-scaled: this lane group supplies the scale of block g4 (head_dim
  // 64 has blocks 0 and 1; the zero k-slots of blocks 2 and 3 take 2^0)
  if constexpr (Q8 && T::MX) q_exp_c = (c < G && g4 < D / 32) ? (int)s_qx[c][g4] : 127;
  if constexpr (!MULTI) {
    if (wave < n_tiles) {
      if constexpr (HALF) {  // keys 0-31 of the tile at t0: sub-blocks 0, 1, PV chunk 0
        const int t0 = t_begin + wave * kTW;
        compute_head(buf, t0);
        const bool okb[4] = {buf.blk_ok[0], buf.blk_ok[1], buf.blk_ok[2], buf.blk_ok[3]};
        attend(buf, t0, Half{}, 0, buf.full, okb);
      } else {
        compute(buf, t_begin + wave * kTile);
      }
    }
  } else if (wave < n_tiles) {
    const int m = (n_tiles - wave + kWaves - 1) / kWaves;  // tiles of this wave
    int tile = wave;
    for (int i = 1; i < m; ++i, tile += kWaves) {
      // the next tile's first part goes into the registers of the half just
      // computed, its second part after the second half
      const int t0 = t_begin + tile * kTile, tn = t0 + kWaves * kTile;
      compute_head(buf, t0);
      const bool full = buf.full;
      const bool okb[4] = {buf.blk_ok[0], buf.blk_ok[1], buf.blk_ok[2], buf.blk_ok[3]};
      compute_half(buf, t0, 0, full, okb);
      load_tile<MODE, D, 0>(buf, a, lo, tn, t_end, tab, e_base, h, lane, true);
      compute_half(buf, t0, 1, full, okb);
      load_tile<MODE, D, 1>(buf, a, lo, tn, t_end, tab, e_base, h, lane, true);
    }
    compute(buf, t_begin + tile * kTile);
  }
  if (APPEND && pos_n >= 0) store_new();

  // --- merge the waves of the work-group: one barrier.  Each wave leaves
  //     its reference, its four lane-group shares of l and its accumulator
  //     (relative to its own reference) in LDS; then every thread combines
  //     the waves for its outputs with power-of-two weights.
  s_l[wave][g4][c] = l_run;
  if (g4 == 0) s_m[wave][c] = m_run;
  if (c < G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t lo4, hi4;
#pragma unroll
      for (int db = 0; db < 4; ++db) lo4[db] = acc[db][i];
      *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][DPR * (4 * g4 + i)]) = lo4;
      if constexpr (DPR == 8) {
#pragma unroll
        for (int db = 0; db < 4; ++db) hi4[db] = acc[4 + db][i];
        *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][DPR * (4 * g4 + i) + 4]) = hi4;
      }
    }
  }
  __syncthreads();
  // the waves' largest reference of head g and their row sum relative to it
  auto ref_of = [&](int g) __attribute__((always_inline)) {
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, s_m[w][g]);
    return ms;
  };
  auto sum_of = [&](int g, float ms) __attribute__((always_inline)) {
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][g];
      if (mw == -INFINITY) continue;
      const float lw = (s_l[w][0][g] + s_l[w][1][g]) + (s_l[w][2][g] + s_l[w][3][g]);
      lsum += ldexpf(lw, (int)(mw - ms));
    }
    return lsum;
  };
  for (int idx = 4 * threadIdx.x; idx < G * D; idx += 4 * blockDim.x) {
    const int g = idx / D, d = idx % D;
    const float ms = ref_of(g);
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][g];
      if (mw == -INFINITY) continue;  // a wave without keys
      sum += ldexpf(1.0f, (int)(mw - ms)) * *reinterpret_cast<const f32x4_t*>(&s_acc[w][g][d]);
    }
    if constexpr (DIRECT) {
      // the merge kernel's result for a single split: its weight is 1 and
      // the other split groups add exact zeros, so it is (acc + 0) / l
      // (which turns a -0 into +0), or 0 for a row without keys
      const float l = sum_of(g, ms);
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
      if (l > 0.0f) o = (sum + 0.0f) / l;
      *reinterpret_cast<f32x4_t*>(out_rows + idx) = o;
    } else {
      *reinterpret_cast<f32x4_t*>(pacc + idx) = sum;
    }
  }
  if constexpr (DIRECT) return;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const float ms = ref_of(g);
    const float lsum = sum_of(g, ms);
    pml[2 * g] = ms;
    pml[2 * g + 1] = lsum;
  }
}

// Second kernel: merge the splits of each (sequence, query head).  One
// single-wave work-group per query head, so a step's merge spreads over
// B * Hkv * G work-groups (the partials of a (sequence, KV head) pair are
// G * (D + 2) * 4 bytes per split; with one work-group per pair, 32 pairs
// would leave the reads to 32 compute units).  The wave's lanes form
// 64 / (D/4) split groups; lane (sg, d4) owns the head's values 4*d4 ..
// 4*d4+3 of the splits sg, sg + NG, sg + 2 NG, ...  Each group consumes its
// splits in batches of MB whose loads are all issued before any is used
// (MB = 4, 8 or 16, the smallest that takes a group's splits in one batch),
// combined online with power-of-two weights; the groups then meet through
// lane swaps, again with power-of-two weights.
//
// The arguments are pointers and scalars only (the divisors' multipliers and
// shifts passed one by one), 13 dwords that the build preloads into scalar
// registers at wave launch: the first loads, of the partials, go out without
// a round trip for the arguments (a structure argument would be loaded from
// memory).
template <int D, int MB>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_acc,
                                                          const float* __restrict__ part_ml,
                                                          float* __restrict__ out, int n_splits,
                                                          uint32_t hkv_m, uint32_t hkv_l, int hkv,
                                                          uint32_t g_m, uint32_t g_l, int group) {
  const FastDiv div_hkv{hkv_m, hkv_l, hkv}, div_group{g_m, g_l, group};
  constexpr int L = D / 4;    // lanes per split group, four values each
  constexpr int NG = 64 / L;  // split groups of the wave
  // Work-group -> (pair, head).  As in the split kernel, when the pairs come
  // in multiples of eight, pair pi = 8k + x runs on XCD x (work-group
  // w = 8q + x), which holds its partials in L2.
  const int w = blockIdx.x;
  const int pairs = div_group.div(gridDim.x);
  int pi, g;
  if ((pairs & 7) == 0) {
    const int q = w >> 3;
    const int qd = div_group.div(q);
    pi = qd * 8 + (w & 7);
    g = q - qd * group;
  } else {
    pi = div_group.div(w);
    g = w - pi * group;
  }
  const int b = div_hkv.div(pi);
  const int bh = b * hkv + rotated_head(pi, b, div_hkv);
  const int lane = threadIdx.x;
  const int sg = lane / L;
  const int d4 = lane % L;
  const float* ml = part_ml + (int64_t)bh * n_splits * group * 2;
  const float* pa = part_acc + (int64_t)bh * n_splits * group * D;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < n_splits; s0 += NG * MB) {
    float m[MB], l[MB];
    f32x4_t x[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int si = s0 + NG * i;
      const int s = si < n_splits ? si : s0;  // s0 < n_splits: in range
      const f32x2_t v = *reinterpret_cast<const f32x2_t*>(ml + ((int64_t)s * group + g) * 2);
      m[i] = si < n_splits ? v[0] : -INFINITY;
      l[i] = v[1];
      x[i] = *reinterpret_cast<const f32x4_t*>(pa + ((int64_t)s * group + g) * D + 4 * d4);
    }
    float mb = m_run;
#pragma unroll
    for (int i = 0; i < MB; ++i) mb = fmaxf(mb, m[i]);
    if (mb == -INFINITY) continue;  // nothing yet
    if (m_run != -INFINITY && mb != m_run) {
      const float alpha = ldexpf(1.0f, (int)(m_run - mb));
      l_run *= alpha;
      acc *= alpha;
    }
    m_run = mb;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (m[i] == -INFINITY) continue;  // empty split: weight 0
      const float wt = ldexpf(1.0f, (int)(m[i] - m_run));
      l_run += wt * l[i];
      acc += wt * x[i];
    }
  }
  // combine the split groups: lanes L, 2L, ... apart hold the same values
#pragma unroll
  for (int off = L; off < 64; off *= 2) {
    const float m2 = __shfl_xor(m_run, off);
    const float l2 = __shfl_xor(l_run, off);
    f32x4_t a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(acc[e], off);
    const float mm = fmaxf(m_run, m2);
    if (mm != -INFINITY) {  // otherwise both are empty and stay so
      const float w1 = m_run == -INFINITY ? 0.0f : ldexpf(1.0f, (int)(m_run - mm));
      const float w2 = m2 == -INFINITY ? 0.0f : ldexpf(1.0f, (int)(m2 - mm));
      l_run = w1 * l_run + w2 * l2;
      acc = w1 * acc + w2 * a2;
      m_run = mm;
    }
  }
  if (sg != 0) return;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  if (l_run > 0.0f) o = acc / l_run;
  // bh = b * hkv + h, output head h * group + g
  *reinterpret_cast<f32x4_t*>(out + ((int64_t)bh * group + g) * D + 4 * d4) = o;
}

template <int MODE, int D, bool APPEND, bool Q8, bool KB, int SHAPE, bool DIRECT>
static void launch_split(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.table)
    hipLaunchKernelGGL((decode_partial_kernel<MODE, D, APPEND, Q8, KB, SHAPE, true, DIRECT>),
                       grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partial_kernel<MODE, D, APPEND, Q8, KB, SHAPE, false, DIRECT>),
                       grid, block, 0, stream, a);
}

template <int MODE, int D, bool APPEND, bool Q8, bool KB>
static void launch_split_shape(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if constexpr (!KB && !k_is_mx(MODE)) {
    if (a.out) {  // one split of at most one tile per wave (direct_output_ok)
      if (a.chunk > kWaves * kTile / 2)
        launch_split<MODE, D, APPEND, Q8, KB, kOne, true>(a, grid, block, stream);
      else
        launch_split<MODE, D, APPEND, Q8, KB, kHalf, true>(a, grid, block, stream);
      return;
    }
  }
  if (a.chunk > kWaves * kTile)
    launch_split<MODE, D, APPEND, Q8, KB, kMulti, false>(a, grid, block, stream);
  else if (a.chunk > kWaves * kTile / 2)
    launch_split<MODE, D, APPEND, Q8, KB, kOne, false>(a, grid, block, stream);
  else
    launch_split<MODE, D, APPEND, Q8, KB, kHalf, false>(a, grid, block, stream);
}

template <int MODE, bool APPEND, bool Q8, bool KB>
static void launch_partial_d(const CacheView& c, const DecodeArgs& a, unsigned n_wg,
                             hipStream_t stream) {
  const dim3 grid(n_wg), block(64 * kWaves);
  if (c.d == 128)
    launch_split_shape<MODE, 128, APPEND, Q8, KB>(a, grid, block, stream);
  else
    launch_split_shape<MODE, 64, APPEND, Q8, KB>(a, grid, block, stream);
}

template <int MODE, bool APPEND, bool Q8>
static void launch_partial_mode(const CacheView& c, const DecodeArgs& a, unsigned n_wg,
                                hipStream_t stream) {
  if constexpr (!Q8 && !k_is_mx(MODE)) {
    if (c.kbias) {
      launch_partial_d<MODE, APPEND, false, true>(c, a, n_wg, stream);
      return;
    }
  }
  launch_partial_d<MODE, APPEND, Q8, false>(c, a, n_wg, stream);
}

template <bool APPEND>
static void launch_partial_append(const CacheView& c, const DecodeArgs& a, unsigned n_wg,
                                  bool q8, hipStream_t stream) {
  if constexpr (!APPEND) {  // block-scaled K: no fused append (checked by the caller)
    if (c.mode == kMXK8V8) {
      if (q8)
        launch_partial_mode<kMXK8V8, false, true>(c, a, n_wg, stream);
      else
        launch_partial_mode<kMXK8V8, false, false>(c, a, n_wg, stream);
      return;
    }
  }
  if (q8) {  // e4m3 K only (checked by the caller)
    if (c.mode == kK8V8)
      launch_partial_mode<kK8V8, APPEND, true>(c, a, n_wg, stream);
    else
      launch_partial_mode<kK8V16, APPEND, true>(c, a, n_wg, stream);
    return;
  }
  switch (c.mode) {
    case kK8V8: launch_partial_mode<kK8V8, APPEND, false>(c, a, n_wg, stream); break;
    case kK16V8: launch_partial_mode<kK16V8, APPEND, false>(c, a, n_wg, stream); break;
    case kK8V16: launch_partial_mode<kK8V16, APPEND, false>(c, a, n_wg, stream); break;
    case kBF16: launch_partial_mode<kBF16, APPEND, false>(c, a, n_wg, stream); break;
    default: break;  // block-scaled K with the fused append: rejected by the caller
  }
}

hipError_t launch_decode_partial(const CacheView& c, const uint16_t* q, int group,
                                 const int32_t* seq_lens, int batch, float c_scale,
                                 int chunk, int n_splits, float* part_acc,
                                 float* part_ml, const float* k_new, const float* v_new,
                                 float* out, bool q8, hipStream_t stream) {
  if (out && !direct_output_ok(c, chunk, n_splits)) return hipErrorInvalidValue;
  const uint64_t rows = (uint64_t)c.num_blocks * c.bs * c.hkv;
  const uint64_t k_bytes = rows * c.d * (k_is_e4m3(c.mode) ? 1 : 2);
  const uint64_t v_bytes = rows * c.d * (v_is_e4m3(c.mode) ? 1 : 2);
  DecodeArgs a{c.k,     c.v,       c.ks,    c.vs,    c.table,  q,       seq_lens,
               part_acc, part_ml,  k_new,   v_new,   c.kbias,  c.kexp,  c_scale,
               c.hkv,   group,     c.bs,    c.mbps,  chunk,    n_splits, c.num_blocks,
               c.layout, slot_stride(c.layout, c.hkv), k_bytes, v_bytes,
               FastDiv::of(c.hkv), FastDiv::of(c.bs), FastDiv::of(n_splits),
               FastDiv::of(batch * c.hkv), out};
  const unsigned n_wg = (unsigned)((int64_t)batch * c.hkv * n_splits);
  if (k_new)
    launch_partial_append<true>(c, a, n_wg, q8, stream);
  else
    launch_partial_append<false>(c, a, n_wg, q8, stream);
  return hipGetLastError();
}

template <int D>
static void launch_merge_d(unsigned n_wg, int hkv, int group, int n_splits,
                           const float* part_acc, const float* part_ml, float* out,
                           hipStream_t stream) {
  constexpr int NG = 64 / (D / 4);  // split groups per wave
  const int per_group = (n_splits + NG - 1) / NG;
  const FastDiv fh = FastDiv::of(hkv), fg = FastDiv::of(group);
  if (per_group <= 4)
    hipLaunchKernelGGL((decode_merge_kernel<D, 4>), dim3(n_wg), dim3(64), 0, stream,
                       part_acc, part_ml, out, n_splits, fh.m, fh.l, fh.d, fg.m, fg.l, fg.d);
  else if (per_group <= 8)
    hipLaunchKernelGGL((decode_merge_kernel<D, 8>), dim3(n_wg), dim3(64), 0, stream,
                       part_acc, part_ml, out, n_splits, fh.m, fh.l, fh.d, fg.m, fg.l, fg.d);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, 16>), dim3(n_wg), dim3(64), 0, stream,
                       part_acc, part_ml, out, n_splits, fh.m, fh.l, fh.d, fg.m, fg.l, fg.d);
}

hipError_t launch_decode_merge(int batch, int hkv, int group, int d, int n_splits,
                               const float* part_acc, const float* part_ml, float* out,
                               hipStream_t stream) {
  const unsigned n_wg = (unsigned)((int64_t)batch * hkv * group);
  if (d == 128)
    launch_merge_d<128>(n_wg, hkv, group, n_splits, part_acc, part_ml, out, stream);
  else
    launch_merge_d<64>(n_wg, hkv, group, n_splits, part_acc, part_ml, out, stream);
  return hipGetLastError();
}

}  // namespace fp8kv
