// Grouped GEMM phases of the block: gate_up + GeGLU, and down + weighted
// scatter.  One kernel serves the experts and the dense MLP: group g < E is
// expert g, whose rows are the (token, slot) pairs routed to it (its pair
// list); group E is the always-on dense MLP, whose rows are the canvas
// positions (the diffgemma contract's MoE-order bullet: the dense MLP runs in
// parallel as the always-on path; the ML@Berkeley post's MOEBlock iterates over
// experts and gathers their tokens).
//
// Work tile (gate_up): up to DG_MT = 32 rows x 128 weight rows (64 gate rows
// and the 64 matching up rows, so GeGLU fuses into the epilogue), over the
// whole input dimension K; the down tiles are described at k_down_q4.
//
// Q4G64 weights (the hot path).  Each of the four waves owns the whole tile
// for a quarter of K: wave w takes the 64-input groups w, w+4, w+8, ...  Per
// group a lane (g16 = lane/16, n16 = lane%16) loads, straight into registers,
//   * the codes of the tile's two 64-row blocks: 32 contiguous bytes each (the
//     four strips of the block, two 32-input halves per strip), and the four
//     (scale|bias) words of its row in each block;
//   * its A fragments: 8 fp16 inputs 64 q + 32 h + 8 g16 .. +7 of row n16 and
//     of row 16 + n16, for both halves h (A rows of an expert are gathered
//     through its pair list);
// dequantises the codes in registers (magic-number nibble expansion and one
// packed fp16 fma per two weights, the value RNE(scale*q + bias)) and feeds
// MFMA 16x16x32 f16 with fp32 accumulation: half h of a group is one MFMA, with
// lane group g16 holding inputs 32h + 8 g16 .. +7 in both operands, so each
// accumulator is the plain dot product.  Three groups are in flight per wave
// and the waves never wait for each other inside a tile; no LDS is used until
// the four partial tiles are added (in wave order) in LDS for the epilogue.
// The first groups of the next tile are requested before that epilogue, so the
// memory pipe does not drain between tiles.
//
// Q4G32 and BF16 weights take the same tiles and bodies (template argument
// WF): Q4G32 reads eight (scale|bias) words per lane and block, BF16 reads
// the lane's 8 inputs of each (strip, half) straight from the row-major
// weight row (256 bytes per lane and block) and converts them to fp16; both
// keep two groups in flight.  A dense MLP in BF16 beside Q4 experts shares
// their launch (k_split_q4: its tiles first, through their own queue).
//
// Tiles: expert g has ceil(rows/DG_MT) row tiles times its column tiles,
// numbered by expert, column tile, row tile; the dense MLP likewise.  Each
// workgroup derives the numbering itself from the per-expert pair counts (an
// exclusive scan in LDS); an expert's act rows start at the sum of the earlier
// experts' counts.  A persistent grid walks the tiles through one work queue
// per XCD, so that tiles sharing an expert's A rows or a weight block run
// under the same L2.
//
// Tile height: batches with many pairs per expert on average take 64-row
// tiles for every group (k_tall_q4); otherwise 32-row tiles, optionally with
// the experts above a pair-count threshold on 64-row tiles in the same launch
// (k_mixed_q4: one scan over the counts on the device builds both tile
// tables, the tall tiles go first through their own queue counters).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace {

static_assert(DG_SYNC_ERR == 4, "flag_error (common.h) writes the error words at word 4");

struct TileCtx {
  int grp, row_start, rows, nt;
  int kc;      // K chunk (the dense MLP's short-tile down tiles; 0 otherwise)
  bool dense;
  // one id per row: gate_up the row's token (experts: of its pair; the dense
  // MLP: the position itself), down the pair t*k + j
  const int32_t* pairs;
};

// ---------------------------------------------------------------- work queues
// Group sizes of this launch, from the per-expert pair counts: s_rows[g],
// s_off[g] (first act row of expert g) and s_tp[g] (first tile of group g,
// for tiles of MT rows and nt_e / nt_d column tiles per row tile),
// s_tp[E + 1] = number of tiles.  Wave 0 scans, five groups per lane.  The
// counts are clamped to the list capacity and fitted into the L*k act rows
// (plan.h), so no count left in the workspace can send a tile out of bounds.
// MIX: experts with at least tall_min rows are counted in a second table
// s_tp2 instead (tiles of MT2 rows, nt2_e column tiles; no dense tiles) and
// have no tiles in s_tp.
constexpr int DG_GPL = 5;  // 5 * 64 >= 257 groups

template <int MT = DG_MT, bool MIX = false, int MT2 = 64>
__device__ __forceinline__ void scan_groups(const GemmPhaseArgs& p, int* s_rows, int* s_off,
                                            int* s_tp, int nt_e, int nt_d, int* s_tp2 = nullptr,
                                            int tall_min = 0, int nt2_e = 0) {
  const int lane = threadIdx.x & 63;
  const int E = p.E, dense_rows = p.dense_rows;
  const int cap = (int)p.list_cap, total = (int)p.pairs;
  if (threadIdx.x < 64) {
    int raw[DG_GPL], nt[DG_GPL], nt2[DG_GPL];
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i)  // every count requested before the first is used
      raw[i] = p.cnt[min(DG_GPL * lane + i, E - 1) * DG_CNT_STRIDE];
    int sr = 0;
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i) {
      const int g = DG_GPL * lane + i;
      raw[i] = g < E && !p.skip_e ? plan_clamp_count(raw[i], cap) : 0;
      sr += raw[i];
    }
    int ir = sr;  // inclusive scan of the clamped counts over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tr = __shfl_up(ir, o, 64);
      if (lane >= o) ir += tr;
    }
    int rows[DG_GPL], first[DG_GPL];
    int excl = ir - sr, st = 0, st2 = 0;
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i) {
      const int g = DG_GPL * lane + i;
      first[i] = plan_first_row(excl, total);
      rows[i] = g < E ? plan_rows(excl, excl + raw[i], total) : (g == E ? dense_rows : 0);
      excl += raw[i];
      const int ntg = g < E ? nt_e : nt_d;
      const bool tl = MIX && g < E && rows[i] >= tall_min;
      nt[i] = g <= E && !tl ? (rows[i] + MT - 1) / MT * ntg : 0;
      nt2[i] = tl ? (rows[i] + MT2 - 1) / MT2 * nt2_e : 0;
      st += nt[i];
      st2 += nt2[i];
    }
    int it = st, it2 = st2;  // inclusive scans of the tile counts
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tt = __shfl_up(it, o, 64);
      const int tt2 = MIX ? __shfl_up(it2, o, 64) : 0;
      if (lane >= o) {
        it += tt;
        it2 += tt2;
      }
    }
    int t0 = it - st, t02 = it2 - st2;
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i) {
      const int g = DG_GPL * lane + i;
      if (g <= E) {
        s_rows[g] = rows[i];
        s_off[g] = g < E ? first[i] : 0;
        s_tp[g] = t0;
        if (g == E) s_tp[g + 1] = t0 + nt[i];
        if (MIX) {
          s_tp2[g] = t02;
          if (g == E) s_tp2[g + 1] = t02;
        }
      }
      t0 += nt[i];
      t02 += nt2[i];
    }
  }
  __syncthreads();
}

// Queue x (x = blockIdx % 8, the workgroup's XCD) holds the dense tiles of
// column tiles x, x+8, ... (all their row tiles) followed by the x-th eighth of
// the expert tiles, so every XCD gets the same share of dense and expert work
// and the tiles of one expert stay under one L2.  A workgroup's first tile is
// fixed (its rank among the workgroups of its queue); after that it takes the
// next tile with an integer atomic on the queue's counter, issued a tile ahead
// of use so the claim's latency is hidden and the claims of a queue are spread
// over time.  Every workgroup leaves once its queue is empty.
template <bool GATEUP_LIST>
struct Queue {
  int x, nd, e0, n, mts_d;
  // parts: which groups' tiles the queue holds (DG_PART_DENSE | DG_PART_EXPERTS)
  __device__ Queue(const GemmPhaseArgs& p, const int* s_tp, int parts = 3) {
    x = blockIdx.x & 7;
    const int te = parts & 2 ? s_tp[p.E] : 0;  // expert tiles
    e0 = (int)((int64_t)te * x / 8);
    const int e1 = (int)((int64_t)te * (x + 1) / 8);
    mts_d = (p.dense_rows + DG_MT - 1) / DG_MT;
    ncol = p.nt_d > x ? (p.nt_d - x + 7) / 8 : 0;
    const int kch = GATEUP_LIST ? 1 : p.kch_d;
    nd = parts & 1 ? mts_d * ncol * kch : 0;
    n = nd + (e1 - e0);
  }
  int ncol;
  __device__ TileCtx tile(const GemmPhaseArgs& p, int j, const int* s_rows, const int* s_off,
                          const int* s_tp) const {
    if (j < nd) {  // row tile fastest (its weights are shared), then column tile, then K chunk
      const int mt = j % mts_d, r = j / mts_d;
      return TileCtx{p.E, mt * DG_MT, min(DG_MT, p.dense_rows - mt * DG_MT), x + 8 * (r % ncol),
                     r / ncol, true, p.rowid + mt * DG_MT};
    }
    const int t = e0 + (j - nd);
    int lo = 0, hi = p.E;  // last expert with s_tp[g] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tp[mid] <= t) lo = mid; else hi = mid;
    }
    // the tile is the same for the whole workgroup: keep it in scalar registers
    const int g = __builtin_amdgcn_readfirstlane(lo);
    const int rows = __builtin_amdgcn_readfirstlane(s_rows[g]);
    const int off = __builtin_amdgcn_readfirstlane(s_off[g]);
    const int local = t - __builtin_amdgcn_readfirstlane(s_tp[g]);
    const int mts = (rows + DG_MT - 1) / DG_MT;
    const int nt = local / mts, mt = local % mts;
    // gate_up reads its A rows through the pairs' tokens, down scatters to the pairs
    const int32_t* ids = GATEUP_LIST ? p.list + (int64_t)p.E * p.list_cap : p.list;
    return TileCtx{g, off + mt * DG_MT, min(DG_MT, rows - mt * DG_MT), nt, 0, false,
                   ids + (int64_t)g * p.list_cap + mt * DG_MT};
  }
};

// ---------------------------------------------------------------- tile row ids
// The 32 row ids of a tile (a wave-uniform address: its slice of a pair list,
// or of the dense MLP's row list) are read through the scalar cache.  Waiting
// for them is then an lgkmcnt wait, which leaves the vector loads in flight
// alone; a vector load here would have to be waited for with vmcnt, and after
// a loop of a variable number of weight loads the compiler can only wait for
// all of them, draining the prefetch ring at every tile.  The reads may run
// up to 31 ids past the tile's last row (still inside the workspace: the row
// lists are followed by other workspace regions); those ids are never used.
struct TileIds {
  int s[32];
};
__device__ __forceinline__ void ids_request(TileIds& t, const int32_t* ids) {
  const uint64_t a = (uint64_t)(uintptr_t)ids;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const __attribute__((address_space(4))) int32_t* c = (const __attribute__((address_space(4))) int32_t*)u;
#pragma unroll
  for (int i = 0; i < 32; ++i) t.s[i] = c[i];
}
// Lane l's ids of rows l % 16 (lo) and 16 + l % 16 (hi); rows at or past
// `rows` take row 0's id.
__device__ __forceinline__ void ids_lanes(const TileIds& t, int rows, int& lo, int& hi) {
  const int n = (int)(threadIdx.x & 15);
  lo = t.s[0];
  hi = 16 < rows ? t.s[16] : t.s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    lo = n == i && i < rows ? t.s[i] : lo;
    hi = n == i && 16 + i < rows ? t.s[16 + i] : hi;
  }
}

// A row feeding tile row m (rows past the tile read row 0 again; their
// results are dropped), in two steps: a_id is the only part that reads
// memory (gate_up: the row's token, the same load for experts and the dense
// MLP) and is issued a tile ahead of use; a_row turns it into the row's address.
template <bool GATEUP>
__device__ __forceinline__ int a_id(const GemmPhaseArgs& p, const TileCtx& tc, int m) {
  const int mm = m < tc.rows ? m : 0;
  if (GATEUP) return plan_clamp_id(tc.pairs[mm], (int)p.n_tok);
  return tc.row_start + mm;  // down: a position, or an expert-sorted act row
}
template <bool GATEUP>
__device__ __forceinline__ const _Float16* a_row(const GemmPhaseArgs& p, const TileCtx& tc, int id,
                                                 int K) {
  return (tc.dense ? p.a_d : p.a_e) + (int64_t)id * K;
}

// ---------------------------------------------------------------- Q4G64 path
constexpr int QRING = 3;             // 64-input groups in flight per wave
constexpr int DG_Q4_WPE = 2;         // waves per SIMD (workgroups per CU) of the Q4G64 GEMMs
constexpr int PT_LD = 2 * 64 + 1;    // LDS row stride (floats) of a partial tile, padded

// Weight formats of the short-tile bodies (template argument WF):
//   WF_Q4G64  codes and one (scale|bias) word per 64 inputs (four per lane and block);
//   WF_Q4G32  the same codes, a (scale|bias) word per 32 inputs (eight per lane and block);
//   WF_BF16   row-major bf16 values: the lane's 8 inputs of each (strip, half)
//             are one 16-byte load from its weight row, converted to fp16 (RNE)
//             in registers; a group the wave does not compute reads the zero
//             words instead, so its products are zero as with a zero scale.
//   WF_Q8G64  row-major 8-bit codes: the lane's 8 codes of each (strip, half)
//             are one 8-byte load from its row, and its row's (scale|bias)
//             word of the group one 4-byte load per strip (the dense MLP only).
//   WF_NVFP4  the Q4G64 code words holding E2M1 codes, and 16 bytes of E4M3
//             scales per lane and block (its row's four strips x four 16-input
//             blocks, in the place of Q4G64's four pairs); the matrix cores
//             take e2m1 * e4m3 (exact in fp16) and the epilogue multiplies the
//             fp32 sums by the matrix's tensor scale.
//   WF_Q6G32  the Q4G64 code words (low 4 bits) and 16 bytes of high bits per
//             lane and block from the high plane; scales as Q4G32.
constexpr int WF_Q4G64 = 0, WF_Q4G32 = 1, WF_BF16 = 2, WF_Q8G64 = 3, WF_NVFP4 = 4, WF_Q6G32 = 5;
// the formats with a (scale|bias) word per 32 inputs
template <int WF> constexpr bool kG32 = WF == WF_Q4G32 || WF == WF_Q6G32;

// A global-memory pointer every lane of the wave holds, moved to scalar
// registers, so that loads from it take the scalar-base + 32-bit lane offset
// form of the global loads.
typedef const __attribute__((address_space(1))) char* gptr_t;
__device__ __forceinline__ gptr_t wave_ptr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return (gptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a));
}
typedef uint32_t gu32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t gu32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(gptr_t base, uint32_t off) {
  const gu32x4_t v = *(const __attribute__((address_space(1))) gu32x4_t*)(base + off);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ gu32x2_t gload8(gptr_t base, uint32_t off) {
  return *(const __attribute__((address_space(1))) gu32x2_t*)(base + off);
}

template <int WF>
struct QGroup {     // one wave's operands for one 64-input group
  // [block][16 bytes]: Q4: words (strip, half) 0..3 and 4..7 of the lane's row;
  // BF16: (strip, half) 2s + h, 8 values each; Q8: strip s, its two halves' 8 codes;
  // Q6: the Q4 words, then the high-plane words of strips 0..3
  uint4 w[2][WF == WF_BF16 ? 8 : WF == WF_Q8G64 ? 4 : WF == WF_Q6G32 ? 3 : 2];
  uint4 sb[2][kG32<WF> ? 2 : 1];  // [block]: (scale | bias << 16) of strips 0..3
                                  // (Q4G32, Q6G32: of (strip, half) 0..3 and 4..7; BF16: unused)
  uint4 a[2][2];    // [row block of 16][half]: 8 fp16 A inputs
};

struct QTile {      // where a tile's operands live
  const uint32_t* codes;  // the group's codes and (scale|bias) pairs
  const uint32_t* sb;
  float gsc;              // NVFP4: the matrix's tensor scale (else 1)
  int64_t hoff;           // Q6G32: words of the low plane (the high plane follows)
  int64_t blk[2];         // 64-row block index of the tile's two blocks
  bool bok1;              // block 1 exists (down: N may end half-way through a tile)
  int G;                  // 64-input groups of K
  const uint32_t* zero;   // 64 zero words: the scales and biases of a group not computed
  const _Float16* arow[2];
};

template <bool GATEUP, int WF>
__device__ __forceinline__ QTile q_tile(const GemmPhaseArgs& p, const TileCtx& tc, int id0,
                                        int id1) {
  QTile q;
  const bool dense = tc.dense;
  const int N = dense ? p.n_d : p.n_e;
  const int K = dense ? p.k_d : p.k_e;
  q.G = K / 64;
  q.zero = p.zero;
  // words of one expert's matrix: codes (BF16: values, two per word) and pairs
  const int64_t words_e = WF == WF_Q6G32 ? (int64_t)p.n_e * p.k_e * 3 / 16
                                          : (int64_t)p.n_e * p.k_e / (WF == WF_BF16 ? 2 : WF == WF_Q8G64 ? 4 : 8);
  // (NVFP4: scale words, and the 16-word trailer)
  const int64_t pairs_e = (int64_t)p.n_e * p.k_e / (kG32<WF> ? 32 : 64) + (WF == WF_NVFP4 ? 16 : 0);
  q.hoff = (int64_t)N * K / 8;
  q.codes = dense ? (const uint32_t*)p.w_d : (const uint32_t*)p.w_e + (int64_t)tc.grp * words_e;
  q.sb = dense ? p.sb_d : p.sb_e + (int64_t)tc.grp * pairs_e;
  q.gsc = WF == WF_NVFP4 ? *(const float*)(q.sb + (int64_t)N * K / 64) : 1.0f;
  if (GATEUP) {
    q.blk[0] = tc.nt;                  // gate rows 64 nt ..
    q.blk[1] = N / 128 + tc.nt;        // the matching up rows N/2 + 64 nt ..
    q.bok1 = true;
  } else {
    q.blk[0] = 2 * tc.nt;
    q.bok1 = 128 * tc.nt + 64 < N;
    q.blk[1] = q.bok1 ? 2 * tc.nt + 1 : 2 * tc.nt;
  }
  q.arow[0] = a_row<GATEUP>(p, tc, id0, K);
  q.arow[1] = a_row<GATEUP>(p, tc, id1, K);
  return q;
}

// Group i of wave w (group index w + 4 i): ten 16-byte loads, always issued,
// so every refill of the ring is the same instruction sequence and each wait
// names exactly the group it needs.  Past the wave's last group (or when K has
// fewer groups than waves) the loads read the wave's last group again (group
// 0 if it has none) and take their scales and biases from the zero words, as
// does a block the tile does not have: every product of such a group is
// exactly zero.  A single-row-block tile still loads its second A block (row
// 0 again) and leaves it unused.
template <int WF>
__device__ __forceinline__ void q_load(QGroup<WF>& d, const QTile& t, int w, int i, int ngw, int g16,
                                       int n16) {
  const bool live = i < ngw;
  const int q = live ? w + 4 * i : (ngw > 0 ? w + 4 * (ngw - 1) : 0);
  if (WF == WF_BF16) {
    // a wave-uniform base (the matrix, or the zero words when the wave does
    // not compute this block) plus a 32-bit lane offset (a matrix is below
    // 2^31 bytes); off blocks read the first 80 bytes of the zero words
    const uint32_t K2 = (uint32_t)t.G * 128;  // bytes of a weight row
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const bool on = live && (bb == 0 || t.bok1);
      const gptr_t base = wave_ptr(on ? (const void*)t.codes : (const void*)t.zero);
      const uint32_t o0 = on ? ((uint32_t)(64 * t.blk[bb]) + n16) * K2 + 128u * q + 16u * g16 : 0u;
      const uint32_t so = on ? 16u * K2 : 0u;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          d.w[bb][2 * s + h] = gload16(base, o0 + s * so + 64u * h);
    }
  } else if (WF == WF_Q8G64) {
    // codes: uniform base + 32-bit lane offset (as BF16, one byte per input);
    // the row's (scale|bias) words of the group: a live block's, or zero words
    const uint32_t K1 = (uint32_t)t.G * 64;  // bytes of a code row
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const bool on = live && (bb == 0 || t.bok1);
      const gptr_t base = wave_ptr(t.codes);
      const uint32_t o0 = ((uint32_t)(64 * t.blk[bb]) + n16) * K1 + 64u * q + 8u * g16;
      uint32_t sbw[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const gu32x2_t c0 = gload8(base, o0 + 16u * s * K1);
        const gu32x2_t c1 = gload8(base, o0 + 16u * s * K1 + 32u);
        d.w[bb][WF == WF_Q8G64 ? s : 0] = make_uint4(c0[0], c0[1], c1[0], c1[1]);
        const int64_t r = 64 * t.blk[bb] + 16 * s + n16;
        sbw[s] = *(on ? t.sb + r * t.G + q : t.zero + 4 * n16);
      }
      d.sb[bb][0] = make_uint4(sbw[0], sbw[1], sbw[2], sbw[3]);
    }
  } else {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int64_t bq = t.blk[bb] * t.G + q;
    const uint4* cw = (const uint4*)(t.codes + ((bq * 4 + g16) * 16 + n16) * 8);
    d.w[bb][0] = cw[0];
    d.w[bb][1] = cw[1];
    const bool on = live && (bb == 0 || t.bok1);
    if (WF == WF_Q6G32)
      d.w[bb][WF == WF_Q6G32 ? 2 : 0] = *(const uint4*)(t.codes + t.hoff + ((bq * 4 + g16) * 16 + n16) * 4);
    if (kG32<WF>) {
      const uint4* ps = (const uint4*)(on ? t.sb + (bq * 16 + n16) * 8 : t.zero + 4 * n16);
      d.sb[bb][0] = ps[0];
      d.sb[bb][kG32<WF> ? 1 : 0] = ps[on ? 1 : 0];
    } else {
      d.sb[bb][0] = *(const uint4*)(on ? t.sb + (bq * 16 + n16) * 4 : t.zero + 4 * n16);
    }
  }
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) d.a[mb][h] = *(const uint4*)(t.arow[mb] + 64 * q + 32 * h + 8 * g16);
}

// acc[block][strip][row block]: lane holds C[m = 16 mb + 4 g16 + i][n = 64 bb + 16 s + n16]
// NVFP4: the byte of the E4M3 scale of (strip s, half h) in a lane's 16 scale
// bytes of a block: word s, byte 2h + (g16 >> 1).
__device__ __forceinline__ uint32_t fp4_scale(const uint4& sb, int s, int h) {
  return u4_get(sb, s) >> (16 * h + 8 * ((threadIdx.x >> 5) & 1));
}

template <int WF>
__device__ __forceinline__ half8_t q_frag(const QGroup<WF>& d, int bb, int s, int h) {
  if (WF == WF_NVFP4) {
    const _Float16 sc = e4m3_half(fp4_scale(d.sb[bb][0], s, h));
    return dequant_fp4_word(u4_get(d.w[bb][s >> 1], 2 * (s & 1) + h), (half2_t){sc, sc});
  }
  if (WF == WF_BF16) return bf16x8_to_half8(d.w[bb][WF == WF_BF16 ? 2 * s + h : 0]);
  if (WF == WF_Q8G64) {
    const uint32_t pr = u4_get(d.sb[bb][0], s);
    const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
    const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
    const uint4 c = d.w[bb][WF == WF_Q8G64 ? s : 0];
    return dequant_q8_pair(h ? c.z : c.x, h ? c.w : c.y, (half2_t){sc, sc}, (half2_t){bi, bi});
  }
  const uint32_t pr = kG32<WF> ? u4_get(d.sb[bb][kG32<WF> ? s >> 1 : 0], 2 * (s & 1) + h)
                                : u4_get(d.sb[bb][0], s);
  const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
  const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
  const uint32_t word = u4_get(d.w[bb][s >> 1], 2 * (s & 1) + h);
  if (WF == WF_Q6G32)
    return dequant_q6_word(word, u4_get(d.w[bb][WF == WF_Q6G32 ? 2 : 0], s) >> (8 * h), (half2_t){sc, sc},
                           (half2_t){bi, bi});
  return dequant_q4_word(word, (half2_t){sc, sc}, (half2_t){bi, bi});
}

template <int WF>
__device__ __forceinline__ void q_compute(const QGroup<WF>& d, float4_t (&acc)[2][4][2], bool two) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half8_t b = q_frag(d, bb, s, h);
        acc[bb][s][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(d.a[0][h]), b,
                                                                acc[bb][s][0], 0, 0, 0);
        if (two)
          acc[bb][s][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(d.a[1][h]), b,
                                                                  acc[bb][s][1], 0, 0, 0);
      }
    }
}

// SCALE (NVFP4): the sums are multiplied by the matrix's tensor scale gsc.
template <bool GATEUP, bool SCALE = false>
__device__ __forceinline__ void q_epilogue(const GemmPhaseArgs& p, const TileCtx& tc,
                                           const float* part, const int* rpair, float gsc = 1.0f) {
  // sum of the four waves' partial tiles, in wave order; one loop (not
  // unrolled; its four columns per step run the same code) so every element
  // runs the same instructions and a row's result does not depend on its
  // place in the tile
  const int tid = threadIdx.x;
  const bool dense = tc.dense;
  const int N = dense ? p.n_d : p.n_e;
  constexpr int WS = DG_MT * PT_LD;  // one wave's partial tile
  if (GATEUP) {
    _Float16* dst = (dense ? p.act_d : p.act_e) + (int64_t)tc.row_start * (N / 2) + tc.nt * DG_NGU;
    // four consecutive columns per thread, one 8-byte store
    constexpr int NQ = DG_NGU / 4;
    float big = 0.f;
#pragma unroll 1
    for (int e = tid; e < tc.rows * NQ; e += 256) {
      const int m = e / NQ, c = 4 * (e % NQ);
      uint16_t h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pg = part + m * PT_LD + c + u;
        float gv = ((pg[0] + pg[WS]) + pg[2 * WS]) + pg[3 * WS];
        const float* pu = pg + 64;
        float uv = ((pu[0] + pu[WS]) + pu[2 * WS]) + pu[3 * WS];
        if (SCALE) {
          gv = __fmul_rn(gv, gsc);
          uv = __fmul_rn(uv, gsc);
        }
        const float av = __fmul_rn(gelu_tanh(gv), uv);
        big = fmaxf(big, fabsf(av));
        h[u] = bitcast<uint16_t>((_Float16)av);
      }
      *(uint2*)(dst + (int64_t)m * (N / 2) + c) =
          make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    }
    if (!(big < DG_F16_LIMIT)) flag_error(p.sync, DG_ERR_RANGE, p.stamp);
  } else {
    // four consecutive columns per thread: one address and one 8-byte (fp16
    // slots) or 16-byte (fp32 h1) store; N and so ncol are multiples of 64
    const int ncol = min(DG_NDN, N - tc.nt * DG_NDN);
    constexpr int NQ = DG_NDN / 4;
    float big = 0.f;
#pragma unroll 1
    for (int e = tid; e < tc.rows * NQ; e += 256) {
      const int m = e / NQ, c = 4 * (e % NQ);
      if (c >= ncol) continue;
      float y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pc = part + m * PT_LD + c + u;
        y[u] = ((pc[0] + pc[WS]) + pc[2 * WS]) + pc[3 * WS];
        if (SCALE) y[u] = __fmul_rn(y[u], gsc);
      }
      const int64_t col = (int64_t)tc.nt * DG_NDN + c;
      if (dense) {
        *(float4*)(p.h1 + (int64_t)(tc.row_start + m) * N + col) = make_float4(y[0], y[1], y[2], y[3]);
      } else {
        big = fmaxf(big, fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))));
        const uint32_t lo = (uint32_t)bitcast<uint16_t>((_Float16)y[0]) |
                            ((uint32_t)bitcast<uint16_t>((_Float16)y[1]) << 16);
        const uint32_t hi = (uint32_t)bitcast<uint16_t>((_Float16)y[2]) |
                            ((uint32_t)bitcast<uint16_t>((_Float16)y[3]) << 16);
        *(uint2*)(p.slots + (int64_t)rpair[m] * N + col) = make_uint2(lo, hi);
      }
    }
    if (!(big < DG_F16_LIMIT)) flag_error(p.sync, DG_ERR_RANGE, p.stamp);
  }
}

// Tile sequence of a workgroup: its first two tiles are fixed (ranks jb and
// jb + nwg of its queue); each later one is claimed with an integer atomic
// issued two tiles ahead of use.  So when a tile starts, the next tile is
// known, and whatever must be read from memory to start it (the row ids that
// locate its gate_up A rows) is requested behind the current tile's operands
// and has arrived by the time the next tile's loads are issued; a down tile's
// own pair ids (its scatter rows) are requested the same way and parked in
// LDS for the epilogue.  Every load of the tile loop is issued on every path
// (clamped to a valid address where it is not needed), so the waits inside
// the loop never cover more than the group about to be used.
// LDS of a short-tile body: the four waves' partial tiles [wave][row][column],
// the next tile claimed, and (down) the pair id of each row of the tile.
struct QLds {
  float part[4 * DG_MT * PT_LD];
  int next;
  int pair[DG_MT];
};

// The tiles of s_tp (from scan_groups), claimed
// through the eight counters at queue.
template <bool GATEUP, int WF = WF_Q4G64>
__device__ __forceinline__ void q_body(const GemmPhaseArgs& p, QLds& L, const int* s_rows,
                                       const int* s_off, const int* s_tp, int* queue,
                                       int parts = 3) {
  float* part = L.part;
  int* s_pair = L.pair;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave: uniform, so its loop bounds are too
  const int g16 = lane >> 4, n16 = lane & 15;
  const int nwg = (int)(gridDim.x >> 3);  // workgroups per queue (the grid is a multiple of 8)
  const Queue<GATEUP> qu(p, s_tp, parts);
  int* ctr = queue + qu.x;

  const int j0 = (int)(blockIdx.x >> 3);
  if (j0 >= qu.n) return;
  TileCtx tc = qu.tile(p, j0, s_rows, s_off, s_tp);
  QTile qt = q_tile<GATEUP, WF>(p, tc, a_id<GATEUP>(p, tc, n16), a_id<GATEUP>(p, tc, 16 + n16));
  bool two = tc.rows > 16;
  int ngw = (qt.G - w + 3) / 4;  // groups of this wave
  // Q4G32, BF16 and Q8G64: two groups in flight (their eight scale words, or
  // 128 to 256 bytes of weights, per block do not fit the register budget of
  // three); NVFP4 loads what Q4G64 loads and keeps three
  constexpr int RING = WF == WF_Q4G64 || WF == WF_NVFP4 ? QRING : 2;
  QGroup<WF> r[RING];
#pragma unroll
  for (int u = 0; u < RING; ++u) q_load(r[u], qt, w, u, ngw, g16, n16);
  // claims: the raw counter value, turned into a tile index only after the
  // barrier, so no instruction next to the atomic waits for its return (an
  // in-order wait that would also cover every load issued before it)
  int nxt = 0;
  if (tid == 0) nxt = atomicAdd(ctr, 1);
  int jn = j0 + nwg;  // the next tile

  while (true) {
    // requested behind this tile's operands, through the scalar cache: the
    // next tile's A row ids (the last tile looks itself up again)
    const TileCtx tn = qu.tile(p, min(jn, qu.n - 1), s_rows, s_off, s_tp);
    TileIds nids;
    ids_request(nids, tn.pairs);
    const int cpair = GATEUP ? 0 : plan_clamp_id(tc.pairs[min(tid, tc.rows - 1)], (int)p.pairs);

    float4_t acc[2][4][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[bb][s][mb] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // the wave's groups, RING in flight, in rounds of RING: while a refill
    // of this tile is still due, a round computes the ring slots and
    // refills each right after its use (groups past the last one read as
    // zero-scale groups); the final round refills the slots with the next
    // tile's first RING groups (after the queue's last tile: zero-scale
    // reads), so the memory pipe never runs dry at a tile boundary.  All of it
    // is straight-line code, so every wait names exactly the group it needs.
    int i0 = 0;
    for (; i0 + RING < ngw; i0 += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) {
        q_compute(r[u], acc, two);
        q_load(r[u], qt, w, i0 + RING + u, ngw, g16, n16);
      }
    }
    const bool more = jn < qu.n;
    int id0, id1;
    ids_lanes(nids, tn.rows, id0, id1);
    const QTile qn = q_tile<GATEUP, WF>(p, tn, plan_clamp_id(id0, (int)p.n_tok),
                                    plan_clamp_id(id1, (int)p.n_tok));
    const bool two_n = tn.rows > 16;
    const int ngw_n = more ? (qn.G - w + 3) / 4 : 0;  // none: zero-scale reads of group 0
    // the final round: slots past the wave's groups hold zero-scale reads and
    // are not computed (their products would be exact zeros)
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      if (i0 + u < ngw) q_compute(r[u], acc, two);
      q_load(r[u], qn, w, u, ngw_n, g16, n16);
    }
    // partial tile of this wave -> LDS
    float* pw = part + w * DG_MT * PT_LD;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if (mb == 1 && !two) break;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pw[(16 * mb + 4 * g16 + i) * PT_LD + 64 * bb + 16 * s + n16] = acc[bb][s][mb][i];
        }
    if (!GATEUP && tid < DG_MT) s_pair[tid] = cpair;
    if (tid == 0) L.next = nxt;
    __syncthreads();
    // the epilogue runs while the next tile's first groups are in flight
    const int jnn = 2 * nwg + L.next;
    const TileCtx cur = tc;
    const float gcur = qt.gsc;
    if (more) {
      tc = tn;
      qt = qn;
      two = two_n;
      ngw = ngw_n;
      if (tid == 0) nxt = atomicAdd(ctr, 1);
    }
    q_epilogue<GATEUP, WF == WF_NVFP4>(p, cur, part, s_pair, gcur);
    __syncthreads();  // the partial tiles and row ids are consumed
    if (!more) break;
    jn = jnn;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the last round's zero-scale reads (vmcnt(0))
}

// ---------------------------------------------------------------- Q4G64 down, short tiles
// Tile: up to DG_MT = 32 rows (an expert's pairs in act order, or positions
// for the dense MLP) x DG_NDN_Q4 = 256 output columns, over the whole K = I
// (a K chunk of about I for the dense MLP).  Wave w owns the 64-row weight
// block 4 nt + w of W_down -- 64 output columns -- for every 64-input group of
// the tile, so no partial sums cross waves.  The tile's act block of each
// group (32 rows x 64 inputs, 4 KB) is loaded once per workgroup, one 16-byte
// piece per thread, and staged in LDS in MFMA fragment order, so each wave
// reads its fragments as contiguous 1 KB sweeps; act blocks are requested
// four positions ahead into registers and written to LDS one position ahead
// (three buffers, one LDS-only barrier per position), weights four positions
// ahead straight into registers, and both streams run on across tile
// boundaries.  A tile has a multiple of four positions (at least four); past
// its groups a position reads its last group again with zero scales and is
// not computed.  The MFMA takes the dequantised weights as its first operand
// and the act fragments as its second, so the lane (g16, n16) accumulates
// weight rows 4 g16 .. 4 g16 + 3 of each strip for row n16 of each 16-row
// block: four consecutive output columns of one row, stored as one 8-byte fp16
// slot write (or 16-byte h1 write).
constexpr int DN_BUF = 3;                  // act buffers in LDS
constexpr int DN_ABYTES = DG_MT * 64 * 2;  // one act block: 32 rows x 64 inputs, fp16

template <int WF>
struct DW {        // one wave's weights of one group
  // Q4: words (strip, half) 0..3 and 4..7 of the lane's row of the block;
  // BF16: (strip, half) 2s + h, 8 values each; Q8: strip s, its two halves' 8 codes;
  // Q6: the Q4 words, then the high-plane words of strips 0..3
  uint4 w[WF == WF_BF16 ? 8 : WF == WF_Q8G64 ? 4 : WF == WF_Q6G32 ? 3 : 2];
  uint4 sb[kG32<WF> ? 2 : 1];  // (scale | bias << 16) of strips 0..3 (Q4G32, Q6G32: of
                               // (strip, half) 0..3, 4..7; BF16: unused)
};

struct DSrc {      // where a tile's operands are read
  const uint32_t* codes;
  const uint32_t* sb;
  int blk;         // the wave's 64-row block of W_down (block 0 when inactive)
  bool active;     // the block lies inside N (N may end within the tile)
  int GT;          // 64-input groups of the whole K (the weights' layout)
  int q0, G;       // the tile's groups: q0 .. q0 + G - 1 (a K chunk for dense tiles)
  const _Float16* arow;  // the act row this thread stages (its piece: see d_src)
  float* out;      // h1, or its partial sum for the tile's K chunk (dense)
  float gsc;       // NVFP4: the matrix's tensor scale (else 1)
  int64_t hoff;    // Q6G32: words of the low plane (the high plane follows)
};

// Thread t stages piece t of each act block: row 16 (t / 128) + t % 16,
// inputs 32 ((t / 64) % 2) + 8 ((t / 16) % 4) .. +7 -- the 16 bytes lane t % 64
// of fragment (row block t / 128, half (t / 64) % 2) holds.
template <int WF>
__device__ __forceinline__ DSrc d_src(const GemmPhaseArgs& p, const TileCtx& tc, int w, int tid,
                                      bool live) {
  DSrc r;
  const bool dense = tc.dense;
  const int N = dense ? p.n_d : p.n_e;
  const int K = dense ? p.k_d : p.k_e;
  r.GT = K / 64;
  if (dense) {  // chunk kc of kch_d: groups [kc * Gc, min((kc + 1) * Gc, GT))
    const int gc = (r.GT + p.kch_d - 1) / p.kch_d;
    r.q0 = min(tc.kc * gc, r.GT - 1);
    r.G = max(1, min(gc, r.GT - r.q0));
    r.out = p.h1 + (int64_t)tc.kc * p.dense_rows * N;
  } else {
    r.q0 = 0;
    r.G = r.GT;
    r.out = p.h1;
  }
  const int64_t words_e = WF == WF_Q6G32 ? (int64_t)p.n_e * p.k_e * 3 / 16
                                          : (int64_t)p.n_e * p.k_e / (WF == WF_BF16 ? 2 : WF == WF_Q8G64 ? 4 : 8);
  const int64_t pairs_e = (int64_t)p.n_e * p.k_e / (kG32<WF> ? 32 : 64) + (WF == WF_NVFP4 ? 16 : 0);
  r.hoff = (int64_t)N * K / 8;
  r.codes = dense ? (const uint32_t*)p.w_d : (const uint32_t*)p.w_e + (int64_t)tc.grp * words_e;
  r.sb = dense ? p.sb_d : p.sb_e + (int64_t)tc.grp * pairs_e;
  r.gsc = WF == WF_NVFP4 ? *(const float*)(r.sb + (int64_t)N * K / 64) : 1.0f;
  const int blk = (DG_NDN_Q4 / 64) * tc.nt + w;
  r.active = live && 64 * blk < N;
  r.blk = r.active ? blk : 0;
  const int m = 16 * (tid >> 7) + (tid & 15);
  const int koff = 32 * ((tid >> 6) & 1) + 8 * ((tid >> 4) & 3);
  r.arow = (dense ? p.a_d : p.a_e) + (int64_t)(tc.row_start + (m < tc.rows ? m : 0)) * K + koff;
  return r;
}

// Position q of a tile: its group (q0 + q, or the last group again past G).
__device__ __forceinline__ int d_group(const DSrc& t, int q) { return t.q0 + min(q, t.G - 1); }

// The wave's weights of position q: two 16-byte code loads and one of scales
// (zero scales past the tile's groups or for an inactive block: every product
// of such a position is zero).
template <int WF>
__device__ __forceinline__ void d_wload(DW<WF>& d, const DSrc& t, const uint32_t* zero, int q, int g16,
                                        int n16) {
  const bool on = t.active && q < t.G;
  if (WF == WF_BF16) {  // uniform base + 32-bit lane offset, as in q_load
    const uint32_t K2 = (uint32_t)t.GT * 128;
    const gptr_t base = wave_ptr(on ? (const void*)t.codes : (const void*)zero);
    const uint32_t o0 = on ? ((uint32_t)(64 * t.blk) + n16) * K2 + 128u * d_group(t, q) + 16u * g16 : 0u;
    const uint32_t so = on ? 16u * K2 : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        d.w[WF == WF_BF16 ? 2 * s + h : 0] = gload16(base, o0 + s * so + 64u * h);
    return;
  }
  if (WF == WF_Q8G64) {  // as in q_load
    const uint32_t K1 = (uint32_t)t.GT * 64;
    const int qg = d_group(t, q);
    const gptr_t base = wave_ptr(t.codes);
    const uint32_t o0 = ((uint32_t)(64 * t.blk) + n16) * K1 + 64u * qg + 8u * g16;
    uint32_t sbw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const gu32x2_t c0 = gload8(base, o0 + 16u * s * K1);
      const gu32x2_t c1 = gload8(base, o0 + 16u * s * K1 + 32u);
      d.w[WF == WF_Q8G64 ? s : 0] = make_uint4(c0[0], c0[1], c1[0], c1[1]);
      const int64_t r = 64 * (int64_t)t.blk + 16 * s + n16;
      sbw[s] = *(on ? t.sb + r * t.GT + qg : zero + 4 * n16);
    }
    d.sb[0] = make_uint4(sbw[0], sbw[1], sbw[2], sbw[3]);
    return;
  }
  const int64_t bq = (int64_t)t.blk * t.GT + d_group(t, q);
  const uint4* cw = (const uint4*)(t.codes + ((bq * 4 + g16) * 16 + n16) * 8);
  d.w[0] = cw[0];
  d.w[1] = cw[1];
  if (WF == WF_Q6G32)
    d.w[WF == WF_Q6G32 ? 2 : 0] = *(const uint4*)(t.codes + t.hoff + ((bq * 4 + g16) * 16 + n16) * 4);
  if (kG32<WF>) {
    const uint4* ps = (const uint4*)(on ? t.sb + (bq * 16 + n16) * 8 : zero + 4 * n16);
    d.sb[0] = ps[0];
    d.sb[kG32<WF> ? 1 : 0] = ps[on ? 1 : 0];
  } else {
    d.sb[0] = *(const uint4*)(on ? t.sb + (bq * 16 + n16) * 4 : zero + 4 * n16);
  }
}

__device__ __forceinline__ uint4 d_aload(const DSrc& t, int q) {
  return *(const uint4*)(t.arow + 64 * d_group(t, q));
}

// acc[strip][row block]: lane holds output columns 16 s + 4 g16 + i (i < 4) of
// the block for row 16 rb + n16; af[row block][half] the act fragments
template <int WF>
__device__ __forceinline__ half8_t d_frag(const DW<WF>& d, int s, int h) {
  if (WF == WF_NVFP4) {
    const _Float16 sc = e4m3_half(fp4_scale(d.sb[0], s, h));
    return dequant_fp4_word(u4_get(d.w[s >> 1], 2 * (s & 1) + h), (half2_t){sc, sc});
  }
  if (WF == WF_BF16) return bf16x8_to_half8(d.w[WF == WF_BF16 ? 2 * s + h : 0]);
  if (WF == WF_Q8G64) {
    const uint32_t pr = u4_get(d.sb[0], s);
    const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
    const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
    const uint4 c = d.w[WF == WF_Q8G64 ? s : 0];
    return dequant_q8_pair(h ? c.z : c.x, h ? c.w : c.y, (half2_t){sc, sc}, (half2_t){bi, bi});
  }
  const uint32_t pr = kG32<WF> ? u4_get(d.sb[kG32<WF> ? s >> 1 : 0], 2 * (s & 1) + h)
                                : u4_get(d.sb[0], s);
  const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
  const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
  const uint32_t word = u4_get(d.w[s >> 1], 2 * (s & 1) + h);
  if (WF == WF_Q6G32)
    return dequant_q6_word(word, u4_get(d.w[WF == WF_Q6G32 ? 2 : 0], s) >> (8 * h), (half2_t){sc, sc},
                           (half2_t){bi, bi});
  return dequant_q4_word(word, (half2_t){sc, sc}, (half2_t){bi, bi});
}

template <int WF>
__device__ __forceinline__ void d_compute(const DW<WF>& d, const uint4 (&af)[2][2], float4_t (&acc)[4][2],
                                          bool two) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8_t wv = d_frag(d, s, h);
      acc[s][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, bitcast<half8_t>(af[0][h]), acc[s][0],
                                                         0, 0, 0);
      if (two)
        acc[s][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, bitcast<half8_t>(af[1][h]),
                                                           acc[s][1], 0, 0, 0);
    }
  }
}

// The wave's 64 columns of the tile: four consecutive columns per lane and
// strip, one store each (rows past the tile and inactive blocks write nothing).
// SCALE (NVFP4): the sums are multiplied by the matrix's tensor scale.
template <bool SCALE = false>
__device__ __forceinline__ void d_epilogue(const GemmPhaseArgs& p, const TileCtx& tc, const DSrc& src,
                                           const float4_t (&acc)[4][2], const int (&pair)[2],
                                           int g16, int n16) {
  if (!src.active) return;
  const int N = tc.dense ? p.n_d : p.n_e;
  float big = 0.f;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int m = 16 * rb + n16;
    if (m >= tc.rows) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t col = 64 * (int64_t)src.blk + 16 * s + 4 * g16;
      float4_t v = acc[s][rb];
      if (SCALE)
        for (int u = 0; u < 4; ++u) v[u] = __fmul_rn(v[u], src.gsc);
      if (tc.dense) {
        *(float4*)(src.out + (int64_t)(tc.row_start + m) * N + col) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        big = fmaxf(big, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        const uint32_t lo = (uint32_t)bitcast<uint16_t>((_Float16)v[0]) |
                            ((uint32_t)bitcast<uint16_t>((_Float16)v[1]) << 16);
        const uint32_t hi = (uint32_t)bitcast<uint16_t>((_Float16)v[2]) |
                            ((uint32_t)bitcast<uint16_t>((_Float16)v[3]) << 16);
        *(uint2*)(p.slots + (int64_t)pair[rb] * N + col) = make_uint2(lo, hi);
      }
    }
  }
  if (!(big < DG_F16_LIMIT)) flag_error(p.sync, DG_ERR_RANGE, p.stamp);
}

// A workgroup barrier that orders LDS accesses only: the vector memory loads
// in flight stay in flight.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Persistent: tiles through one work queue per XCD as in q_body (first two
// tiles of a workgroup fixed, later ones claimed two tiles ahead).
struct DLds {
  uint4 a[DN_BUF * DN_ABYTES / 16];
  int next;
};

template <int WF = WF_Q4G64>
__device__ __forceinline__ void d_body(const GemmPhaseArgs& p, DLds& L, const int* s_rows,
                                       const int* s_off, const int* s_tp, int* queue,
                                       int parts = 3) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, n16 = lane & 15;
  const int nwg = (int)(gridDim.x >> 3);
  const Queue<false> qu(p, s_tp, parts);
  int* ctr = queue + qu.x;
  const int j0 = (int)(blockIdx.x >> 3);
  if (j0 >= qu.n) return;

  uint4* sa = L.a;
  auto a_store = [&](const uint4& v, int b) { sa[b * (DN_ABYTES / 16) + tid] = v; };
  auto frag_read = [&](uint4 (&af)[2][2], int b) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) af[rb][h] = sa[b * (DN_ABYTES / 16) + (2 * rb + h) * 64 + lane];
  };

  TileCtx tc = qu.tile(p, j0, s_rows, s_off, s_tp);
  DSrc src = d_src<WF>(p, tc, w, tid, true);
  bool two = tc.rows > 16;
  // staged act blocks (position q in register set q % 4) and the weight ring
  // (position q in slot q % 4), four positions ahead
  uint4 x0 = d_aload(src, 0), x1 = d_aload(src, 1), x2 = d_aload(src, 2), x3 = d_aload(src, 3);
  DW<WF> r0, r1, r2, r3;
  d_wload(r0, src, p.zero, 0, g16, n16);
  d_wload(r1, src, p.zero, 1, g16, n16);
  d_wload(r2, src, p.zero, 2, g16, n16);
  d_wload(r3, src, p.zero, 3, g16, n16);
  a_store(x0, 0);
  lds_sync();
  uint4 af[2][2];  // fragments of the position in hand
  frag_read(af, 0);
  int buf = 0;
  int nxt = 0;
  if (tid == 0) nxt = atomicAdd(ctr, 1);
  int jn = j0 + nwg;

  float4_t acc[4][2];
  // Position q of the tile: act block q + 1 into LDS from its staging set,
  // that set refilled with block q + 4 (of this tile, or of the next tile
  // past this one's positions); a barrier; position q's MFMAs on the
  // fragments read one position earlier (when q is one of the tile's groups);
  // the fragments of block q + 1; the weight slot refilled with position
  // q + 4.  A buffer is rewritten two positions after its fragments were read,
  // and every wave has read them before the barrier in between.
  auto step = [&](DW<WF>& rw, uint4& st, uint4& ld, int q, const DSrc& l, int lq) {
    const int nb = buf == DN_BUF - 1 ? 0 : buf + 1;
    a_store(st, nb);
    ld = d_aload(l, lq);
    lds_sync();
    if (q < src.G) d_compute(rw, af, acc, two);
    frag_read(af, nb);
    d_wload(rw, l, p.zero, lq, g16, n16);
    buf = nb;
  };
  while (true) {
    // requested behind this tile's operands, through the scalar cache: its
    // rows' pair ids (the scatter rows of the epilogue; unused for the dense MLP)
    TileIds pids;
    ids_request(pids, tc.pairs);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s][0] = acc[s][1] = (float4_t){0.f, 0.f, 0.f, 0.f};
    const int G4 = (src.G + 3) & ~3;  // positions of the tile
    int q0 = 0;
    for (; q0 + 4 < G4; q0 += 4) {
      step(r0, x1, x0, q0, src, q0 + 4);
      step(r1, x2, x1, q0 + 1, src, q0 + 5);
      step(r2, x3, x2, q0 + 2, src, q0 + 6);
      step(r3, x0, x3, q0 + 3, src, q0 + 7);
    }
    // the last four positions request the next tile's first ones (after the
    // queue's last tile: a stand-in with zero scales, never computed)
    const bool more = jn < qu.n;
    const TileCtx tn = qu.tile(p, min(jn, qu.n - 1), s_rows, s_off, s_tp);
    const DSrc sn = d_src<WF>(p, tn, w, tid, more);
    step(r0, x1, x0, q0, sn, 0);
    step(r1, x2, x1, q0 + 1, sn, 1);
    step(r2, x3, x2, q0 + 2, sn, 2);
    step(r3, x0, x3, q0 + 3, sn, 3);
    int pair[2];
    ids_lanes(pids, tc.rows, pair[0], pair[1]);
    pair[0] = plan_clamp_id(pair[0], (int)p.pairs);
    pair[1] = plan_clamp_id(pair[1], (int)p.pairs);
    d_epilogue<WF == WF_NVFP4>(p, tc, src, acc, pair, g16, n16);
    if (!more) break;
    if (tid == 0) L.next = nxt;
    lds_sync();
    const int jnn = 2 * nwg + L.next;
    if (tid == 0) nxt = atomicAdd(ctr, 1);
    lds_sync();  // the claim is read before it is written again
    tc = tn;
    src = sn;
    two = tn.rows > 16;
    jn = jnn;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the stream's reads past the last tile (vmcnt(0))
}

// ---------------------------------------------------------------- Q4G64, tall tiles
// With many rows per expert (from about 32 pairs per expert; a batch of
// canvases has about 128 at 2048 positions) the GEMMs turn compute-bound, and
// what limits the short tiles above is the dequantisation per MFMA: a
// dequantised weight fragment feeds only the tile's two 16-row blocks.  Tall tiles: BT_M = 64 rows, and
// each wave owns 64 weight rows for the whole K (gate_up: 32 gate rows and the
// 32 matching up rows, so GeGLU is formed in registers; down: 64 output
// columns), so each fragment feeds four MFMAs.  The four waves share the A
// rows through LDS: per 64-input group the workgroup stages the 64 x 64 fp16
// block in fragment order (16-byte chunk (row block, half, lane group, lane)
// at 16 * chunk), so each fragment read is one contiguous 1 KB sweep of a
// wave.  A blocks are requested four groups ahead into registers, written to
// LDS one group ahead (three buffers, one barrier per group) and read into
// fragments one group ahead; weight groups are requested four ahead straight
// into registers.  Tiles are numbered as for the short tiles (group, column
// tile, row tile) and each XCD's work queue holds a contiguous share of them,
// so the row tiles that share a weight block, and the column tiles that share
// an expert's A rows, meet in one L2.
constexpr int BT_M = 64;     // rows per tile
constexpr int BT_RING = 4;   // weight groups in flight per wave
constexpr int BT_BUF = 3;    // A buffers in LDS
constexpr int BT_ABYTES = BT_M * 64 * 2;  // one A block: 64 rows x 64 inputs, fp16

// Column tiles per row tile: gate_up 128 act columns (two 64-row gate blocks
// and their up blocks), down 256 output columns (four 64-row blocks).
template <bool GATEUP>
__host__ __device__ __forceinline__ int bt_ncol(int N) {
  return GATEUP ? (N / 128 + 1) / 2 : (N / 64 + 3) / 4;
}

struct BtGroup {
  uint4 w[2];  // gate_up: the gate block's, then the up block's four words of the wave's strip pair;
               // down: words 0..3 and 4..7 of the block
  uint4 sb;    // (scale|bias) of the four pseudo-strips j (gate_up: gate 2sh, 2sh+1, up 2sh, 2sh+1)
};

// A tile of the tall GEMMs as one wave and one thread see it (the weight and
// A addresses follow from the group, so little has to stay live for the
// next tile).
struct TallTile {
  int grp;                // expert, or E for the dense MLP
  int blk0, blk1;         // this wave's weight blocks (gate_up: gate and up; down: the block twice)
  int G;                  // 64-input groups
  int rows, row_start, cb;
  bool dense, active;
  bool live;              // a real tile (not the stand-in after a queue's last tile)
  int id0, id1;           // A rows of this thread's two staging chunks
  int pair;               // down, experts: the pair id of tile row tid % 64
};

// Work queue x (x = blockIdx % 8, the workgroup's XCD) holds the x-th eighth
// of all tiles in their numbering (experts, then the dense MLP; each group by
// column tile, then row tile), the eighths cut by work: a tile costs its
// number of 64-input groups (dense down tiles have three times the K of
// expert down tiles).
struct TallQueue {
  int e0, n;
  __device__ TallQueue(const GemmPhaseArgs& p, const int* s_tp) {
    const int x = blockIdx.x & 7;
    const int te = s_tp[p.E], T = s_tp[p.E + 1];
    const int64_t ge = (p.k_e / 64 + 3) & ~3, gd = (p.k_d / 64 + 3) & ~3;
    const int64_t total = (int64_t)te * ge + (int64_t)(T - te) * gd;
    auto cut = [&](int y) -> int {  // first tile at or past work total * y / 8
      if (y <= 0) return 0;
      if (y >= 8) return T;
      const int64_t w = total * y / 8;
      const int64_t t = w <= te * ge ? (w + ge - 1) / ge : te + (w - te * ge + gd - 1) / gd;
      return t < T ? (int)t : T;
    };
    e0 = cut(x);
    n = cut(x + 1) - e0;
  }
};

template <bool GATEUP>
__device__ __forceinline__ TallTile tall_tile(const GemmPhaseArgs& p, const TallQueue& tq, int j,
                                              const int* s_rows, const int* s_off, const int* s_tp,
                                              int w, int n16) {
  const int E = p.E;
  const int t = tq.e0 + j;
  int lo = 0, hi = E + 1;  // last group with s_tp[g] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tp[mid] <= t) lo = mid; else hi = mid;
  }
  const int g = __builtin_amdgcn_readfirstlane(lo);
  const int mts = (__builtin_amdgcn_readfirstlane(s_rows[g]) + BT_M - 1) / BT_M;
  const int local = t - __builtin_amdgcn_readfirstlane(s_tp[g]);
  const int nt = local / mts, mt = local % mts;
  TallTile c;
  c.grp = g;
  c.live = true;
  c.dense = g == E;
  const int rows_g = __builtin_amdgcn_readfirstlane(s_rows[g]);
  c.row_start = (c.dense ? 0 : __builtin_amdgcn_readfirstlane(s_off[g])) + mt * BT_M;
  c.rows = min(BT_M, rows_g - mt * BT_M);
  const int N = c.dense ? p.n_d : p.n_e;
  c.G = (c.dense ? p.k_d : p.k_e) / 64;
  if (GATEUP) {
    const int nblk = N / 128;  // 64-column act blocks
    c.cb = 2 * nt + (w >> 1);
    c.active = c.cb < nblk;
    c.blk0 = c.active ? c.cb : 0;
    c.blk1 = c.active ? nblk + c.cb : 0;
  } else {
    c.cb = 4 * nt + w;
    c.active = c.cb < N / 64;
    c.blk0 = c.blk1 = c.active ? c.cb : 0;
  }
  const int r0 = 16 * (w >> 1) + n16, r1 = r0 + 32;
  const int m0 = r0 < c.rows ? r0 : 0, m1 = r1 < c.rows ? r1 : 0;
  if (GATEUP) {  // rows gathered through the tokens (experts) or the positions (dense)
    const int32_t* ids = c.dense ? p.rowid + mt * BT_M
                                 : p.list + (int64_t)(E + g) * p.list_cap + mt * BT_M;
    c.id0 = plan_clamp_id(ids[m0], (int)p.n_tok);
    c.id1 = plan_clamp_id(ids[m1], (int)p.n_tok);
    c.pair = 0;
  } else {
    c.id0 = c.row_start + m0;
    c.id1 = c.row_start + m1;
    c.pair = c.dense ? 0
                     : plan_clamp_id(p.list[(int64_t)g * p.list_cap + mt * BT_M +
                                            min((int)(threadIdx.x & 63), c.rows - 1)],
                                     (int)p.pairs);
  }
  return c;
}

// Weight group q of a tile (past its groups, or for a tile that is not live:
// zero-scale reads of its last group).  Addresses are a uniform base plus a
// 32-bit byte offset (the host keeps every offset below 2^31).
template <bool GATEUP>
__device__ __forceinline__ void bt_load(BtGroup& d, const uint32_t* codes, const uint32_t* sb,
                                        const uint32_t* zero, int blk0, int blk1, int G, bool live,
                                        int q, int sh, int g16, int n16) {
  const bool on = live && q < G;
  const int qc = min(q, G - 1);
  const uint32_t b0 = (uint32_t)(blk0 * G + qc), b1 = (uint32_t)(blk1 * G + qc);
  const uint32_t lw = (uint32_t)((g16 * 16 + n16) * 8);  // the lane's words within a (block, group)
  const char* cb = (const char*)codes;
  const char* sbb = (const char*)sb;
  const uint4* c0 = (const uint4*)(cb + (b0 * 512u + lw) * 4u);
  const uint4* c1 = (const uint4*)(cb + (b1 * 512u + lw) * 4u);
  if (GATEUP) {
    d.w[0] = c0[sh];
    d.w[1] = c1[sh];
    const uint2 s0 = *(const uint2*)(on ? sbb + ((b0 * 16u + n16) * 4u + 2u * sh) * 4u
                                        : (const char*)(zero + 4 * n16));
    const uint2 s1 = *(const uint2*)(on ? sbb + ((b1 * 16u + n16) * 4u + 2u * sh) * 4u
                                        : (const char*)(zero + 4 * n16));
    d.sb = make_uint4(s0.x, s0.y, s1.x, s1.y);
  } else {
    d.w[0] = c0[0];
    d.w[1] = c0[1];
    d.sb = *(const uint4*)(on ? sbb + (b0 * 16u + n16) * 16u : (const char*)(zero + 4 * n16));
  }
}

// Half h (inputs 32h .. 32h+31) of a group: acc[j][mb], lane holding
// C[m = 16 mb + 4 g16 + i][pseudo-strip j, column n16]
__device__ __forceinline__ void bt_compute(const BtGroup& d, const uint4 (&af)[4][2],
                                           float4_t (&acc)[4][4], int h) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t pr = u4_get(d.sb, j);
    const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
    const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
    const half8_t b = dequant_q4_word(u4_get(d.w[j >> 1], 2 * (j & 1) + h), (half2_t){sc, sc},
                                      (half2_t){bi, bi});
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      acc[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(af[mb][h]), b,
                                                          acc[j][mb], 0, 0, 0);
  }
}

template <bool GATEUP>
__device__ __forceinline__ void bt_epilogue(const GemmPhaseArgs& p, const TallTile& c,
                                            const float4_t (&acc)[4][4], const int* spair, int sh,
                                            int g16, int n16) {
  if (!c.active) return;
  const int N = c.dense ? p.n_d : p.n_e;
  float big = 0.f;
  if (GATEUP) {
    _Float16* dst = (c.dense ? p.act_d : p.act_e) + (int64_t)c.row_start * (N / 2) + 64 * c.cb + 32 * sh;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * mb + 4 * g16 + i;
          if (m < c.rows) {
            const float av = __fmul_rn(gelu_tanh(acc[s2][mb][i]), acc[2 + s2][mb][i]);
            big = fmaxf(big, fabsf(av));
            dst[(int64_t)m * (N / 2) + 16 * s2 + n16] = (_Float16)av;
          }
        }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * mb + 4 * g16 + i;
          if (m >= c.rows) continue;
          const int64_t col = 64 * c.cb + 16 * j + n16;
          if (c.dense) {
            p.h1[(int64_t)(c.row_start + m) * N + col] = acc[j][mb][i];
          } else {
            big = fmaxf(big, fabsf(acc[j][mb][i]));
            p.slots[(int64_t)spair[m] * N + col] = (_Float16)acc[j][mb][i];
          }
        }
  }
  if (!(big < DG_F16_LIMIT)) flag_error(p.sync, DG_ERR_RANGE, p.stamp);
}

// Persistent: the grid walks the tiles through one work queue per XCD (first
// two tiles of a workgroup fixed, each later one claimed a tile ahead), and a
// workgroup's streams of weight groups and A blocks run on across its tile
// boundaries: the last groups of a tile request the next tile's first ones,
// and that tile's first A block is in LDS (its fragments in registers) when
// the tile starts.  A tile's own row ids are read a tile ahead as well.
struct TLds {
  uint4 a[BT_BUF * BT_ABYTES / 16];
  int pair[2 * BT_M];  // down: the pair ids of the current and the next tile
  int claim;
};

template <bool GATEUP>
__device__ __forceinline__ void t_body(const GemmPhaseArgs& p, TLds& L, const int* s_rows,
                                       const int* s_off, const int* s_tp, int* queue) {
  int* s_pair = L.pair;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, n16 = lane & 15;
  const int sh = GATEUP ? (w & 1) : 0;
  const int nwg = (int)(gridDim.x >> 3);
  const TallQueue tq(p, s_tp);
  int* ctr = queue + (blockIdx.x & 7);
  const int j0 = (int)(blockIdx.x >> 3);
  if (j0 >= tq.n) return;

  TallTile c = tall_tile<GATEUP>(p, tq, j0, s_rows, s_off, s_tp, w, n16);
  TallTile n = c;
  n.live = false;
  if (j0 + nwg < tq.n) n = tall_tile<GATEUP>(p, tq, j0 + nwg, s_rows, s_off, s_tp, w, n16);
  int claim = 0;
  if (tid == 0 && n.live) claim = atomicAdd(ctr, 1);

  const int koff = 32 * (w & 1) + 8 * g16;  // the chunk's inputs within a group
  uint4* sa = L.a;
  const int64_t words_e = (int64_t)p.n_e * p.k_e / 8, pairs_e = (int64_t)p.n_e * p.k_e / 64;
  // Where a tile's loads read: this thread's two A rows (at its chunk's
  // inputs) and the wave's weights.
  struct Src {
    const char* abase;
    uint32_t a0, a1;  // byte offsets of this thread's two A rows (at its chunk's inputs)
    const uint32_t* codes;
    const uint32_t* sb;
    int blk0, blk1, G;
    bool live;
  };
  auto src_of = [&](const TallTile& t) {
    Src r;
    const uint32_t K = 64u * (uint32_t)t.G;
    r.abase = (const char*)(t.dense ? p.a_d : p.a_e);
    r.a0 = ((uint32_t)t.id0 * K + koff) * 2u;
    r.a1 = ((uint32_t)t.id1 * K + koff) * 2u;
    r.codes = t.dense ? (const uint32_t*)p.w_d : (const uint32_t*)p.w_e + t.grp * words_e;
    r.sb = t.dense ? p.sb_d : p.sb_e + t.grp * pairs_e;
    r.blk0 = t.blk0;
    r.blk1 = t.blk1;
    r.G = t.G;
    r.live = t.live;
    return r;
  };
  // A block q of a tile into a staging pair (past the tile's groups: its last
  // group again, unused); four pairs, A(q) in pair q % 4, named so they stay
  // in registers
  auto a_load = [&](uint4& d0, uint4& d1, const Src& sr, int q) {
    const uint32_t off = 128u * (uint32_t)min(q, sr.G - 1);
    d0 = *(const uint4*)(sr.abase + (sr.a0 + off));
    d1 = *(const uint4*)(sr.abase + (sr.a1 + off));
  };
  auto a_store = [&](const uint4& d0, const uint4& d1, int b) {
    sa[b * (BT_ABYTES / 16) + tid] = d0;
    sa[b * (BT_ABYTES / 16) + 256 + tid] = d1;
  };
  auto w_load = [&](BtGroup& d, const Src& sr, int q) {
    bt_load<GATEUP>(d, sr.codes, sr.sb, p.zero, sr.blk0, sr.blk1, sr.G, sr.live, q, sh, g16, n16);
  };
  auto frag_read = [&](uint4 (&af)[4][2], int b, int h) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[mb][h] = sa[b * (BT_ABYTES / 16) + (2 * mb + h) * 64 + lane];
  };

  Src sc = src_of(c);
  uint4 x0, x1, y0, y1, z0, z1, u0, u1;
  static_assert(BT_RING == 4, "the weight ring is four named slots");
  BtGroup r0_, r1_, r2_, r3_;  // the weight ring, slot q % BT_RING
  a_load(x0, x1, sc, 0);
  a_load(y0, y1, sc, 1);
  a_load(z0, z1, sc, 2);
  a_load(u0, u1, sc, 3);
  w_load(r0_, sc, 0);
  w_load(r1_, sc, 1);
  w_load(r2_, sc, 2);
  w_load(r3_, sc, 3);
  a_store(x0, x1, 0);
  if (tid < BT_M) s_pair[tid] = c.pair;
  lds_barrier();
  uint4 af[4][2];  // A fragments of the group in hand
  frag_read(af, 0, 0);
  frag_read(af, 0, 1);

  // One stream position q of the current tile: A(q + 1) into LDS from its
  // staging pair, and pair q % 4 (stored one position earlier) refilled with
  // the block four positions on; a barrier; group q's MFMAs half by half on
  // the fragments read one position earlier, each half's fragments of
  // A(q + 1) requested as soon as that half is done (so the LDS reads overlap
  // the MFMAs); the ring slot refilled with the weights four positions on.  Four positions on is group q + 4 of this tile, or, in the
  // tile's last four positions, group q + 4 - G4 of the next tile (every tile
  // has at least four positions, so nothing reaches past the next tile).  A
  // buffer is rewritten two positions after its fragments were read, and
  // every wave has used those before the barrier in between.
  int buf = 0, par = 0;
  float4_t acc[4][4];
  auto step = [&](BtGroup& rs, uint4& s0, uint4& s1, uint4& l0, uint4& l1, int q, const Src& ld,
                  int lq) {
    const int nb = buf == BT_BUF - 1 ? 0 : buf + 1;
    a_store(s0, s1, nb);
    a_load(l0, l1, ld, lq);
    lds_barrier();
    if (!GATEUP && q == 0 && tid < BT_M) s_pair[(par ^ 1) * BT_M + tid] = n.pair;
    if (c.active) bt_compute(rs, af, acc, 0);
    frag_read(af, nb, 0);
    if (c.active) bt_compute(rs, af, acc, 1);
    frag_read(af, nb, 1);
    w_load(rs, ld, lq);
    buf = nb;
  };
  while (true) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[jj][mb] = (float4_t){0.f, 0.f, 0.f, 0.f};
    const int G4 = (c.G + 3) & ~3;  // past G: zero-scale groups
    int q0 = 0;
    for (; q0 + 4 < G4; q0 += 4) {
      step(r0_, y0, y1, x0, x1, q0, sc, q0 + 4);
      step(r1_, z0, z1, y0, y1, q0 + 1, sc, q0 + 5);
      step(r2_, u0, u1, z0, z1, q0 + 2, sc, q0 + 6);
      step(r3_, x0, x1, u0, u1, q0 + 3, sc, q0 + 7);
    }
    const Src sn = src_of(n);  // the last four positions request the next tile's first groups
    step(r0_, y0, y1, x0, x1, q0, sn, 0);
    step(r1_, z0, z1, y0, y1, q0 + 1, sn, 1);
    step(r2_, u0, u1, z0, z1, q0 + 2, sn, 2);
    step(r3_, x0, x1, u0, u1, q0 + 3, sn, 3);
    bt_epilogue<GATEUP>(p, c, acc, s_pair + par * BT_M, sh, g16, n16);
    if (!n.live) break;
    if (tid == 0) L.claim = claim;
    lds_barrier();
    const int jn = 2 * nwg + L.claim;
    c = n;
    sc = sn;
    n.live = false;
    if (jn < tq.n) n = tall_tile<GATEUP>(p, tq, jn, s_rows, s_off, s_tp, w, n16);
    if (tid == 0 && n.live) claim = atomicAdd(ctr, 1);
    par ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the stream's reads past the last tile (vmcnt(0))
}

struct GroupsLds {
  int rows[DG_MAX_GROUPS], off[DG_MAX_GROUPS], tp[DG_MAX_GROUPS + 1], tp2[DG_MAX_GROUPS + 1];
};

template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_tall_q4(GemmPhaseArgs p) {
  __shared__ GroupsLds gl;
  __shared__ TLds L;
  scan_groups<BT_M>(p, gl.rows, gl.off, gl.tp, bt_ncol<GATEUP>(p.n_e), bt_ncol<GATEUP>(p.n_d));
  t_body<GATEUP>(p, L, gl.rows, gl.off, gl.tp, p.queue);
}

// Q4G64: two workgroups per CU (the partial tiles take 66 KB of LDS each), two
// waves per SIMD and their register budget for the three-group ring.
// WF: the weight format (WF_Q4G64, WF_Q4G32 or WF_BF16).
template <bool GATEUP, int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DG_Q4_WPE, DG_Q4_WPE)))
void k_grouped_q4(GemmPhaseArgs p) {
  __shared__ GroupsLds gl;
  __shared__ QLds L;
  scan_groups(p, gl.rows, gl.off, gl.tp, p.nt_e, p.nt_d);
  q_body<GATEUP, WF>(p, L, gl.rows, gl.off, gl.tp, p.queue);
}

template <int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DG_Q4_WPE, DG_Q4_WPE)))
void k_down_q4(GemmPhaseArgs p) {
  __shared__ GroupsLds gl;
  __shared__ DLds L;
  scan_groups(p, gl.rows, gl.off, gl.tp, p.nt_e, p.nt_d);
  d_body<WF>(p, L, gl.rows, gl.off, gl.tp, p.queue);
}

// The experts in one format and the dense MLP in another, one launch: the
// dense MLP's tiles first, through their own eight queue counters (its tiles
// are the longest, so they are taken first), then the experts' tiles; the
// workgroups that find the dense queue empty go straight to the experts.
template <bool GATEUP, int WFE, int WFD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DG_Q4_WPE, DG_Q4_WPE)))
void k_split_q4(GemmPhaseArgs p) {
  __shared__ GroupsLds gl;
  __shared__ typename std::conditional<GATEUP, QLds, DLds>::type L;
  scan_groups(p, gl.rows, gl.off, gl.tp, p.nt_e, p.nt_d);
  if constexpr (GATEUP) {
    q_body<true, WFD>(p, L, gl.rows, gl.off, gl.tp, p.queue + 32, 1);
    __syncthreads();
    q_body<true, WFE>(p, L, gl.rows, gl.off, gl.tp, p.queue, 2);
  } else {
    d_body<WFD>(p, L, gl.rows, gl.off, gl.tp, p.queue + 32, 1);
    __syncthreads();
    d_body<WFE>(p, L, gl.rows, gl.off, gl.tp, p.queue, 2);
  }
}

union MixGuLds {
  TLds t;
  QLds q;
};
union MixDnLds {
  TLds t;
  DLds d;
};

// Short and tall tiles in one launch, the tile height chosen per expert from
// its pair count: experts with at least p.tall_min pairs take the tall tiles
// (first, through their own eight queue counters), the other experts and the
// dense MLP the short ones.  One scan gives both tile tables; the two bodies'
// LDS overlay each other (a barrier between them).
template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DG_Q4_WPE, DG_Q4_WPE)))
void k_mixed_q4(GemmPhaseArgs p) {
  __shared__ GroupsLds gl;
  __shared__ typename std::conditional<GATEUP, MixGuLds, MixDnLds>::type L;
  scan_groups<DG_MT, true, BT_M>(p, gl.rows, gl.off, gl.tp, p.nt_e, p.nt_d, gl.tp2, p.tall_min,
                                 bt_ncol<GATEUP>(p.n_e));
  t_body<GATEUP>(p, L.t, gl.rows, gl.off, gl.tp2, p.queue + 16);
  __syncthreads();
  if constexpr (GATEUP) q_body<true>(p, L.q, gl.rows, gl.off, gl.tp, p.queue);
  else d_body(p, L.d, gl.rows, gl.off, gl.tp, p.queue);
}


template <bool GATEUP>
hipError_t launch_phase(const GemmPhaseArgs& a, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  // the launch's format: the experts' (the dense MLP, when it is in the same
  // launch, has the same one, or is BF16 beside Q4 experts on short tiles:
  // k_split_q4; checked on the host), or the dense MLP's alone
  const int fmt = a.skip_e ? a.wfmt_d : a.wfmt_e;
  if (!a.skip_e && a.dense_rows > 0 && a.wfmt_e != a.wfmt_d) {
    const bool bf = a.wfmt_d == DGMOE_BF16;
    if ((!bf && a.wfmt_d != DGMOE_Q8G64) ||
        (fmt != DGMOE_Q4G64 && fmt != DGMOE_Q4G32 && fmt != DGMOE_NVFP4 && fmt != DGMOE_Q6G32) ||
        a.tall || a.tall_min > 0)
      return hipErrorInvalidValue;
    int grid = (a.max_tiles + 7) / 8 * 8;
    grid = std::max(8, std::min(grid, 256 * DG_Q4_WPE));
    const dim3 g(grid), b(256);
    if (fmt == DGMOE_Q4G64 && bf) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q4G64, WF_BF16>), g, b, 0, st, a);
    else if (fmt == DGMOE_Q4G64) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q4G64, WF_Q8G64>), g, b, 0, st, a);
    else if (fmt == DGMOE_Q4G32 && bf) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q4G32, WF_BF16>), g, b, 0, st, a);
    else if (fmt == DGMOE_Q4G32) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q4G32, WF_Q8G64>), g, b, 0, st, a);
    else if (fmt == DGMOE_NVFP4 && bf) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_NVFP4, WF_BF16>), g, b, 0, st, a);
    else if (fmt == DGMOE_NVFP4) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_NVFP4, WF_Q8G64>), g, b, 0, st, a);
    else if (bf) hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q6G32, WF_BF16>), g, b, 0, st, a);
    else hipLaunchKernelGGL((k_split_q4<GATEUP, WF_Q6G32, WF_Q8G64>), g, b, 0, st, a);
    return hipGetLastError();
  }
  const bool q4 = fmt == DGMOE_Q4G64, g32 = fmt == DGMOE_Q4G32, q8 = fmt == DGMOE_Q8G64;
  const bool f4 = fmt == DGMOE_NVFP4, q6 = fmt == DGMOE_Q6G32;
  if (q4 && a.tall) {  // persistent: up to two workgroups per CU, none idle from the start
    const int64_t mt_e = (a.pairs + BT_M - 1) / BT_M + a.E, mt_d = (a.dense_rows + BT_M - 1) / BT_M;
    const int64_t tiles = mt_e * bt_ncol<GATEUP>(a.n_e) + mt_d * bt_ncol<GATEUP>(a.n_d);
    const int64_t grid = std::min<int64_t>(256 * 2, std::max<int64_t>(8, (tiles + 7) / 8 * 8));
    hipLaunchKernelGGL((k_tall_q4<GATEUP>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (!q4 && (a.tall || a.tall_min > 0)) return hipErrorInvalidValue;  // Q4G64 only
  int grid = (a.max_tiles + 7) / 8 * 8;
  const int cap = 256 * DG_Q4_WPE;  // resident workgroups
  if (grid > cap) grid = cap;
  if (grid < 8) grid = 8;
  dim3 g(grid), b(256);
  if (q4 && a.tall_min > 0) hipLaunchKernelGGL((k_mixed_q4<GATEUP>), g, b, 0, st, a);
  else if (q4 && GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_Q4G64>), g, b, 0, st, a);
  else if (g32 && GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_Q4G32>), g, b, 0, st, a);
  else if (q8 && GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_Q8G64>), g, b, 0, st, a);
  else if (f4 && GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_NVFP4>), g, b, 0, st, a);
  else if (q6 && GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_Q6G32>), g, b, 0, st, a);
  else if (GATEUP) hipLaunchKernelGGL((k_grouped_q4<true, WF_BF16>), g, b, 0, st, a);
  else if (q4) hipLaunchKernelGGL((k_down_q4<WF_Q4G64>), g, b, 0, st, a);
  else if (g32) hipLaunchKernelGGL((k_down_q4<WF_Q4G32>), g, b, 0, st, a);
  else if (q8) hipLaunchKernelGGL((k_down_q4<WF_Q8G64>), g, b, 0, st, a);
  else if (f4) hipLaunchKernelGGL((k_down_q4<WF_NVFP4>), g, b, 0, st, a);
  else if (q6) hipLaunchKernelGGL((k_down_q4<WF_Q6G32>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_down_q4<WF_BF16>), g, b, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<true>(a, st); }
hipError_t launch_down(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<false>(a, st); }
