// Grouped GEMM phases of the block: gate_up + GeGLU, and down + weighted
// scatter.  One kernel body serves the experts and the dense MLP: group g < E
// is expert g, whose rows are the (token, slot) pairs routed to it (its pair
// list); group E is the always-on dense MLP, whose rows
// are the canvas positions (the diffgemma contract's MoE-order bullet: the
// dense MLP runs in parallel as the always-on path; the ML@Berkeley post's
// MOEBlock iterates over experts and gathers their tokens).
//
// Work tile: up to DG_MT = 32 rows x 128 weight rows (gate_up: 64 gate rows
// and the 64 matching up rows, so GeGLU fuses into the epilogue; down: 128
// output columns).  Four waves, each owning two 16-row weight strips.  The K
// loop runs in stages of 256 inputs (four 64-input quantisation groups):
//   * the workgroup stages the tile's A rows (fp16, gathered through the
//     expert's pair list) for the stage in LDS, double-buffered, so the four waves
//     share one copy;
//   * each lane loads the packed weights it feeds to the matrix core straight
//     from HBM into registers, one stage ahead of use: lane (g = l/16, n = l%16)
//     holds group g of the stage for weight row n (32 bytes of Q4G64 codes plus
//     its fp16 scale and bias);
//   * it dequantises them in registers (magic-number nibble expansion and one
//     packed fp16 fma per two weights, the value RNE(scale*q + bias)) and feeds
//     MFMA 16x16x32 f16 with fp32 accumulation.  MFMA step j of a stage takes
//     inputs 64g + 8j .. 64g + 8j + 7 in lane group g; the A fragments follow
//     the same order, so each accumulator is the plain dot product.
// Tiles: expert g has ceil(rows/DG_MT) row tiles times its column tiles,
// numbered by expert, column tile, row tile; the dense MLP likewise.
// Each workgroup derives the numbering itself from the per-expert pair counts
// (an exclusive scan in LDS), and an expert's rows are the pairs the router
// listed for it; its act rows start at the sum of the earlier experts' counts.
// A persistent grid walks the tiles through one work queue per XCD, so that
// tiles sharing an expert's A rows or a weight strip run under the same L2.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int KS = 256;        // inputs per stage
constexpr int LDA = KS + 8;    // LDS row stride (halves), padded against bank conflicts
constexpr int EG_LD = 2 * DG_NGU + 2;  // epilogue row stride (floats): gate/up pairs, padded
static_assert(DG_MT * EG_LD * 4 <= 2 * DG_MT * LDA * 2, "the GeGLU epilogue reuses the A buffers");

template <int WFMT>
struct WStage;

template <>
struct WStage<DGMOE_Q4G64> {
  uint4 w[2][2];    // [strip][16-byte half]: the 64 inputs of one group of one row
  uint32_t sb[2];   // fp16 scale | fp16 bias << 16 (0 for an idle lane)
};

template <>
struct WStage<DGMOE_BF16> {
  uint4 w[2][8];       // [strip][8 inputs]
  bool on[2];
};

// Branch-free: every lane loads from a valid address (row 0 / group 0 when
// idle) so that the loads stay in straight-line code and the compiler's
// wait-count tracking keeps the next stage in flight; idle lanes are zeroed
// where the values are used.
// Q4G64 (tiled): the chunk of (row 16*strip + n, group q) starts at chunk index
// (strip * groups + q) * 16 + n: 32 bytes of codes and one (scale|bias) word,
// so one wave's 16 rows x 4 groups of a stage are 2 KB of contiguous codes and
// 256 contiguous bytes of scale_bias.  BF16 stays row-major.
// Branch-free: every lane loads from a valid address (row 0 / group 0 when
// idle) so that the loads stay in straight-line code and the compiler's
// wait-count tracking keeps the next stages in flight; idle lanes are zeroed
// where the values are used.
template <int WFMT>
__device__ __forceinline__ void load_stage(WStage<WFMT>& ws, const void* W, const uint32_t* SB,
                                           const int64_t* row, const bool* sok, int K, int grp,
                                           bool active) {
  const int gq = active ? grp : 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const bool on = active && sok[s];
    const int64_t r = sok[s] ? row[s] : (row[s] & 15);  // a row of strip 0 when idle
    if constexpr (WFMT == DGMOE_Q4G64) {
      const int64_t c = ((r >> 4) * (K / 64) + gq) * 16 + (r & 15);
      const uint4* p = (const uint4*)W + c * 2;
      ws.w[s][0] = p[0];
      ws.w[s][1] = p[1];
      const uint32_t sb = SB[c];
      ws.sb[s] = on ? sb : 0u;
    } else {
      const uint4* p = (const uint4*)((const uint16_t*)W + r * K + gq * 64);
#pragma unroll
      for (int j = 0; j < 8; ++j) ws.w[s][j] = p[j];
      ws.on[s] = on;
    }
  }
}

template <int WFMT>
__device__ __forceinline__ half8_t stage_b(const WStage<WFMT>& ws, int s, int j) {
  if constexpr (WFMT == DGMOE_Q4G64) {
    const uint4 q = ws.w[s][j >> 2];
    const uint32_t word = (j & 3) == 0 ? q.x : (j & 3) == 1 ? q.y : (j & 3) == 2 ? q.z : q.w;
    const _Float16 sc = bitcast<_Float16>((uint16_t)(ws.sb[s] & 0xFFFFu));
    const _Float16 bi = bitcast<_Float16>((uint16_t)(ws.sb[s] >> 16));
    return dequant_q4_word(word, (half2_t){sc, sc}, (half2_t){bi, bi});
  } else {
    const half8_t zero = {};
    const half8_t v = bf16x8_to_half8(ws.w[s][j]);
    return ws.on[s] ? v : zero;
  }
}

struct AChunk {  // one thread's four 16-byte chunks of A for one stage
  uint4 v0, v1, v2, v3;
};

struct TileCtx {
  int grp, row_start, rows, nt;
  bool dense;
  const int32_t* pairs;  // experts: the tile's pairs (t*k + j), one per row
};

template <int WFMT, bool GATEUP>
__device__ __forceinline__ void run_tile(const GemmPhaseArgs& p, const TileCtx& tc,
                                         _Float16 (*lds)[DG_MT][LDA]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, n16 = lane & 15;
  const bool dense = tc.dense;
  const int N = dense ? p.n_d : p.n_e;
  const int K = dense ? p.k_d : p.k_e;
  const int64_t ebytes = (WFMT == DGMOE_Q4G64) ? (int64_t)p.n_e * p.k_e / 2
                                               : (int64_t)p.n_e * p.k_e * 2;
  const void* W = dense ? p.w_d : (const void*)((const uint8_t*)p.w_e + (int64_t)tc.grp * ebytes);
  const int64_t sbo = (int64_t)tc.grp * p.n_e * (p.k_e / 64);
  const uint32_t* SB = dense ? p.sb_d : (p.sb_e ? p.sb_e + sbo : nullptr);

  // the two 16-row weight strips of this wave
  int64_t srow[2];
  bool sok[2];
  if (GATEUP) {
    const int c0 = tc.nt * DG_NGU + 16 * wave;
    srow[0] = c0 + n16;
    srow[1] = N / 2 + c0 + n16;
    sok[0] = sok[1] = true;
  } else {
    const int n0 = tc.nt * DG_NDN + 32 * wave;
    srow[0] = n0 + n16;
    srow[1] = n0 + 16 + n16;
    sok[0] = n0 < N;
    sok[1] = n0 + 16 < N;
  }

  // A rows this thread stages: row tid/8, and the 16-byte chunks (tid%8) + 8i
  // (i = 0..3) of each 256-input stage, so that the eight threads of a row
  // write neighbouring chunks (no LDS bank conflicts).  Rows past the tile
  // stage row 0 again (their outputs are dropped).
  const int ar = tid >> 3, ac = tid & 7;
  const int arow = ar < tc.rows ? ar : 0;
  int64_t r;
  if (dense) r = tc.row_start + arow;
  else if (GATEUP) r = tc.pairs[arow] / p.topk;               // token of the pair
  else r = tc.row_start + arow;                                // expert-sorted act row
  const _Float16* asrc = (dense ? p.a_d : p.a_e) + r * K;
  const int ngroups = K / 64;
  const int nstages = (ngroups + 3) / 4;
  const bool two = tc.rows > 16;

  float4_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[mb][s] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // chunk c of stage st, clamped to chunk 0 past the stage's valid groups
  // (the clamped copies land in columns that only idle lanes read, as zeros)
  auto a_load = [&](int st) {
    const int valid = 8 * min(4, ngroups - 4 * st);
    const _Float16* base = asrc + (int64_t)st * KS;
    AChunk r;
    r.v0 = *(const uint4*)(base + 8 * (ac < valid ? ac : 0));
    r.v1 = *(const uint4*)(base + 8 * (ac + 8 < valid ? ac + 8 : 0));
    r.v2 = *(const uint4*)(base + 8 * (ac + 16 < valid ? ac + 16 : 0));
    r.v3 = *(const uint4*)(base + 8 * (ac + 24 < valid ? ac + 24 : 0));
    return r;
  };
  auto a_store = [&](int buf, const AChunk& v) {
    *(uint4*)&lds[buf][ar][8 * ac] = v.v0;
    *(uint4*)&lds[buf][ar][8 * (ac + 8)] = v.v1;
    *(uint4*)&lds[buf][ar][8 * (ac + 16)] = v.v2;
    *(uint4*)&lds[buf][ar][8 * (ac + 24)] = v.v3;
  };
  auto compute = [&](int st, const WStage<WFMT>& wc, bool partial) {
    const int buf = st & 1;
    const bool lane_on = g16 < min(4, ngroups - 4 * st);
    if (!sok[0]) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const half8_t b0 = stage_b<WFMT>(wc, 0, j);
      const half8_t b1 = stage_b<WFMT>(wc, 1, j);
      const half8_t zero = {};
      half8_t a0 = *(const half8_t*)&lds[buf][n16][64 * g16 + 8 * j];
      if (partial && !lane_on) a0 = zero;
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[0][0], 0, 0, 0);
      if (sok[1]) acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b1, acc[0][1], 0, 0, 0);
      if (two) {
        half8_t a1 = *(const half8_t*)&lds[buf][16 + n16][64 * g16 + 8 * j];
        if (partial && !lane_on) a1 = zero;
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b0, acc[1][0], 0, 0, 0);
        if (sok[1]) acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[1][1], 0, 0, 0);
      }
    }
  };

  // Weights and A both run two stages ahead of the math: the weights in a ring
  // of three register sets; A in one register set that is written to the LDS
  // double buffer at the start of the stage before its use (that buffer was
  // last read in the previous stage, which the barrier closed).  A stage that
  // does not exist is "loaded" from valid addresses (group 0 of the lane's
  // rows with zeroed scales for weights, the last stage for A) so the code
  // stays straight-line.
  WStage<WFMT> wcur, wnext, wnext2;
  load_stage<WFMT>(wcur, W, SB, srow, sok, K, g16, g16 < ngroups);
  const int g1 = min(4, ngroups - 4);
  load_stage<WFMT>(wnext, W, SB, srow, sok, K, g1 > 0 ? 4 + g16 : 0, g16 < g1);
  a_store(0, a_load(0));
  AChunk anext = a_load(min(1, nstages - 1));
  __syncthreads();

  // every stage but the last holds four full groups
  for (int st = 0; st + 1 < nstages; ++st) {
    a_store((st + 1) & 1, anext);                              // A of the next stage
    anext = a_load(min(st + 2, nstages - 1));                  // A two stages on ...
    const int g2 = min(4, ngroups - 4 * (st + 2));
    load_stage<WFMT>(wnext2, W, SB, srow, sok, K, g2 > 0 ? 4 * (st + 2) + g16 : 0,
                     g16 < g2);                                 // ... and the weights
    compute(st, wcur, false);
    __syncthreads();
    wcur = wnext;
    wnext = wnext2;
  }
  if (ngroups % 4 == 0) compute(nstages - 1, wcur, false);
  else compute(nstages - 1, wcur, true);
  __syncthreads();  // the A buffers are free: the epilogue reuses them

  if (GATEUP) {
    // GeGLU through LDS: lane (g16, n16) of wave w holds gate and up of row
    // m = 16 mb + 4 g16 + i, column 16 w + n16; they go to LDS, and one loop
    // (not unrolled, so every element runs the same instructions and a row's
    // result does not depend on its place in the tile) writes act rows of 64
    // contiguous fp16.
    float* eg = reinterpret_cast<float*>(&lds[0][0][0]);  // [DG_MT][EG_LD]: (gate, up) pairs
    const int c = 16 * wave + n16;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb == 1 && !two) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mb * 16 + 4 * g16 + i;
        eg[m * EG_LD + 2 * c] = acc[mb][0][i];
        eg[m * EG_LD + 2 * c + 1] = acc[mb][1][i];
      }
    }
    __syncthreads();
    _Float16* dst = (dense ? p.act_d : p.act_e) + (int64_t)tc.row_start * (N / 2) + tc.nt * DG_NGU;
#pragma unroll 1
    for (int e = tid; e < tc.rows * DG_NGU; e += 256) {
      const int m = e / DG_NGU, cc = e % DG_NGU;
      const float gv = eg[m * EG_LD + 2 * cc], uv = eg[m * EG_LD + 2 * cc + 1];
      dst[(int64_t)m * (N / 2) + cc] = (_Float16)__fmul_rn(gelu_tanh(gv), uv);
    }
    __syncthreads();  // LDS is free for the next tile
    return;
  }

  if (!sok[0]) return;
  // down epilogue: lane holds C[m = 16 mb + 4 g16 + i][n = n16] of each strip;
  // one rounded multiply per element, the same in every position
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb == 1 && !two) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mb * 16 + 4 * g16 + i;
      if (m >= tc.rows) continue;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!sok[s]) continue;
        const int64_t col = srow[s];
        const float y = acc[mb][s][i];
        if (dense) {
          p.h1[(int64_t)(tc.row_start + m) * N + col] = y;
        } else {
          const int pair = tc.pairs[m];
          p.slots[(int64_t)pair * N + col] = __fmul_rn(p.route_w[pair], y);
        }
      }
    }
  }
}

// Group sizes of this launch, from the per-expert pair counts: s_rows[g],
// s_off[g] (first act row of expert g) and s_tp[g] (first tile of group g),
// s_tp[E + 1] = number of tiles.  Wave 0 scans, five groups per lane.
constexpr int DG_GPL = 5;  // 5 * 64 >= 257 groups

__device__ __forceinline__ void scan_groups(const GemmPhaseArgs& p, int* s_rows, int* s_off,
                                            int* s_tp) {
  const int lane = threadIdx.x & 63;
  const int E = p.E, nt_e = p.nt_e, nt_d = p.nt_d, dense_rows = p.dense_rows;
  if (threadIdx.x < 64) {
    int rows[DG_GPL], nt[DG_GPL];
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i)  // every count requested before the first is used
      rows[i] = p.cnt[min(DG_GPL * lane + i, E - 1)];
    int sr = 0, st = 0;
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i) {
      const int g = DG_GPL * lane + i;
      rows[i] = g < E ? rows[i] : (g == E ? dense_rows : 0);
      const int ntg = g < E ? nt_e : nt_d;
      nt[i] = g <= E ? (rows[i] + DG_MT - 1) / DG_MT * ntg : 0;
      sr += g < E ? rows[i] : 0;
      st += nt[i];
    }
    int ir = sr, it = st;  // inclusive scans over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tr = __shfl_up(ir, o, 64), tt = __shfl_up(it, o, 64);
      if (lane >= o) { ir += tr; it += tt; }
    }
    int r0 = ir - sr, t0 = it - st;
#pragma unroll
    for (int i = 0; i < DG_GPL; ++i) {
      const int g = DG_GPL * lane + i;
      if (g <= E) {
        s_rows[g] = rows[i];
        s_off[g] = g < E ? r0 : 0;
        s_tp[g] = t0;
        if (g == E) s_tp[g + 1] = t0 + nt[i];
      }
      r0 += g < E ? rows[i] : 0;
      t0 += nt[i];
    }
  }
  __syncthreads();
}

// Work queues: queue x (x = blockIdx % 8, the workgroup's XCD) holds the
// dense tiles of column tiles x, x+8, ... (all their row tiles) followed by
// the x-th eighth of the expert tiles, so every XCD gets the same share of
// dense and expert work and the tiles of one expert stay under one L2.
// A workgroup's first tile is fixed (its rank among the workgroups of its
// queue); after that it takes the next tile with an integer atomic on the
// queue's counter, issued when a tile starts and read when it ends, so the
// claim's latency is hidden and the claims of a queue are spread over time.
// Every workgroup leaves once its queue is empty.
template <int WFMT_E, int WFMT_D, bool GATEUP>
__device__ __forceinline__ void grouped_body(const GemmPhaseArgs& p) {
  __shared__ _Float16 lds[2][DG_MT][LDA];
  __shared__ int s_rows[DG_MAX_GROUPS], s_off[DG_MAX_GROUPS], s_tp[DG_MAX_GROUPS + 1];
  __shared__ int s_next;
  const int x = blockIdx.x & 7;
  const int nwg = (int)(gridDim.x >> 3);  // workgroups per queue (the grid is a multiple of 8)
  int* ctr = p.queue + x;
  scan_groups(p, s_rows, s_off, s_tp);
  const int E = p.E;
  const int te = s_tp[E];  // expert tiles (dense tiles are counted here)
  const int e0 = (int)((int64_t)te * x / 8), e1 = (int)((int64_t)te * (x + 1) / 8);
  const int mts_d = (p.dense_rows + DG_MT - 1) / DG_MT;
  const int ncol = p.nt_d > x ? (p.nt_d - x + 7) / 8 : 0;
  const int nd = mts_d * ncol;
  const int n = nd + (e1 - e0);
  int j = (int)(blockIdx.x >> 3);
  while (j < n) {
    int nxt = 0;
    if (threadIdx.x == 0) nxt = nwg + atomicAdd(ctr, 1);
    if (j < nd) {
      const int mt = j % mts_d;
      TileCtx tc{E, mt * DG_MT, min(DG_MT, p.dense_rows - mt * DG_MT), x + 8 * (j / mts_d), true,
                 nullptr};
      run_tile<WFMT_D, GATEUP>(p, tc, lds);
    } else {
      const int t = e0 + (j - nd);
      int lo = 0, hi = E;  // last expert with s_tp[g] <= t
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
      TileCtx tc{g, off + mt * DG_MT, min(DG_MT, rows - mt * DG_MT), nt, false,
                 p.list + (int64_t)g * p.list_cap + mt * DG_MT};
      run_tile<WFMT_E, GATEUP>(p, tc, lds);
    }
    if (threadIdx.x == 0) s_next = nxt;
    __syncthreads();
    j = s_next;
  }
}

// All-Q4G64 weights: the register budget of three waves per SIMD holds the
// three-deep weight ring without spilling.
template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 4)))
void k_grouped_q4(GemmPhaseArgs p) {
  grouped_body<DGMOE_Q4G64, DGMOE_Q4G64, GATEUP>(p);
}

template <int WFMT_E, int WFMT_D, bool GATEUP>
__global__ __launch_bounds__(256) void k_grouped(GemmPhaseArgs p) {
  grouped_body<WFMT_E, WFMT_D, GATEUP>(p);
}

template <bool GATEUP>
hipError_t launch_phase(const GemmPhaseArgs& a, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  int grid = (a.max_tiles + 7) / 8 * 8;
  const int cap = 256 * 3;  // three resident workgroups per CU
  if (grid > cap) grid = cap;
  if (grid < 8) grid = 8;
  dim3 g(grid), b(256);
  const bool eq = a.wfmt_e == DGMOE_Q4G64, dq = a.wfmt_d == DGMOE_Q4G64;
  if (eq && dq) hipLaunchKernelGGL((k_grouped_q4<GATEUP>), g, b, 0, st, a);
  else if (eq) hipLaunchKernelGGL((k_grouped<DGMOE_Q4G64, DGMOE_BF16, GATEUP>), g, b, 0, st, a);
  else if (dq) hipLaunchKernelGGL((k_grouped<DGMOE_BF16, DGMOE_Q4G64, GATEUP>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_grouped<DGMOE_BF16, DGMOE_BF16, GATEUP>), g, b, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<true>(a, st); }
hipError_t launch_down(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<false>(a, st); }
