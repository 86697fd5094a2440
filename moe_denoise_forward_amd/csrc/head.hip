// The tied embedding table E [V, D] (Q4G64) at both ends of a denoising
// forward: the forward tail after the last decoder layer, and the soft
// embedding and canvas input of self-conditioning before the first (the
// diffgemma contract, Part II section 4 "Denoise step" items 1 and 3, section
// 5 "Self-conditioning (SC)", section 6 "Sampler" item 2; "DiffusionGemma
// Explained", "Complete DiffusionGemma model" and "Logit Softcapping").
//
// Tail.  The head is the GEMM [L, D] x [D, V] against the table read as V rows
// of D inputs, the table's own orientation.  It is bound by the matrix cores
// (2 L D V flops against D V / 2 bytes of codes, ~900 flops per byte at
// L = 256), so a tile holds every row of a canvas (up to 256) and each
// dequantised weight feeds all of them.  A tile is up to 256 rows x 256
// vocabulary rows; wave w owns table block 4 c + w (64 vocabulary rows) over
// the whole K = D:
//   * per 64-input group a lane loads its 32 contiguous bytes of the block's
//     codes and its four (scale | bias) words (three groups in flight),
//     dequantises them in registers and feeds MFMA 16x16x32 f16 against every
//     16-row block of A, fp32 accumulation;
//   * the A rows of a group (up to 256 x 64 fp16) go through LDS in MFMA
//     fragment order (three buffers, one barrier per group), requested two
//     groups ahead.
// Epilogue in registers: y = softcap(z) / T, and for every row the tile's max,
// lowest argmax, sum exp(y - m) and sum exp(y - m)(y - m) -- DPP within rows of
// 16 lanes, then the four waves in order through LDS.  The logits are written
// only when the caller asks for them.  A merge over the tiles gives the row
// statistics; the logits matrix itself never has to exist.
//
// Soft embedding.  soft = softmax(y) E sqrt(D) contracts over the vocabulary,
// the table's row dimension: K = V is large and the output [L, D] small, so
// the sum over V is split into pieces.  Per (row, piece) the probabilities are
// stored once as fp16 2^14 exp(y - m_piece) (values in (0, 2^14], the tail of
// the row far above the fp16 subnormals) with the piece's max and sum.  A
// workgroup takes one piece, one 256-row tile and 256 columns of D; per 64-row
// block of the table it dequantises the block's four groups (a wave each) into
// LDS transposed to [d][v], stages the probabilities [256 rows x 64] in
// fragment order, and each wave runs 128 MFMAs on a 128 x 128 corner of the
// output; loads run two blocks ahead, LDS is double-buffered.  The partial
// sums are rescaled to the row's max and added in piece order by the reduce.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 30 tanh(z / 30) / T, as (30 - 60 / (1 + exp(z / 15))) / T with the hardware
// exp2 and reciprocal; it saturates through inf / 0 to +-30 / T.
__device__ __forceinline__ float softcap_t(float z, float inv_t) {
  const float e = __builtin_amdgcn_exp2f(z * (LOG2E / 15.0f));
  return (30.0f - 60.0f * __builtin_amdgcn_rcpf(1.0f + e)) * inv_t;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, bitcast<float>(dpp32<0xB1>(bitcast<uint32_t>(v))));
  v = fmaxf(v, bitcast<float>(dpp32<0x4E>(bitcast<uint32_t>(v))));
  v = fmaxf(v, bitcast<float>(dpp32<0x141>(bitcast<uint32_t>(v))));
  v = fmaxf(v, bitcast<float>(dpp32<0x140>(bitcast<uint32_t>(v))));
  return v;
}

// Largest value and its lowest index within each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = bitcast<float>(dpp32<CTRL>(bitcast<uint32_t>(v)));
  const int oi = (int)dpp32<CTRL>((uint32_t)i);
  const bool take = ov > v || (ov == v && oi < i);
  v = take ? ov : v;
  i = take ? oi : i;
}
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_step<0xB1>(v, i);
  argmax_step<0x4E>(v, i);
  argmax_step<0x141>(v, i);
  argmax_step<0x140>(v, i);
}

// Softmax statistics of a set of columns: m its largest y, l = sum exp(y - m),
// s = sum exp(y - m) (y - m), best the lowest column holding m; l == 0 marks
// the empty set.  Merging two disjoint sets rescales both to the larger max.
// The merge is symmetric bit for bit (products and sums commute), so a
// butterfly leaves the same result in every lane.
struct RowStat {
  float m, l, s;
  int best;
};
__device__ __forceinline__ RowStat stat_merge(RowStat a, RowStat b) {
  if (b.l == 0.f) return a;
  if (a.l == 0.f) return b;
  const float m = fmaxf(a.m, b.m);
  const float da = a.m - m, db = b.m - m;
  const float ea = __builtin_amdgcn_exp2f(da * LOG2E), eb = __builtin_amdgcn_exp2f(db * LOG2E);
  RowStat r;
  r.m = m;
  r.l = a.l * ea + b.l * eb;
  r.s = (a.s + a.l * da) * ea + (b.s + b.l * db) * eb;
  r.best = (b.m > a.m || (b.m == a.m && b.best < a.best)) ? b.best : a.best;
  return r;
}

// ================================================================ tail
constexpr int LH_RING = 3;  // weight groups in flight per wave
constexpr int LH_BUF = 3;   // A buffers in LDS (== LH_RING: the unrolled loop indexes both statically)

struct LhGroup {
  uint4 w[2];  // the lane's words 2 s + h of one group: w[0] strips 0-1, w[1] strips 2-3
  uint4 sb;    // (scale | bias << 16) of strips 0..3 (table rows 16 s + lane % 16)
};

// A tile is 16 MB RH rows x 256 vocabulary rows, 4 RH waves: wave w owns
// table block 4 c + w % 4 for rows 16 MB (w / 4) .. +16 MB - 1, so two waves
// run on each SIMD (RH = 2: one workgroup of eight waves per CU; RH = 1: two
// workgroups) and one wave's waits overlap the other's MFMAs.
template <int MB, int RH>
__global__ __launch_bounds__(256 * RH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_lmhead_q4(TailArgs a) {
  constexpr int NT = 256 * RH;
  constexpr int ROWS = 16 * MB * RH;
  constexpr int ABYTES = ROWS * 128;  // one group of A: ROWS x 64 inputs, fp16
  constexpr int CH = ROWS * 8 / NT;   // 16-byte A chunks per thread and group (MB / 2)
  __shared__ __attribute__((aligned(16))) unsigned char s_a[LH_BUF * ABYTES];
  __shared__ float4 s_st[4 * ROWS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wb = w & 3, wr = w >> 2;
  const int g16 = lane >> 4, n16 = lane & 15;
  const int64_t L = a.L;
  const int D = a.D, G = D / 64, nblk = a.V / 64;
  const int nrt = (int)((L + ROWS - 1) / ROWS), nct = (nblk + 3) / 4;
  // tiles numbered row tile fastest; each XCD (blockIdx % 8) takes a
  // contiguous eighth, so the row tiles of a table block meet in one L2
  const int n = nrt * nct, per = (n + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (t >= n) return;
  const int ct = t / nrt, rt = t - ct * nrt;
  const int blk = 4 * ct + wb;
  const bool active = blk < nblk;  // a wave past the table's end loads block nblk-1 and computes nothing
  const uint32_t blkc = (uint32_t)(active ? blk : nblk - 1);
  const int64_t r0 = (int64_t)rt * ROWS;
  const int rows = (int)min((int64_t)ROWS, L - r0);

  // A chunk c = tid + NT i of a group: fragment f = c / 64 = 2 (row block) + h
  // and lane position p = c % 64, i.e. row 16 (f / 2) + p % 16 (rows past the
  // tile's last read that last row again) and inputs 32 h + 8 (p / 16) .. +7
  const _Float16* xb = a.xn + r0 * D;
  uint32_t aoff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i, f = c >> 6, p = c & 63;
    const int r = min(16 * (f >> 1) + (p & 15), rows - 1);
    aoff[i] = (uint32_t)(r * D + 32 * (f & 1) + 8 * (p >> 4));
  }
  u32x4 areg[CH];  // group q + 1 between its load and its store to LDS
  auto a_load = [&](int q) {
#pragma unroll
    for (int i = 0; i < CH; ++i) areg[i] = *(const u32x4*)(xb + aoff[i] + 64 * q);
  };
  auto a_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) *(u32x4*)(s_a + buf * ABYTES + (tid + NT * i) * 16) = areg[i];
  };
  const uint32_t* codes = a.codes;
  const uint32_t* sbw = a.sb;
  auto w_load = [&](LhGroup& d, int q) {  // groups past the last re-read the last
    const uint32_t bq = blkc * (uint32_t)G + (uint32_t)min(q, G - 1);
    const uint4* c = (const uint4*)(codes + ((bq * 4u + (uint32_t)g16) * 16u + (uint32_t)n16) * 8u);
    d.w[0] = c[0];
    d.w[1] = c[1];
    d.sb = *(const uint4*)(sbw + (bq * 16u + (uint32_t)n16) * 4u);
  };

  float4_t acc[4][MB];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[s][mb] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // acc[s][mb]: lane holds z[row 16 (MB wr + mb) + 4 g16 + i][table row 64 blk + 16 s + n16]
  // A fragments are read from LDS ahead of their MFMAs (the scheduler's
  // MFMA / LDS-read interleaving strategy keeps reads in flight), so the LDS
  // latency hides behind the four MFMAs of each fragment.
  auto compute = [&](const LhGroup& d, int buf) {
    const unsigned char* ab = s_a + buf * ABYTES + MB * wr * 2 * 64 * 16;
    auto frag = [&](int i) {  // fragment i: half i / MB, row block i % MB of the wave
      return bitcast<half8_t>(*(const uint4*)(ab + ((2 * (i % MB) + i / MB) * 64 + lane) * 16));
    };
    half8_t f0 = frag(0), f1 = frag(1), f2 = frag(2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      half8_t b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t pr = u4_get(d.sb, s);
        const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
        const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
        b[s] = dequant_q4_word(u4_get(d.w[s >> 1], 2 * (s & 1) + h), (half2_t){sc, sc},
                               (half2_t){bi, bi});
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int i = MB * h + mb;
        const half8_t fn = i + 3 < 2 * MB ? frag(i + 3) : f0;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[s][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f0, b[s], acc[s][mb], 0, 0, 0);
        f0 = f1;
        f1 = f2;
        f2 = fn;
      }
    }
    __builtin_amdgcn_iglp_opt(0);
  };

  // Every load is unconditional (past the last group: the last again,
  // unused), so the compiler can count them; the weight ring is three named
  // slots (an array indexed in the loop would live in scratch memory), and
  // the prologue issues in the steps' order (a group's weights, then A).
  LhGroup g0, g1, g2;
  w_load(g0, 0);
  a_load(0);
  a_store(0);
  w_load(g1, 1);
  w_load(g2, 2);
  a_load(min(1, G - 1));
  __syncthreads();
  auto step = [&](int q, LhGroup& g, int buf) {  // group q: weights in g, A in buffer buf
    if (active) compute(g, buf);
    w_load(g, q + LH_RING);
    a_store(buf == LH_BUF - 1 ? 0 : buf + 1);    // group q + 1
    a_load(min(q + 2, G - 1));
    lds_barrier();
  };
  for (int q0 = 0; q0 < G; q0 += LH_RING) {
    step(q0, g0, 0);
    if (q0 + 1 < G) step(q0 + 1, g1, 1);
    if (q0 + 2 < G) step(q0 + 2, g2, 2);
  }

  // epilogue: per row, this wave's 64 columns, then the four blocks in order
  const float inv_t = a.inv_t;
  float* lg = a.logits;
  if (active) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (MB * wr + mb) + 4 * g16 + i;
        float y[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) y[s] = softcap_t(acc[s][mb][i], inv_t);
        float m = y[0];
        int best = 64 * blk + n16;
#pragma unroll
        for (int s = 1; s < 4; ++s)
          if (y[s] > m) { m = y[s]; best = 64 * blk + 16 * s + n16; }
        row16_argmax(m, best);
        float l = 0.f, sm = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float d = y[s] - m;
          const float e = __builtin_amdgcn_exp2f(d * LOG2E);
          l += e;
          sm += e * d;
        }
        l = row16_sum(l);
        sm = row16_sum(sm);
        if (n16 == 0) s_st[wb * ROWS + row] = make_float4(m, l, sm, bitcast<float>(best));
        if (lg && row < rows) {
          float* dst = lg + (r0 + row) * (int64_t)a.V + 64 * blk + n16;
#pragma unroll
          for (int s = 0; s < 4; ++s) dst[16 * s] = y[s];
        }
      }
    }
  }
  __syncthreads();
  for (int row = tid; row < rows; row += NT) {
    float4 v = s_st[row];  // block 4 ct always exists
    RowStat st{v.x, v.y, v.z, bitcast<int>(v.w)};
#pragma unroll
    for (int bb = 1; bb < 4; ++bb) {
      if (4 * ct + bb < nblk) {
        v = s_st[bb * ROWS + row];
        st = stat_merge(st, RowStat{v.x, v.y, v.z, bitcast<int>(v.w)});
      }
    }
    a.pstat[(int64_t)ct * L + r0 + row] = make_float4(st.m, st.l, st.s, bitcast<float>(st.best));
  }
}

// One wave per row: the tiles' statistics merged (lanes take every 64th tile,
// then a butterfly), entropy = ln l - s / l.
__global__ __launch_bounds__(64) void k_tail_merge(TailArgs a) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int nct = (a.V / 64 + 3) / 4;
  RowStat st{0.f, 0.f, 0.f, 0};
  for (int c = lane; c < nct; c += 64) {
    const float4 v = a.pstat[(int64_t)c * a.L + row];
    st = stat_merge(st, RowStat{v.x, v.y, v.z, bitcast<int>(v.w)});
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const RowStat ot{__shfl_xor(st.m, o, 64), __shfl_xor(st.l, o, 64), __shfl_xor(st.s, o, 64),
                     __shfl_xor(st.best, o, 64)};
    st = stat_merge(st, ot);
  }
  if (lane == 0) {
    a.entropy[row] = logf(st.l) - st.s / st.l;
    a.argmax[row] = st.best;
    if (a.row_max) a.row_max[row] = st.m;
    if (a.row_sum) a.row_sum[row] = st.l;
  }
}

// ================================================================ soft embedding
constexpr float SOFT_SCALE = 16384.0f;  // 2^14: the stored probabilities are 2^14 exp(y - m_piece)

// Piece p of a row: its 64-row blocks [b0, b1).
__device__ __forceinline__ void piece_range(int p, int pieces, int nblk, int& b0, int& b1) {
  b0 = (int)((int64_t)p * nblk / pieces);
  b1 = (int)((int64_t)(p + 1) * nblk / pieces);
}

// Block-wide max / sum of 256 threads, the same value in every thread (fixed order).
__device__ __forceinline__ float block_max(float v, float* s_red) {
  v = row16_max(v);
  v = fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* s_red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

// grid (L, pieces): one (row, piece) per workgroup, the piece held in
// registers.  Within each 64-row block of the table the probabilities are
// stored in the GEMM's order: the one of table row v = 16 s + n goes to slot
// 4 n + s, so a lane of the GEMM's table staging (table rows 16 s + n, s < 4)
// writes its four values for one column as one 8-byte LDS store.  Thread t
// takes column n = t % 16 of blocks t / 16 + 16 i.
__global__ __launch_bounds__(256) void k_soft_probs(SoftArgs a) {
  __shared__ float s_red[4];
  const int64_t row = blockIdx.x;
  const int p = blockIdx.y, tid = threadIdx.x;
  if (row == 0 && p == 0 && tid == 0) *(uint64_t*)(a.sync + DG_SYNC_CALL) = a.stamp;
  int b0, b1;
  piece_range(p, a.pieces, a.V / 64, b0, b1);
  const int nb = b1 - b0, n = tid & 15;  // at most DG_SOFT_MAXBLK blocks
  const float* src = a.logits + row * a.V + (int64_t)b0 * 64 + n;
  float v[DG_SOFT_MAXBLK / 16][4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < DG_SOFT_MAXBLK / 16; ++i) {
    const int j = (tid >> 4) + 16 * i;
    if (j < nb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v[i][s] = src[64 * j + 16 * s];
        m = fmaxf(m, v[i][s]);
      }
    }
  }
  m = block_max(m, s_red);
  float l = 0.f;
  uint2* dst = (uint2*)(a.p16 + row * a.V + (int64_t)b0 * 64 + 4 * n);
#pragma unroll
  for (int i = 0; i < DG_SOFT_MAXBLK / 16; ++i) {
    const int j = (tid >> 4) + 16 * i;
    if (j < nb) {
      float e[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) e[s] = __builtin_amdgcn_exp2f((v[i][s] - m) * LOG2E);
      l += (e[0] + e[1]) + (e[2] + e[3]);
      const half2_t h01 = {(_Float16)(e[0] * SOFT_SCALE), (_Float16)(e[1] * SOFT_SCALE)};
      const half2_t h23 = {(_Float16)(e[2] * SOFT_SCALE), (_Float16)(e[3] * SOFT_SCALE)};
      dst[16 * j] = make_uint2(bitcast<uint32_t>(h01), bitcast<uint32_t>(h23));
    }
  }
  l = block_sum(l, s_red);
  if (tid == 0) a.pst[(int64_t)p * a.L + row] = make_float2(m, l);
}

constexpr int SG_EST = 144;                      // LDS bytes per column d of the E tile: 64 v fp16 + 16 pad
constexpr int SG_EBYTES = 256 * SG_EST;          // E tile: 256 columns d x 64 table rows v
constexpr int SG_PBYTES = DG_SOFT_ROWS * 128;    // P tile: 256 rows x 64 v fp16, fragment order
constexpr int SG_STAGE = SG_EBYTES + SG_PBYTES;

struct SgE {
  uint4 w;   // the lane's words of its two strips (2 s + h for s = 2 sp, 2 sp + 1)
  uint2 sb;  // (scale | bias << 16) of those two strips' table rows
};
constexpr int SG_ERING = 3;  // table blocks in flight (registers)

// Eight waves, two per SIMD.  Staging: wave w dequantises strips 2 (w / 4),
// +1 of group 4 db + w % 4 of each table block; the probabilities go through
// registers (four 16-byte chunks per thread).  Compute: wave w takes rows
// 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63 of the tile.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_soft_gemm(SoftArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[2 * SG_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, n16 = lane & 15;
  const int64_t L = a.L;
  const int D = a.D, G = D / 64, V = a.V, nblk = V / 64;
  const int nrt = (int)((L + DG_SOFT_ROWS - 1) / DG_SOFT_ROWS), ndb = (G + 3) / 4;
  // workgroups numbered column block fastest, then row tile, then piece; each
  // XCD takes a contiguous eighth, so the column blocks sharing a P tile meet
  // in one L2
  const int n = a.pieces * nrt * ndb, per = (n + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (t >= n) return;
  const int db = t % ndb, rest = t / ndb, rt = rest % nrt, p = rest / nrt;
  int b0, b1;
  piece_range(p, a.pieces, nblk, b0, b1);
  const int64_t r0 = (int64_t)rt * DG_SOFT_ROWS;
  const int rows = (int)min((int64_t)DG_SOFT_ROWS, L - r0);
  // E: group q = 4 db + w % 4 (a wave past D stores nothing; the columns it
  // would fill are never written out), strips 2 sp, 2 sp + 1
  const int qe = 4 * db + (w & 3), sp = w >> 2;
  const bool eon = qe < G;
  // P: chunk c = tid + 512 i is row 16 (c / 128) + c % 16 (rows past the
  // tile's last are zero), inputs 8 pc .. +7 with pc = (c / 16) % 8; in LDS it
  // sits at fragment (row / 16, half pc / 4), lane position 16 (pc % 4) +
  // row % 16.  So the 16 lanes of a store pass write 16 rows of one chunk,
  // 16 different 16-byte slots modulo 256 bytes (no bank conflicts)
  const int pr0 = (tid & 15) + 16 * (tid >> 7), pc = (tid >> 4) & 7;
  const _Float16* pb = a.p16 + r0 * V + 8 * pc;
  uint32_t prow[4];  // element offsets of the thread's rows pr0 + 64 i within the tile
#pragma unroll
  for (int i = 0; i < 4; ++i) prow[i] = (uint32_t)min(pr0 + 64 * i, rows - 1) * (uint32_t)V;
  const int plds0 = ((((pr0 >> 4) * 2 + (pc >> 2)) * 64) + (pc & 3) * 16 + (pr0 & 15)) * 16;

  // Loads are unconditional (clamped addresses), so the compiler can count
  // them: a load under a branch would make it wait for every load in flight.
  const uint32_t qec = (uint32_t)(eon ? qe : G - 1);
  auto e_load = [&](SgE& d, int b) {  // blocks past the piece re-read its last
    const uint32_t bq = (uint32_t)min(b, b1 - 1) * (uint32_t)G + qec;
    d.w = *(const uint4*)(a.codes + ((bq * 4u + (uint32_t)g16) * 16u + (uint32_t)n16) * 8u + 4u * sp);
    d.sb = *(const uint2*)(a.sb + (bq * 16u + (uint32_t)n16) * 4u + 2u * sp);
  };
  uint4 preg[4];
  auto p_load = [&](int b) {  // rows past the tile's last read its last row (stored as zero);
                              // blocks past the piece re-read its last (unused)
    const int bc = min(b, b1 - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) preg[i] = *(const uint4*)(pb + prow[i] + 64 * bc);
  };
  auto store = [&](const SgE& d, unsigned char* st) {
    if (eon) {
      // table row v = 16 s + n16 is slot 4 n16 + s; column d = 64 (w % 4) + 32 h + 8 g16 + j:
      // E tile [d][slot], the lane's two slots of a column in one 4-byte store
      unsigned char* ecol = st + (64 * (w & 3) + 8 * g16) * SG_EST + 8 * n16 + 4 * sp;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        half8_t v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t pr = k ? d.sb.y : d.sb.x;
          const _Float16 sc = bitcast<_Float16>((uint16_t)(pr & 0xFFFFu));
          const _Float16 bi = bitcast<_Float16>((uint16_t)(pr >> 16));
          v[k] = dequant_q4_word(u4_get(d.w, 2 * k + h), (half2_t){sc, sc}, (half2_t){bi, bi});
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const half2_t pair = {v[0][j], v[1][j]};
          *(uint32_t*)(ecol + (32 * h + j) * SG_EST) = bitcast<uint32_t>(pair);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = pr0 + 64 * i < rows;
      const uint4 v = preg[i];
      *(uint4*)(st + SG_EBYTES + plds0 + 8192 * i) =
          make_uint4(on ? v.x : 0u, on ? v.y : 0u, on ? v.z : 0u, on ? v.w : 0u);
    }
  };

  const int th = w >> 2, dq = w & 3;
  float4_t acc[8][4];
#pragma unroll
  for (int tb = 0; tb < 8; ++tb)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[tb][dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // acc[tb][dt]: lane holds out[row 128 th + 16 tb + 4 g16 + i][column 64 dq + 16 dt + n16]
  auto compute = [&](const unsigned char* st) {
    auto afrag = [&](int i) {  // P fragment i: half i / 8, row block i % 8
      return bitcast<half8_t>(*(const uint4*)(st + SG_EBYTES + (((8 * th + i % 8) * 2 + i / 8) * 64 + lane) * 16));
    };
    half8_t f0 = afrag(0), f1 = afrag(1), f2 = afrag(2);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      half8_t bf[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        bf[dt] = bitcast<half8_t>(*(const uint4*)(st + (64 * dq + 16 * dt + n16) * SG_EST + 64 * h2 + 16 * g16));
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const int i = 8 * h2 + tb;
        const half8_t fn = i + 3 < 16 ? afrag(i + 3) : f0;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          acc[tb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f0, bf[dt], acc[tb][dt], 0, 0, 0);
        f0 = f1;
        f1 = f2;
        f2 = fn;
      }
    }
    __builtin_amdgcn_iglp_opt(0);  // interleave the LDS reads with the MFMAs
  };

  // table codes run three blocks ahead in registers, probabilities one; LDS
  // is double-buffered (block b in stage (b - b0) % 2)
  SgE er[SG_ERING];
#pragma unroll
  for (int r = 0; r < SG_ERING; ++r) e_load(er[r], b0 + r);
  p_load(b0);
  store(er[0], s_buf);
  p_load(b0 + 1);
  __syncthreads();
  for (int bb = b0; bb < b1; bb += SG_ERING) {
#pragma unroll
    for (int r = 0; r < SG_ERING; ++r) {
      const int b = bb + r;  // codes of b in er[r] (already in LDS), of b + 1 in er[(r + 1) % 3]
      if (b < b1) {
        e_load(er[r], b + SG_ERING);
        const int k = (b - b0) & 1;
        compute(s_buf + k * SG_STAGE);
        if (b + 1 < b1) store(er[(r + 1) % SG_ERING], s_buf + (k ^ 1) * SG_STAGE);
        p_load(b + 2);
        lds_barrier();
      }
    }
  }

  float* dst = a.part + ((int64_t)p * L + r0) * D + 256 * db + 64 * dq + n16;
#pragma unroll
  for (int tb = 0; tb < 8; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 128 * th + 16 * tb + 4 * g16 + i;
      if (row < rows) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          if (256 * db + 64 * dq + 16 * dt < D) dst[(int64_t)row * D + 16 * dt] = acc[tb][dt][i];
      }
    }
}

// grid L: soft[row] = sum_p e^(m_p - m) part[p][row] * sqrt(D) / (2^14 l), with
// m = max_p m_p and l = sum_p e^(m_p - m) l_p; pieces added in order.
__global__ __launch_bounds__(256) void k_soft_reduce(SoftArgs a) {
  __shared__ float s_f[DG_SOFT_MAXPIECES];
  __shared__ float s_red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, P = a.pieces, D = a.D;
  float m = -INFINITY;
  for (int p = tid; p < P; p += 256) m = fmaxf(m, a.pst[(int64_t)p * a.L + row].x);
  m = block_max(m, s_red);
  float l = 0.f;
  for (int p = tid; p < P; p += 256) {
    const float2 v = a.pst[(int64_t)p * a.L + row];
    const float f = __builtin_amdgcn_exp2f((v.x - m) * LOG2E);
    s_f[p] = f;
    l += f * v.y;
  }
  l = block_sum(l, s_red);  // ends with a barrier: s_f is complete
  const float inv = sqrtf((float)D) / (l * SOFT_SCALE);
  const float* src = a.part + row * D;
  const int64_t pstride = a.L * (int64_t)D;
  for (int d = tid; d < D; d += 256) {
    float acc = 0.f;
    for (int p = 0; p < P; ++p) acc += s_f[p] * src[(int64_t)p * pstride + d];
    a.soft[row * D + d] = acc * inv;
  }
}

// ================================================================ canvas input
constexpr int SC_WORDS = 4;  // code words per thread of a row: D <= 8192 = 8 * 256 * 4
// grid L: e = E[id] sqrt(D) (+ the partial sums of h1), out = e / sqrt(mean(e^2) + eps).
// Thread t takes the words k = t + 256 j (inputs 8 k .. 8 k + 7) of the row.
__global__ __launch_bounds__(256) void k_sc_out(const int32_t* __restrict__ ids, int64_t L, int D, int V,
                                                const uint32_t* __restrict__ codes,
                                                const uint32_t* __restrict__ sbw, const float* h1,
                                                int h1_parts, float eps, float* out, uint32_t* sync,
                                                uint64_t stamp, int first) {
  __shared__ float s_red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  if (first && row == 0 && tid == 0) *(uint64_t*)(sync + DG_SYNC_CALL) = stamp;
  int id = ids[row];
  if (id < 0 || id >= V) {
    if (tid == 0) flag_error(sync, DG_ERR_INDEX, stamp);
    id = 0;
  }
  const int G = D / 64, nw = D / 8;
  const uint32_t b = (uint32_t)id >> 6, s = ((uint32_t)id >> 4) & 3u, nn = (uint32_t)id & 15u;
  const float sq = sqrtf((float)D);
  float v[SC_WORDS][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < SC_WORDS; ++j) {
    const int k = tid + 256 * j;
    if (k < nw) {
      const uint32_t q = (uint32_t)k >> 3, h = ((uint32_t)k >> 2) & 1u, g = (uint32_t)k & 3u;
      const uint32_t bq = b * (uint32_t)G + q;
      const uint32_t word = codes[((bq * 4u + g) * 16u + nn) * 8u + 2u * s + h];
      const uint32_t pr = sbw[(bq * 16u + nn) * 4u + s];
      const float sc = half_bits_to_float((uint16_t)(pr & 0xFFFFu));
      const float bi = half_bits_to_float((uint16_t)(pr >> 16));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {  // input 8 k + jj: nibble at bits 4 (jj / 2) + 16 (jj % 2)
        const float qv = (float)((word >> (4 * (jj >> 1) + 16 * (jj & 1))) & 15u);
        float e = fmaf(sc, qv, bi) * sq;
        for (int c = 0; c < h1_parts; ++c) e += h1[((int64_t)c * L + row) * D + 8 * k + jj];
        v[j][jj] = e;
        ss += e * e;
      }
    }
  }
  ss = block_sum(ss, s_red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int j = 0; j < SC_WORDS; ++j) {
    const int k = tid + 256 * j;
    if (k < nw) {
      float4* o = (float4*)(out + row * D + 8 * k);
      o[0] = make_float4(v[j][0] * r, v[j][1] * r, v[j][2] * r, v[j][3] * r);
      o[1] = make_float4(v[j][4] * r, v[j][5] * r, v[j][6] * r, v[j][7] * r);
    }
  }
}

}  // namespace

hipError_t launch_tail(const TailArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  if (a.L <= 0) return hipSuccess;
  if (a.D % 64 || a.V % 64 || a.D < 64 || a.V < 64) return hipErrorInvalidValue;
  const int64_t nct = (a.V / 64 + 3) / 4;
  auto grid = [&](int rows) {
    const int64_t n = (a.L + rows - 1) / rows * nct;
    return dim3((unsigned)(8 * ((n + 7) / 8)));
  };
  if (a.L <= 64) hipLaunchKernelGGL((k_lmhead_q4<4, 1>), grid(64), dim3(256), 0, st, a);
  else if (a.L <= 128) hipLaunchKernelGGL((k_lmhead_q4<8, 1>), grid(128), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_lmhead_q4<8, 2>), grid(256), dim3(512), 0, st, a);
  hipLaunchKernelGGL(k_tail_merge, dim3((unsigned)a.L), dim3(64), 0, st, a);
  return hipGetLastError();
}

int soft_pieces(int64_t L, int D, int V) {
  const int64_t nblk = V / 64, nrt = (L + DG_SOFT_ROWS - 1) / DG_SOFT_ROWS, ndb = (D / 64 + 3) / 4;
  int64_t s = 256 / (nrt * ndb);
  s = std::max<int64_t>(s, (nblk + DG_SOFT_MAXBLK - 1) / DG_SOFT_MAXBLK);
  s = std::min<int64_t>(s, nblk);
  s = std::min<int64_t>(s, DG_SOFT_MAXPIECES);
  return (int)std::max<int64_t>(s, 1);
}

hipError_t launch_soft_embed(const SoftArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  if (a.L <= 0) return hipSuccess;
  const int nblk = a.V / 64;
  if (a.D % 64 || a.V % 64 || a.D < 64 || a.V < 64 || !a.sync) return hipErrorInvalidValue;
  if (a.pieces < 1 || a.pieces > DG_SOFT_MAXPIECES || a.pieces > nblk ||
      (nblk + a.pieces - 1) / a.pieces > DG_SOFT_MAXBLK)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_soft_probs, dim3((unsigned)a.L, (unsigned)a.pieces), dim3(256), 0, st, a);
  const int64_t nrt = (a.L + DG_SOFT_ROWS - 1) / DG_SOFT_ROWS, ndb = (a.D / 64 + 3) / 4;
  const int64_t n = a.pieces * nrt * ndb;
  hipLaunchKernelGGL(k_soft_gemm, dim3((unsigned)(8 * ((n + 7) / 8))), dim3(512), 0, st, a);
  hipLaunchKernelGGL(k_soft_reduce, dim3((unsigned)a.L), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sc_out(const int32_t* ids, int64_t L, int D, int V, const uint32_t* codes,
                         const uint32_t* sb, const float* h1, int h1_parts, float eps, float* out,
                         uint32_t* sync, uint64_t stamp, bool first, hipStream_t st) {
  (void)hipGetLastError();
  if (L <= 0) return hipSuccess;
  if (D % 64 || D < 64 || D > 8 * 256 * SC_WORDS || V % 64 || V < 64 || !sync) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sc_out, dim3((unsigned)L), dim3(256), 0, st, ids, L, D, V, codes, sb, h1,
                     h1 ? h1_parts : 0, eps, out, sync, stamp, first ? 1 : 0);
  return hipGetLastError();
}
