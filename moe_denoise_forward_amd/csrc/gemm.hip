// Grouped GEMM phases of the block: gate_up + GeGLU, and down + weighted
// scatter.  One kernel body serves the 128 experts and the dense MLP: group
// g < E is expert g, whose rows are the (token, slot) pairs routed to it in
// the plan's expert-major order; group E is the always-on dense MLP, whose rows
// are the canvas positions (the diffgemma contract's MoE-order bullet: "the
// dense MLP runs in parallel as the always-on path"; the ML@Berkeley post's
// MOEBlock iterates over experts and gathers their tokens).
//
// Weights stream from HBM straight into registers: each lane loads the 16
// inputs of one weight row it feeds to the matrix core, dequantises them to
// fp16 in registers (Q4G64: magic-number nibble expansion + one packed fma per
// two weights; BF16: conversion), and the MFMA 16x16x32 f16 accumulates in
// fp32.  A 64-input group is one chunk: lane (g = l/16, n = l%16) covers inputs
// kb + 16g .. kb + 16g + 15 of row n, and MFMA j (j = 0, 1) takes inputs
// kb + 16g + 8j .. +7 -- the A operand uses the same order, so the product is
// the plain dot product over the group.
//
// Work tiles are DG_MT rows x (gate_up: 64 gate + 64 up columns | down: 128
// columns); 4 waves per workgroup, each owning two 16-column strips.  A
// persistent grid walks the tile table; tiles are dealt to the 8 XCDs in
// contiguous ranges so that tiles sharing an expert's A rows or a weight strip
// run on the same L2.
#include "common.h"
#include "kernels.h"

template <int WFMT>
__device__ __forceinline__ void load_b(const void* w, const uint16_t* sc, const uint16_t* bi,
                                       int64_t row, int K, int kb, int g, half8_t& b0,
                                       half8_t& b1) {
  if constexpr (WFMT == DGMOE_Q4G64) {
    const uint8_t* rp = (const uint8_t*)w + row * (K / 2);
    const uint2 v = *(const uint2*)(rp + kb / 2 + 8 * g);
    const int64_t gi = row * (K / 64) + kb / 64;
    const _Float16 s = bitcast<_Float16>(sc[gi]);
    const _Float16 b = bitcast<_Float16>(bi[gi]);
    const half2_t s2 = {s, s}, b2 = {b, b};
    b0 = dequant_q4_word(v.x, s2, b2);
    b1 = dequant_q4_word(v.y, s2, b2);
  } else {  // BF16
    const uint16_t* rp = (const uint16_t*)w + row * K + kb + 16 * g;
    b0 = bf16x8_to_half8(*(const uint4*)rp);
    b1 = bf16x8_to_half8(*(const uint4*)(rp + 8));
  }
}

template <int WFMT, bool GATEUP>
__device__ __forceinline__ void run_tile(const GemmPhaseArgs& p, int tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g16 = lane >> 4, n16 = lane & 15;
  // ---- locate the tile: group, row tile, column tile
  int lo = 0, hi = p.E + 1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.pref[mid] <= tile) lo = mid; else hi = mid;
  }
  const int grp = lo;
  const bool dense = grp == p.E;
  const int rows_g = p.grp_cnt[grp];
  const int mtiles = (rows_g + DG_MT - 1) / DG_MT;
  const int local = tile - p.pref[grp];
  const int nt = local / mtiles, mt = local % mtiles;
  const int row0 = mt * DG_MT;
  const int rows = min(DG_MT, rows_g - row0);
  const int goff = dense ? 0 : p.grp_off[grp];

  const int N = dense ? p.n_d : p.n_e;
  const int K = dense ? p.k_d : p.k_e;
  // bytes of one expert matrix: Q4G64 half a byte per weight, BF16 two bytes
  const int64_t ebytes = (WFMT == DGMOE_Q4G64) ? (int64_t)p.n_e * p.k_e / 2
                                               : (int64_t)p.n_e * p.k_e * 2;
  const void* W = dense ? p.w_d : (const void*)((const uint8_t*)p.w_e + (int64_t)grp * ebytes);
  const uint16_t* S = dense ? p.s_d : (p.s_e ? p.s_e + (int64_t)grp * p.n_e * (p.k_e / 64) : nullptr);
  const uint16_t* B = dense ? p.b_d : (p.b_e ? p.b_e + (int64_t)grp * p.n_e * (p.k_e / 64) : nullptr);

  // ---- the two 16-row weight strips of this wave
  int64_t srow[2];
  bool sok[2];
  if (GATEUP) {
    const int c0 = nt * DG_NGU + 16 * wave;
    srow[0] = c0 + n16;              // gate row
    srow[1] = N / 2 + c0 + n16;      // matching up row
    sok[0] = sok[1] = true;
  } else {
    const int n0 = nt * DG_NDN + 32 * wave;
    srow[0] = n0 + n16;
    srow[1] = n0 + 16 + n16;
    sok[0] = n0 < N;
    sok[1] = n0 + 16 < N;
  }
  if (!sok[0]) return;  // whole wave idle (down tail tile)

  // ---- A row pointers for the two 16-row blocks (rows past the tile reuse row 0)
  const _Float16* arow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int m = mb * 16 + n16;
    if (m >= rows) m = 0;
    int64_t r;
    if (dense) {
      r = row0 + m;
      arow[mb] = p.a_d + r * K;
    } else if (GATEUP) {
      r = p.perm[goff + row0 + m] / p.topk;  // token of the pair
      arow[mb] = p.a_e + r * K;
    } else {
      r = goff + row0 + m;                   // expert-sorted act row
      arow[mb] = p.a_e + r * K;
    }
  }
  const bool two = rows > 16;

  float4_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[mb][s] = (float4_t){0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < K; kb += 64) {
    half8_t bw[2][2];
    load_b<WFMT>(W, S, B, srow[0], K, kb, g16, bw[0][0], bw[0][1]);
    if (sok[1]) load_b<WFMT>(W, S, B, srow[1], K, kb, g16, bw[1][0], bw[1][1]);
    half8_t av[2][2];
    av[0][0] = *(const half8_t*)(arow[0] + kb + 16 * g16);
    av[0][1] = *(const half8_t*)(arow[0] + kb + 16 * g16 + 8);
    if (two) {
      av[1][0] = *(const half8_t*)(arow[1] + kb + 16 * g16);
      av[1][1] = *(const half8_t*)(arow[1] + kb + 16 * g16 + 8);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[0][j], bw[0][j], acc[0][0], 0, 0, 0);
      if (sok[1]) acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[0][j], bw[1][j], acc[0][1], 0, 0, 0);
      if (two) {
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1][j], bw[0][j], acc[1][0], 0, 0, 0);
        if (sok[1]) acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1][j], bw[1][j], acc[1][1], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds C[m = 16 mb + 4 g16 + i][n = n16] of each strip
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb == 1 && !two) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mb * 16 + 4 * g16 + i;
      if (m >= rows) continue;
      if (GATEUP) {
        const float gv = acc[mb][0][i], uv = acc[mb][1][i];
        const _Float16 hv = (_Float16)(gelu_tanh(gv) * uv);
        const int col = nt * DG_NGU + 16 * wave + n16;
        if (dense) p.act_d[(int64_t)(row0 + m) * (N / 2) + col] = hv;
        else p.act_e[(int64_t)(goff + row0 + m) * (N / 2) + col] = hv;
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (!sok[s]) continue;
          const int64_t col = srow[s];
          const float y = acc[mb][s][i];
          if (dense) {
            p.h1[(int64_t)(row0 + m) * N + col] = y;
          } else {
            const int pair = p.perm[goff + row0 + m];
            p.slots[(int64_t)pair * N + col] = p.route_w[pair] * y;
          }
        }
      }
    }
  }
}

template <int WFMT_E, int WFMT_D, bool GATEUP>
__global__ __launch_bounds__(256) void k_grouped(GemmPhaseArgs p) {
  const int total = p.pref[p.E + 1];
  const int per = (total + 7) / 8;
  const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3, g8 = gridDim.x >> 3;
  for (int i = jb; i < per; i += g8) {
    const int t = xcd * per + i;
    if (t >= total) break;
    // the dense group sits at the end of the table
    if (t >= p.pref[p.E]) run_tile<WFMT_D, GATEUP>(p, t);
    else run_tile<WFMT_E, GATEUP>(p, t);
  }
}

template <bool GATEUP>
static hipError_t launch_phase(const GemmPhaseArgs& a, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  int grid = (a.max_tiles + 7) / 8 * 8;
  const int cap = 256 * 4;
  if (grid > cap) grid = cap;
  if (grid < 8) grid = 8;
  dim3 g(grid), b(256);
  const bool eq = a.wfmt_e == DGMOE_Q4G64, dq = a.wfmt_d == DGMOE_Q4G64;
  if (eq && dq) hipLaunchKernelGGL((k_grouped<DGMOE_Q4G64, DGMOE_Q4G64, GATEUP>), g, b, 0, st, a);
  else if (eq) hipLaunchKernelGGL((k_grouped<DGMOE_Q4G64, DGMOE_BF16, GATEUP>), g, b, 0, st, a);
  else if (dq) hipLaunchKernelGGL((k_grouped<DGMOE_BF16, DGMOE_Q4G64, GATEUP>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_grouped<DGMOE_BF16, DGMOE_BF16, GATEUP>), g, b, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gate_up(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<true>(a, st); }
hipError_t launch_down(const GemmPhaseArgs& a, hipStream_t st) { return launch_phase<false>(a, st); }
