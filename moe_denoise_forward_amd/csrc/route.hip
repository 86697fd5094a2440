// Front of the block: RMSNorm, router logits, top-k selection and the
// per-expert lists of routed pairs.
//
// The router follows the diffgemma contract (Part II section 2.1, MoE-order
// bullet): weightless RMSNorm of the block input, times router_scale and
// hidden^-1/2, a linear map to E logits, the top-k by logit with ties going to
// the lower expert index, and softmax weights over the selected k times
// per_expert_scale (the mlx-bun dossier's Router takes the softmax over the
// selected scores, which is the same quantity).  Logits stay fp32 (the
// contract's precision policy keeps router logits in f32: routing is control
// flow).
//
//   k_front   grid (row blocks of 16, expert tiles of 16, or pairs of tiles
//             at large L): the norm, the router logits of its 16 x 16 tile(s)
//             over the whole input (fp32 MFMA, the input split over the eight
//             waves) and its share of the fp16 GEMM operands
//             a = xh*pre_ff_norm, b = xh*pre_ff_norm_2;
//             the last workgroup of each row block to finish selects the
//             top-k, the weights and the per-expert pair lists (an integer
//             atomic counter per expert gives the position): the pair id
//             t*k + j at list[e*cap + i], its token t at list[(E + e)*cap + i].
//   k_norm    the norm and the operands only (routing given by the caller).
//   k_assign  the pair lists from a routing given by the caller.
// Each kernel issues its global loads before it first waits on one (the
// front kernel in batches of steps, kept in step order), so a launch costs
// about one memory latency plus its arithmetic.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int FR_ROWS = DG_FRONT_ROWS;  // rows per front workgroup
constexpr int FR_THREADS = 512;         // 8 waves
constexpr int FR_WAVES = FR_THREADS / 64;
constexpr int FR_TILE = 16;             // experts per front workgroup
constexpr int FR_MAX_D = 8192;

template <typename XT>
__device__ __forceinline__ void load8(const XT* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const uint4 a = *(const uint4*)p;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bitcast<float>(w[i] << 16);
    v[2 * i + 1] = bitcast<float>(w[i] & 0xFFFF0000u);
  }
}

// Eight fp16 operands v*w; returns whether every one of them fits fp16.
__device__ __forceinline__ bool store8h(_Float16* p, const float* v, const float* w) {
  half8_t h;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = v[i] * w[i];
    m = fmaxf(m, fabsf(o));
    h[i] = (_Float16)o;
  }
  *(half8_t*)p = h;
  return m < DG_F16_LIMIT;  // false for inf and NaN too
}

// Eight consecutive router weights W[e][k..k+7] (k a multiple of 8), as
// loaded, and their fp32 values (the exact dequant for Q8).
template <int RFMT>
struct RouterRaw;
template <>
struct RouterRaw<DGMOE_F32> { float4 v[2]; };
template <>
struct RouterRaw<DGMOE_BF16> { uint4 v; };
template <>
struct RouterRaw<DGMOE_Q8G64> { uint2 v; uint32_t sb; };

template <int RFMT>
__device__ __forceinline__ void router_load8(RouterRaw<RFMT>& r, const dgmoe_matrix& w, int D, int e, int k) {
  if constexpr (RFMT == DGMOE_F32) {
    const float4* p = (const float4*)((const float*)w.data + (int64_t)e * D + k);
    r.v[0] = p[0];
    r.v[1] = p[1];
  } else if constexpr (RFMT == DGMOE_BF16) {
    r.v = *(const uint4*)((const uint16_t*)w.data + (int64_t)e * D + k);
  } else {  // Q8G64: row-major bytes, (scale, bias) pairs row-major per group
    r.v = *(const uint2*)((const uint8_t*)w.data + (int64_t)e * D + k);
    r.sb = ((const uint32_t*)w.scale_bias)[(int64_t)e * (D / 64) + k / 64];
  }
}

template <int RFMT>
__device__ __forceinline__ float router_value(const RouterRaw<RFMT>& r, int i) {
  if constexpr (RFMT == DGMOE_F32) {
    const float4 q = r.v[i >> 2];
    return (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
  } else if constexpr (RFMT == DGMOE_BF16) {
    const int j = i >> 1;
    const uint32_t u = j == 0 ? r.v.x : j == 1 ? r.v.y : j == 2 ? r.v.z : r.v.w;
    return bitcast<float>((i & 1) ? (u & 0xFFFF0000u) : (u << 16));
  } else {
    const uint32_t u = i < 4 ? r.v.x : r.v.y;
    const float sc = half_bits_to_float((uint16_t)(r.sb & 0xFFFFu));
    const float bi = half_bits_to_float((uint16_t)(r.sb >> 16));
    return fmaf(sc, (float)((u >> (8 * (i & 3))) & 0xFFu), bi);
  }
}

// Order-preserving 32-bit image of a logit (-0 taken as +0, so equal logits
// tie); 0 is below the image of every logit that is not a NaN with its sign
// bit set, and stands for "no expert".
__device__ __forceinline__ uint32_t order_u32(float z) {
  const uint32_t f = bitcast<uint32_t>(z + 0.0f);  // -0 -> +0
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}
__device__ __forceinline__ float u32_logit(uint32_t o) {
  return bitcast<float>((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Largest (smallest) value within each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp32<0x141>(v));  // row_half_mirror
  v = max(v, dpp32<0x140>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ int row16_min_i32(int v) {
  v = min(v, (int)dpp32<0xB1>((uint32_t)v));
  v = min(v, (int)dpp32<0x4E>((uint32_t)v));
  v = min(v, (int)dpp32<0x141>((uint32_t)v));
  v = min(v, (int)dpp32<0x140>((uint32_t)v));
  return v;
}
constexpr int SEL_MAX_E = 256;  // experts a selection handles (16 per lane)
constexpr int SEL_MAX_K = 32;   // choices (two per lane of a row group)
static_assert(DG_SYNC_ERR == 4, "flag_error (common.h) writes the error words at word 4");

// One 32-input step of a wave: lane (m = lane%16, g = lane/16) holds inputs
// 32 s + 8 g .. +7 of row m (the A operand) and of expert 16 et + m (B).
template <typename XT>
struct XRaw;
template <>
struct XRaw<float> { float4 v[2]; };
template <>
struct XRaw<uint16_t> { uint4 v; };
__device__ __forceinline__ void x_load8(XRaw<float>& r, const float* p) {
  r.v[0] = *(const float4*)p;
  r.v[1] = *(const float4*)(p + 4);
}
__device__ __forceinline__ void x_load8(XRaw<uint16_t>& r, const uint16_t* p) { r.v = *(const uint4*)p; }
__device__ __forceinline__ float x_value(const XRaw<float>& r, int t) {
  const float4 q = r.v[t >> 2];
  return (t & 3) == 0 ? q.x : (t & 3) == 1 ? q.y : (t & 3) == 2 ? q.z : q.w;
}
__device__ __forceinline__ float x_value(const XRaw<uint16_t>& r, int t) {
  const int j = t >> 1;
  const uint32_t u = j == 0 ? r.v.x : j == 1 ? r.v.y : j == 2 ? r.v.z : r.v.w;
  return bitcast<float>((t & 1) ? (u & 0xFFFF0000u) : (u << 16));
}

template <typename XT, int RFMT, int NT>
struct FrStep {
  XRaw<XT> x;
  RouterRaw<RFMT> w[NT];  // the same 8 inputs of the workgroup's NT expert tiles
};

// Steps in flight per wave.  More is not faster: at canvas 256 a 2816-wide
// input in one batch of 11 steps took 24.6 us, in batches of 3, 4 or 6 steps
// 22.6-22.9 us (the loads of a batch queue on the CU's address path, and the
// first MFMAs wait for the whole queue ahead of them).  With two expert
// tiles each step also holds a second router slice.
template <typename XT, int RFMT, int NT>
constexpr int fr_batch() {
  return NT == 1 ? 6 : (RFMT == DGMOE_F32 ? 2 : RFMT == DGMOE_BF16 ? 3 : 4);
}

// One of the lane's two choices (choice m + 16 q of its row group).
struct Choice {
  int e = 0;       // expert (never outside [0, E) unless the logits hold NaNs)
  int slot = 0;    // its claimed place in the expert's pair list
  bool on = false; // a choice of a real row
};

// Top-k of one row per 16-lane group (row srow; rows past L read row0 and
// write nothing).  Lane m holds the order-preserving images of the logits of
// experts NKL m .. NKL m + NKL - 1 (0 past E).  Round j: the row's largest
// image (DPP maximum within the 16 lanes), the lowest expert holding it (DPP
// minimum of each lane's lowest match), that expert's image retired; lane
// j % 16 keeps choice j.  Then the softmax over the chosen logits (the
// largest first; the denominator is the row-of-16 sum of choices 0..15 plus
// that of choices 16..31), times pes; each choice claims its list slot with
// an integer atomic before the softmax, so the round trip overlaps it.
template <int NKL>
__device__ __forceinline__ void select_row(const FrontArgs& fa, int64_t srow, int64_t row0, int m, Choice (&ch)[2],
                                           const float* s_pes) {
  const int E = fa.E, k = fa.k;
  const int64_t L = fa.L;
  const int64_t rr = srow < L ? srow : row0;
  float zv[NKL];
  uint32_t key[NKL];
#pragma unroll
  for (int i = 0; i < NKL; ++i) zv[i] = ld_agent(&fa.plog[rr * E + min(NKL * m + i, E - 1)]);
#pragma unroll
  for (int i = 0; i < NKL; ++i) key[i] = NKL * m + i < E ? order_u32(zv[i]) : 0u;
  if (fa.logits && srow < L)
#pragma unroll
    for (int i = 0; i < NKL; ++i)
      if (NKL * m + i < E) fa.logits[srow * E + NKL * m + i] = zv[i];
  uint32_t top = 0, ck[2] = {0u, 0u};
  int ce[2] = {0, 0};
  for (int j = 0; j < k; ++j) {
    uint32_t mx = key[0];
#pragma unroll
    for (int i = 1; i < NKL; ++i) mx = max(mx, key[i]);
    const uint32_t best = row16_max_u32(mx);
    if (j == 0) top = best;
    int cand = 0x7FFFFFFF;  // the lane's lowest expert holding the maximum
#pragma unroll
    for (int i = NKL - 1; i >= 0; --i) cand = key[i] == best ? NKL * m + i : cand;
    const int win = row16_min_i32(cand);
#pragma unroll
    for (int i = 0; i < NKL; ++i) key[i] = NKL * m + i == win ? 0u : key[i];
    if (m == (j & 15)) {
      if (j < 16) { ce[0] = win; ck[0] = best; }
      else { ce[1] = win; ck[1] = best; }
    }
  }
  // the claims first (a choice outside [0, E) can only come from NaN logits
  // and is not listed)
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = m + 16 * q;
    ch[q].e = ce[q];
    ch[q].on = c < k && srow < L;
    const bool in = ch[q].on && ce[q] >= 0 && ce[q] < E;
    if (fa.list && c < k) ch[q].slot = atomicAdd(&fa.cnt[(in ? ce[q] : 0) * DG_CNT_STRIDE], in ? 1 : 0);
  }
  const float topz = u32_logit(top);
  float ex[2], pe[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    ex[q] = m + 16 * q < k ? expf(u32_logit(ck[q]) - topz) : 0.f;
    pe[q] = s_pes[min(max(ce[q], 0), E - 1)];
  }
  const float den = row16_sum(ex[0]) + row16_sum(ex[1]);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (ch[q].on) {
      fa.idx[srow * k + m + 16 * q] = ce[q];
      fa.w[srow * k + m + 16 * q] = (ex[q] / den) * pe[q];
    }
}

// Grid (row blocks of 16, groups of NT expert tiles of 16), 8 waves.
//   * Wave w takes the 32-input steps w, w + 8, ... of the input.  Per step a
//     lane loads 8 inputs of its row and the same 8 weights of its expert in
//     each of the NT tiles;
//     MFMA t (fp32 16x16x4) takes input 8g + t of the step in lane group g,
//     for A = (x*router_scale)*D^-1/2 (router_scale staged in LDS) and B
//     alike, so each accumulator is the plain dot product; the same inputs
//     give the lane's share of the row's sum of squares.
//   * The eight partial tiles and row sums are added in wave order through
//     LDS: r = 1/sqrt(mean + eps) is the same bit for bit in every workgroup
//     of the row block, and z = r*(u'.W) + bias is the logit of
//     u = (xh*router_scale)*D^-1/2 (the router scale folded before the norm).
//   * Each workgroup stores its 16 x 16 NT logits and counts its arrival.
//   * The last of the row block to arrive selects for the block's 16 rows,
//     one row per 16-lane group of waves 0..3 (select_row: k rounds of DPP
//     maxima and minima within the group); softmax over the k chosen logits
//     (the largest first) times pes; the pair lists.
//   * Then every workgroup writes its share of a and b: step s of the input
//     belongs to workgroup (s/8) % (workgroups of the row block).
// The arrival counters and the expert counts are zeroed in the same launch by
// workgroup (0, 0), which then publishes the call's stamp; a workgroup counts
// its arrival only after it has seen the stamp (requested early, so it is
// almost always there; a bounded wait, and workgroup (0, 0) never waits on
// anything), so no counter is touched before it is zero.
template <typename XT, int RFMT, int NT>
__global__ __launch_bounds__(FR_THREADS) void k_front(FrontArgs fa, dgmoe_matrix wr, float rc) {
  constexpr int NB = fr_batch<XT, RFMT, NT>();
  constexpr int NE = NT * FR_TILE;  // experts of the workgroup
  __shared__ float s_rs[FR_MAX_D];
  __shared__ float s_red[FR_WAVES][FR_ROWS][NE + 1];
  __shared__ float s_ss[FR_WAVES][FR_ROWS];
  __shared__ float s_r[FR_ROWS];
  __shared__ int s_last;
  __shared__ float s_pes[SEL_MAX_E];
  const XT* __restrict__ x = (const XT*)fa.x;
  const int64_t L = fa.L;
  const int D = fa.D, E = fa.E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * FR_ROWS;
  const int et = blockIdx.y, nwg = gridDim.y;  // workgroups of a row block
  uint32_t* arrive = fa.sync + DG_SYNC_HEAD;
  uint64_t* stamp = (uint64_t*)fa.sync;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    if (fa.cnt)
      for (int i = tid; i < DG_CLEAR_WORDS; i += FR_THREADS) st_agent(&fa.cnt[dg_clear_word(i)], 0);
    for (int64_t i = tid; i < (int64_t)gridDim.x; i += FR_THREADS) st_agent(&arrive[i], 0u);
    if (tid == 0) st_agent((uint64_t*)(fa.sync + DG_SYNC_CALL), fa.stamp);
    drain_then_sync();
    if (tid == 0 && fa.publish) st_agent(stamp, fa.stamp);
  }
  if (fa.rowid && et == 0 && tid < FR_ROWS && row0 + tid < L) fa.rowid[row0 + tid] = (int32_t)(row0 + tid);

  // loads of the first batch of steps, router_scale into LDS
  const int S = D / 32;
  const int ns = wave < S ? (S - wave + FR_WAVES - 1) / FR_WAVES : 0;  // steps of this wave
  const XT* xr = x + (row0 + m < L ? row0 + m : row0) * (int64_t)D;   // rows past L redo row0
  int ew[NT];  // the lane's expert in each tile (past E: expert E-1 again, dropped)
#pragma unroll
  for (int t = 0; t < NT; ++t) ew[t] = min(NE * et + FR_TILE * t + m, E - 1);
  FrStep<XT, RFMT, NT> st[NB];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // past the wave's steps: its last again (a wave with none: the last step
      // of the input); unused either way
      const int s = min(wave + FR_WAVES * max(min(b0 + i, ns - 1), 0), S - 1);
      const int k0 = 32 * s + 8 * g;
      x_load8(st[i].x, xr + k0);
#pragma unroll
      for (int t = 0; t < NT; ++t) router_load8<RFMT>(st[i].w[t], wr, D, ew[t], k0);
      // in step order, so the wait for a step covers no later step's loads
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // router_scale into LDS, requested before the batch so that its wait does
  // not cover the batch (a wave's loads complete in order); the barrier orders
  // LDS only, so the batch stays in flight into the MFMA loop
  static_assert(FR_MAX_D == 4 * 4 * FR_THREADS, "four router_scale chunks per thread");
  auto rs_at = [&](int j) { const int i = 4 * (tid + j * FR_THREADS); return i < D ? i : 0; };
  const float4 rs0 = *(const float4*)(fa.router_scale + rs_at(0));
  const float4 rs1 = *(const float4*)(fa.router_scale + rs_at(1));
  const float4 rs2 = *(const float4*)(fa.router_scale + rs_at(2));
  const float4 rs3 = *(const float4*)(fa.router_scale + rs_at(3));
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the batch
  load_batch(0);  // on every path, so the waits below count the same loads on all of them
  // the call's stamp, requested early
  uint64_t seen = 0;
  if (tid == 0) seen = ld_agent(stamp);
  *(float4*)&s_rs[rs_at(0)] = rs0;  // chunks past D rewrite chunk 0 with its own value
  *(float4*)&s_rs[rs_at(1)] = rs1;
  *(float4*)&s_rs[rs_at(2)] = rs2;
  *(float4*)&s_rs[rs_at(3)] = rs3;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  float4_t acc[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  for (int b0 = 0; b0 < ns; b0 += NB) {
    if (b0 > 0) load_batch(b0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (b0 + i >= ns) break;  // uniform
      const int k0 = 32 * (wave + FR_WAVES * (b0 + i)) + 8 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xv = x_value(st[i].x, t);
        ss += xv * xv;
        const float a = (xv * s_rs[k0 + t]) * rc;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          acc[tt][i & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, router_value<RFMT>(st[i].w[tt], t),
                                                                acc[tt][i & 1], 0, 0, 0);
      }
    }
  }
  // partial tiles and row sums of squares -> LDS, added in wave order
  ss += __shfl_xor(ss, 16, DG_WAVE);
  ss += __shfl_xor(ss, 32, DG_WAVE);
  if (g == 0) s_ss[wave][m] = ss;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const float4_t t = acc[tt][0] + acc[tt][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][4 * g + i][FR_TILE * tt + m] = t[i];
  }
  __syncthreads();
  if (tid < FR_ROWS) {
    float v = 0.f;
    for (int w = 0; w < FR_WAVES; ++w) v += s_ss[w][tid];
    s_r[tid] = 1.0f / sqrtf(v / (float)D + fa.eps);
  }
  __syncthreads();
  for (int i = tid; i < FR_ROWS * NE; i += FR_THREADS) {
    const int mm = i / NE, nn = i % NE;
    const int64_t row = row0 + mm;
    const int e = NE * et + nn;
    float v = 0.f;
    for (int w = 0; w < FR_WAVES; ++w) v += s_red[w][mm][nn];
    float z = v * s_r[mm];
    if (e < E && fa.bias) z += fa.bias[e];
    if (row < L && e < E) st_agent(&fa.plog[row * E + e], z);
  }
  // arrival: once every logit store of the workgroup has completed, and the
  // counters have been cleared for this call.  The wait is bounded: a
  // workgroup that gives up flags the call and does not arrive, so the row
  // block's selection and list appends never run (nothing is counted on
  // counters that may not have been cleared).
  drain_then_sync();
  if (tid == 0) {
    for (int spins = 0; seen != fa.stamp && spins < fa.spin_limit; ++spins) {
      __builtin_amdgcn_s_sleep(2);
      seen = ld_agent(stamp);
    }
    if (seen == fa.stamp) {
      s_last = atomicAdd(&arrive[blockIdx.x], 1u) == (uint32_t)(nwg - 1);
    } else {
      flag_error(fa.sync, DG_ERR_SYNC, fa.stamp);
      s_last = 0;
    }
  }
  __syncthreads();
  const int k = fa.k;
  // the last arriver's selection: row srow of the block per 16-lane group of
  // waves 0..3; lane m of the group ends with choices m and m + 16
  const bool sel = s_last && wave < FR_ROWS / 4;
  const int64_t srow = row0 + 4 * wave + g;
  Choice ch[2];
  if (s_last) {
    // pes of every expert into LDS, where the choices read theirs
    if (tid < E) s_pes[tid] = fa.pes[tid];
    __syncthreads();
    if (sel) {
      if (E <= 128) select_row<8>(fa, srow, row0, m, ch, s_pes);
      else select_row<16>(fa, srow, row0, m, ch, s_pes);
    }
  }

  // this workgroup's share of the fp16 operands: the steps s = wave + 8 i of
  // the whole input with i % (workgroups of the row block) == blockIdx.y,
  // rows m of the block, inputs 32 s + 8 g ..
  if (fa.a || fa.b) {
    const int64_t row = row0 + m;
    const float r = s_r[m];
    const int nsw = wave < S ? (S - wave + FR_WAVES - 1) / FR_WAVES : 0;
    bool fits = true;
    for (int i = blockIdx.y; i < nsw; i += nwg) {
      const int k0 = 32 * (wave + FR_WAVES * i) + 8 * g;
      float xv[8], w[8];
      load8<XT>(xr + k0, xv);
#pragma unroll
      for (int t = 0; t < 8; ++t) xv[t] *= r;
      if (row < L) {
        if (fa.a) { load8<float>(fa.w_pre + k0, w); fits &= store8h(fa.a + row * D + k0, xv, w); }
        if (fa.b) { load8<float>(fa.w_pre2 + k0, w); fits &= store8h(fa.b + row * D + k0, xv, w); }
      }
    }
    if (!fits) flag_error(fa.sync, DG_ERR_RANGE, fa.stamp);
  }
  // the last arriver's list entries, in the slots claimed above
  // (a position names an expert at most once, so a list never holds more than
  // L = cap entries; the check only guards the bound)
  if (sel && fa.list)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (ch[q].on && ch[q].e >= 0 && ch[q].e < E) {
        if (ch[q].slot >= fa.cap) {
          flag_error(fa.sync, DG_ERR_ROUTE, fa.stamp);
          continue;
        }
        const int64_t at = (int64_t)ch[q].e * fa.cap + ch[q].slot;
        fa.list[at] = (int32_t)(srow * k + m + 16 * q);
        fa.list[(int64_t)E * fa.cap + at] = (int32_t)srow;  // the pair's token
      }
}

// RMSNorm and the fp16 operands only (no router), 16 rows per workgroup of
// eight waves.  The row's sum of squares is added in exactly the order k_front
// adds it (lane (m, g) of wave w sums inputs 32 s + 8 g .. + 7 of its steps
// s = w + 8 i in step order, then the four g lanes pairwise, then the waves in
// order), so r, a and b are the same bits on every path.  Workgroup 0 zeroes
// the counter block for the launches that follow; rowid[t] = t.
template <typename XT>
__global__ __launch_bounds__(FR_THREADS) void k_norm(FrontArgs fa) {
  __shared__ float s_ss[FR_WAVES][FR_ROWS];
  __shared__ float s_r[FR_ROWS];
  const XT* __restrict__ x = (const XT*)fa.x;
  const int64_t L = fa.L;
  const int D = fa.D, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * FR_ROWS;
  if (fa.cnt && blockIdx.x == 0)
    for (int i = tid; i < DG_CLEAR_WORDS; i += FR_THREADS) fa.cnt[dg_clear_word(i)] = 0;
  if (blockIdx.x == 0 && tid == 0) *(uint64_t*)(fa.sync + DG_SYNC_CALL) = fa.stamp;
  if (fa.rowid && tid < FR_ROWS && row0 + tid < L) fa.rowid[row0 + tid] = (int32_t)(row0 + tid);
  const int S = D / 32;
  const int ns = wave < S ? (S - wave + FR_WAVES - 1) / FR_WAVES : 0;  // steps of this wave
  const int64_t row = row0 + m;
  const XT* xr = x + (row < L ? row : row0) * (int64_t)D;  // rows past L redo row0
  float ss = 0.f;
  for (int i = 0; i < ns; ++i) {
    float v[8];
    load8<XT>(xr + 32 * (wave + FR_WAVES * i) + 8 * g, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) ss += v[t] * v[t];
  }
  ss += __shfl_xor(ss, 16, DG_WAVE);
  ss += __shfl_xor(ss, 32, DG_WAVE);
  if (g == 0) s_ss[wave][m] = ss;
  __syncthreads();
  if (tid < FR_ROWS) {
    float v = 0.f;
    for (int w = 0; w < FR_WAVES; ++w) v += s_ss[w][tid];
    s_r[tid] = 1.0f / sqrtf(v / (float)D + fa.eps);
  }
  __syncthreads();
  if (row >= L) return;
  const float r = s_r[m];
  bool fits = true;
  for (int i = 0; i < ns; ++i) {
    const int k0 = 32 * (wave + FR_WAVES * i) + 8 * g;
    float v[8], w[8];
    load8<XT>(xr + k0, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] *= r;
    if (fa.a) { load8<float>(fa.w_pre + k0, w); fits &= store8h(fa.a + row * D + k0, v, w); }
    if (fa.b) { load8<float>(fa.w_pre2 + k0, w); fits &= store8h(fa.b + row * D + k0, v, w); }
  }
  if (!fits) flag_error(fa.sync, DG_ERR_RANGE, fa.stamp);
}

__global__ __launch_bounds__(256) void k_assign(const int32_t* __restrict__ idx, int64_t Lk, int k,
                                                int E, int32_t* __restrict__ cnt,
                                                int32_t* __restrict__ list, int64_t cap,
                                                uint32_t* sync, uint64_t stamp) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= Lk) return;
  const int e = idx[p];
  if (e >= 0 && e < E) {
    const int slot = atomicAdd(&cnt[e * DG_CNT_STRIDE], 1);
    if (slot < cap) {
      const int64_t at = (int64_t)e * cap + slot;
      list[at] = (int32_t)p;
      list[(int64_t)E * cap + at] = (int32_t)(p / k);  // the pair's token
    } else {
      flag_error(sync, DG_ERR_ROUTE, stamp);  // the GEMMs clamp the count to cap
    }
  }
}

}  // namespace

hipError_t launch_front(const FrontArgs& fa, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  if (fa.D > FR_MAX_D || fa.D % 64) return hipErrorInvalidValue;
  if (!fa.sync) return hipErrorInvalidValue;
  if (!fa.wr) {
    dim3 grid((unsigned)((fa.L + FR_ROWS - 1) / FR_ROWS)), block(FR_THREADS);
    if (fa.x_dtype == DGMOE_F32) hipLaunchKernelGGL((k_norm<float>), grid, block, 0, st, fa);
    else hipLaunchKernelGGL((k_norm<uint16_t>), grid, block, 0, st, fa);
    return hipGetLastError();
  }
  if (!fa.sync || fa.E > SEL_MAX_E || fa.k > SEL_MAX_K || fa.spin_limit < 1) return hipErrorInvalidValue;
  const float rc = (float)(1.0 / sqrt((double)fa.D));
  // Workgroups of two expert tiles once that still gives two workgroups per
  // CU: the x rows are then loaded once for two tiles instead of once per tile.
  // (Measured at 2048 positions: two tiles 44 us, four 46 us, eight 109 us, one
  // 68 us.)
  const int64_t rb = (fa.L + FR_ROWS - 1) / FR_ROWS;
  const int tiles = (fa.E + FR_TILE - 1) / FR_TILE;
  const int nt = rb * ((tiles + 1) / 2) >= 512 ? 2 : 1;
  dim3 grid((unsigned)rb, (unsigned)((tiles + nt - 1) / nt)), block(FR_THREADS);
  const dgmoe_matrix m = *fa.wr;
#define DG_FR(XT, RF)                                                                  \
  do {                                                                                 \
    if (nt == 2) hipLaunchKernelGGL((k_front<XT, RF, 2>), grid, block, 0, st, fa, m, rc); \
    else hipLaunchKernelGGL((k_front<XT, RF, 1>), grid, block, 0, st, fa, m, rc);         \
  } while (0)
#define DG_FR_X(XT)                                   \
  switch (m.dtype) {                                  \
    case DGMOE_F32: DG_FR(XT, DGMOE_F32); break;      \
    case DGMOE_BF16: DG_FR(XT, DGMOE_BF16); break;    \
    case DGMOE_Q8G64: DG_FR(XT, DGMOE_Q8G64); break;  \
    default: return hipErrorInvalidValue;             \
  }
  if (fa.x_dtype == DGMOE_F32) {
    DG_FR_X(float)
  } else {
    DG_FR_X(uint16_t)
  }
#undef DG_FR_X
#undef DG_FR
  return hipGetLastError();
}

hipError_t launch_assign(const int32_t* idx, int64_t L, int k, int E, int32_t* cnt, int32_t* list,
                         int64_t cap, uint32_t* sync, uint64_t stamp, hipStream_t st) {
  (void)hipGetLastError();
  const int64_t Lk = L * k;
  hipLaunchKernelGGL(k_assign, dim3((unsigned)((Lk + 255) / 256)), dim3(256), 0, st, idx, Lk, k, E,
                     cnt, list, cap, sync, stamp);
  return hipGetLastError();
}
