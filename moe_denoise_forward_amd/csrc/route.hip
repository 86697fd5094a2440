// RMSNorm, router logits, top-k selection and the expert-major plan.
//
// The router follows the diffgemma contract (Part II section 2.1, MoE-order
// bullet): weightless RMSNorm of the block input, times router_scale and
// hidden^-1/2, a linear map to E logits, the top-k by logit with ties going to
// the lower expert index, and softmax weights over the selected k times
// per_expert_scale (the mlx-bun dossier's Router takes the softmax over the
// selected scores, which is the same quantity).  Logits stay fp32 (the
// contract's precision policy keeps router logits in f32: routing is control
// flow).
#include "common.h"
#include "kernels.h"

// ---------------------------------------------------------------- RMSNorm
// One wave per row.  Sum of squares in fp32 (lane-strided partials, then a
// fixed butterfly), r = 1/sqrt(mean + eps).
template <typename XT>
__device__ __forceinline__ float load_x(const XT* p, int64_t i);
template <>
__device__ __forceinline__ float load_x<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}

// One workgroup of 256 threads per row; each thread owns 8-wide chunks
// c = tid + 256 j of the row (at most 4 chunks: D <= 8192), loaded once into
// registers with 16-byte loads.
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

__device__ __forceinline__ void store8h(_Float16* p, const float* v, const float* w) {
  half8_t h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)(v[i] * w[i]);
  *(half8_t*)p = h;
}

template <typename XT>
__global__ __launch_bounds__(256) void k_norm(const XT* __restrict__ x, int64_t L, int D, float eps,
                                              const float* __restrict__ w_pre,
                                              const float* __restrict__ w_pre2,
                                              const float* __restrict__ router_scale, float rc,
                                              _Float16* __restrict__ a, _Float16* __restrict__ b,
                                              float* __restrict__ u) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nch = D / 8;
  float v[4][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nch) {
      load8<XT>(x + row * D + 8 * c, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[j][i] * v[j][i];
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(tot / (float)D + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c >= nch) continue;
    float xh[8], w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xh[i] = v[j][i] * r;
    const int64_t o = row * D + 8 * c;
    if (a) { load8<float>(w_pre + 8 * c, w); store8h(a + o, xh, w); }
    if (b) { load8<float>(w_pre2 + 8 * c, w); store8h(b + o, xh, w); }
    if (u) {
      load8<float>(router_scale + 8 * c, w);
      float4 p0, p1;
      p0.x = (xh[0] * w[0]) * rc; p0.y = (xh[1] * w[1]) * rc; p0.z = (xh[2] * w[2]) * rc; p0.w = (xh[3] * w[3]) * rc;
      p1.x = (xh[4] * w[4]) * rc; p1.y = (xh[5] * w[5]) * rc; p1.z = (xh[6] * w[6]) * rc; p1.w = (xh[7] * w[7]) * rc;
      *(float4*)(u + o) = p0;
      *(float4*)(u + o + 4) = p1;
    }
  }
}

hipError_t launch_norm(const void* x, int x_dtype, int64_t L, int D, float eps,
                       const float* w_pre, const float* w_pre2, const float* router_scale,
                       _Float16* a, _Float16* b, float* u, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const float rc = (float)(1.0 / sqrt((double)D));
  dim3 grid((unsigned)L), block(256);
  if (x_dtype == DGMOE_F32)
    hipLaunchKernelGGL(k_norm<float>, grid, block, 0, st, (const float*)x, L, D, eps, w_pre,
                       w_pre2, router_scale, rc, a, b, u);
  else
    hipLaunchKernelGGL(k_norm<uint16_t>, grid, block, 0, st, (const uint16_t*)x, L, D, eps,
                       w_pre, w_pre2, router_scale, rc, a, b, u);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router logits
// Tile: 16 rows x 16 experts per workgroup; the 4 waves split K into quarters
// and the partial tiles are summed in LDS in a fixed order.  fp32 MFMA
// 16x16x4: lane l holds A[m=l%16][k=l/16], B[k=l/16][n=l%16] and produces
// C[m=4*(l/16)+i][n=l%16].  Each lane loads 4 consecutive k (a float4) and the
// 4 MFMAs of a 16-wide k block take them in turn: MFMA j's slot g carries
// k = k0 + 4g + j, for A and B alike.
template <int RFMT>
__device__ __forceinline__ float4_t router_w4(const dgmoe_matrix& w, int D, int e, int k) {
  float4_t r;
  if constexpr (RFMT == DGMOE_F32) {
    const float4 v = *(const float4*)((const float*)w.data + (int64_t)e * D + k);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  } else if constexpr (RFMT == DGMOE_BF16) {
    const uint2 v = *(const uint2*)((const uint16_t*)w.data + (int64_t)e * D + k);
    r[0] = bitcast<float>(v.x << 16); r[1] = bitcast<float>(v.x & 0xFFFF0000u);
    r[2] = bitcast<float>(v.y << 16); r[3] = bitcast<float>(v.y & 0xFFFF0000u);
  } else {  // Q8G64: row-major bytes, (scale, bias) pairs row-major per group
    const uint32_t v = *(const uint32_t*)((const uint8_t*)w.data + (int64_t)e * D + k);
    const uint32_t sb = ((const uint32_t*)w.scale_bias)[(int64_t)e * (D / 64) + k / 64];
    const float s = half_bits_to_float((uint16_t)(sb & 0xFFFFu));
    const float b = half_bits_to_float((uint16_t)(sb >> 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = fmaf(s, (float)((v >> (8 * j)) & 0xFFu), b);
  }
  return r;
}

template <int RFMT>
__global__ __launch_bounds__(256) void k_router(const float* __restrict__ u, int64_t L, int D,
                                                int E, dgmoe_matrix w,
                                                const float* __restrict__ bias,
                                                float* __restrict__ logits) {
  __shared__ float part[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int e0 = blockIdx.y * 16;
  const int m = lane & 15, g = lane >> 4;
  const int64_t arow = row0 + m;
  const int be = e0 + m;  // expert this lane feeds as B column n = lane % 16
  const bool a_ok = arow < L, b_ok = be < E;
  const int kq = D / 4;
  const int kbeg = wave * kq, kend = kbeg + kq;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  // two 16-wide k blocks per iteration, the next pair loaded before the MFMAs
  // of the current one (kq is a multiple of 16; an odd last block is handled
  // by the tail)
  auto load_a = [&](int k, float4_t& av) {
    av = (float4_t){0.f, 0.f, 0.f, 0.f};
    if (a_ok && k < kend) {
      const float4 t = *(const float4*)(u + arow * D + k + 4 * g);
      av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
    }
  };
  auto load_b = [&](int k, float4_t& bv) {
    bv = (float4_t){0.f, 0.f, 0.f, 0.f};
    if (b_ok && k < kend) bv = router_w4<RFMT>(w, D, be, k + 4 * g);
  };
  float4_t a0, a1, b0, b1;
  load_a(kbeg, a0); load_b(kbeg, b0);
  load_a(kbeg + 16, a1); load_b(kbeg + 16, b1);
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    float4_t na0, na1, nb0, nb1;
    load_a(k0 + 32, na0); load_b(k0 + 32, nb0);
    load_a(k0 + 48, na1); load_b(k0 + 48, nb1);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], b1[j], acc, 0, 0, 0);
    a0 = na0; a1 = na1; b0 = nb0; b1 = nb1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][lane * 4 + i] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = ((part[0][lane * 4 + i] + part[1][lane * 4 + i]) + part[2][lane * 4 + i]) +
                      part[3][lane * 4 + i];
      const int64_t r = row0 + 4 * g + i;
      const int e = e0 + m;
      if (r < L && e < E) logits[r * E + e] = s + (bias ? bias[e] : 0.f);
    }
  }
}

hipError_t launch_router(const float* u, int64_t L, int D, int E, const dgmoe_matrix* wr,
                         const float* bias, float* logits, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  dim3 grid((unsigned)((L + 15) / 16), (unsigned)((E + 15) / 16)), block(256);
  switch (wr->dtype) {
    case DGMOE_F32:
      hipLaunchKernelGGL(k_router<DGMOE_F32>, grid, block, 0, st, u, L, D, E, *wr, bias, logits);
      break;
    case DGMOE_BF16:
      hipLaunchKernelGGL(k_router<DGMOE_BF16>, grid, block, 0, st, u, L, D, E, *wr, bias, logits);
      break;
    default:
      hipLaunchKernelGGL(k_router<DGMOE_Q8G64>, grid, block, 0, st, u, L, D, E, *wr, bias, logits);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k
// One wave per row.  Each lane holds up to 4 logits (expert lane + 64c); k
// rounds of a wave arg-max with the order (logit desc, index asc); the owner
// of each winner drops it.  Lane j keeps round j's winner.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t L, int E,
                                              int k, const float* __restrict__ pes,
                                              int32_t* __restrict__ idx_out,
                                              float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= L) return;
  float v[4];
  bool live[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    live[c] = e < E;
    v[c] = live[c] ? logits[row * E + e] : 0.f;
  }
  int my_e = 0;
  float my_z = 0.f;
  float top = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (live[c] && (bi == 0x7fffffff || better(v[c], lane + 64 * c, bv, bi))) {
        bv = v[c];
        bi = lane + 64 * c;
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the winner (bv, bi)
    if (j == 0) top = bv;
    if (lane == j) { my_e = bi; my_z = bv; }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c == bi) live[c] = false;
  }
  const float ex = (lane < k) ? expf(my_z - top) : 0.f;
  const float den = wave_sum(ex);
  if (lane < k) {
    idx_out[row * k + lane] = my_e;
    w_out[row * k + lane] = (ex / den) * pes[my_e];
  }
}

hipError_t launch_topk(const float* logits, int64_t L, int E, int k, const float* pes,
                       int32_t* idx, float* w, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  dim3 grid((unsigned)((L + 3) / 4)), block(256);
  hipLaunchKernelGGL(k_topk, grid, block, 0, st, logits, L, E, k, pes, idx, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- plan
// One workgroup of 1024 threads turns the routing into an expert-major order
// of the L*k (token, slot) pairs -- the pages' "iterate over the experts, gather
// the tokens routed to each, run them once, send the results back".
//   1. counts per expert (integer LDS atomics, order-free), exclusive scan;
//   2. rank of each pair among the earlier pairs of its expert, chunk by chunk:
//      every pair of the chunk sets its bit in a per-expert bit mask, and its
//      rank is the popcount of the bits below it (plus the rows of earlier
//      chunks), so rows of an expert stay in ascending pair order;
//   3. the tile tables: group g (expert g, or the dense MLP as group E) has
//      ceil(rows/DG_MT) row tiles times its column tiles; entry t of a table is
//      {group, first row, rows, column tile}, ordered by group, column tile,
//      row tile.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = s_wave[w];
      s_wave[w] = run;
      run += t;
    }
    s_wave[nw] = run;
  }
  __syncthreads();
  const int res = s_wave[wave] + inc - v;
  if (total) *total = s_wave[nw];
  __syncthreads();
  return res;
}

__device__ void write_tiles(int total, const int* s_pref, const int* s_rows, const int* s_off,
                            int ngroups, int nt_exp, int nt_dense, int E, int4* table) {
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    int lo = 0, hi = ngroups;  // last group with s_pref[g] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= t) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int mts = (s_rows[g] + DG_MT - 1) / DG_MT;
    const int local = t - s_pref[g];
    const int nt = local / mts, mt = local % mts;
    (void)nt_exp; (void)nt_dense; (void)E;
    table[t] = make_int4(g, s_off[g] + mt * DG_MT, min(DG_MT, s_rows[g] - mt * DG_MT), nt);
  }
}

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ idx, int64_t L, int k,
                                               int E, int nt_gu_exp, int nt_gu_dense, int nt_dn,
                                               int dense_rows, PlanOut out) {
  __shared__ uint32_t s_mask[256][33];
  __shared__ int s_cnt[258], s_off[258], s_base[258], s_pg[258], s_pd[258];
  __shared__ int s_wave[17];
  const int tid = threadIdx.x;
  const int64_t Lk = L * k;
  for (int e = tid; e < 258; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int64_t p = tid; p < Lk; p += 1024) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  // rows per group (dense last), exclusive offsets of the expert rows
  int rows = 0;
  if (tid < E) rows = s_cnt[tid];
  else if (tid == E) rows = dense_rows;
  const int off = block_exclusive_scan(tid < E ? rows : 0, s_wave, nullptr);
  if (tid <= E) {
    s_off[tid] = tid < E ? off : 0;
    s_base[tid] = off;
    s_cnt[tid] = rows;
  }
  __syncthreads();
  // stable ranks, 1024 pairs at a time
  for (int64_t c0 = 0; c0 < Lk; c0 += 1024) {
    for (int w = tid; w < E * 32; w += 1024) s_mask[w >> 5][w & 31] = 0u;
    __syncthreads();
    const int64_t p = c0 + tid;
    const int e = p < Lk ? idx[p] : -1;
    const bool valid = e >= 0 && e < E;
    const int wi = tid >> 5, bi = tid & 31;
    if (valid) atomicOr(&s_mask[e][wi], 1u << bi);
    __syncthreads();
    if (valid) {
      int r = __popc(s_mask[e][wi] & ((1u << bi) - 1u));
      for (int w = 0; w < wi; ++w) r += __popc(s_mask[e][w]);
      out.perm[s_base[e] + r] = (int32_t)p;
    }
    __syncthreads();
    if (tid < E) {
      int c = 0;
      for (int w = 0; w < 32; ++w) c += __popc(s_mask[tid][w]);
      s_base[tid] += c;
    }
    __syncthreads();
  }
  // tile counts and tables
  const int mt = (tid <= E) ? (s_cnt[tid] + DG_MT - 1) / DG_MT : 0;
  const int tg = (tid <= E) ? mt * (tid < E ? nt_gu_exp : nt_gu_dense) : 0;
  const int td = (tid <= E) ? mt * nt_dn : 0;
  int tot_g = 0, tot_d = 0;
  const int pg = block_exclusive_scan(tg, s_wave, &tot_g);
  const int pd = block_exclusive_scan(td, s_wave, &tot_d);
  if (tid <= E) {
    s_pg[tid] = pg;
    s_pd[tid] = pd;
    out.grp_off[tid] = s_off[tid];
    out.grp_cnt[tid] = s_cnt[tid];
  }
  if (tid == E) {  // the dense group is last: its first entry closes the expert range
    out.n_tiles[0] = tot_g;
    out.n_tiles[1] = 0;
    out.n_tiles[2] = pg;
    out.n_tiles[3] = 0;
    out.n_tiles[4] = tot_d;
    out.n_tiles[5] = 0;
    out.n_tiles[6] = pd;
    out.n_tiles[7] = 0;
  }
  __syncthreads();
  write_tiles(tot_g, s_pg, s_cnt, s_off, E + 1, nt_gu_exp, nt_gu_dense, E, out.tiles_gu);
  write_tiles(tot_d, s_pd, s_cnt, s_off, E + 1, nt_dn, nt_dn, E, out.tiles_dn);
}

hipError_t launch_plan(const int32_t* idx, int64_t L, int k, int E, int nt_gu_exp,
                       int nt_gu_dense, int nt_dn, int dense_rows, const PlanOut& out,
                       hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, idx, L, k, E, nt_gu_exp, nt_gu_dense,
                     nt_dn, dense_rows, out);
  return hipGetLastError();
}
