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

template <typename XT>
__global__ __launch_bounds__(256) void k_norm(const XT* __restrict__ x, int64_t L, int D, float eps,
                                              const float* __restrict__ w_pre,
                                              const float* __restrict__ w_pre2,
                                              const float* __restrict__ router_scale, float rc,
                                              _Float16* __restrict__ a, _Float16* __restrict__ b,
                                              float* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= L) return;
  const XT* xr = x + row * D;
  float ss = 0.f;
  for (int i = lane; i < D; i += 64) {
    float v = load_x<XT>(xr, i);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  for (int i = lane; i < D; i += 64) {
    float xh = load_x<XT>(xr, i) * r;
    if (a) a[row * D + i] = (_Float16)(xh * w_pre[i]);
    if (b) b[row * D + i] = (_Float16)(xh * w_pre2[i]);
    if (u) u[row * D + i] = (xh * router_scale[i]) * rc;
  }
}

hipError_t launch_norm(const void* x, int x_dtype, int64_t L, int D, float eps,
                       const float* w_pre, const float* w_pre2, const float* router_scale,
                       _Float16* a, _Float16* b, float* u, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const float rc = (float)(1.0 / sqrt((double)D));
  dim3 grid((unsigned)((L + 3) / 4)), block(256);
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
  } else if constexpr (RFMT == DGMOE_Q8G64) {
    const uint32_t v = *(const uint32_t*)((const uint8_t*)w.data + (int64_t)e * D + k);
    const int64_t gi = (int64_t)e * (D / 64) + k / 64;
    const float s = half_bits_to_float(w.scales[gi]), b = half_bits_to_float(w.biases[gi]);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = fmaf(s, (float)((v >> (8 * j)) & 0xFFu), b);
  } else {  // Q4G64: inputs k..k+3 of word k/8, elements 8w + 2p + h at bits 4p + 16h
    const uint32_t v = *((const uint32_t*)w.data + ((int64_t)e * D + k) / 8);
    const int64_t gi = (int64_t)e * (D / 64) + k / 64;
    const float s = half_bits_to_float(w.scales[gi]), b = half_bits_to_float(w.biases[gi]);
    const int c0 = k & 7;  // 0 or 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + j, p = c >> 1, h = c & 1;
      r[j] = fmaf(s, (float)((v >> (4 * p + 16 * h)) & 0xFu), b);
    }
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
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    const int k = k0 + 4 * g;
    float4_t av = {0.f, 0.f, 0.f, 0.f}, bv = {0.f, 0.f, 0.f, 0.f};
    if (a_ok) {
      const float4 t = *(const float4*)(u + arow * D + k);
      av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
    }
    if (b_ok) bv = router_w4<RFMT>(w, D, be, k);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
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
    case DGMOE_Q8G64:
      hipLaunchKernelGGL(k_router<DGMOE_Q8G64>, grid, block, 0, st, u, L, D, E, *wr, bias, logits);
      break;
    default:
      hipLaunchKernelGGL(k_router<DGMOE_Q4G64>, grid, block, 0, st, u, L, D, E, *wr, bias, logits);
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
// One workgroup of 1024 threads.  Thread (e, part) owns expert e and a
// contiguous slice of positions; it counts the pairs (t, j) with idx == e,
// a block-wide exclusive scan over (e, part) gives each its first row, and a
// second pass writes the pair indices.  Rows of an expert are therefore in
// ascending pair order (a stable counting sort; the pages' "iterate over the
// experts, gather their tokens, send results back").  The tile tables follow:
// group g has ceil(rows/DG_MT) row tiles times its column tiles.
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

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ idx, int64_t L, int k,
                                               int E, int P, int nt_gu_exp, int nt_gu_dense,
                                               int nt_dn, int dense_rows, PlanOut out) {
  __shared__ int s_wave[17];
  __shared__ int s_cnt[1024];
  __shared__ int s_base[1024];
  const int tid = threadIdx.x;
  const int e = tid / P, part = tid % P;
  const bool active = e < E;
  const int64_t chunk = (L + P - 1) / P;
  const int64_t t0 = (int64_t)part * chunk;
  const int64_t t1 = t0 + chunk < L ? t0 + chunk : L;
  int c = 0;
  if (active)
    for (int64_t t = t0; t < t1; ++t)
      for (int j = 0; j < k; ++j) c += (idx[t * k + j] == e);
  s_cnt[tid] = c;
  const int base = block_exclusive_scan(c, s_wave, nullptr);
  s_base[tid] = base;
  if (active) {
    int pos = base;
    for (int64_t t = t0; t < t1; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[t * k + j] == e) out.perm[pos++] = (int32_t)(t * k + j);
  }
  __syncthreads();
  // per group: rows, offset and tile counts (group E = dense)
  int rows = 0, off = 0;
  if (tid < E) {
    off = s_base[tid * P];
    for (int p = 0; p < P; ++p) rows += s_cnt[tid * P + p];
  } else if (tid == E) {
    rows = dense_rows;
  }
  const int mt = (rows + DG_MT - 1) / DG_MT;
  const int tg = (tid <= E) ? mt * (tid < E ? nt_gu_exp : nt_gu_dense) : 0;
  const int td = (tid <= E) ? mt * nt_dn : 0;
  int tot_g = 0, tot_d = 0;
  const int pg = block_exclusive_scan(tg, s_wave, &tot_g);
  const int pd = block_exclusive_scan(td, s_wave, &tot_d);
  if (tid <= E) {
    out.grp_off[tid] = off;
    out.grp_cnt[tid] = rows;
    out.pref_gu[tid] = pg;
    out.pref_dn[tid] = pd;
  }
  if (tid == 0) {
    out.pref_gu[E + 1] = tot_g;
    out.pref_dn[E + 1] = tot_d;
  }
}

hipError_t launch_plan(const int32_t* idx, int64_t L, int k, int E, int nt_gu_exp,
                       int nt_gu_dense, int nt_dn, int dense_rows, const PlanOut& out,
                       hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const int P = 1024 / E;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, idx, L, k, E, P, nt_gu_exp, nt_gu_dense,
                     nt_dn, dense_rows, out);
  return hipGetLastError();
}
