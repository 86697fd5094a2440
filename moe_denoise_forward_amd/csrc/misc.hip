// Combine + post-norms + residual + layer_scalar, and the GPU packer/unpacker.
#include <algorithm>

#include "common.h"
#include "kernels.h"

// ---------------------------------------------------------------- combine
// One workgroup per position t:
//   moe = sum_{j=0..k-1} w[t*k + j] * slots[t*k + j]   (fp16 slot rows widened
//         exactly; slot order, fixed;
//         each product rounded once before it is added)
//   h   = rms(h1) * post_ff_norm_1 + rms(moe) * post_ff_norm_2
//   y   = layer_scalar * (x + rms(h) * post_ff_norm)
// (the ML@Berkeley MOEBlock's last two lines and the model's x * layer_scalar;
// the mlx-bun dossier's DecoderLayer: post_feedforward_layernorm(h1 + h2),
// residual, then layer_scalar).  With moe_out set it stops after the sum.
//
// The workgroup has one thread per 8 columns of the row (D <= 8192, so at
// most 1024 threads), so the row lives in registers and every load of a
// thread (16 bytes each) is issued before the first add.  Block sums go
// through one LDS slot per wave and are added in wave order, so results do
// not depend on timing.
constexpr int CB_MAX_THREADS = 1024;

template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float (*red)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red[wave][i] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w)
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += red[w][i];
}

// Eight consecutive x values as two float4.
template <typename XT>
__device__ __forceinline__ void ld_x8(const XT* p, float4& a, float4& b);
template <>
__device__ __forceinline__ void ld_x8<float>(const float* p, float4& a, float4& b) {
  a = ((const float4*)p)[0];
  b = ((const float4*)p)[1];
}
__device__ __forceinline__ float4 bf16x4(uint32_t lo, uint32_t hi) {
  return make_float4(bitcast<float>(lo << 16), bitcast<float>(lo & 0xFFFF0000u),
                     bitcast<float>(hi << 16), bitcast<float>(hi & 0xFFFF0000u));
}
template <>
__device__ __forceinline__ void ld_x8<uint16_t>(const uint16_t* p, float4& a, float4& b) {
  const uint4 v = *(const uint4*)p;
  a = bf16x4(v.x, v.y);
  b = bf16x4(v.z, v.w);
}

__device__ __forceinline__ float4 half4_to_float4(uint32_t lo, uint32_t hi) {
  return make_float4((float)bitcast<_Float16>((uint16_t)(lo & 0xFFFFu)), (float)bitcast<_Float16>((uint16_t)(lo >> 16)),
                     (float)bitcast<_Float16>((uint16_t)(hi & 0xFFFFu)), (float)bitcast<_Float16>((uint16_t)(hi >> 16)));
}

__device__ __forceinline__ float dot4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(__fadd_rn(a.x, b.x), __fadd_rn(a.y, b.y), __fadd_rn(a.z, b.z),
                     __fadd_rn(a.w, b.w));
}
__device__ __forceinline__ float4 mul4(float s, float4 v) {
  return make_float4(__fmul_rn(s, v.x), __fmul_rn(s, v.y), __fmul_rn(s, v.z), __fmul_rn(s, v.w));
}
__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }

// h = rms(h1) * w1 + rms(moe) * w2 for four columns
__device__ __forceinline__ float4 branch_sum(float4 hv, float4 m, float4 w1, float4 w2, float r1, float r2) {
  return make_float4((hv.x * r1) * w1.x + (m.x * r2) * w2.x, (hv.y * r1) * w1.y + (m.y * r2) * w2.y,
                     (hv.z * r1) * w1.z + (m.z * r2) * w2.z, (hv.w * r1) * w1.w + (m.w * r2) * w2.w);
}
// y = layer_scalar * (x + rms(h) * w) for four columns
__device__ __forceinline__ float4 residual(float ls, float4 x, float4 h, float4 w, float r3) {
  return make_float4(ls * (x.x + (h.x * r3) * w.x), ls * (x.y + (h.y * r3) * w.y),
                     ls * (x.z + (h.z * r3) * w.z), ls * (x.w + (h.w * r3) * w.w));
}

// bitwise choice between two float4: a where keep is all ones, b where it is zero
__device__ __forceinline__ float4 pick4(float4 a, float4 b, uint32_t keep) {
  auto f = [keep](float x, float y) {
    return bitcast<float>((bitcast<uint32_t>(x) & keep) | (bitcast<uint32_t>(y) & ~keep));
  };
  return make_float4(f(a.x, b.x), f(a.y, b.y), f(a.z, b.z), f(a.w, b.w));
}

template <typename XT, bool MOE_ONLY>
__global__ __launch_bounds__(CB_MAX_THREADS) void k_combine(
    const _Float16* __restrict__ slots, const float* __restrict__ h1, int h1_parts, int64_t L,
    const int32_t* __restrict__ idx,
    const float* __restrict__ rw, const XT* __restrict__ x, int D, int k, int E, float eps, const float* __restrict__ wp1,
    const float* __restrict__ wp2, const float* __restrict__ wp, float ls,
    float* __restrict__ moe_out, void* y, int y_dtype) {
  __shared__ float red2[CB_MAX_THREADS / 64][2];
  __shared__ float red1[CB_MAX_THREADS / 64][1];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int nc = D / 8;  // 8-column chunks, one per thread
  const bool on = (int)threadIdx.x < nc;
  const int c = on ? (int)threadIdx.x : nc - 1;  // past the row: the last chunk again, dropped
  const int64_t col = 8 * (int64_t)c;
  // Every operand is requested before the first is used, in one round trip:
  // the row's k expert indices and weights (lane j holds slot j's, k <= 32),
  // its first eight slot rows and, for the block, h1, x and the three norm
  // weights.  Nothing below branches on a loaded value, so no load is moved
  // behind another's wait.
  const int jl = lane < k ? lane : k - 1;
  const int e_l = idx[t * k + jl];
  const float w_l = rw[t * k + jl];
  const uint4* srow = (const uint4*)(slots + t * k * D);  // 8 fp16 per chunk
  uint4 v[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) v[jj] = srow[(int64_t)min(jj, k - 1) * nc + c];
  float4 hv0, hv1, xv0, xv1, w1a, w1b, w2a, w2b, w3a, w3b;
  if (!MOE_ONLY) {
    // h1 = its partial sums over the dense down projection's K chunks, in order
    hv0 = ld4(h1 + t * D + col);
    hv1 = ld4(h1 + t * D + col + 4);
    for (int q = 1; q < h1_parts; ++q) {
      const float* hp = h1 + (int64_t)q * L * D + t * D + col;
      hv0 = add4(hv0, ld4(hp));
      hv1 = add4(hv1, ld4(hp + 4));
    }
    ld_x8<XT>(x + t * D + col, xv0, xv1);
    w1a = ld4(wp1 + col); w1b = ld4(wp1 + col + 4);
    w2a = ld4(wp2 + col); w2b = ld4(wp2 + col + 4);
    w3a = ld4(wp + col); w3b = ld4(wp + col + 4);
  }
  // slots in order j = 0 .. k-1, each product rounded once before it is added;
  // a slot whose expert index is outside [0, E) (its row was never written)
  // leaves the sum as it is, as do the padding steps j >= k
  float4 m0 = make_float4(0.f, 0.f, 0.f, 0.f), m1 = m0;
  for (int j0 = 0; j0 < k; j0 += 8) {
    if (j0 > 0)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v[jj] = srow[(int64_t)min(j0 + jj, k - 1) * nc + c];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      const int e = __builtin_amdgcn_readlane(e_l, j & 63);
      const float wj = bitcast<float>(__builtin_amdgcn_readlane(bitcast<int>(w_l), j & 63));
      const uint32_t keep = (j < k && e >= 0 && e < E) ? 0xFFFFFFFFu : 0u;
      const float4 n0 = add4(m0, mul4(wj, half4_to_float4(v[jj].x, v[jj].y)));
      const float4 n1 = add4(m1, mul4(wj, half4_to_float4(v[jj].z, v[jj].w)));
      m0 = pick4(n0, m0, keep);
      m1 = pick4(n1, m1, keep);
    }
  }
  if (MOE_ONLY) {
    if (on) {
      ((float4*)(moe_out + t * D + col))[0] = m0;
      ((float4*)(moe_out + t * D + col))[1] = m1;
    }
    return;
  }
  float ss[2] = {on ? dot4(hv0) + dot4(hv1) : 0.f, on ? dot4(m0) + dot4(m1) : 0.f};  // h1, moe
  block_sum<2>(ss, red2);
  const float r1 = 1.0f / sqrtf(ss[0] / (float)D + eps);
  const float r2 = 1.0f / sqrtf(ss[1] / (float)D + eps);
  const float4 h0 = branch_sum(hv0, m0, w1a, w2a, r1, r2), hh1 = branch_sum(hv1, m1, w1b, w2b, r1, r2);
  float sh[1] = {on ? dot4(h0) + dot4(hh1) : 0.f};
  block_sum<1>(sh, red1);
  const float r3 = 1.0f / sqrtf(sh[0] / (float)D + eps);
  if (!on) return;
  const float4 o0 = residual(ls, xv0, h0, w3a, r3), o1 = residual(ls, xv1, hh1, w3b, r3);
  if (y_dtype == DGMOE_F32) {
    ((float4*)((float*)y + t * D + col))[0] = o0;
    ((float4*)((float*)y + t * D + col))[1] = o1;
  } else {
    const uint32_t a = (uint32_t)float_to_bf16_bits(o0.x) | ((uint32_t)float_to_bf16_bits(o0.y) << 16);
    const uint32_t b = (uint32_t)float_to_bf16_bits(o0.z) | ((uint32_t)float_to_bf16_bits(o0.w) << 16);
    const uint32_t cc = (uint32_t)float_to_bf16_bits(o1.x) | ((uint32_t)float_to_bf16_bits(o1.y) << 16);
    const uint32_t d = (uint32_t)float_to_bf16_bits(o1.z) | ((uint32_t)float_to_bf16_bits(o1.w) << 16);
    *(uint4*)((uint16_t*)y + t * D + col) = make_uint4(a, b, cc, d);
  }
}

hipError_t launch_combine(const _Float16* slots, const float* h1, int h1_parts, const int32_t* idx,
                          const float* w, const void* x,
                          int x_dtype, int64_t L, int D, int k, int E, float eps,
                          const float* wp1, const float* wp2,
                          const float* wp, float layer_scalar, float* moe_out, void* y,
                          int y_dtype, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const int nc = D / 8;  // one thread per 8 columns (D <= 8192)
  if (nc > CB_MAX_THREADS) return hipErrorInvalidValue;
  const int threads = (nc + 63) / 64 * 64;
  dim3 grid((unsigned)L), block(threads);
#define DG_CB(XT, MO)                                                                          \
  hipLaunchKernelGGL((k_combine<XT, MO>), grid, block, 0, st, slots, h1, h1_parts, L, idx, w, (const XT*)x, D, k, \
                     E, eps, wp1, wp2, wp, layer_scalar, moe_out, y, y_dtype)
  if (moe_out) {
    if (x_dtype == DGMOE_F32) DG_CB(float, true);
    else DG_CB(uint16_t, true);
  } else {
    if (x_dtype == DGMOE_F32) DG_CB(float, false);
    else DG_CB(uint16_t, false);
  }
#undef DG_CB
  return hipGetLastError();
}

// ---------------------------------------------------------------- pack
// One thread per (row, group) of GS = 64 inputs (Q4G64, Q8G64) or 32 (Q4G32).
// Min/max affine quantiser with fp32 arithmetic and fp16 scale/bias (the
// mlx-bun dossier's affine group-64 quantisation; the diffgemma contract's q4
// group-32 experts; the min/max rule is this library's reading):
//   scale = fp16((max - min) / qmax), bias = fp16(min)
//   q = clamp(rint((w - bias) / scale), 0, qmax), q = 0 when scale == 0.
// __fsub_rn / __fdiv_rn keep every step a single IEEE-rounded operation.
// Output positions follow the layouts of include/dgmoe.h: Q4G64 and Q4G32
// tiled by blocks of 64 rows (the same code words), Q8G64 row-major.
// Q4G64 word holding inputs 64q + 32h + 8g + (0..7) of a row, and the index of
// the row's (scale, bias) pair of group q (Q4G64) or of half h of group q
// (Q4G32); groups counts 64-input groups.
__device__ __forceinline__ int64_t q4_word(int64_t row, int64_t q, int g, int h, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return (((b * groups + q) * 4 + g) * 16 + n) * 8 + 2 * s + h;
}
__device__ __forceinline__ int64_t q4_pair(int64_t row, int64_t q, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return ((b * groups + q) * 16 + n) * 4 + s;
}
__device__ __forceinline__ int64_t q4g32_pair(int64_t row, int64_t q, int h, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return ((b * groups + q) * 16 + n) * 8 + 2 * s + h;
}

// Q6G32 high-plane word of row `row`, 64-input group q, lane group g (its
// bit 2 (4h + p) + 16t holds the high bits of input 64q + 32h + 8g + 2p + t)
__device__ __forceinline__ int64_t q6_high_word(int64_t row, int64_t q, int g, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return (((b * groups + q) * 4 + g) * 16 + n) * 4 + s;
}

template <int FMT> struct PackFmt;
template <> struct PackFmt<DGMOE_Q4G64> { static constexpr int GS = 64, BITS = 4; };
template <> struct PackFmt<DGMOE_Q4G32> { static constexpr int GS = 32, BITS = 4; };
template <> struct PackFmt<DGMOE_Q8G64> { static constexpr int GS = 64, BITS = 8; };

template <int FMT>
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int64_t rows,
                                              int64_t cols, void* __restrict__ codes,
                                              uint32_t* __restrict__ scale_bias) {
  constexpr int GS = PackFmt<FMT>::GS, BITS = PackFmt<FMT>::BITS;
  const int64_t ng = cols / GS, groups = cols / 64;
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * ng) return;
  const int64_t row = gi / ng, qq = gi % ng;
  const float* src = w + gi * GS;
  float lo = src[0], hi = src[0];
  for (int i = 1; i < GS; ++i) {
    const float v = src[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float qmax = (float)((1 << BITS) - 1);
  const _Float16 s16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), qmax);
  const _Float16 b16 = (_Float16)lo;
  const uint32_t pair = (uint32_t)bitcast<uint16_t>(s16) | ((uint32_t)bitcast<uint16_t>(b16) << 16);
  const float s = (float)s16, b = (float)b16;
  uint32_t qv[GS];
  for (int i = 0; i < GS; ++i) {
    float r = 0.f;
    if (s != 0.f) r = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(src[i], b), s)), 0.f), qmax);
    qv[i] = (uint32_t)r;
  }
  if (BITS == 4) {
    // the 64-input group q and the first word of this group within it
    const int64_t q = GS == 64 ? qq : qq >> 1;
    const int wd0 = GS == 64 ? 0 : 4 * (int)(qq & 1);
    if (GS == 64) scale_bias[q4_pair(row, q, groups)] = pair;
    else scale_bias[q4g32_pair(row, q, (int)(qq & 1), groups)] = pair;
    for (int u = 0; u < GS / 8; ++u) {  // inputs 8 wd .. 8 wd + 7 of the 64-group: h = wd / 4, g = wd % 4
      const int wd = wd0 + u;
      uint32_t v = 0;
      for (int p = 0; p < 4; ++p)
        for (int t = 0; t < 2; ++t) v |= qv[8 * u + 2 * p + t] << (4 * p + 16 * t);
      ((uint32_t*)codes)[q4_word(row, q, wd & 3, wd >> 2, groups)] = v;
    }
  } else {
    scale_bias[gi] = pair;
    uint32_t* out = (uint32_t*)codes + gi * 16;
    for (int wd = 0; wd < 16; ++wd)
      out[wd] = qv[4 * wd] | (qv[4 * wd + 1] << 8) | (qv[4 * wd + 2] << 16) | (qv[4 * wd + 3] << 24);
  }
}

// ---------------------------------------------------------------- NVFP4
// The codecs of the NVFP4 format (include/dgmoe.h): E4M3 scales (bias 7,
// 3 mantissa bits, subnormals m * 2^-9, largest 448) and E2M1 codes (bit 3
// the sign; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).  Every step is an exact or
// single-rounding fp32 operation.

// E4M3 byte of t >= 0: round to nearest even; above 448 saturates to 448.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  t = fminf(t, 896.0f);
  if (t < 0x1p-6f) return (uint32_t)rintf(t * 512.0f);  // steps of 2^-9; 8 is the smallest normal
  int ex;
  const float mant = frexpf(t, &ex);  // t = mant * 2^ex, mant in [0.5, 1)
  int e = ex - 1;
  int m = (int)rintf((2.0f * mant - 1.0f) * 8.0f);
  if (m == 8) {
    e += 1;
    m = 0;
  }
  return t > 448.0f ? 0x7Eu : (uint32_t)min(((e + 7) << 3) | m, 0x7E);
}
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
}
// E2M1 code of x: nearest magnitude, ties to the even code, above 6 -> 6.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(x) >> 31) << 3);
}
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float v = m < 4 ? 0.5f * (float)m : (float)(2u << ((m - 4) >> 1)) * (1.0f + 0.5f * (float)(m & 1));
  return (c & 8u) ? -v : v;
}
// byte of the E4M3 scale of row `row`, 16-input block j of 64-input group q
__device__ __forceinline__ int64_t fp4_scale_byte(int64_t row, int64_t q, int j, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return (((b * groups + q) * 16 + n) * 4 + s) * 4 + j;
}

// The trailer (64 bytes after the rows*cols/16 scale bytes): cleared, then
// word 1 collects amax (non-negative floats order as their bits), then word 0
// gets gs = amax / 2688 from the quantising kernel.
__global__ __launch_bounds__(64) void k_fp4_clear(uint32_t* __restrict__ trailer) {
  if (threadIdx.x < 16) trailer[threadIdx.x] = 0u;
}

// One atomic per workgroup (the maximum is exact in any order).
__global__ __launch_bounds__(256) void k_fp4_amax(const float* __restrict__ w, int64_t n,
                                                  uint32_t* __restrict__ trailer) {
  __shared__ float wmax[4];
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    m = fmaxf(m, fabsf(w[i]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(trailer + 1, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

// One thread per (row, 16-input block).
__global__ __launch_bounds__(256) void k_pack_fp4(const float* __restrict__ w, int64_t rows,
                                                  int64_t cols, uint32_t* __restrict__ codes,
                                                  uint8_t* __restrict__ sbytes,
                                                  uint32_t* __restrict__ trailer) {
  const int64_t nb16 = cols / 16, groups = cols / 64;
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * nb16) return;
  const int64_t row = gi / nb16, blk = gi % nb16, q = blk >> 2;
  const int j = (int)(blk & 3);
  const float amax = __uint_as_float(trailer[1]);
  const float gs = __fdiv_rn(amax, 2688.0f);
  if (gi == 0) trailer[0] = __float_as_uint(gs);
  const float* src = w + gi * 16;
  float bmax = 0.0f;
  for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(src[i]));
  const float t = gs > 0.0f ? __fdiv_rn(bmax, __fmul_rn(6.0f, gs)) : 0.0f;
  const uint32_t byte = e4m3_encode(t);
  const float es = __fmul_rn(e4m3_value(byte), gs);
  sbytes[fp4_scale_byte(row, q, j, groups)] = (uint8_t)byte;
  // inputs 16 j + 8 u .. +7 of the group: word (g = 2 (j & 1) + u, h = j >> 1)
  for (int u = 0; u < 2; ++u) {
    uint32_t v = 0;
    for (int p = 0; p < 4; ++p)
      for (int tt = 0; tt < 2; ++tt) {
        const float x = src[8 * u + 2 * p + tt];
        const uint32_t c = es > 0.0f ? e2m1_encode(__fdiv_rn(x, es)) : 0u;
        v |= c << (4 * p + 16 * tt);
      }
    codes[q4_word(row, q, 2 * (j & 1) + u, j >> 1, groups)] = v;
  }
}

// Q6G32: one thread per (row, 64-input group); each 32-input half is
// quantised like the affine formats above with 6-bit codes; the thread writes
// the group's eight low-plane words, its four high-plane words and two pairs.
__global__ __launch_bounds__(256) void k_pack_q6(const float* __restrict__ w, int64_t rows,
                                                 int64_t cols, uint32_t* __restrict__ codes,
                                                 uint32_t* __restrict__ scale_bias) {
  const int64_t groups = cols / 64;
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * groups) return;
  const int64_t row = gi / groups, q = gi % groups;
  uint32_t hw[4] = {0u, 0u, 0u, 0u};
  for (int h = 0; h < 2; ++h) {
    const float* src = w + gi * 64 + 32 * h;
    float lo = src[0], hi = src[0];
    for (int i = 1; i < 32; ++i) {
      lo = fminf(lo, src[i]);
      hi = fmaxf(hi, src[i]);
    }
    const _Float16 s16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), 63.0f);
    const _Float16 b16 = (_Float16)lo;
    scale_bias[q4g32_pair(row, q, h, groups)] =
        (uint32_t)bitcast<uint16_t>(s16) | ((uint32_t)bitcast<uint16_t>(b16) << 16);
    const float s = (float)s16, b = (float)b16;
    for (int g = 0; g < 4; ++g) {
      uint32_t v = 0;
      for (int p = 0; p < 4; ++p)
        for (int t = 0; t < 2; ++t) {
          float r = 0.f;
          if (s != 0.f) r = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(src[8 * g + 2 * p + t], b), s)), 0.f), 63.f);
          const uint32_t c = (uint32_t)r;
          v |= (c & 15u) << (4 * p + 16 * t);
          hw[g] |= (c >> 4) << (2 * (4 * h + p) + 16 * t);
        }
      codes[q4_word(row, q, g, h, groups)] = v;
    }
  }
  uint32_t* high = codes + rows * cols / 8;
  for (int g = 0; g < 4; ++g) high[q6_high_word(row, q, g, groups)] = hw[g];
}

hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, int fmt, void* codes,
                       uint16_t* scale_bias, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  if (fmt == DGMOE_Q6G32) {
    const int64_t ng = rows * (cols / 64);
    hipLaunchKernelGGL(k_pack_q6, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, w, rows,
                       cols, (uint32_t*)codes, (uint32_t*)scale_bias);
    return hipGetLastError();
  }
  if (fmt == DGMOE_NVFP4) {
    uint8_t* sb = (uint8_t*)scale_bias;
    uint32_t* trailer = (uint32_t*)(sb + rows * cols / 16);
    hipLaunchKernelGGL(k_fp4_clear, dim3(1), dim3(64), 0, st, trailer);
    const int64_t n = rows * cols;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(k_fp4_amax, dim3((unsigned)blocks), dim3(256), 0, st, w, n, trailer);
    const int64_t nb = rows * (cols / 16);
    hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, w, rows,
                       cols, (uint32_t*)codes, sb, trailer);
    return hipGetLastError();
  }
  const int64_t ng = rows * (cols / (fmt == DGMOE_Q4G32 ? 32 : 64));
  dim3 grid((unsigned)((ng + 255) / 256)), block(256);
  uint32_t* sb = (uint32_t*)scale_bias;
  if (fmt == DGMOE_Q4G64)
    hipLaunchKernelGGL(k_pack<DGMOE_Q4G64>, grid, block, 0, st, w, rows, cols, codes, sb);
  else if (fmt == DGMOE_Q4G32)
    hipLaunchKernelGGL(k_pack<DGMOE_Q4G32>, grid, block, 0, st, w, rows, cols, codes, sb);
  else
    hipLaunchKernelGGL(k_pack<DGMOE_Q8G64>, grid, block, 0, st, w, rows, cols, codes, sb);
  return hipGetLastError();
}

// ---------------------------------------------------------------- unpack
// One thread per 8 inputs of the row-major output.  F32: fmaf(scale, q, bias),
// the exact value rounded once to fp32.  F16: for Q4G64 and Q4G32 exactly the
// in-register dequantisation the GEMM kernels use; for Q8G64 the same
// single-rounding fp16 fma.
template <int FMT, bool F16OUT>
__global__ __launch_bounds__(256) void k_unpack(const void* __restrict__ codes,
                                                const uint32_t* __restrict__ scale_bias,
                                                int64_t rows, int64_t cols,
                                                void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-input chunk
  const int64_t per_row = cols / 8, groups = cols / 64;
  if (i >= rows * per_row) return;
  const int64_t row = i / per_row, c8 = i % per_row, q = c8 / 8, wd = c8 % 8;
  uint32_t pair, qv[8];
  if (FMT == DGMOE_NVFP4) {
    const uint8_t* sb = (const uint8_t*)scale_bias;
    const float gs = __uint_as_float(((const uint32_t*)(sb + rows * cols / 16))[0]);
    const float sc = e4m3_value(sb[fp4_scale_byte(row, q, (int)(wd >> 1), groups)]);
    const uint32_t v = ((const uint32_t*)codes)[q4_word(row, q, (int)(wd & 3), (int)(wd >> 2), groups)];
    for (int p = 0; p < 4; ++p)
      for (int h = 0; h < 2; ++h) {
        // e2m1 * e4m3 is exact in fp32; times gs: one rounding.  The empty asm
        // keeps the fp32 product: without it the multiply and the fp16
        // conversion fuse into one mixed fma that rounds once, straight to fp16.
        float val = __fmul_rn(__fmul_rn(e2m1_value((v >> (4 * p + 16 * h)) & 0xFu), sc), gs);
        asm volatile("" : "+v"(val));
        if (F16OUT) ((_Float16*)out)[i * 8 + 2 * p + h] = (_Float16)val;
        else ((float*)out)[i * 8 + 2 * p + h] = val;
      }
    return;
  }
  if (FMT == DGMOE_Q6G32) {
    const int h = (int)(wd >> 2), g = (int)(wd & 3);
    pair = scale_bias[q4g32_pair(row, q, h, groups)];
    const uint32_t v = ((const uint32_t*)codes)[q4_word(row, q, g, h, groups)];
    const uint32_t hw = ((const uint32_t*)codes)[rows * cols / 8 + q6_high_word(row, q, g, groups)] >> (8 * h);
    if (F16OUT) {
      const _Float16 s = bitcast<_Float16>((uint16_t)(pair & 0xFFFFu));
      const _Float16 b = bitcast<_Float16>((uint16_t)(pair >> 16));
      *(half8_t*)((_Float16*)out + i * 8) = dequant_q6_word(v, hw, (half2_t){s, s}, (half2_t){b, b});
      return;
    }
    for (int p = 0; p < 4; ++p)
      for (int t = 0; t < 2; ++t)
        qv[2 * p + t] = ((v >> (4 * p + 16 * t)) & 0xFu) | (((hw >> (2 * p + 16 * t)) & 3u) << 4);
  } else if (FMT == DGMOE_Q4G64 || FMT == DGMOE_Q4G32) {
    pair = FMT == DGMOE_Q4G64 ? scale_bias[q4_pair(row, q, groups)]
                              : scale_bias[q4g32_pair(row, q, (int)(wd >> 2), groups)];
    const uint32_t v = ((const uint32_t*)codes)[q4_word(row, q, (int)(wd & 3), (int)(wd >> 2), groups)];
    if (F16OUT) {
      const _Float16 s = bitcast<_Float16>((uint16_t)(pair & 0xFFFFu));
      const _Float16 b = bitcast<_Float16>((uint16_t)(pair >> 16));
      *(half8_t*)((_Float16*)out + i * 8) = dequant_q4_word(v, (half2_t){s, s}, (half2_t){b, b});
      return;
    }
    for (int p = 0; p < 4; ++p)
      for (int h = 0; h < 2; ++h) qv[2 * p + h] = (v >> (4 * p + 16 * h)) & 0xFu;
  } else {
    pair = scale_bias[row * groups + q];
    const uint2 v = ((const uint2*)codes)[i];
    for (int c = 0; c < 4; ++c) {
      qv[c] = (v.x >> (8 * c)) & 0xFFu;
      qv[4 + c] = (v.y >> (8 * c)) & 0xFFu;
    }
  }
  if (F16OUT) {
    const _Float16 s = bitcast<_Float16>((uint16_t)(pair & 0xFFFFu));
    const _Float16 b = bitcast<_Float16>((uint16_t)(pair >> 16));
    for (int c = 0; c < 8; ++c)
      ((_Float16*)out)[i * 8 + c] = __builtin_elementwise_fma((_Float16)(float)qv[c], s, b);
  } else {
    const float s = half_bits_to_float((uint16_t)(pair & 0xFFFFu));
    const float b = half_bits_to_float((uint16_t)(pair >> 16));
    for (int c = 0; c < 8; ++c) ((float*)out)[i * 8 + c] = fmaf(s, (float)qv[c], b);
  }
}

hipError_t launch_unpack(const void* codes, const uint16_t* scale_bias, int64_t rows,
                         int64_t cols, int fmt, int out_dtype, void* out, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const int64_t n8 = rows * cols / 8;
  dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  const bool f16 = out_dtype == DGMOE_F16;
  const uint32_t* sb = (const uint32_t*)scale_bias;
  if (fmt == DGMOE_Q4G64) {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_Q4G64, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_Q4G64, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  } else if (fmt == DGMOE_Q4G32) {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_Q4G32, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_Q4G32, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  } else if (fmt == DGMOE_Q6G32) {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_Q6G32, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_Q6G32, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  } else if (fmt == DGMOE_NVFP4) {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_NVFP4, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_NVFP4, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  } else {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_Q8G64, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_Q8G64, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  }
  return hipGetLastError();
}
