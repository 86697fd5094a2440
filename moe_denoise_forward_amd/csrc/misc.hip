// Combine + post-norms + residual + layer_scalar, and the GPU packer/unpacker.
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
// The workgroup has one thread per float4 chunk of the row (up to 1024
// threads; a thread owns chunks c = tid and tid + blockDim, D <= 8192), so
// the row lives in registers and every slot load of a thread is issued before
// the first add.  Block sums go through one LDS slot per wave and are added in
// wave order, so results do not depend on timing.
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

template <typename XT>
__device__ __forceinline__ float4 ld_x4(const XT* p);
template <>
__device__ __forceinline__ float4 ld_x4<float>(const float* p) { return *(const float4*)p; }
template <>
__device__ __forceinline__ float4 ld_x4<uint16_t>(const uint16_t* p) {
  const uint2 v = *(const uint2*)p;
  return make_float4(bitcast<float>(v.x << 16), bitcast<float>(v.x & 0xFFFF0000u),
                     bitcast<float>(v.y << 16), bitcast<float>(v.y & 0xFFFF0000u));
}

__device__ __forceinline__ float4 half4_to_float4(uint2 v) {
  return make_float4((float)bitcast<_Float16>((uint16_t)(v.x & 0xFFFFu)), (float)bitcast<_Float16>((uint16_t)(v.x >> 16)),
                     (float)bitcast<_Float16>((uint16_t)(v.y & 0xFFFFu)), (float)bitcast<_Float16>((uint16_t)(v.y >> 16)));
}

__device__ __forceinline__ float dot4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(__fadd_rn(a.x, b.x), __fadd_rn(a.y, b.y), __fadd_rn(a.z, b.z),
                     __fadd_rn(a.w, b.w));
}
__device__ __forceinline__ float4 mul4(float s, float4 v) {
  return make_float4(__fmul_rn(s, v.x), __fmul_rn(s, v.y), __fmul_rn(s, v.z), __fmul_rn(s, v.w));
}

template <typename XT>
__global__ __launch_bounds__(CB_MAX_THREADS) void k_combine(
    const _Float16* __restrict__ slots, const float* __restrict__ h1, const int32_t* __restrict__ idx,
    const float* __restrict__ rw, const XT* __restrict__ x, int D, int k, int E, float eps, const float* __restrict__ wp1,
    const float* __restrict__ wp2, const float* __restrict__ wp, float ls,
    float* __restrict__ moe_out, void* y, int y_dtype) {
  __shared__ float red2[CB_MAX_THREADS / 64][2];
  __shared__ float red1[CB_MAX_THREADS / 64][1];
  const int64_t t = blockIdx.x;
  const int nc = D / 4, nt = blockDim.x;
  const int nq = (nc + nt - 1) / nt;  // chunks per thread (uniform): 1 or 2
  uint32_t valid = 0;  // slots whose expert index is in range
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e >= 0 && e < E) valid |= 1u << j;
  }
  const uint2* srow = (const uint2*)(slots + t * k * D);  // 4 fp16 per chunk
  // Every operand of the thread's chunks is loaded before the first reduction:
  // the k slot rows and their weights, h1, x and the three norm weights.  Chunk indices past the
  // row are clamped to the last chunk (valid addresses) and dropped.
  float4 m[2], hv[2], xv[2], w1[2], w2[2], w3[2];
  bool on[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c0 = threadIdx.x + nt * q;
    on[q] = c0 < nc;
    const int c = on[q] ? c0 : nc - 1;
    m[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    hv[q] = xv[q] = w1[q] = w2[q] = w3[q] = m[q];
    if (q >= nq) continue;  // uniform: no second chunk anywhere in the row
    for (int j0 = 0; j0 < k; j0 += 8) {
      uint2 v[8];
      float wj[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {  // addresses clamped to a real slot: loads stay unconditional
        const int j = min(j0 + jj, k - 1);
        v[jj] = srow[(int64_t)j * nc + c];
        wj[jj] = rw[t * k + j];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k && (valid >> (j0 + jj) & 1u)) m[q] = add4(m[q], mul4(wj[jj], half4_to_float4(v[jj])));
    }
    if (!moe_out) {
      hv[q] = ((const float4*)(h1 + t * D))[c];
      xv[q] = ld_x4<XT>(x + t * D + 4 * c);
      w1[q] = ((const float4*)wp1)[c];
      w2[q] = ((const float4*)wp2)[c];
      w3[q] = ((const float4*)wp)[c];
    }
  }
  if (moe_out) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (on[q]) ((float4*)(moe_out + t * D))[threadIdx.x + nt * q] = m[q];
    return;
  }
  float ss[2] = {0.f, 0.f};  // h1, moe
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (on[q]) {
      ss[0] += dot4(hv[q]);
      ss[1] += dot4(m[q]);
    }
  block_sum<2>(ss, red2);
  const float r1 = 1.0f / sqrtf(ss[0] / (float)D + eps);
  const float r2 = 1.0f / sqrtf(ss[1] / (float)D + eps);
  float sh[1] = {0.f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float4 h;
    h.x = (hv[q].x * r1) * w1[q].x + (m[q].x * r2) * w2[q].x;
    h.y = (hv[q].y * r1) * w1[q].y + (m[q].y * r2) * w2[q].y;
    h.z = (hv[q].z * r1) * w1[q].z + (m[q].z * r2) * w2[q].z;
    h.w = (hv[q].w * r1) * w1[q].w + (m[q].w * r2) * w2[q].w;
    m[q] = h;
    if (on[q]) sh[0] += dot4(h);
  }
  block_sum<1>(sh, red1);
  const float r3 = 1.0f / sqrtf(sh[0] / (float)D + eps);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!on[q]) continue;
    const int c = threadIdx.x + nt * q;
    const float4 h = m[q], w = w3[q];
    const float o[4] = {ls * (xv[q].x + (h.x * r3) * w.x), ls * (xv[q].y + (h.y * r3) * w.y),
                        ls * (xv[q].z + (h.z * r3) * w.z), ls * (xv[q].w + (h.w * r3) * w.w)};
    if (y_dtype == DGMOE_F32) {
      ((float4*)y)[t * nc + c] = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      const uint32_t lo = (uint32_t)float_to_bf16_bits(o[0]) | ((uint32_t)float_to_bf16_bits(o[1]) << 16);
      const uint32_t hi = (uint32_t)float_to_bf16_bits(o[2]) | ((uint32_t)float_to_bf16_bits(o[3]) << 16);
      ((uint2*)y)[t * nc + c] = make_uint2(lo, hi);
    }
  }
}

hipError_t launch_combine(const _Float16* slots, const float* h1, const int32_t* idx, const float* w,
                          const void* x,
                          int x_dtype, int64_t L, int D, int k, int E, float eps,
                          const float* wp1, const float* wp2,
                          const float* wp, float layer_scalar, float* moe_out, void* y,
                          int y_dtype, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const int nc = D / 4;
  int threads = (nc + 63) / 64 * 64;
  if (threads > CB_MAX_THREADS) threads = CB_MAX_THREADS;
  dim3 grid((unsigned)L), block(threads);
  if (x_dtype == DGMOE_F32)
    hipLaunchKernelGGL(k_combine<float>, grid, block, 0, st, slots, h1, idx, w, (const float*)x,
                       D, k, E, eps, wp1, wp2, wp, layer_scalar, moe_out, y, y_dtype);
  else
    hipLaunchKernelGGL(k_combine<uint16_t>, grid, block, 0, st, slots, h1, idx, w,
                       (const uint16_t*)x, D, k, E, eps, wp1, wp2, wp, layer_scalar, moe_out, y,
                       y_dtype);
  return hipGetLastError();
}

// ---------------------------------------------------------------- pack
// One thread per (row, 64-input group).  Min/max affine quantiser with fp32
// arithmetic and fp16 scale/bias (the mlx-bun dossier's affine group-64
// quantisation; the min/max rule is this library's reading):
//   scale = fp16((max - min) / qmax), bias = fp16(min)
//   q = clamp(rint((w - bias) / scale), 0, qmax), q = 0 when scale == 0.
// __fsub_rn / __fdiv_rn keep every step a single IEEE-rounded operation.
// Output positions follow the layouts of include/dgmoe.h: Q4G64 tiled by
// blocks of 64 rows, Q8G64 row-major.
// Q4G64 word holding inputs 64q + 32h + 8g + (0..7) of a row, and the index of
// the row's (scale, bias) pair of group q.
__device__ __forceinline__ int64_t q4_word(int64_t row, int64_t q, int g, int h, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return (((b * groups + q) * 4 + g) * 16 + n) * 8 + 2 * s + h;
}
__device__ __forceinline__ int64_t q4_pair(int64_t row, int64_t q, int64_t groups) {
  const int64_t b = row >> 6, s = (row >> 4) & 3, n = row & 15;
  return ((b * groups + q) * 16 + n) * 4 + s;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int64_t rows,
                                              int64_t groups, void* __restrict__ codes,
                                              uint32_t* __restrict__ scale_bias) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * groups) return;
  const int64_t row = gi / groups, q = gi % groups;
  const float* src = w + gi * 64;
  float lo = src[0], hi = src[0];
  for (int i = 1; i < 64; ++i) {
    const float v = src[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float qmax = (float)((1 << BITS) - 1);
  const _Float16 s16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), qmax);
  const _Float16 b16 = (_Float16)lo;
  const uint32_t pair = (uint32_t)bitcast<uint16_t>(s16) | ((uint32_t)bitcast<uint16_t>(b16) << 16);
  const float s = (float)s16, b = (float)b16;
  uint32_t qv[64];
  for (int i = 0; i < 64; ++i) {
    float r = 0.f;
    if (s != 0.f) r = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(src[i], b), s)), 0.f), qmax);
    qv[i] = (uint32_t)r;
  }
  if (BITS == 4) {
    scale_bias[q4_pair(row, q, groups)] = pair;
    for (int wd = 0; wd < 8; ++wd) {  // inputs 8 wd .. 8 wd + 7 of the group: h = wd / 4, g = wd % 4
      uint32_t v = 0;
      for (int p = 0; p < 4; ++p)
        for (int t = 0; t < 2; ++t) v |= qv[8 * wd + 2 * p + t] << (4 * p + 16 * t);
      ((uint32_t*)codes)[q4_word(row, q, wd & 3, wd >> 2, groups)] = v;
    }
  } else {
    scale_bias[gi] = pair;
    uint32_t* out = (uint32_t*)codes + gi * 16;
    for (int wd = 0; wd < 16; ++wd)
      out[wd] = qv[4 * wd] | (qv[4 * wd + 1] << 8) | (qv[4 * wd + 2] << 16) | (qv[4 * wd + 3] << 24);
  }
}

hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, int fmt, void* codes,
                       uint16_t* scale_bias, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const int64_t groups = cols / 64, ng = rows * groups;
  dim3 grid((unsigned)((ng + 255) / 256)), block(256);
  if (fmt == DGMOE_Q4G64)
    hipLaunchKernelGGL(k_pack<4>, grid, block, 0, st, w, rows, groups, codes, (uint32_t*)scale_bias);
  else
    hipLaunchKernelGGL(k_pack<8>, grid, block, 0, st, w, rows, groups, codes, (uint32_t*)scale_bias);
  return hipGetLastError();
}

// ---------------------------------------------------------------- unpack
// One thread per 8 inputs of the row-major output.  F32: fmaf(scale, q, bias),
// the exact value rounded once to fp32.  F16: for Q4G64 exactly the
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
  if (FMT == DGMOE_Q4G64) {
    pair = scale_bias[q4_pair(row, q, groups)];
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
  } else {
    if (f16) hipLaunchKernelGGL((k_unpack<DGMOE_Q8G64, true>), grid, block, 0, st, codes, sb, rows, cols, out);
    else hipLaunchKernelGGL((k_unpack<DGMOE_Q8G64, false>), grid, block, 0, st, codes, sb, rows, cols, out);
  }
  return hipGetLastError();
}
