// Denoise attention of one decoder layer: the canvas rows attend to the
// committed window of the KV cache and bidirectionally to the whole canvas.
//
// What it computes ("diffgemma -- architecture & implemented contract", Part
// II section 2 "Two attention phases" (Denoise) and section 2.1 (Norms, RoPE,
// no 1/sqrt(d) scale, full layers without v_proj); "DiffusionGemma
// Explained", the attention section (rotate, AttentionBlock.forward); the
// mlx-bun port dossier section 2, Attention.__call__ and _make_decoder_masks):
//   q = rope(rms(q_raw) * w_q), k = rope(rms(k_raw) * w_k), v = rms(v_raw)
//   (full layers: v = rms(k_raw)), per head, at position kv_len + t;
//   o = softmax(q . K^T) V over [cache rows s0 .. kv_len-1 | canvas rows],
//   unit scale, query head h reading KV head h / (H / H_kv).
//
//   k_attn_prep     one workgroup per canvas row: the cos / sin of the row's
//                   rotated pairs (angles in fp64) into LDS, then one wave per
//                   head vector: RMSNorm (weights for q, k), the split-half
//                   rotation through LDS, fp16 q / k / v into the workspace.
//   k_attn          flash attention per (64 query rows of one KV head, key
//                   range).  The rows are the (query head, canvas row) pairs
//                   of the KV head's query group, so every K / V tile in LDS
//                   serves all of its query heads (GQA).  Per 32-key tile a
//                   wave of 16 rows computes S^T = K Q^T (MFMA 16x16x32 f16,
//                   fp32 accumulation; K fragments from LDS, Q^T fragments
//                   held in registers), so the query sits on lane % 16 and
//                   the online softmax's max and rescale stay per lane (two
//                   cross-lane-group maxima per tile); then O^T += V^T P^T
//                   with P^T taken straight from the score registers: the
//                   MFMA's k index runs over the keys in the order the score
//                   layout holds them (lane group g: keys 4g..4g+3 of each
//                   16-key block), and V^T is staged in LDS in that order.
//                   K and V^T tiles are double-buffered: the next tile's
//                   loads are in flight while the current one is computed.
//   k_attn_combine  the key ranges of a row merged in a fixed order
//                   (rescaled to the row's max), divided by the sum of
//                   exponentials, written as fp32 or bf16.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int AT_KT = DG_ATTN_KT;
constexpr int AT_ROWS = DG_ATTN_ROWS;

template <typename XT>
__device__ __forceinline__ float at_load(const XT* p);
template <>
__device__ __forceinline__ float at_load<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float at_load<uint16_t>(const uint16_t* p) { return bf16_bits_to_float(*p); }

// ---------------------------------------------------------------- prep
template <typename XT, int HD>
__global__ __launch_bounds__(256) void k_attn_prep(AttnArgs a) {
  constexpr int PER = HD / 64;  // elements per lane: d = lane + 64 i
  __shared__ float s_cos[HD / 2], s_sin[HD / 2];
  __shared__ float s_y[4][HD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t = blockIdx.x;
  const double pos = (double)(a.kv_len + t);
  const double lt = log((double)a.theta);
  for (int j = tid; j < a.n_rot; j += 256) {
    double sn, cs;
    sincos(pos * exp(-2.0 * (double)j / (double)a.den * lt), &sn, &cs);
    s_cos[j] = (float)cs;
    s_sin[j] = (float)sn;
  }
  __syncthreads();
  const int nvec = a.H + 2 * a.Hkv;
  for (int c = w; c < nvec; c += 4) {
    const bool isq = c < a.H, isk = !isq && c < a.H + a.Hkv;
    const int head = isq ? c : isk ? c - a.H : c - a.H - a.Hkv;
    const void* src = isq ? a.q : (isk || !a.v) ? a.k : a.v;
    const int64_t ld = (int64_t)(isq ? a.H : a.Hkv) * HD;
    const XT* row = (const XT*)src + t * ld + (int64_t)head * HD;
    float x[PER];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x[i] = at_load<XT>(row + lane + 64 * i);
      ss += x[i] * x[i];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
    const float* wv = isq ? a.wq : isk ? a.wk : nullptr;
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = wv ? (x[i] * r) * wv[lane + 64 * i] : x[i] * r;
    _Float16* dst = (isq ? a.qp + ((int64_t)head * a.L + t) * HD
                         : (isk ? a.kp : a.vp) + ((int64_t)head * a.L + t) * HD);
    if (!isq && !isk) {  // v: no rotation
#pragma unroll
      for (int i = 0; i < PER; ++i) dst[lane + 64 * i] = (_Float16)x[i];
      continue;
    }
    // the rotation reads each element's partner through LDS (one wave's row;
    // a wave's LDS accesses are performed in order)
#pragma unroll
    for (int i = 0; i < PER; ++i) s_y[w][lane + 64 * i] = x[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      float o = x[i];
      if (d < a.n_rot) {
        o = x[i] * s_cos[d] - s_y[w][d + a.stride] * s_sin[d];
      } else if (d >= a.stride && d < a.stride + a.n_rot) {
        const int j = d - a.stride;
        o = x[i] * s_cos[j] + s_y[w][j] * s_sin[j];
      }
      dst[d] = (_Float16)o;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();  // every lane has read s_y before the next vector rewrites it
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

// ---------------------------------------------------------------- flash attention
// Register arrays of 16-byte pieces as ext vectors, so they stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t u4_half(const u32x4& v, int e) {
  return (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int KLD = HD + 8;         // K tile row stride (halfs), padded
  constexpr int VLD = AT_KT + 8;      // V^T row stride (halfs), padded
  constexpr int NC = HD / 32;         // 32-wide head_dim chunks of a score MFMA chain
  constexpr int NB = HD / 16;         // 16-wide output blocks
  constexpr int C8 = HD / 8;          // 16-byte pieces of a row
  constexpr int KU = (AT_KT * C8 + 255) / 256;  // K pieces per thread
  constexpr int VU = (HD + 255) / 256;          // V units (4 keys x 8 columns) per thread
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][AT_KT * KLD];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][HD * VLD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, n16 = lane & 15;
  const int n = blockIdx.y, ch = blockIdx.z;
  const int G = a.H / a.Hkv;
  const int64_t M = (int64_t)G * a.L;
  const int64_t r = (int64_t)blockIdx.x * AT_ROWS + 16 * w + n16;
  const bool rvalid = r < M;
  const int64_t rq = rvalid ? r : M - 1;  // rows past the group redo its last row, unwritten
  const int gq = (int)(rq / a.L);
  const int64_t t = rq - (int64_t)gq * a.L;
  const int h = n * G + gq;

  // Q^T fragments: lane (head_dim 32 cc + 8 g16 .. +7, query n16)
  u32x4 qf[NC];
  const _Float16* qrow = a.qp + ((int64_t)h * a.L + t) * HD + 8 * g16;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = *(const u32x4*)(qrow + 32 * cc);

  const int64_t nk = a.n_enc + a.L;
  const int T = (int)((nk + AT_KT - 1) / AT_KT);
  const int tb = ch * a.tiles_per_chunk;
  const int te = min(T, tb + a.tiles_per_chunk);

  // key kj of this KV head: a committed cache row, or a canvas row (padding
  // keys past nk read the last canvas row and are masked / zeroed); chosen
  // by selects, so that every load is issued on every path
  auto key_row = [&](int64_t kj, const _Float16* cache, const _Float16* canvas) -> const _Float16* {
    const bool enc = kj < a.n_enc;
    const int64_t row = enc ? (int64_t)n * a.cap + a.s0 + kj
                            : (int64_t)n * a.L + min(kj - a.n_enc, a.L - 1);
    return (enc ? cache : canvas) + row * HD;
  };
  u32x4 kreg[KU];
  u32x4 vreg[VU * 4];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = min(tid + 256 * i, AT_KT * C8 - 1);
      kreg[i] = *(const u32x4*)(key_row((int64_t)tile * AT_KT + u / C8, a.kc, a.kp) + 8 * (u % C8));
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = min(tid + 256 * i, HD - 1);
      const int quad = u / C8, c8 = u % C8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vreg[4 * i + kk] = *(const u32x4*)(key_row((int64_t)tile * AT_KT + 4 * quad + kk, a.vc, a.vp) + 8 * c8);
    }
  };
  auto store_tile = [&](int buf, int tile) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + 256 * i;
      if (u < AT_KT * C8) *(u32x4*)&sK[buf][(u / C8) * KLD + 8 * (u % C8)] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + 256 * i;
      if (u >= HD) continue;
      const int quad = u / C8, c8 = u % C8;
      const int slot0 = quad < 4 ? 8 * quad : 8 * (quad - 4) + 4;  // keys 16b + 4g + i -> slot 8g + 4b + i
      u32x4 vv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bool live = (int64_t)tile * AT_KT + 4 * quad + kk < nk;
        vv[kk] = live ? vreg[4 * i + kk] : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = u4_half(vv[0], e) | (u4_half(vv[1], e) << 16);
        const uint32_t hi = u4_half(vv[2], e) | (u4_half(vv[3], e) << 16);
        *(uint2*)&sV[buf][(8 * c8 + e) * VLD + slot0] = make_uint2(lo, hi);
      }
    }
  };

  float4_t o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  if (tb < te) {
    load_tile(tb);
    store_tile(0, tb);
  }
  __syncthreads();
  int buf = 0;
  for (int tile = tb; tile < te; ++tile) {
    const bool more = tile + 1 < te;
    if (more) load_tile(tile + 1);
    // S^T = K Q^T: lane holds keys 16 b + 4 g16 + i for query n16
    float4_t s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const u32x4 kf = *(const u32x4*)&sK[buf][(16 * b + n16) * KLD + 32 * cc + 8 * g16];
        s[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(kf), bitcast<half8_t>(qf[cc]),
                                                      s[b], 0, 0, 0);
      }
    }
    float mx = -1e30f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((int64_t)tile * AT_KT + 16 * b + 4 * g16 + i >= nk) s[b][i] = -1e30f;
        mx = fmaxf(mx, s[b][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, DG_WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, DG_WAVE));
    const float m_new = fmaxf(m_run, mx);
    const float sc = expf(m_run - m_new);
    m_run = m_new;
    half8_t P;
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = expf(s[b][i] - m_new);
        ps += p;
        P[4 * b + i] = (_Float16)p;
      }
    l_run = l_run * sc + ps;
    if (__ballot(sc != 1.0f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] *= sc;
    }
    // O^T += V^T P^T: lane holds head_dim columns 16 b + 4 g16 + i for query n16
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const u32x4 vf = *(const u32x4*)&sV[buf][(16 * b + n16) * VLD + 8 * g16];
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(vf), P, o[b], 0, 0, 0);
    }
    if (more) store_tile(buf ^ 1, tile + 1);
    __syncthreads();
    buf ^= 1;
  }
  l_run += __shfl_xor(l_run, 16, DG_WAVE);
  l_run += __shfl_xor(l_run, 32, DG_WAVE);
  if (rvalid) {
    float* op = a.opart + (((int64_t)ch * a.H + h) * a.L + t) * HD + 4 * g16;
#pragma unroll
    for (int b = 0; b < NB; ++b) *(float4_t*)(op + 16 * b) = o[b];
    if (g16 == 0) a.ml[((int64_t)ch * a.H + h) * a.L + t] = make_float2(m_run, l_run);
  }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y, HD = a.hd;
  float m = -1e30f;
  for (int c = 0; c < a.chunks; ++c) m = fmaxf(m, a.ml[((int64_t)c * a.H + h) * a.L + t].x);
  float den = 0.f;
  for (int c = 0; c < a.chunks; ++c) {
    const float2 v = a.ml[((int64_t)c * a.H + h) * a.L + t];
    den += expf(v.x - m) * v.y;
  }
  const float inv = 1.0f / den;
  for (int d4 = threadIdx.x; d4 < HD / 4; d4 += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < a.chunks; ++c) {
      const int64_t row = ((int64_t)c * a.H + h) * a.L + t;
      const float wgt = expf(a.ml[row].x - m);
      const float4 v = *(const float4*)(a.opart + row * HD + 4 * d4);
      acc.x += wgt * v.x;
      acc.y += wgt * v.y;
      acc.z += wgt * v.z;
      acc.w += wgt * v.w;
    }
    const float y[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    const int64_t at = t * (int64_t)a.H * HD + (int64_t)h * HD + 4 * d4;
    if (a.out_dtype == DGMOE_F32) {
      *(float4*)((float*)a.out + at) = make_float4(y[0], y[1], y[2], y[3]);
    } else {
      const uint32_t lo = (uint32_t)float_to_bf16_bits(y[0]) | ((uint32_t)float_to_bf16_bits(y[1]) << 16);
      const uint32_t hi = (uint32_t)float_to_bf16_bits(y[2]) | ((uint32_t)float_to_bf16_bits(y[3]) << 16);
      *(uint2*)((uint16_t*)a.out + at) = make_uint2(lo, hi);
    }
  }
}

template <int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  const dim3 blk(256);
  if (a.in_dtype == DGMOE_F32) hipLaunchKernelGGL((k_attn_prep<float, HD>), dim3((unsigned)a.L), blk, 0, st, a);
  else hipLaunchKernelGGL((k_attn_prep<uint16_t, HD>), dim3((unsigned)a.L), blk, 0, st, a);
  const int64_t M = (int64_t)(a.H / a.Hkv) * a.L;
  hipLaunchKernelGGL((k_attn<HD>), dim3((unsigned)((M + AT_ROWS - 1) / AT_ROWS), (unsigned)a.Hkv,
                                         (unsigned)a.chunks), blk, 0, st, a);
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)a.L, (unsigned)a.H), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int attn_chunks(int64_t L, int H, int Hkv, int hd, int64_t n_keys) {
  const int64_t M = (int64_t)(H / Hkv) * L;
  const int64_t base = (M + AT_ROWS - 1) / AT_ROWS * Hkv;  // workgroups per key range
  const int per_cu = hd >= 512 ? 1 : hd >= 256 ? 2 : 4;   // resident workgroups per CU (LDS)
  const int64_t T = (n_keys + AT_KT - 1) / AT_KT;
  int64_t c = (256 * per_cu + base - 1) / base;
  c = std::max<int64_t>(1, std::min<int64_t>(c, std::min<int64_t>(T, DG_ATTN_MAXCHUNKS)));
  const int64_t tpc = (T + c - 1) / c;  // every range non-empty
  return (int)((T + tpc - 1) / tpc);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  switch (a.hd) {
    case 64: return launch_hd<64>(a, st);
    case 128: return launch_hd<128>(a, st);
    case 256: return launch_hd<256>(a, st);
    case 512: return launch_hd<512>(a, st);
    default: return hipErrorInvalidValue;
  }
}
