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
constexpr float AT_LOG2E = 1.4426950408889634f;
constexpr int AT_RING = 4;  // LDS fragments read ahead of their MFMA
constexpr float AT_SLACK2 = 11.5f;  // lazy-rescale margin of the running max, base 2 (about e^8)

template <typename XT>
__device__ __forceinline__ float at_load(const XT* p);
template <>
__device__ __forceinline__ float at_load<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float at_load<uint16_t>(const uint16_t* p) { return bf16_bits_to_float(*p); }

// ---------------------------------------------------------------- prep
// Grid (canvas rows, groups of four head vectors): wave w of workgroup
// (t, y) takes vector 4 y + w of row t (query heads, then KV heads' k, then
// their v).
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
  for (int c = 4 * (int)blockIdx.y + w; c < min(nvec, 4 * (int)blockIdx.y + 4); c += 4) {
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

// CS waves share each 16-row group: every one computes the group's scores,
// and wave slice cs accumulates the output columns [cs HD/CS, (cs+1) HD/CS),
// so each wave holds 1/CS of the output accumulators (4 CS waves).  PF: the
// number of tiles whose loads are in flight.
template <int HD, int CS, int PF>
__global__ __launch_bounds__(256 * CS) void k_attn(AttnArgs a) {
  constexpr int NT = 256 * CS;        // threads
  constexpr int KLD = HD + 8;         // K tile row stride (halfs), padded
  constexpr int VLD = AT_KT + 8;      // V^T row stride (halfs), padded
  constexpr int NC = HD / 32;         // 32-wide head_dim chunks of a score MFMA chain
  constexpr int NB = HD / 16 / CS;    // 16-wide output blocks of a wave
  constexpr int C8 = HD / 8;          // 16-byte pieces of a row
  constexpr int KU = (AT_KT * C8 + NT - 1) / NT;  // K pieces per thread
  constexpr int VU = (HD + NT - 1) / NT;          // V units (4 keys x 8 columns) per thread
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][AT_KT * KLD];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][HD * VLD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wv & 3, cs = wv >> 2;  // row group, output column slice
  const int g16 = lane >> 4, n16 = lane & 15;
  // grid (KV head x key range, row tile): workgroups are dealt to the XCDs
  // round robin by linear id, so with a multiple of 8 (head, range) pairs
  // every row tile of a pair runs on one XCD and its K / V tiles are shared
  // through that XCD's L2
  const int n = (int)blockIdx.x % a.Hkv, ch = (int)blockIdx.x / a.Hkv;
  const int G = a.H / a.Hkv;
  const int64_t M = (int64_t)G * a.L;
  const int64_t r = (int64_t)blockIdx.y * AT_ROWS + 16 * w + n16;
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

  // The keys in tiles of AT_KT: first the committed rows s0 .. kv_len-1
  // (Tenc tiles, the last one ragged), then the canvas rows (the rest, the
  // last one ragged), so that a tile is wholly in the cache or wholly in the
  // canvas and its rows are a uniform base plus small per-thread offsets.
  // Rows past a tile's valid count re-read its last valid row; their scores
  // are masked and their values zeroed.
  const int Tenc = (int)((a.n_enc + AT_KT - 1) / AT_KT);
  const int T = Tenc + (int)((a.L + AT_KT - 1) / AT_KT);
  const int tb = ch * a.tiles_per_chunk;
  const int te = min(T, tb + a.tiles_per_chunk);
  struct TileSrc {
    const _Float16* kb;
    const _Float16* vb;
    int valid;
  };
  auto tile_src = [&](int tile) {
    const bool enc = tile < Tenc;
    const int64_t j0 = (int64_t)AT_KT * (enc ? tile : tile - Tenc);
    const int64_t row = enc ? (int64_t)n * a.cap + a.s0 + j0 : (int64_t)n * a.L + j0;
    TileSrc ts;
    ts.kb = (enc ? a.kc : a.kp) + row * HD;
    ts.vb = (enc ? a.vc : a.vp) + row * HD;
    ts.valid = (int)min((int64_t)AT_KT, (enc ? a.n_enc : a.L) - j0);
    return ts;
  };
  // a tile's K and V pieces between their loads and their stores to LDS
  struct Stage {
    u32x4 k[KU];
    u32x4 v[VU * 4];
  };
  auto load_tile = [&](Stage& sg, const TileSrc& ts) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = min(tid + NT * i, AT_KT * C8 - 1);
      const int key = min(u / C8, ts.valid - 1);
      sg.k[i] = *(const u32x4*)(ts.kb + key * HD + 8 * (u % C8));
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = min(tid + NT * i, HD - 1);
      const int quad = u & 7, c8 = u >> 3;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = min(4 * quad + kk, ts.valid - 1);
        sg.v[4 * i + kk] = *(const u32x4*)(ts.vb + key * HD + 8 * c8);
      }
    }
  };
  auto store_tile = [&](const Stage& sg, int buf, int valid) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + NT * i;
      if (u < AT_KT * C8) *(u32x4*)&sK[buf][(u / C8) * KLD + 8 * (u % C8)] = sg.k[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + NT * i;
      if (u >= HD) continue;
      // consecutive lanes take consecutive key quads: the eight quads of a
      // row are eight different bank pairs (16 banks); a 16-lane pass also
      // holds the next chunk's lanes, whose rows are 8 rows = 160 banks on,
      // so those lanes write their rows in the order e ^ 4 (16 banks further)
      // and the pass covers all 32 banks once
      const int quad = u & 7, c8 = u >> 3;
      const int slot0 = quad < 4 ? 8 * quad : 8 * (quad - 4) + 4;  // keys 16b + 4g + i -> slot 8g + 4b + i
      const bool flip = (c8 & 1) != 0;
      u32x4 vv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vv[kk] = sg.v[4 * i + kk];
      if (valid < AT_KT) {  // a ragged tile: values past the valid rows are zero
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          if (4 * quad + kk >= valid) vv[kk] = (u32x4){0u, 0u, 0u, 0u};
      }
      // column e of the four keys as two words (keys 0,1 and 2,3), one byte
      // permute each: selector 0x05040100 takes the low halves of both
      // sources, 0x07060302 the high halves
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        lo[e] = __builtin_amdgcn_perm(vv[1][e >> 1], vv[0][e >> 1], sel);
        hi[e] = __builtin_amdgcn_perm(vv[3][e >> 1], vv[2][e >> 1], sel);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int er = flip ? (e ^ 4) : e;
        const uint32_t l2 = flip ? lo[e ^ 4] : lo[e];
        const uint32_t h2 = flip ? hi[e ^ 4] : hi[e];
        *(uint2*)&sV[buf][(8 * c8 + er) * VLD + slot0] = make_uint2(l2, h2);
      }
    }
  };

  float4_t o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // the running max and the exponentials in base 2 (scores times log2 e)
  float m_run = -1e30f, l_run = 0.f;

  // one tile from LDS buffer buf: the scores, the online softmax, the output
  auto compute = [&](int buf, int valid) {
    // S^T = K Q^T: lane holds keys 16 b + 4 g16 + i for query n16.  The two
    // 16-key blocks' chains alternate (step j: block j & 1, head_dim chunk
    // j >> 1) and each K fragment is read from LDS four steps ahead.
    const _Float16* kbase = &sK[buf][n16 * KLD + 8 * g16];
    auto kfrag = [&](int j) {
      return *(const u32x4*)(kbase + 16 * (j & 1) * KLD + 32 * (j >> 1));
    };
    float4_t s[2] = {(float4_t){0.f, 0.f, 0.f, 0.f}, (float4_t){0.f, 0.f, 0.f, 0.f}};
    {
      u32x4 kr[AT_RING];
#pragma unroll
      for (int j = 0; j < AT_RING; ++j) kr[j] = kfrag(j);
#pragma unroll
      for (int j = 0; j < 2 * NC; ++j) {
        const u32x4 f = kr[j % AT_RING];
        if (j + AT_RING < 2 * NC) kr[j % AT_RING] = kfrag(j + AT_RING);
        s[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(f), bitcast<half8_t>(qf[j >> 1]),
                                                          s[j & 1], 0, 0, 0);
      }
    }
    float mx = -1e30f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[b][i] *= AT_LOG2E;
        if (valid < AT_KT && 16 * b + 4 * g16 + i >= valid) s[b][i] = -1e30f;
        mx = fmaxf(mx, s[b][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, DG_WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, DG_WAVE));
    // the reference max moves only when a score passes it by more than
    // AT_SLACK2, so the probabilities stay below 2^AT_SLACK2 (fp16 holds
    // them) and the accumulators are rarely rescaled
    const bool up = mx > m_run + AT_SLACK2;
    const float m_new = up ? mx : m_run;
    const float sc = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    half8_t P;
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[b][i] - m_new);
        ps += p;
        P[4 * b + i] = (_Float16)p;
      }
    l_run = l_run * sc + ps;
    if (__ballot(up)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] *= sc;
    }
    // O^T += V^T P^T: lane holds head_dim columns 16 b + 4 g16 + i for query
    // n16; each V^T fragment read four blocks ahead
    {
      const _Float16* vbase = &sV[buf][(16 * NB * cs + n16) * VLD + 8 * g16];
      u32x4 vr[AT_RING];
#pragma unroll
      for (int j = 0; j < AT_RING; ++j) vr[j] = *(const u32x4*)(vbase + 16 * j * VLD);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4 f = vr[b % AT_RING];
        if (b + AT_RING < NB) vr[b % AT_RING] = *(const u32x4*)(vbase + 16 * (b + AT_RING) * VLD);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(f), P, o[b], 0, 0, 0);
      }
    }
  };

  // The stream of tiles: LDS buffers alternate; the loads of a tile are
  // issued PF tiles ahead of its compute (PF register stages), and a tile is
  // stored to LDS at the end of the step before its compute.
  Stage A, B;
  if (tb < te) {
    load_tile(A, tile_src(tb));
    if (PF == 2 && tb + 1 < te) load_tile(B, tile_src(tb + 1));
    store_tile(A, 0, tile_src(tb).valid);
  }
  // the Q fragments have arrived before the loop (the wait for tile tb
  // covers them), so no wait inside the loop covers more than tile loads
  if (PF == 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  // step of tile `tile` from buffer buf: `mine` is free (its last tile is
  // stored), `other` holds tile + 1 (PF 2; PF 1 uses one stage)
  auto step = [&](int tile, Stage& mine, Stage& other, int buf) {
    const bool has1 = tile + 1 < te, has2 = tile + 2 < te;
    const TileSrc t1 = tile_src(min(tile + 1, te - 1));
    if (PF == 2) {
      if (has2) load_tile(mine, tile_src(tile + 2));
    } else {
      if (has1) load_tile(other, t1);
    }
    compute(buf, tile_src(tile).valid);
    if (has1) store_tile(other, buf ^ 1, t1.valid);
    __syncthreads();
  };
  for (int tile = tb; tile < te; tile += 2) {
    if (PF == 2) {
      step(tile, A, B, 0);
      if (tile + 1 < te) step(tile + 1, B, A, 1);
    } else {
      step(tile, A, A, 0);
      if (tile + 1 < te) step(tile + 1, A, A, 1);
    }
  }
  l_run += __shfl_xor(l_run, 16, DG_WAVE);
  l_run += __shfl_xor(l_run, 32, DG_WAVE);
  if (rvalid) {
    float* op = a.opart + (((int64_t)ch * a.H + h) * a.L + t) * HD + 16 * NB * cs + 4 * g16;
#pragma unroll
    for (int b = 0; b < NB; ++b) *(float4_t*)(op + 16 * b) = o[b];
    if (g16 == 0 && cs == 0) a.ml[((int64_t)ch * a.H + h) * a.L + t] = make_float2(m_run, l_run);
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
    den += exp2f(v.x - m) * v.y;
  }
  const float inv = 1.0f / den;
  for (int d4 = threadIdx.x; d4 < HD / 4; d4 += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < a.chunks; ++c) {
      const int64_t row = ((int64_t)c * a.H + h) * a.L + t;
      const float wgt = exp2f(a.ml[row].x - m);
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
  const dim3 pg((unsigned)a.L, (unsigned)((a.H + 2 * a.Hkv + 3) / 4));
  if (a.in_dtype == DGMOE_F32) hipLaunchKernelGGL((k_attn_prep<float, HD>), pg, blk, 0, st, a);
  else hipLaunchKernelGGL((k_attn_prep<uint16_t, HD>), pg, blk, 0, st, a);
  const int64_t M = (int64_t)(a.H / a.Hkv) * a.L;
  constexpr int CS = HD >= 256 ? 2 : 1;
  // tiles of loads in flight (register stages): two where registers allow;
  // at head_dim 256 a second stage measured no faster (the loads of the
  // stage in flight are waited for anyway when its registers are reused)
  constexpr int PF = HD <= 128 ? 2 : 1;
  hipLaunchKernelGGL((k_attn<HD, CS, PF>), dim3((unsigned)(a.Hkv * a.chunks), (unsigned)((M + AT_ROWS - 1) / AT_ROWS)),
                     dim3(256 * CS), 0, st, a);
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)a.L, (unsigned)a.H), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int attn_tiles(int64_t n_enc, int64_t L) {
  return (int)((n_enc + AT_KT - 1) / AT_KT + (L + AT_KT - 1) / AT_KT);
}

int attn_chunks(int64_t L, int H, int Hkv, int hd, int64_t T) {
  const int64_t M = (int64_t)(H / Hkv) * L;
  const int64_t base = (M + AT_ROWS - 1) / AT_ROWS * Hkv;  // workgroups per key range
  // resident workgroups per CU: one of eight waves at head_dim 256 and 512
  // (registers and LDS), about four of four waves below
  const int per_cu = hd >= 256 ? 1 : 4;
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
