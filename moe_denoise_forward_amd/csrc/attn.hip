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
//                   16-key block), and the V^T operand is read in that order
//                   from the row-major V tile by transposing LDS reads.  K
//                   and V tiles go from global memory to LDS by DMA (no
//                   registers), swizzled for conflict-free fragment reads,
//                   one or two tiles ahead of the tile being computed.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// K and V tiles go from global memory straight to LDS (global_load_lds, 16
// bytes per lane, 1 KB per wave instruction), with no registers and no
// transposition: both stay row-major ([key][head_dim], rows of R = 2 HD bytes)
// with their 16-byte chunks swizzled so the MFMA fragment reads are free of
// bank conflicts.  An LDS pass serves 256 bytes (64 banks of 4 bytes):
//   K: 16 lanes read the same chunk of 16 consecutive rows; chunk c of row r
//      sits at 16-byte slot c ^ fk(r), fk(r) = r & 15 (rows of 256 bytes or
//      more), (r >> 1) & 7 at head_dim 64 (rows of 128 bytes: odd rows fill
//      the other half of a 256-byte window);
//   V: 32 lanes read 32 bytes of each of 8 consecutive rows (the transposing
//      reads below); 32-byte slot m of row r sits at m ^ fv(r), fv(r) = r & 7,
//      or (r >> 1) & 3 at head_dim 64.
// A DMA instruction writes 64 consecutive 16-byte LDS slots; each lane loads
// the global chunk that belongs in its slot (the swizzles are involutions).
template <int HD>
__device__ __forceinline__ int k_swz(int r, int c) {
  return c ^ (HD >= 128 ? (r & 15) : ((r >> 1) & 7));
}
template <int HD>
__device__ __forceinline__ int v_slot(int r, int m) {
  return m ^ (HD >= 128 ? (r & 7) : ((r >> 1) & 3));
}
template <int HD>
__device__ __forceinline__ int v_swz(int r, int c) {
  return (v_slot<HD>(r, c >> 1) << 1) | (c & 1);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i & 3 of the 4 x 16-bit block addressed by lane 4 e + (i >> 2), as its
// element e (e < 4).  So if lane 4 e + d of the group addresses 4 consecutive
// head_dim values 4 d .. 4 d + 3 of key row k_e, lane i receives V[k_e][i]
// for e = 0..3: the transposed fragment the MFMA takes, read from a row-major
// V tile.
__device__ __forceinline__ s16x4 ds_read_tr16(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// CS waves share each 16-row group: every one computes the group's scores,
// and wave slice cs accumulates the output columns [cs HD/CS, (cs+1) HD/CS),
// so each wave holds 1/CS of the output accumulators (4 CS waves).  NS: LDS
// stages of the K / V tiles (the DMA for tile i + NS - 1 is issued while tile
// i is computed).
template <int HD, int CS, int NS>
__global__ __launch_bounds__(256 * CS) void k_attn(AttnArgs a) {
  constexpr int NW = 4 * CS;          // waves
  constexpr int R = 2 * HD;           // bytes of a row
  constexpr int NC = HD / 32;         // 32-wide head_dim chunks of a score MFMA chain
  constexpr int NB = HD / 16 / CS;    // 16-wide output blocks of a wave
  constexpr int TB = AT_KT * R;       // bytes of one K (or V) tile
  constexpr int NI = 2 * TB / 1024;   // DMA instructions per tile (K, then V)
  constexpr int NIW = NI / NW;        // ... per wave
  static_assert(NI % NW == 0, "whole DMA instructions per wave");
  static_assert(NS == 2 || NS == 3, "the waits below count at most one later tile");
  __shared__ __attribute__((aligned(1024))) unsigned char sKV[NS][2 * TB];
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
  // wait for them here, before the tile DMAs: a wait inside the loop would
  // count the DMAs too and drain them
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) asm volatile("" : "+v"(qf[cc]));

  // The keys in tiles of AT_KT: first the committed rows s0 .. kv_len-1
  // (Tenc tiles, the last one ragged), then the canvas rows (the rest, the
  // last one ragged), so that a tile is wholly in the cache or wholly in the
  // canvas and its rows are a uniform base plus small per-lane offsets.  Rows
  // past a tile's valid count re-read its last valid row; their scores are
  // masked, so their (finite) values are multiplied by zero.
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
  // the wave's NIW DMA instructions of a tile into stage st: instruction
  // ii = wv + NW i writes LDS bytes [1024 ii, 1024 ii + 1024) of the stage
  // (K in the first TB bytes, V in the next)
  auto dma_tile = [&](int tile, int st) {
    const TileSrc ts = tile_src(tile);
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int ii = wv + NW * i;
      const bool isv = ii >= NI / 2;
      const int pos = 1024 * (isv ? ii - NI / 2 : ii) + 16 * lane;  // byte in the K or V tile
      const int row = pos / R, p = (pos % R) / 16;
      const int c = isv ? v_swz<HD>(row, p) : k_swz<HD>(row, p);
      const int key = min(row, ts.valid - 1);
      const _Float16* src = (isv ? ts.vb : ts.kb) + (int64_t)key * HD + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)&sKV[st][1024 * ii], 16, 0, 0);
    }
  };

  float4_t o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // the running max and the exponentials in base 2 (scores times log2 e)
  float m_run = -1e30f, l_run = 0.f;

  // one tile from LDS stage st: the scores, the online softmax, the output
  auto compute = [&](int st, int valid) {
    const unsigned char* kt = sKV[st];
    const unsigned char* vt = sKV[st] + TB;
    // S^T = K Q^T: lane holds keys 16 b + 4 g16 + i for query n16.  The two
    // 16-key blocks' chains alternate (step j: block j & 1, head_dim chunk
    // j >> 1, i.e. 16-byte chunk 4 (j >> 1) + g16 of row 16 (j & 1) + n16)
    // and each K fragment is read from LDS AT_RING steps ahead.
    auto kfrag = [&](int j) {
      const int row = 16 * (j & 1) + n16;
      return *(const u32x4*)(kt + row * R + 16 * k_swz<HD>(row, 4 * (j >> 1) + g16));
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
    // O^T += V^T P^T.  The MFMA's k slot 8 g16 + 4 b + i is key 16 b + 4 g16 + i
    // (the score registers' order), so the V^T fragment of output block ob
    // (head_dim 16 ob ..) is two transposing reads: lane 4 e + d of group g16
    // addresses head_dim 16 ob + 4 d .. +3 of key 4 g16 + e (then 16 + 4 g16 + e).
    // Fragments are read AT_RING blocks ahead.
    const int rv = 4 * g16 + (n16 >> 2);
    auto vaddr = [&](int row, int ob) {
      return (const _Float16*)(vt + row * R + 32 * v_slot<HD>(row, ob) + 8 * (n16 & 3));
    };
    auto vfrag = [&](int ob) {
      return __builtin_shufflevector(ds_read_tr16(vaddr(rv, ob)), ds_read_tr16(vaddr(rv + 16, ob)), 0, 1, 2, 3, 4, 5,
                                     6, 7);
    };
    {
      s16x8 vr[AT_RING];
#pragma unroll
      for (int j = 0; j < AT_RING; ++j) vr[j] = vfrag(NB * cs + j);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const s16x8 f = vr[b % AT_RING];
        if (b + AT_RING < NB) vr[b % AT_RING] = vfrag(NB * cs + b + AT_RING);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(f), P, o[b], 0, 0, 0);
      }
    }
  };

  // The stream of tiles: stage i % NS holds tile tb + i.  Per step: wait for
  // this wave's DMA of the tile (the NS - 2 later tiles' DMAs stay in flight),
  // a barrier (every wave's part of the tile has landed, and every wave is
  // done with the stage the next DMA overwrites), the DMA of tile + NS - 1,
  // then the tile's compute.  The DMAs are the only vector-memory operations
  // of the loop, so vmcnt counts exactly them.
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (tb + i < te) dma_tile(tb + i, i);
  for (int tile = tb, st = 0; tile < te; ++tile, st = st == NS - 1 ? 0 : st + 1) {
    // DMAs issued after this tile's: those of the tiles tile + 1 .. tile + NS - 2
    const int later = min(te - 1 - tile, NS - 2);
    if (later <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
    else if (NS == 3 || later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (NIW & 15) | ((NIW >> 4) << 14));
    // the empty asm statements keep the compiler from moving LDS accesses
    // across the barrier (it is not a memory fence: a fence would wait for
    // every DMA in flight)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (tile + NS - 1 < te) dma_tile(tile + NS - 1, st == 0 ? NS - 1 : st - 1);
    compute(st, tile_src(tile).valid);
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
  // LDS stages of K / V tiles: three (two tiles in flight) where they fit,
  // two at head_dim 512 (64 KB a tile)
  constexpr int NS = HD >= 512 ? 2 : 3;
  hipLaunchKernelGGL((k_attn<HD, CS, NS>), dim3((unsigned)(a.Hkv * a.chunks), (unsigned)((M + AT_ROWS - 1) / AT_ROWS)),
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
