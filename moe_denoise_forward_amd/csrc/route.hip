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
//   k_prologue  grid (row blocks of 16, input chunks of 256).  Every
//               workgroup takes the full-row RMS of its 16 rows, writes its
//               chunk of the fp16 GEMM operands a = xh*pre_ff_norm and
//               b = xh*pre_ff_norm_2, and the router's partial logits over its
//               chunk (fp32 MFMA) into plog[row][expert][chunk].
//   k_topk      one wave per row sums the partial logits in chunk order,
//               selects the top k, writes the weights and appends each chosen
//               (token, slot) pair to its expert's list (an integer atomic
//               counter per expert gives the position): the pair id t*k + j
//               at list[e*cap + i], its token t at list[(E + e)*cap + i].
//   k_assign    the same lists from a routing given by the caller.
// Each kernel issues its global loads before it first waits on one, so a
// launch costs about one memory latency plus its arithmetic.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PR_ROWS = 16;      // rows per prologue workgroup
constexpr int PR_KC = 256;       // inputs per prologue chunk
constexpr int PR_THREADS = 512;  // 8 waves
constexpr int TK_THREADS = 256;  // top-k: 4 rows per workgroup, one wave each

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

// Sixteen consecutive router weights W[e][k..k+15] of one 64-input group, as
// loaded (raw), and their fp32 values (exact dequant for Q8).
template <int RFMT>
struct RouterRaw;
template <>
struct RouterRaw<DGMOE_F32> { float4 v[4]; };
template <>
struct RouterRaw<DGMOE_BF16> { uint4 v[2]; };
template <>
struct RouterRaw<DGMOE_Q8G64> { uint4 v; uint32_t sb; };

template <int RFMT>
__device__ __forceinline__ void router_load16(RouterRaw<RFMT>& r, const dgmoe_matrix& w, int D, int e, int k) {
  if constexpr (RFMT == DGMOE_F32) {
    const float4* p = (const float4*)((const float*)w.data + (int64_t)e * D + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = p[i];
  } else if constexpr (RFMT == DGMOE_BF16) {
    const uint4* p = (const uint4*)((const uint16_t*)w.data + (int64_t)e * D + k);
    r.v[0] = p[0];
    r.v[1] = p[1];
  } else {  // Q8G64: row-major bytes, (scale, bias) pairs row-major per group
    r.v = *(const uint4*)((const uint8_t*)w.data + (int64_t)e * D + k);
    r.sb = ((const uint32_t*)w.scale_bias)[(int64_t)e * (D / 64) + k / 64];
  }
}

template <int RFMT>
__device__ __forceinline__ float router_value(const RouterRaw<RFMT>& r, int i) {
  if constexpr (RFMT == DGMOE_F32) {
    const float4 q = r.v[i >> 2];
    return (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
  } else if constexpr (RFMT == DGMOE_BF16) {
    const uint4 q = r.v[i >> 3];
    const int j = (i & 7) >> 1;
    const uint32_t u = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    return bitcast<float>((i & 1) ? (u & 0xFFFF0000u) : (u << 16));
  } else {
    const int j = i >> 2;
    const uint32_t u = j == 0 ? r.v.x : j == 1 ? r.v.y : j == 2 ? r.v.z : r.v.w;
    const float s = half_bits_to_float((uint16_t)(r.sb & 0xFFFFu));
    const float b = half_bits_to_float((uint16_t)(r.sb >> 16));
    return fmaf(s, (float)((u >> (8 * (i & 3))) & 0xFFu), b);
  }
}

constexpr int NO_ROUTER = -1;

// ---------------------------------------------------------------- prologue
// Router weights of one 16-expert tile for the chunk's (up to) four 64-input
// groups; groups past the chunk reload its last group (their products are
// zeroed).
constexpr int PR_GROUPS = PR_KC / 64;

template <int RFMT>
__device__ __forceinline__ void load_router_chunk(RouterRaw<RFMT> (&bv)[PR_GROUPS], const dgmoe_matrix& wr,
                                                  int D, int e, int kc0, int ngroups, int g) {
#pragma unroll
  for (int q = 0; q < PR_GROUPS; ++q)
    router_load16<RFMT>(bv[q], wr, D, e, kc0 + 64 * min(q, ngroups - 1) + 16 * g);
}

// Phase 1: each half-wave sums the squares of one full row (fp32, lane-strided
// partials, then a fixed butterfly), r = 1/sqrt(mean + eps).  Every workgroup
// of a row block computes the same r bit for bit.
// Phase 2: thread (row t/32, 8 inputs at 8*(t%32)) of the chunk writes the
// fp16 operands and u = (xh*router_scale)*D^-1/2 into LDS.
// Phase 3: wave w computes the 16 rows x 16 experts tiles w, w+8, ... over the
// chunk with fp32 MFMA 16x16x4: lane l holds A[m=l%16][k=l/16],
// B[k=l/16][n=l%16] and produces C[m=4*(l/16)+i][n=l%16].  Within a 64-input
// group, lane group g owns inputs 16g .. 16g+15 (one 16-byte load of the
// weights) and MFMA i of the group takes input 16g + i in lane group g, for A
// and B alike, so each accumulator is the plain dot product.
// The router weights of the first tile are requested before phase 1, so their
// latency overlaps the norm.
template <typename XT, int RFMT>
__global__ __launch_bounds__(PR_THREADS) void k_prologue(
    const XT* __restrict__ x, int64_t L, int D, float eps, const float* __restrict__ w_pre,
    const float* __restrict__ w_pre2, const float* __restrict__ rs, float rc, dgmoe_matrix wr,
    int E, int sp, float* __restrict__ plog, _Float16* __restrict__ a, _Float16* __restrict__ b,
    int32_t* __restrict__ cnt, int32_t* __restrict__ rowid) {
  __shared__ float s_r[PR_ROWS];
  __shared__ float s_u[PR_ROWS][PR_KC + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * PR_ROWS;
  const int chunk = blockIdx.y;
  const int kc0 = chunk * PR_KC;
  const int kc = min(PR_KC, D - kc0);  // a multiple of 64
  const int ngroups = kc / 64;         // 1 to 4 groups of 64 inputs
  const int m = lane & 15, g = lane >> 4;
  if (cnt && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < DG_COUNTERS; i += PR_THREADS) cnt[i] = 0;
  if (rowid && blockIdx.y == 0 && tid < PR_ROWS && row0 + tid < L) rowid[row0 + tid] = (int32_t)(row0 + tid);

  using Raw = RouterRaw<RFMT == NO_ROUTER ? DGMOE_Q8G64 : RFMT>;
  Raw bv[PR_GROUPS];
  if constexpr (RFMT != NO_ROUTER) {
    const int e = wave * 16 + m;
    load_router_chunk<RFMT>(bv, wr, D, e < E ? e : 0, kc0, ngroups, g);
  }

  {  // phase 1: up to sixteen 16-byte loads of a lane in flight at a time
    const int rl = 2 * wave + (lane >> 5), hl = lane & 31;
    const int64_t row = row0 + rl;
    const int nch = D / 8;
    float ss = 0.f;
    if (row < L) {
      const XT* xr = x + row * D;
      for (int c0 = hl; c0 < nch; c0 += 32 * 16) {
        float v[16][8];
#pragma unroll
        for (int u = 0; u < 16; ++u) load8<XT>(xr + 8 * min(c0 + 32 * u, nch - 1), v[u]);
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (c0 + 32 * u < nch)
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += v[u][i] * v[u][i];
      }
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, DG_WAVE);
    if (hl == 0) s_r[rl] = row < L ? 1.0f / sqrtf(ss / (float)D + eps) : 0.f;
  }
  __syncthreads();

  {  // phase 2
    const int rl = tid >> 5, c8 = tid & 31;
    const int64_t row = row0 + rl;
    const int col = kc0 + 8 * c8;
    if (8 * c8 < kc) {
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (row < L) load8<XT>(x + row * D + col, v);
      const float r = s_r[rl];
      float xh[8], w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xh[i] = v[i] * r;
      if (row < L) {
        if (a) { load8<float>(w_pre + col, w); store8h(a + row * D + col, xh, w); }
        if (b) { load8<float>(w_pre2 + col, w); store8h(b + row * D + col, xh, w); }
      }
      if constexpr (RFMT != NO_ROUTER) {
        load8<float>(rs + col, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) s_u[rl][8 * c8 + i] = (xh[i] * w[i]) * rc;
      }
    }
  }
  if constexpr (RFMT != NO_ROUTER) {
    __syncthreads();
    for (int nb = wave; nb * 16 < E; nb += PR_THREADS / 64) {
      const int e = nb * 16 + m;
      const bool eok = e < E;
      if (nb != wave) load_router_chunk<RFMT>(bv, wr, D, eok ? e : 0, kc0, ngroups, g);
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < PR_GROUPS; ++q) {
        const bool on = eok && q < ngroups;
        const float* ap = &s_u[m][64 * min(q, ngroups - 1) + 16 * g];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4_t a4 = *(const float4_t*)(ap + 4 * i4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float bw = on ? router_value<RFMT>(bv[q], 4 * i4 + i) : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[i], bw, acc, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + 4 * g + i;
        if (row < L && eok) plog[(row * E + e) * sp + chunk] = acc[i];
      }
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wave per row.  z_e = sum over chunks (ascending) of the partial logits,
// plus the bias.  Each expert gets a 64-bit key whose unsigned order is the
// selection order (logit desc, index asc): the logit's bits mapped to an
// order-preserving unsigned integer (with -0 taken as +0, so equal logits tie)
// above the complement of the index.  The row's keys go to LDS, and each lane
// counts for each of its experts (lane + 64c) the keys above its own: that
// count is the expert's rank, a permutation of 0..E-1, and rank j < k is the
// j-th choice.
constexpr int TK_QMAX = 8;  // float4s of partial logits per expert: chunks <= 32

__device__ __forceinline__ uint64_t order_key(float z, int e) {
  const uint32_t f = bitcast<uint32_t>(z + 0.0f);  // -0 -> +0
  const uint32_t o = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__global__ __launch_bounds__(TK_THREADS) void k_topk(
    const float* __restrict__ plog, int nchunks, int sp, int64_t L, int E, int k,
    const float* __restrict__ bias, const float* __restrict__ pes, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, float* __restrict__ logits_out, int32_t* __restrict__ cnt,
    int32_t* __restrict__ list, int64_t cap) {
  __shared__ uint64_t s_key[TK_THREADS / 64][256];  // the row's keys, 0 past E
  __shared__ int s_se[TK_THREADS / 64][32];
  __shared__ float s_sz[TK_THREADS / 64][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (TK_THREADS / 64) + wave;
  const bool live_row = row < L;
  const int64_t rr = live_row ? row : L - 1;
  // all partial logits of the lane's experts are requested at once (experts
  // past E and float4s past the chunks re-read valid entries and are dropped)
  const int nq = sp / 4;
  float4 t[4][TK_QMAX];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4* pp = (const float4*)(plog + (rr * E + min(lane + 64 * c, E - 1)) * sp);
#pragma unroll
    for (int q = 0; q < TK_QMAX; ++q) t[c][q] = pp[min(q, nq - 1)];
  }
  float z[4];
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < TK_QMAX; ++q) {
      if (4 * q + 0 < nchunks) v += t[c][q].x;
      if (4 * q + 1 < nchunks) v += t[c][q].y;
      if (4 * q + 2 < nchunks) v += t[c][q].z;
      if (4 * q + 3 < nchunks) v += t[c][q].w;
    }
    if (e < E) {
      if (bias) v += bias[e];
      if (logits_out && live_row) logits_out[row * E + e] = v;
    }
    z[c] = v;
    key[c] = e < E ? order_key(v, e) : 0ull;
    s_key[wave][e] = key[c];
  }
  __syncthreads();
  const int e2 = (E + 1) / 2;  // 16-byte pairs of keys that hold experts
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    if (64 * c >= E) break;  // uniform
    int rank = 0;
    for (int j0 = 0; j0 < e2; j0 += 8) {
      ulonglong2 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = ((const ulonglong2*)s_key[wave])[min(j0 + u, 127)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = j0 + u < e2;
        rank += (in && q[u].x > key[c]) ? 1 : 0;
        rank += (in && q[u].y > key[c]) ? 1 : 0;
      }
    }
    if (e < E && rank < k) {
      s_se[wave][rank] = e;
      s_sz[wave][rank] = z[c];
    }
  }
  __syncthreads();
  const int my_e = lane < k ? s_se[wave][lane] : 0;
  const float my_z = lane < k ? s_sz[wave][lane] : 0.f;
  const float top = s_sz[wave][0];
  const float ex = (lane < k) ? expf(my_z - top) : 0.f;
  const float den = wave_sum(ex);
  if (lane < k && live_row) {
    idx_out[row * k + lane] = my_e;
    w_out[row * k + lane] = (ex / den) * pes[my_e];
    if (cnt) {
      const int64_t at = (int64_t)my_e * cap + atomicAdd(&cnt[my_e], 1);
      list[at] = (int32_t)(row * k + lane);
      list[(int64_t)E * cap + at] = (int32_t)row;  // the pair's token
    }
  }
}

__global__ __launch_bounds__(256) void k_assign(const int32_t* __restrict__ idx, int64_t Lk, int k,
                                                int E, int32_t* __restrict__ cnt,
                                                int32_t* __restrict__ list, int64_t cap) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= Lk) return;
  const int e = idx[p];
  if (e >= 0 && e < E) {
    const int64_t at = (int64_t)e * cap + atomicAdd(&cnt[e], 1);
    list[at] = (int32_t)p;
    list[(int64_t)E * cap + at] = (int32_t)(p / k);  // the pair's token
  }
}

}  // namespace

hipError_t launch_prologue(const void* x, int x_dtype, int64_t L, int D, float eps,
                           const float* w_pre, const float* w_pre2, _Float16* a, _Float16* b,
                           const float* router_scale, const dgmoe_matrix* wr, int E, float* plog,
                           int32_t* cnt, int32_t* rowid, hipStream_t st) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls (e.g. a not-ready query)
  const float rc = (float)(1.0 / sqrt((double)D));
  const int sp = prologue_stride(D);
  dim3 grid((unsigned)((L + PR_ROWS - 1) / PR_ROWS), (unsigned)prologue_chunks(D)), block(PR_THREADS);
  dgmoe_matrix none{};
  const int rf = wr ? wr->dtype : NO_ROUTER;
  const dgmoe_matrix m = wr ? *wr : none;
#define DG_PRO(XT, RF)                                                                          \
  hipLaunchKernelGGL((k_prologue<XT, RF>), grid, block, 0, st, (const XT*)x, L, D, eps, w_pre, \
                     w_pre2, router_scale, rc, m, E, sp, plog, a, b, cnt, rowid)
#define DG_PRO_X(XT)                                   \
  switch (rf) {                                        \
    case DGMOE_F32: DG_PRO(XT, DGMOE_F32); break;      \
    case DGMOE_BF16: DG_PRO(XT, DGMOE_BF16); break;    \
    case DGMOE_Q8G64: DG_PRO(XT, DGMOE_Q8G64); break;  \
    default: DG_PRO(XT, NO_ROUTER); break;             \
  }
  if (x_dtype == DGMOE_F32) {
    DG_PRO_X(float)
  } else {
    DG_PRO_X(uint16_t)
  }
#undef DG_PRO_X
#undef DG_PRO
  return hipGetLastError();
}

hipError_t launch_topk(const float* plog, int64_t L, int D, int E, int k, const float* bias,
                       const float* pes, int32_t* idx, float* w, float* logits, int32_t* cnt,
                       int32_t* list, int64_t cap, hipStream_t st) {
  (void)hipGetLastError();
  dim3 grid((unsigned)((L + TK_THREADS / 64 - 1) / (TK_THREADS / 64))), block(TK_THREADS);
  hipLaunchKernelGGL(k_topk, grid, block, 0, st, plog, prologue_chunks(D), prologue_stride(D), L, E,
                     k, bias, pes, idx, w, logits, cnt, list, cap);
  return hipGetLastError();
}

hipError_t launch_assign(const int32_t* idx, int64_t L, int k, int E, int32_t* cnt, int32_t* list,
                         int64_t cap, hipStream_t st) {
  (void)hipGetLastError();
  const int64_t Lk = L * k;
  hipLaunchKernelGGL(k_assign, dim3((unsigned)((Lk + 255) / 256)), dim3(256), 0, st, idx, Lk, k, E,
                     cnt, list, cap);
  return hipGetLastError();
}
