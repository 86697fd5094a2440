// The C ABI of libdgmoe: host-side argument checks, workspace carving and the
// launch sequence of each entry point.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include <algorithm>
#include "../../include/dgmoe.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxL = int64_t(1) << 20;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

bool dims_ok(const dgmoe_dims* d) {
  auto m64 = [](int v, int hi) { return v >= 64 && v <= hi && v % 64 == 0; };
  if (!m64(d->hidden, 8192) || !m64(d->expert_inter, 16384) || !m64(d->dense_inter, 16384)) return false;
  if (d->n_experts < 1 || d->n_experts > 256) return false;
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 32) return false;
  if (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)) return false;
  return true;
}

// Workspace carve-up; every region 256-byte aligned.
struct Layout {
  size_t a, b, plog, idx, wts, cnt, sync, rowid, list, act, act_d, slots, h1, total;
  int64_t list_cap;        // slots per expert in the pair lists (L)
  int64_t max_gu, max_dn;  // upper bounds on the tiles of the two GEMM phases
};

// Upper bounds on the tile counts: sum_e ceil(rows_e / DG_MT) <= ceil(L*k / DG_MT) + E.
void tile_bounds(const dgmoe_dims* d, int64_t L, int64_t* gu, int64_t* dn) {
  const int64_t exp_mt = (L * d->top_k + DG_MT - 1) / DG_MT + d->n_experts;
  const int64_t den_mt = (L + DG_MT - 1) / DG_MT;
  const int64_t nt_dn = (d->hidden + DG_NDN - 1) / DG_NDN;
  *gu = exp_mt * (d->expert_inter / DG_NGU) + den_mt * (d->dense_inter / DG_NGU);
  *dn = (exp_mt + den_mt) * nt_dn;
}

Layout layout(const dgmoe_dims* d, int64_t L) {
  const size_t D = d->hidden, E = d->n_experts, k = d->top_k, I = d->expert_inter, Id = d->dense_inter;
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  l.a = take(L * D * 2);
  l.b = take(L * D * 2);
  l.plog = take(L * E * 4);  // router logits
  l.idx = take(L * k * 4);
  l.wts = take(L * k * 4);
  l.cnt = take(DG_COUNTERS * 4);
  l.sync = take(front_sync_words(L) * 4);
  l.rowid = take(L * 4);
  // A position names an expert at most once (the router's top-k is a set), so
  // an expert's list never holds more than L pairs; a caller routing that
  // names one expert more than L times in total overfills it, and the extra
  // pairs are dropped and flagged (DGMOE_FLAG_ROUTE_OVERFLOW).
  l.list_cap = L;
  l.list = take(2 * E * L * 4);  // pair ids, then their tokens
  tile_bounds(d, L, &l.max_gu, &l.max_dn);
  l.act = take(L * k * I * 2);
  l.act_d = take(L * Id * 2);
  l.slots = take(L * k * D * 2);
  l.h1 = take(dense_down_chunks(I, Id) * L * D * 4);  // partial sums of the dense down projection
  l.total = off;
  return l;
}

dgmoe_status check_matrix(const dgmoe_matrix& m, bool allow_f32, bool allow_q8, bool allow_q4) {
  if (!m.data) return DGMOE_ERR_NULL_ARG;
  const int f = m.dtype;
  // the MFMA-tiled formats (4- and 6-bit)
  const bool q4 = f == DGMOE_Q4G64 || f == DGMOE_Q4G32 || f == DGMOE_NVFP4 || f == DGMOE_Q6G32;
  const bool packed = q4 || f == DGMOE_Q8G64;
  if (f == DGMOE_F32 && !allow_f32) return DGMOE_ERR_BAD_DTYPE;
  if (f == DGMOE_Q8G64 && !allow_q8) return DGMOE_ERR_BAD_DTYPE;
  if (q4 && !allow_q4) return DGMOE_ERR_BAD_DTYPE;
  if (f != DGMOE_F32 && f != DGMOE_BF16 && !packed) return DGMOE_ERR_BAD_DTYPE;
  if (packed && !m.scale_bias) return DGMOE_ERR_NULL_ARG;
  if (!aligned(m.data, 64)) return DGMOE_ERR_MISALIGNED;
  if (packed && !aligned(m.scale_bias, 64)) return DGMOE_ERR_MISALIGNED;
  return DGMOE_OK;
}

// [D] weight vectors are read with 16-byte loads; [E] vectors element-wise.
dgmoe_status check_vec(const float* p, uintptr_t align = 16) {
  if (!p) return DGMOE_ERR_NULL_ARG;
  if (!aligned(p, align)) return DGMOE_ERR_MISALIGNED;
  return DGMOE_OK;
}

#define DG_TRY(expr)                        \
  do {                                      \
    dgmoe_status s_ = (expr);               \
    if (s_ != DGMOE_OK) return s_;          \
  } while (0)

dgmoe_status check_router(const dgmoe_block_weights* w) {
  DG_TRY(check_matrix(w->router, true, true, false));
  DG_TRY(check_vec(w->router_scale));
  DG_TRY(check_vec(w->per_expert_scale, 4));
  if (w->router_bias && !aligned(w->router_bias, 4)) return DGMOE_ERR_MISALIGNED;
  return DGMOE_OK;
}

// allow_q8: the dense MLP's pair may be Q8G64 (the experts' may not: the
// diffgemma contract's section 8.2 gives the expert class q4, q6 and nvfp4
// only, and the OptiQ checkpoint of the mlx-bun dossier stores the dense MLP
// at 8 bits).
dgmoe_status check_pair(const dgmoe_matrix& gu, const dgmoe_matrix& dn, bool allow_q8 = false) {
  DG_TRY(check_matrix(gu, false, allow_q8, true));
  DG_TRY(check_matrix(dn, false, allow_q8, true));
  if (gu.dtype != dn.dtype) return DGMOE_ERR_BAD_DTYPE;
  return DGMOE_OK;
}

dgmoe_status check_common(const dgmoe_dims* d, const dgmoe_block_weights* w, const void* x,
                          int32_t x_dtype, int64_t L, void* ws, size_t ws_bytes) {
  if (!d || !w) return DGMOE_ERR_NULL_ARG;
  if (!dims_ok(d) || L < 0 || L > kMaxL) return DGMOE_ERR_BAD_DIMS;
  if (x_dtype != DGMOE_F32 && x_dtype != DGMOE_BF16) return DGMOE_ERR_BAD_DTYPE;
  if (L == 0) return DGMOE_OK;
  if (!x) return DGMOE_ERR_NULL_ARG;
  if (!aligned(x, 16)) return DGMOE_ERR_MISALIGNED;
  if (!ws) return DGMOE_ERR_NULL_ARG;
  if (!aligned(ws, 256)) return DGMOE_ERR_MISALIGNED;
  if (ws_bytes < layout(d, L).total) return DGMOE_ERR_WORKSPACE;
  return DGMOE_OK;
}

// The last HIP error this thread saw inside the library (diagnostics only).
thread_local hipError_t g_last_hip = hipSuccess;

// Diagnostics only (dgmoe_debug_force_stamp_timeout): 0, or the stamp-wait
// poll limit of this thread's next front launches, whose stamp is then never
// published.
thread_local int g_debug_spin = 0;
constexpr int kSpinLimit = 1 << 20;  // polls of the front kernel's stamp wait (~50 ms)

// Pairs from which an expert takes tall tiles in a short-tile launch
// (dgmoe_debug_set_tall_min; 0: none do).
thread_local int g_mix_tall_min = DG_MIX_TALL_MIN;

inline dgmoe_status hip_ok(hipError_t e) {
  if (e == hipSuccess) return DGMOE_OK;
  g_last_hip = e;
  return DGMOE_ERR_HIP;
}

// A stamp for each call, distinct for every call in the process: the front
// kernel's workgroup (0, 0) publishes it once it has cleared the workspace's
// counters, and the other workgroups wait for it before counting.  It starts
// from the clock so that a workspace left by another library instance does
// not already hold it.
uint64_t next_stamp() {
  static std::atomic<uint64_t> ctr{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
  return ctr.fetch_add(2, std::memory_order_relaxed);
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

// Optional per-kernel HIP events: mark() records the next one on the stream.
struct Marks {
  hipEvent_t* ev = nullptr;
  int n = 0, i = 0;
  dgmoe_status mark(hipStream_t st) {
    if (!ev || i >= n) return DGMOE_OK;
    return hip_ok(hipEventRecord(ev[i++], st));
  }
};

// Which groups a pair of GEMM launches computes: the experts and the dense
// MLP together (one format), the experts only, or the dense MLP only (its own
// format, its own queue counters).
enum class Part { kAll, kExperts, kDense };

// The gate_up and down launch arguments for the groups of `part`.
// h1_parts: the K chunks of the dense down projection's partial sums (set when
// the part includes the dense MLP).
void phase_args(const dgmoe_dims* d, const dgmoe_block_weights* w, int64_t L, const Layout& l,
                void* ws, Part part, uint64_t stamp, GemmPhaseArgs& g, GemmPhaseArgs& dn,
                int* h1_parts) {
  const int D = d->hidden, E = d->n_experts, k = d->top_k, I = d->expert_inter, Id = d->dense_inter;
  const bool dense = part != Part::kExperts, experts = part != Part::kDense;
  g = GemmPhaseArgs{};
  g.wfmt_d = dense ? w->dense_gate_up.dtype : w->expert_gate_up.dtype;
  g.wfmt_e = experts ? w->expert_gate_up.dtype : g.wfmt_d;
  g.skip_e = experts ? 0 : 1;
  const int fmt = experts ? g.wfmt_e : g.wfmt_d;  // the format of the launches
  g.cnt = at<int32_t>(ws, l.cnt);
  g.list = at<int32_t>(ws, l.list);
  g.list_cap = l.list_cap;
  g.rowid = at<int32_t>(ws, l.rowid);
  g.zero = (const uint32_t*)(at<int32_t>(ws, l.cnt) + DG_ZERO_OFF);
  g.E = E; g.topk = k;
  g.dense_rows = dense ? (int)L : 0;
  // queue counters: gate_up +0 (tall tiles of a mixed launch +16), down +8
  // (+24); the dense MLP alone +32 and +40
  int32_t* queues = at<int32_t>(ws, l.cnt) + DG_QUEUE_OFF + (experts ? 0 : 32);
  g.pairs = L * k;
  g.n_tok = L;
  g.sync = at<uint32_t>(ws, l.sync);
  g.stamp = stamp;
  // tall tiles address their operands with 32-bit byte offsets
  const int64_t widest = std::max<int64_t>(D, std::max(I, Id));
  const bool fits32 = (L * k + L) * widest * 2 < (int64_t(1) << 31) &&
                      (int64_t)E * 2 * std::max(I, D) * widest / 2 < (int64_t(1) << 31);
  // Q4G64 only: tall tiles from an average of DG_TALL_MIN_ROWS pairs per expert
  g.tall = fmt == DGMOE_Q4G64 && L * k >= (int64_t)DG_TALL_MIN_ROWS * E && fits32;
  // below the all-tall average, the experts with many pairs still take tall tiles
  g.tall_min = fmt == DGMOE_Q4G64 && experts && !g.tall && fits32 ? g_mix_tall_min : 0;
  const int64_t exp_mt = experts ? (L * k + DG_MT - 1) / DG_MT + E : 0;
  const int64_t den_mt = dense ? (L + DG_MT - 1) / DG_MT : 0;
  dn = g;
  // gate_up
  g.w_e = w->expert_gate_up.data; g.sb_e = (const uint32_t*)w->expert_gate_up.scale_bias;
  g.n_e = 2 * I; g.k_e = D;
  if (dense) {
    g.w_d = w->dense_gate_up.data; g.sb_d = (const uint32_t*)w->dense_gate_up.scale_bias;
  }
  g.n_d = 2 * Id; g.k_d = D;
  g.a_e = at<_Float16>(ws, l.b);
  g.a_d = at<_Float16>(ws, l.a);
  g.nt_e = I / DG_NGU;
  g.nt_d = Id / DG_NGU;
  g.queue = queues;
  g.act_e = at<_Float16>(ws, l.act);
  g.act_d = at<_Float16>(ws, l.act_d);
  g.max_tiles = (int)std::min<int64_t>(l.max_gu, exp_mt * (I / DG_NGU) + den_mt * (Id / DG_NGU));
  // down
  dn.w_e = w->expert_down.data; dn.sb_e = (const uint32_t*)w->expert_down.scale_bias;
  dn.n_e = D; dn.k_e = I;
  if (dense) {
    dn.w_d = w->dense_down.data; dn.sb_d = (const uint32_t*)w->dense_down.scale_bias;
  }
  dn.n_d = D; dn.k_d = Id;
  dn.a_e = at<_Float16>(ws, l.act);
  dn.a_d = at<_Float16>(ws, l.act_d);
  dn.nt_e = dn.nt_d = (int)cdiv(D, DG_NDN_Q4);
  dn.queue = queues + 8;
  dn.slots = at<_Float16>(ws, l.slots);
  dn.h1 = at<float>(ws, l.h1);
  dn.kch_d = !g.tall ? dense_down_chunks(I, Id) : 1;
  dn.max_tiles = (int)std::min<int64_t>(l.max_dn, (exp_mt + den_mt * dn.kch_d) * dn.nt_e);
  if (dense) *h1_parts = dn.kch_d;
}

// gate_up + down once the pair lists are built: for the experts alone
// (with_dense false), or for the experts and the dense MLP -- in one pair of
// launches when the two have one format, or a BF16 or Q8G64 dense MLP beside
// 4-bit experts on short tiles (one kernel holds both bodies), else the experts'
// gate_up, the dense MLP's gate_up, the experts' down, the dense MLP's down.
dgmoe_status run_gemms(const dgmoe_dims* d, const dgmoe_block_weights* w, int64_t L, const Layout& l,
                       void* ws, bool with_dense, uint64_t stamp, hipStream_t st, Marks& mk,
                       int* h1_parts) {
  GemmPhaseArgs gu[2], dn[2];
  int n = 1;
  const int fe = w->expert_gate_up.dtype, fd = w->dense_gate_up.dtype;
  if (!with_dense) {
    phase_args(d, w, L, l, ws, Part::kExperts, stamp, gu[0], dn[0], h1_parts);
  } else {
    phase_args(d, w, L, l, ws, Part::kAll, stamp, gu[0], dn[0], h1_parts);
    const bool one = fe == fd || ((fd == DGMOE_BF16 || fd == DGMOE_Q8G64) &&
                                  (fe == DGMOE_Q4G64 || fe == DGMOE_Q4G32 || fe == DGMOE_NVFP4 ||
                                   fe == DGMOE_Q6G32) &&
                                  !gu[0].tall && gu[0].tall_min == 0);
    if (!one) {
      phase_args(d, w, L, l, ws, Part::kExperts, stamp, gu[0], dn[0], h1_parts);
      phase_args(d, w, L, l, ws, Part::kDense, stamp, gu[1], dn[1], h1_parts);
      n = 2;
    }
  }
  DG_TRY(mk.mark(st));
  for (int i = 0; i < n; ++i) DG_TRY(hip_ok(launch_gate_up(gu[i], st)));
  DG_TRY(mk.mark(st));
  for (int i = 0; i < n; ++i) DG_TRY(hip_ok(launch_down(dn[i], st)));
  return DGMOE_OK;
}

// The front kernel's stamp fields for one call.
void set_stamp(FrontArgs& fa, void* ws, const Layout& l, uint64_t stamp) {
  fa.sync = at<uint32_t>(ws, l.sync);
  fa.stamp = stamp;
  fa.spin_limit = g_debug_spin > 0 ? g_debug_spin : kSpinLimit;
  fa.publish = g_debug_spin > 0 ? 0 : 1;
}

// ---------------------------------------------------------------- head
bool head_dims_ok(const dgmoe_head_dims* h) {
  auto m64 = [](int v, int hi) { return v >= 64 && v <= hi && v % 64 == 0; };
  if (!m64(h->hidden, 8192) || !m64(h->vocab, 1 << 20) || !m64(h->sc_inter, 16384)) return false;
  return h->rms_eps >= 0.f && std::isfinite(h->rms_eps);
}

// The self-conditioning MLP runs through the block's GEMM phases as the dense
// MLP of a block with one expert that no position is routed to.
dgmoe_dims sc_dims(const dgmoe_head_dims* h) {
  dgmoe_dims d{};
  d.hidden = h->hidden;
  d.n_experts = 1;
  d.top_k = 1;
  d.expert_inter = h->sc_inter;
  d.dense_inter = h->sc_inter;
  d.rms_eps = h->rms_eps;
  return d;
}

// Head workspace: that block's workspace at offset 0 (its sync region holds
// the call stamp and the error words of every head call), then the head's own
// regions.
struct HeadLayout {
  Layout blk;
  size_t xn, tstat, p16, pst, part, soft, total;
  int pieces;
};

HeadLayout head_layout(const dgmoe_head_dims* h, int64_t L) {
  HeadLayout hl{};
  const dgmoe_dims d = sc_dims(h);
  hl.blk = layout(&d, L);
  size_t off = hl.blk.total;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  const size_t D = h->hidden, V = h->vocab;
  hl.pieces = soft_pieces(L, h->hidden, h->vocab);
  hl.xn = take(L * D * 2);                                       // fp16 x_hat * final_norm
  hl.tstat = take((V / 64 + 3) / 4 * L * 16);                    // per-tile row statistics
  hl.p16 = take(L * V * 2);                                      // 2^14 exp(y - m_piece), fp16
  hl.pst = take((size_t)hl.pieces * L * 8);                      // (m_piece, l_piece)
  hl.part = take((size_t)hl.pieces * L * D * 4);                 // partial soft embeddings
  hl.soft = take(L * D * 4);                                     // the soft embedding
  hl.total = off;
  return hl;
}

dgmoe_status check_head(const dgmoe_head_dims* h, const dgmoe_head_weights* w, int64_t L,
                        void* ws, size_t ws_bytes) {
  if (!h || !w) return DGMOE_ERR_NULL_ARG;
  if (!head_dims_ok(h) || L < 0 || L > kMaxL) return DGMOE_ERR_BAD_DIMS;
  DG_TRY(check_matrix(w->embed, false, false, true));
  if (w->embed.dtype != DGMOE_Q4G64) return DGMOE_ERR_BAD_DTYPE;
  if (L == 0) return DGMOE_OK;
  if (!ws) return DGMOE_ERR_NULL_ARG;
  if (!aligned(ws, 256)) return DGMOE_ERR_MISALIGNED;
  if (ws_bytes < head_layout(h, L).total) return DGMOE_ERR_WORKSPACE;
  return DGMOE_OK;
}

SoftArgs soft_args(const dgmoe_head_dims* h, const dgmoe_head_weights* w, const float* sc_logits,
                   int64_t L, void* ws, const HeadLayout& hl, float* soft, uint64_t stamp) {
  SoftArgs sa{};
  sa.logits = sc_logits;
  sa.L = L;
  sa.D = h->hidden;
  sa.V = h->vocab;
  sa.codes = (const uint32_t*)w->embed.data;
  sa.sb = (const uint32_t*)w->embed.scale_bias;
  sa.pieces = hl.pieces;
  sa.p16 = at<_Float16>(ws, hl.p16);
  sa.pst = at<float2>(ws, hl.pst);
  sa.part = at<float>(ws, hl.part);
  sa.soft = soft;
  sa.sync = at<uint32_t>(ws, hl.blk.sync);
  sa.stamp = stamp;
  return sa;
}

// Host, synchronous: flags of the last call from the sync region at sync_off.
dgmoe_status read_flags(const void* ws, size_t sync_off, uint32_t* flags, void* stream) {
  *flags = 0;
  DG_TRY(hip_ok(hipStreamSynchronize(static_cast<hipStream_t>(stream))));
  uint64_t words[DG_SYNC_HEAD / 2];
  DG_TRY(hip_ok(hipMemcpy(words, static_cast<const uint8_t*>(ws) + sync_off, sizeof(words),
                          hipMemcpyDeviceToHost)));
  const uint64_t call = words[DG_SYNC_CALL / 2];
  static_assert(DGMOE_FLAG_SYNC_TIMEOUT == 1u << DG_ERR_SYNC, "flag bits follow the error kinds");
  static_assert(DGMOE_FLAG_FP16_RANGE == 1u << DG_ERR_RANGE, "flag bits follow the error kinds");
  static_assert(DGMOE_FLAG_ROUTE_OVERFLOW == 1u << DG_ERR_ROUTE, "flag bits follow the error kinds");
  static_assert(DGMOE_FLAG_INDEX == 1u << DG_ERR_INDEX, "flag bits follow the error kinds");
  for (int i = 0; i < DG_ERR_KINDS; ++i)
    if (words[DG_SYNC_ERR / 2 + i] == call) *flags |= 1u << i;
  return *flags ? DGMOE_ERR_DEVICE : DGMOE_OK;
}

// ---------------------------------------------------------------- scratch
// The workspace of dgmoe_block_forward_noalloc: a file-scope device array that
// each GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory; its device address
// is looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (nullptr on failure).
dgmoe_status scratch_ptr(void** out) {
  int dev = -1;
  DG_TRY(hip_ok(hipGetDevice(&dev)));
  if (dev < 0 || dev >= kMaxDevices) return DGMOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DG_TRY(hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))));
    if (!p) return DGMOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DGMOE_OK;
}

// ---------------------------------------------------------------- attention
bool attn_dims_ok(const dgmoe_attn_dims* a) {
  const int hd = a->head_dim;
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512) return false;
  if (a->n_heads < 1 || a->n_heads > 256 || a->n_kv_heads < 1 || a->n_heads % a->n_kv_heads) return false;
  if (a->window < 0) return false;
  if (a->rope_pairs < 0 || a->rope_pairs > hd / 2 || a->rope_stride < a->rope_pairs ||
      a->rope_pairs + a->rope_stride > hd)
    return false;
  if (!(a->rope_theta > 0.f) || !std::isfinite(a->rope_theta)) return false;
  if (!(a->rope_den > 0.f) || !std::isfinite(a->rope_den)) return false;
  return a->rms_eps >= 0.f && std::isfinite(a->rms_eps);
}

struct AttnLayout {
  size_t qp, kp, vp, opart, ml, total;
  int chunks, tiles_per_chunk;
  int64_t s0, n_enc;
};

AttnLayout attn_layout(const dgmoe_attn_dims* a, int64_t L, int64_t kv_len) {
  AttnLayout al{};
  const size_t H = a->n_heads, Hkv = a->n_kv_heads, hd = a->head_dim;
  al.s0 = a->window > 0 ? std::max<int64_t>(0, kv_len - a->window) : 0;
  al.n_enc = kv_len - al.s0;
  const int64_t T = attn_tiles(al.n_enc, L);
  al.chunks = attn_chunks(L, a->n_heads, a->n_kv_heads, a->head_dim, T);
  al.tiles_per_chunk = (int)((T + al.chunks - 1) / al.chunks);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  al.qp = take(H * L * hd * 2);
  al.kp = take(Hkv * L * hd * 2);
  al.vp = take(Hkv * L * hd * 2);
  al.opart = take((size_t)al.chunks * H * L * hd * 4);
  al.ml = take((size_t)al.chunks * H * L * 8);
  al.total = off;
  return al;
}

}  // namespace

extern "C" {

size_t dgmoe_attn_workspace_size(const dgmoe_attn_dims* a, int64_t L, int64_t kv_len) {
  if (!a || !attn_dims_ok(a) || L < 0 || L > kMaxL || kv_len < 0 || kv_len > (int64_t(1) << 30)) return 0;
  return attn_layout(a, L, kv_len).total;
}

dgmoe_status dgmoe_attn_denoise(const dgmoe_attn_dims* a, const void* q, const void* k,
                                const void* v, int32_t in_dtype, int64_t L, const float* q_norm,
                                const float* k_norm, const uint16_t* k_cache,
                                const uint16_t* v_cache, int64_t cache_rows, int64_t kv_len,
                                void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!a) return DGMOE_ERR_NULL_ARG;
  if (!attn_dims_ok(a) || L < 0 || L > kMaxL || kv_len < 0 || kv_len > cache_rows ||
      cache_rows > (int64_t(1) << 30))
    return DGMOE_ERR_BAD_DIMS;
  if (in_dtype != DGMOE_F32 && in_dtype != DGMOE_BF16) return DGMOE_ERR_BAD_DTYPE;
  if (out_dtype != DGMOE_F32 && out_dtype != DGMOE_BF16) return DGMOE_ERR_BAD_DTYPE;
  // row tiles of a KV head's query group are a grid dimension (at most 65535)
  if (((int64_t)(a->n_heads / a->n_kv_heads) * L + DG_ATTN_ROWS - 1) / DG_ATTN_ROWS > 65535)
    return DGMOE_ERR_BAD_DIMS;
  if (L == 0) return DGMOE_OK;
  if (!q || !k || !q_norm || !k_norm || !out || !ws) return DGMOE_ERR_NULL_ARG;
  if (kv_len > 0 && (!k_cache || !v_cache)) return DGMOE_ERR_NULL_ARG;
  if (!aligned(q, 4) || !aligned(k, 4) || (v && !aligned(v, 4)) || !aligned(q_norm, 4) ||
      !aligned(k_norm, 4) || (k_cache && !aligned(k_cache, 16)) || (v_cache && !aligned(v_cache, 16)) ||
      !aligned(out, 16) || !aligned(ws, 256))
    return DGMOE_ERR_MISALIGNED;
  const AttnLayout al = attn_layout(a, L, kv_len);
  if (ws_bytes < al.total) return DGMOE_ERR_WORKSPACE;
  AttnArgs aa{};
  aa.q = q; aa.k = k; aa.v = v; aa.in_dtype = in_dtype;
  aa.L = L; aa.H = a->n_heads; aa.Hkv = a->n_kv_heads; aa.hd = a->head_dim;
  aa.wq = q_norm; aa.wk = k_norm;
  aa.qp = at<_Float16>(ws, al.qp); aa.kp = at<_Float16>(ws, al.kp); aa.vp = at<_Float16>(ws, al.vp);
  // with no committed rows the cache is never read; the canvas stands in for it
  aa.kc = kv_len > 0 ? reinterpret_cast<const _Float16*>(k_cache) : aa.kp;
  aa.vc = kv_len > 0 ? reinterpret_cast<const _Float16*>(v_cache) : aa.vp;
  aa.cap = kv_len > 0 ? cache_rows : 0;
  aa.kv_len = kv_len; aa.s0 = al.s0; aa.n_enc = al.n_enc;
  aa.n_rot = a->rope_pairs; aa.stride = a->rope_stride;
  aa.theta = a->rope_theta; aa.den = a->rope_den; aa.eps = a->rms_eps;
  aa.chunks = al.chunks; aa.tiles_per_chunk = al.tiles_per_chunk;
  aa.opart = at<float>(ws, al.opart); aa.ml = at<float2>(ws, al.ml);
  aa.out = out; aa.out_dtype = out_dtype;
  return hip_ok(launch_attn(aa, static_cast<hipStream_t>(stream)));
}

int dgmoe_abi_version(void) { return DGMOE_ABI_VERSION; }

const char* dgmoe_status_str(dgmoe_status s) {
  switch (s) {
    case DGMOE_OK: return "ok";
    case DGMOE_ERR_NULL_ARG: return "a required pointer is NULL";
    case DGMOE_ERR_BAD_DIMS: return "a dimension is out of range or not a multiple of 64";
    case DGMOE_ERR_BAD_DTYPE: return "unsupported dtype or format combination";
    case DGMOE_ERR_MISALIGNED: return "a pointer breaks the alignment rule";
    case DGMOE_ERR_WORKSPACE: return "workspace too small";
    case DGMOE_ERR_HIP: return "HIP launch failure";
    case DGMOE_ERR_DEVICE: return "the last call on the workspace reported a device-side error";
  }
  return "unknown status";
}

const char* dgmoe_last_hip_error(void) {
  return g_last_hip == hipSuccess ? "none" : hipGetErrorName(g_last_hip);
}

size_t dgmoe_workspace_size(const dgmoe_dims* d, int64_t L) {
  if (!d || !dims_ok(d) || L < 0 || L > kMaxL) return 0;
  return layout(d, L).total;
}

size_t dgmoe_packed_bytes(int64_t rows, int64_t cols, int32_t fmt) {
  if (rows < 0 || cols <= 0 || cols % 64) return 0;
  if (fmt == DGMOE_Q4G64 || fmt == DGMOE_Q4G32 || fmt == DGMOE_NVFP4) return (size_t)(rows * cols / 2);
  if (fmt == DGMOE_Q6G32) return (size_t)(rows * cols / 4 * 3);
  if (fmt == DGMOE_Q8G64) return (size_t)(rows * cols);
  return 0;
}

dgmoe_status dgmoe_route(const dgmoe_dims* d, const dgmoe_block_weights* w, const void* x,
                         int32_t x_dtype, int64_t L, int32_t* topk_idx, float* topk_w,
                         float* logits, void* ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_common(d, w, x, x_dtype, L, ws, ws_bytes));
  DG_TRY(check_router(w));
  if (L == 0) return DGMOE_OK;
  if (!topk_idx || !topk_w) return DGMOE_ERR_NULL_ARG;
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || (logits && !aligned(logits, 4)))
    return DGMOE_ERR_MISALIGNED;
  const Layout l = layout(d, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the router needs no GEMM operands and no pair lists
  FrontArgs fa{};
  fa.x = x; fa.x_dtype = x_dtype; fa.L = L; fa.D = d->hidden; fa.eps = d->rms_eps;
  fa.router_scale = w->router_scale; fa.wr = &w->router; fa.E = d->n_experts;
  fa.plog = at<float>(ws, l.plog);
  fa.k = d->top_k; fa.bias = w->router_bias; fa.pes = w->per_expert_scale;
  fa.idx = topk_idx; fa.w = topk_w; fa.logits = logits;
  set_stamp(fa, ws, l, next_stamp());
  DG_TRY(hip_ok(launch_front(fa, st)));
  return DGMOE_OK;
}

dgmoe_status dgmoe_moe_ffn(const dgmoe_dims* d, const dgmoe_block_weights* w, const void* x,
                           int32_t x_dtype, int64_t L, const int32_t* topk_idx,
                           const float* topk_w, float* moe_out, void* ws, size_t ws_bytes,
                           void* stream) {
  DG_TRY(check_common(d, w, x, x_dtype, L, ws, ws_bytes));
  DG_TRY(check_pair(w->expert_gate_up, w->expert_down));
  DG_TRY(check_vec(w->pre_ff_norm_2));
  if (L == 0) return DGMOE_OK;
  if (!topk_idx || !topk_w || !moe_out) return DGMOE_ERR_NULL_ARG;
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(moe_out, 16)) return DGMOE_ERR_MISALIGNED;
  const Layout l = layout(d, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  FrontArgs fa{};
  fa.x = x; fa.x_dtype = x_dtype; fa.L = L; fa.D = d->hidden; fa.eps = d->rms_eps;
  fa.w_pre2 = w->pre_ff_norm_2; fa.b = at<_Float16>(ws, l.b); fa.E = d->n_experts;
  fa.cnt = at<int32_t>(ws, l.cnt); fa.rowid = at<int32_t>(ws, l.rowid);
  const uint64_t stamp = next_stamp();
  set_stamp(fa, ws, l, stamp);
  DG_TRY(hip_ok(launch_front(fa, st)));
  DG_TRY(hip_ok(launch_assign(topk_idx, L, d->top_k, d->n_experts, at<int32_t>(ws, l.cnt),
                              at<int32_t>(ws, l.list), l.list_cap, fa.sync, stamp, st)));
  Marks none;
  int parts = 1;
  DG_TRY(run_gemms(d, w, L, l, ws, false, stamp, st, none, &parts));
  DG_TRY(hip_ok(launch_combine(at<_Float16>(ws, l.slots), nullptr, 0, topk_idx, topk_w, x, x_dtype, L, d->hidden,
                               d->top_k, d->n_experts, d->rms_eps, nullptr, nullptr, nullptr, 0.f,
                               moe_out, nullptr, DGMOE_F32, st)));
  return DGMOE_OK;
}

static dgmoe_status block_forward(const dgmoe_dims* d, const dgmoe_block_weights* w, const void* x,
                                  int32_t x_dtype, int64_t L, const int32_t* force_idx,
                                  const float* force_w, void* y, int32_t y_dtype,
                                  int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                  size_t ws_bytes, void* stream, Marks& mk) {
  DG_TRY(check_common(d, w, x, x_dtype, L, ws, ws_bytes));
  const bool forced = force_idx && force_w;
  if (!forced) DG_TRY(check_router(w));
  DG_TRY(check_pair(w->expert_gate_up, w->expert_down));
  DG_TRY(check_pair(w->dense_gate_up, w->dense_down, true));
  DG_TRY(check_vec(w->pre_ff_norm));
  DG_TRY(check_vec(w->pre_ff_norm_2));
  DG_TRY(check_vec(w->post_ff_norm_1));
  DG_TRY(check_vec(w->post_ff_norm_2));
  DG_TRY(check_vec(w->post_ff_norm));
  if (!std::isfinite(w->layer_scalar)) return DGMOE_ERR_BAD_DIMS;
  if (y_dtype != DGMOE_F32 && y_dtype != DGMOE_BF16) return DGMOE_ERR_BAD_DTYPE;
  if (L == 0) return DGMOE_OK;
  if (!y) return DGMOE_ERR_NULL_ARG;
  if (!aligned(y, 16)) return DGMOE_ERR_MISALIGNED;
  if ((force_idx && !aligned(force_idx, 4)) || (force_w && !aligned(force_w, 4)) ||
      (topk_idx_out && !aligned(topk_idx_out, 4)) || (topk_w_out && !aligned(topk_w_out, 4)))
    return DGMOE_ERR_MISALIGNED;
  const Layout l = layout(d, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t nk = L * d->top_k;
  const int32_t* idx;
  const float* wts;
  _Float16* a = at<_Float16>(ws, l.a);
  _Float16* b = at<_Float16>(ws, l.b);
  int32_t* cnt = at<int32_t>(ws, l.cnt);
  int32_t* list = at<int32_t>(ws, l.list);
  FrontArgs fa{};
  fa.x = x; fa.x_dtype = x_dtype; fa.L = L; fa.D = d->hidden; fa.eps = d->rms_eps;
  fa.w_pre = w->pre_ff_norm; fa.w_pre2 = w->pre_ff_norm_2; fa.a = a; fa.b = b;
  fa.E = d->n_experts; fa.cnt = cnt; fa.rowid = at<int32_t>(ws, l.rowid);
  const uint64_t stamp = next_stamp();
  set_stamp(fa, ws, l, stamp);
  if (forced) {
    DG_TRY(mk.mark(st));
    DG_TRY(hip_ok(launch_front(fa, st)));
    idx = force_idx;
    wts = force_w;
    if (topk_idx_out)
      DG_TRY(hip_ok(hipMemcpyAsync(topk_idx_out, force_idx, nk * 4, hipMemcpyDeviceToDevice, st)));
    if (topk_w_out)
      DG_TRY(hip_ok(hipMemcpyAsync(topk_w_out, force_w, nk * 4, hipMemcpyDeviceToDevice, st)));
    DG_TRY(hip_ok(launch_assign(idx, L, d->top_k, d->n_experts, cnt, list, l.list_cap, fa.sync,
                                stamp, st)));
  } else {
    int32_t* ri = topk_idx_out ? topk_idx_out : at<int32_t>(ws, l.idx);
    float* rw = topk_w_out ? topk_w_out : at<float>(ws, l.wts);
    fa.router_scale = w->router_scale; fa.wr = &w->router; fa.plog = at<float>(ws, l.plog);
    fa.k = d->top_k; fa.bias = w->router_bias; fa.pes = w->per_expert_scale;
    fa.idx = ri; fa.w = rw; fa.list = list; fa.cap = l.list_cap;
    DG_TRY(mk.mark(st));
    DG_TRY(hip_ok(launch_front(fa, st)));
    idx = ri;
    wts = rw;
  }
  int parts = 1;
  DG_TRY(run_gemms(d, w, L, l, ws, true, stamp, st, mk, &parts));
  DG_TRY(mk.mark(st));
  DG_TRY(hip_ok(launch_combine(at<_Float16>(ws, l.slots), at<float>(ws, l.h1), parts, idx, wts, x, x_dtype, L,
                               d->hidden, d->top_k, d->n_experts, d->rms_eps, w->post_ff_norm_1,
                               w->post_ff_norm_2, w->post_ff_norm, w->layer_scalar, nullptr, y,
                               y_dtype, st)));
  DG_TRY(mk.mark(st));
  return DGMOE_OK;
}

dgmoe_status dgmoe_block_forward(const dgmoe_dims* d, const dgmoe_block_weights* w, const void* x,
                                 int32_t x_dtype, int64_t L, const int32_t* force_idx,
                                 const float* force_w, void* y, int32_t y_dtype,
                                 int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                 size_t ws_bytes, void* stream) {
  Marks none;
  return block_forward(d, w, x, x_dtype, L, force_idx, force_w, y, y_dtype, topk_idx_out,
                       topk_w_out, ws, ws_bytes, stream, none);
}

dgmoe_status dgmoe_block_forward_noalloc(const dgmoe_dims* d, const dgmoe_block_weights* w,
                                         const void* x, int32_t x_dtype, int64_t L,
                                         const int32_t* force_idx, const float* force_w, void* y,
                                         int32_t y_dtype, int32_t* topk_idx_out, float* topk_w_out,
                                         void* stream) {
  if (!d) return DGMOE_ERR_NULL_ARG;
  const size_t need = dgmoe_workspace_size(d, L);
  if (need == 0 && L != 0) return DGMOE_ERR_BAD_DIMS;
  if (need > kScratchBytes) return DGMOE_ERR_WORKSPACE;
  if (L == 0) {
    Marks none;
    return block_forward(d, w, x, x_dtype, L, force_idx, force_w, y, y_dtype, topk_idx_out,
                         topk_w_out, nullptr, 0, stream, none);
  }
  void* ws = nullptr;
  DG_TRY(scratch_ptr(&ws));
  Marks none;
  return block_forward(d, w, x, x_dtype, L, force_idx, force_w, y, y_dtype, topk_idx_out,
                       topk_w_out, ws, kScratchBytes, stream, none);
}

size_t dgmoe_noalloc_max_bytes(void) { return kScratchBytes; }

dgmoe_status dgmoe_block_forward_profiled(const dgmoe_dims* d, const dgmoe_block_weights* w,
                                          const void* x, int32_t x_dtype, int64_t L, void* y,
                                          int32_t y_dtype, void* ws, size_t ws_bytes,
                                          void* stream, void** events, int32_t n_events) {
  if (!events) return DGMOE_ERR_NULL_ARG;
  if (n_events != DGMOE_PROFILE_EVENTS) return DGMOE_ERR_BAD_DIMS;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return DGMOE_ERR_NULL_ARG;
  Marks mk;
  mk.ev = reinterpret_cast<hipEvent_t*>(events);
  mk.n = n_events;
  return block_forward(d, w, x, x_dtype, L, nullptr, nullptr, y, y_dtype, nullptr, nullptr, ws,
                       ws_bytes, stream, mk);
}

dgmoe_status dgmoe_pack(const float* w, int64_t rows, int64_t cols, int32_t fmt, void* codes,
                        uint16_t* scale_bias, void* stream) {
  if (fmt != DGMOE_Q4G64 && fmt != DGMOE_Q4G32 && fmt != DGMOE_Q8G64 && fmt != DGMOE_NVFP4 &&
      fmt != DGMOE_Q6G32)
    return DGMOE_ERR_BAD_DTYPE;
  if (rows < 1 || cols < 64 || cols % 64 || rows * (cols / 64) > (int64_t(1) << 40)) return DGMOE_ERR_BAD_DIMS;
  if (fmt != DGMOE_Q8G64 && rows % 64) return DGMOE_ERR_BAD_DIMS;
  if (!w || !codes || !scale_bias) return DGMOE_ERR_NULL_ARG;
  if (!aligned(w, 16) || !aligned(codes, 64) || !aligned(scale_bias, 64)) return DGMOE_ERR_MISALIGNED;
  return hip_ok(launch_pack(w, rows, cols, fmt, codes, scale_bias, static_cast<hipStream_t>(stream)));
}

dgmoe_status dgmoe_unpack(const void* codes, const uint16_t* scale_bias, int64_t rows, int64_t cols,
                          int32_t fmt, int32_t out_dtype, void* out, void* stream) {
  if (fmt != DGMOE_Q4G64 && fmt != DGMOE_Q4G32 && fmt != DGMOE_Q8G64 && fmt != DGMOE_NVFP4 &&
      fmt != DGMOE_Q6G32)
    return DGMOE_ERR_BAD_DTYPE;
  if (out_dtype != DGMOE_F32 && out_dtype != DGMOE_F16) return DGMOE_ERR_BAD_DTYPE;
  if (rows < 1 || cols < 64 || cols % 64 || rows * (cols / 64) > (int64_t(1) << 40)) return DGMOE_ERR_BAD_DIMS;
  if (fmt != DGMOE_Q8G64 && rows % 64) return DGMOE_ERR_BAD_DIMS;
  if (!codes || !scale_bias || !out) return DGMOE_ERR_NULL_ARG;
  if (!aligned(codes, 64) || !aligned(scale_bias, 64) || !aligned(out, 16)) return DGMOE_ERR_MISALIGNED;
  return hip_ok(launch_unpack(codes, scale_bias, rows, cols, fmt, out_dtype, out,
                              static_cast<hipStream_t>(stream)));
}

dgmoe_status dgmoe_check_workspace(const dgmoe_dims* d, int64_t L, const void* ws,
                                   uint32_t* flags, void* stream) {
  if (!d || !ws || !flags) return DGMOE_ERR_NULL_ARG;
  if (!dims_ok(d) || L < 1 || L > kMaxL) return DGMOE_ERR_BAD_DIMS;
  if (!aligned(ws, 256)) return DGMOE_ERR_MISALIGNED;
  *flags = 0;
  return read_flags(ws, layout(d, L).sync, flags, stream);
}

size_t dgmoe_head_workspace_size(const dgmoe_head_dims* h, int64_t L) {
  if (!h || !head_dims_ok(h) || L < 0 || L > kMaxL) return 0;
  return head_layout(h, L).total;
}

dgmoe_status dgmoe_tail(const dgmoe_head_dims* h, const dgmoe_head_weights* w, const void* x,
                        int32_t x_dtype, int64_t L, float temperature, float* entropy,
                        int32_t* argmax, float* row_max, float* row_sum, float* logits, void* ws,
                        size_t ws_bytes, void* stream) {
  DG_TRY(check_head(h, w, L, ws, ws_bytes));
  if (x_dtype != DGMOE_F32 && x_dtype != DGMOE_BF16) return DGMOE_ERR_BAD_DTYPE;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return DGMOE_ERR_BAD_DIMS;
  DG_TRY(check_vec(w->final_norm));
  if (L == 0) return DGMOE_OK;
  if (!x || !entropy || !argmax) return DGMOE_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(entropy, 4) || !aligned(argmax, 4) ||
      (row_max && !aligned(row_max, 4)) || (row_sum && !aligned(row_sum, 4)) ||
      (logits && !aligned(logits, 16)))
    return DGMOE_ERR_MISALIGNED;
  const HeadLayout hl = head_layout(h, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  FrontArgs fa{};
  fa.x = x; fa.x_dtype = x_dtype; fa.L = L; fa.D = h->hidden; fa.eps = h->rms_eps;
  fa.w_pre = w->final_norm; fa.a = at<_Float16>(ws, hl.xn);
  set_stamp(fa, ws, hl.blk, next_stamp());
  DG_TRY(hip_ok(launch_front(fa, st)));
  TailArgs ta{};
  ta.xn = fa.a; ta.L = L; ta.D = h->hidden; ta.V = h->vocab;
  ta.codes = (const uint32_t*)w->embed.data; ta.sb = (const uint32_t*)w->embed.scale_bias;
  ta.inv_t = 1.0f / temperature;
  ta.logits = logits;
  ta.pstat = at<float4>(ws, hl.tstat);
  ta.entropy = entropy; ta.argmax = argmax; ta.row_max = row_max; ta.row_sum = row_sum;
  DG_TRY(hip_ok(launch_tail(ta, st)));
  return DGMOE_OK;
}

dgmoe_status dgmoe_soft_embed(const dgmoe_head_dims* h, const dgmoe_head_weights* w,
                              const float* sc_logits, int64_t L, float* soft, void* ws,
                              size_t ws_bytes, void* stream) {
  DG_TRY(check_head(h, w, L, ws, ws_bytes));
  if (L == 0) return DGMOE_OK;
  if (!sc_logits || !soft) return DGMOE_ERR_NULL_ARG;
  if (!aligned(sc_logits, 16) || !aligned(soft, 16)) return DGMOE_ERR_MISALIGNED;
  const HeadLayout hl = head_layout(h, L);
  const SoftArgs sa = soft_args(h, w, sc_logits, L, ws, hl, soft, next_stamp());
  DG_TRY(hip_ok(launch_soft_embed(sa, static_cast<hipStream_t>(stream))));
  return DGMOE_OK;
}

dgmoe_status dgmoe_sc_input(const dgmoe_head_dims* h, const dgmoe_head_weights* w,
                            const int32_t* canvas_ids, const float* sc_logits, int64_t L,
                            float* out, void* ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_head(h, w, L, ws, ws_bytes));
  if (sc_logits) {
    DG_TRY(check_pair(w->sc_gate_up, w->sc_down));
    if (w->sc_gate_up.dtype != DGMOE_Q4G64) return DGMOE_ERR_BAD_DTYPE;
    DG_TRY(check_vec(w->sc_pre_norm));
  }
  if (L == 0) return DGMOE_OK;
  if (!canvas_ids || !out) return DGMOE_ERR_NULL_ARG;
  if (!aligned(canvas_ids, 4) || !aligned(out, 16) || (sc_logits && !aligned(sc_logits, 16)))
    return DGMOE_ERR_MISALIGNED;
  const HeadLayout hl = head_layout(h, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t stamp = next_stamp();
  uint32_t* sync = at<uint32_t>(ws, hl.blk.sync);
  const uint32_t* codes = (const uint32_t*)w->embed.data;
  const uint32_t* sb = (const uint32_t*)w->embed.scale_bias;
  if (!sc_logits) {  // no previous prediction: the signal is zero and so is the MLP's output
    DG_TRY(hip_ok(launch_sc_out(canvas_ids, L, h->hidden, h->vocab, codes, sb, nullptr, 0,
                                h->rms_eps, out, sync, stamp, true, st)));
    return DGMOE_OK;
  }
  float* soft = at<float>(ws, hl.soft);
  DG_TRY(hip_ok(launch_soft_embed(soft_args(h, w, sc_logits, L, ws, hl, soft, stamp), st)));
  // n = fp16(rms(soft) * sc_pre_norm) as the dense operand; clears the GEMM counters
  FrontArgs fa{};
  fa.x = soft; fa.x_dtype = DGMOE_F32; fa.L = L; fa.D = h->hidden; fa.eps = h->rms_eps;
  fa.w_pre = w->sc_pre_norm; fa.a = at<_Float16>(ws, hl.blk.a);
  fa.cnt = at<int32_t>(ws, hl.blk.cnt); fa.rowid = at<int32_t>(ws, hl.blk.rowid);
  set_stamp(fa, ws, hl.blk, stamp);
  DG_TRY(hip_ok(launch_front(fa, st)));
  dgmoe_block_weights bw{};
  bw.expert_gate_up = bw.dense_gate_up = w->sc_gate_up;
  bw.expert_down = bw.dense_down = w->sc_down;
  const dgmoe_dims d = sc_dims(h);
  Marks none;
  int parts = 1;
  DG_TRY(run_gemms(&d, &bw, L, hl.blk, ws, true, stamp, st, none, &parts));
  DG_TRY(hip_ok(launch_sc_out(canvas_ids, L, h->hidden, h->vocab, codes, sb, at<float>(ws, hl.blk.h1),
                              parts, h->rms_eps, out, sync, stamp, false, st)));
  return DGMOE_OK;
}

dgmoe_status dgmoe_head_check_workspace(const dgmoe_head_dims* h, int64_t L, const void* ws,
                                        uint32_t* flags, void* stream) {
  if (!h || !ws || !flags) return DGMOE_ERR_NULL_ARG;
  if (!head_dims_ok(h) || L < 1 || L > kMaxL) return DGMOE_ERR_BAD_DIMS;
  if (!aligned(ws, 256)) return DGMOE_ERR_MISALIGNED;
  return read_flags(ws, head_layout(h, L).blk.sync, flags, stream);
}

void dgmoe_debug_force_stamp_timeout(int32_t spin_limit) { g_debug_spin = spin_limit > 0 ? spin_limit : 0; }

int32_t dgmoe_debug_set_tall_min(int32_t rows) {
  const int prev = g_mix_tall_min;
  g_mix_tall_min = rows < 0 ? DG_MIX_TALL_MIN : rows;
  return prev;
}

}  // extern "C"
