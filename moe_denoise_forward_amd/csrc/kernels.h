// Internal launchers of libdgmoe (host side).  Each returns the HIP status of
// its launch; the C ABI in dgmoe_api.cpp maps failures to DGMOE_ERR_HIP.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgmoe.h"

// Rows of one GEMM work tile and the column widths of the two GEMM phases.
constexpr int DG_MT = 32;       // rows (token-expert pairs) per tile
constexpr int DG_NGU = 64;      // gate columns per gate_up tile (and 64 matching up columns)
constexpr int DG_NDN = 128;     // output columns per down tile (bf16 weights)
constexpr int DG_NDN_Q4 = 256;  // output columns per down tile (Q4G64 short tiles)
// K chunks of the dense MLP's down projection in the short-tile q4 path: about
// I_d / I, at most 8 (every chunk at least one 64-input group)
__host__ __device__ constexpr int dense_down_chunks(int expert_inter, int dense_inter) {
  return dense_inter / expert_inter < 1 ? 1 : (dense_inter / expert_inter > 8 ? 8 : dense_inter / expert_inter);
}

// Groups of the grouped GEMMs: the experts, then the dense MLP.
constexpr int DG_MAX_GROUPS = 257;
// The counter block: the pair count of expert e at word e * DG_CNT_STRIDE
// (e < 256; one 128-byte line per expert, so the appends of different experts
// do not queue on one line), the GEMM work-queue counters (8 per launch:
// gate_up, down, the tall tiles of a mixed launch's gate_up and down, then the
// dense MLP's own gate_up and down when its format differs from the experts')
// at [DG_QUEUE_OFF, +48), and at [DG_ZERO_OFF, +64), on cache lines of their own,
// 64 words that stay zero (the scales and biases a GEMM wave reads for a
// group it does not own); the first launch of a call zeroes the counts, the
// queue counters and the zero words.
constexpr int DG_CNT_STRIDE = 32;
constexpr int DG_QUEUE_OFF = 256 * DG_CNT_STRIDE;
constexpr int DG_ZERO_OFF = DG_QUEUE_OFF + 128;
constexpr int DG_ZERO_WORDS = 64;
constexpr int DG_COUNTERS = DG_ZERO_OFF + DG_ZERO_WORDS;
// Words of the counter block that must be zero at the start of a call: the
// counts (i < 256: word i * DG_CNT_STRIDE), then the rest from DG_QUEUE_OFF.
constexpr int DG_CLEAR_WORDS = 256 + (DG_COUNTERS - DG_QUEUE_OFF);
__host__ __device__ constexpr int dg_clear_word(int i) {
  return i < 256 ? i * DG_CNT_STRIDE : DG_QUEUE_OFF + (i - 256);
}

constexpr int DG_FRONT_ROWS = 16;  // rows per front workgroup
// The sync region of the workspace, in 32-bit words:
//   [0, 2)   the stamp the front kernel's workgroup (0, 0) publishes once it
//            has cleared the counters (the other workgroups wait for it);
//   [2, 4)   the call stamp: the stamp of the last call that ran on the
//            workspace (written by the first kernel of every call);
//   [4, 4 + 2 DG_ERR_KINDS)  one 64-bit error word per kind: the stamp of the
//            last call in which that error happened (no word is ever cleared:
//            a stale error carries an older stamp);
//   then one arrival counter per front row block.
// A call hit error kind i iff error word i equals the call stamp.
constexpr int DG_ERR_SYNC = 0;    // a front workgroup gave up waiting for the stamp
constexpr int DG_ERR_RANGE = 1;   // an fp16 intermediate would have overflowed
constexpr int DG_ERR_ROUTE = 2;   // a caller routing overfilled an expert's pair list
constexpr int DG_ERR_INDEX = 3;   // a canvas token id outside [0, V)
constexpr int DG_ERR_KINDS = 4;
constexpr int DG_SYNC_CALL = 2;
constexpr int DG_SYNC_ERR = 4;
constexpr int DG_SYNC_HEAD = DG_SYNC_ERR + 2 * DG_ERR_KINDS;
inline int64_t front_sync_words(int64_t L) { return DG_SYNC_HEAD + (L + DG_FRONT_ROWS - 1) / DG_FRONT_ROWS; }

// Largest magnitude that converts to a finite fp16 under round-to-nearest-even
// (65504 is the largest fp16; from 65520 on the conversion gives inf).
constexpr float DG_F16_LIMIT = 65520.0f;

// The front of the block in one launch, grid (row blocks of 16, groups of
// expert tiles of 16):
//   * RMSNorm of x; a = fp16(xh*w_pre) and b = fp16(xh*w_pre2) where non-null;
//   * if wr is non-null, the router's logits (+ bias) for the workgroup's
//     experts into plog[L][E], and, in the last workgroup of each row block to
//     arrive, the top-k by (logit desc, index asc), the softmax over the k
//     times pes into idx/w (logits too if non-null) and, if list is non-null,
//     each chosen pair p = t*k + j appended to its expert's list
//     (i = atomicAdd(&cnt[e], 1): list[e*cap + i] = p, list[(E + e)*cap + i]
//     = t; the order within an expert is whatever the atomics give and results
//     do not depend on it);
//   * the counter block cnt (if non-null: expert counts and GEMM queues) and
//     the row-block arrival counters are zeroed by workgroup (0, 0), which then
//     publishes `stamp` (distinct for every call on a workspace) in sync[0..1];
//     no workgroup counts its arrival before it has seen the stamp;
//   * rowid[t] = t (if non-null): the dense MLP's row list.
//   * the wait for the stamp is bounded (spin_limit polls); a workgroup that
//     gives up flags DG_ERR_SYNC and neither counts its arrival nor appends to
//     the lists (so the routing of its row block is never written and the
//     call's results are not to be used; the GEMMs clamp every count and row
//     id they read, so nothing is read or written out of bounds);
//   * publish = 0 (diagnostics only) suppresses the stamp, so that every
//     waiting workgroup gives up;
//   * an operand whose value does not fit fp16 flags DG_ERR_RANGE.
// k_norm (no router) writes the call stamp and clears the counters itself.
struct FrontArgs {
  const void* x; int x_dtype; int64_t L; int D; float eps;
  const float* w_pre; const float* w_pre2; _Float16* a; _Float16* b;
  const float* router_scale; const dgmoe_matrix* wr; int E; float* plog;
  int k; const float* bias; const float* pes; int32_t* idx; float* w; float* logits;
  int32_t* cnt; int32_t* list; int64_t cap; int32_t* rowid;
  uint32_t* sync; uint64_t stamp; int spin_limit; int publish;
};
hipError_t launch_front(const FrontArgs& a, hipStream_t st);

// The same pair lists from a given routing (indices outside [0, E) are
// skipped; a pair past its expert's list capacity is dropped and flags
// DG_ERR_ROUTE).
hipError_t launch_assign(const int32_t* idx, int64_t L, int k, int E, int32_t* cnt, int32_t* list,
                         int64_t cap, uint32_t* sync, uint64_t stamp, hipStream_t st);

// Grouped GEMM phases.  Group g < E is expert g (rows = its pairs), group E is
// the dense MLP (rows = positions).
struct GemmPhaseArgs {
  // weights of the experts [E, N_e, K_e] and of the dense MLP [N_d, K_d]; a
  // launch with both groups has one format for both
  int wfmt_e, wfmt_d;
  // 1: the experts have no rows in this launch (the dense MLP alone, in its
  // own format); their pair counts are ignored
  int skip_e;
  const void* w_e; const uint32_t* sb_e;   // codes (or bf16 values), (scale|bias<<16) pairs
  const void* w_d; const uint32_t* sb_d;
  int n_e, k_e, n_d, k_d;    // matrix rows (out) and cols (in)
  // A operands [rows, K] fp16
  const _Float16* a_e;       // gate_up: b [L, D] gathered via perm; down: act [L*k, I]
  const _Float16* a_d;       // gate_up: a [L, D]; down: act_d [L, I_d]
  // routing: per-expert pair counts and lists (pair ids at list[e*list_cap + i],
  // their tokens at list[(E + e)*list_cap + i]); the
  // dense MLP's rows 0..L-1 (rowid[t] = t); DG_ZERO_WORDS zero words
  const int32_t* cnt;
  const int32_t* list;
  const int32_t* rowid;
  const uint32_t* zero;
  int64_t list_cap;
  int E, topk;
  int* queue;              // this phase's 8 work-queue counters (zero at launch)
  int dense_rows;          // rows of the dense group (0: none)
  int nt_e, nt_d;          // column tiles per expert / per dense row tile
  // outputs
  _Float16* act_e; _Float16* act_d;    // gate_up outputs [L*k, I], [L, I_d]
  _Float16* slots; float* h1;           // down outputs [L*k, D] (fp16), [L, D]
  // down, short q4 tiles: the dense MLP's K is cut into kch_d chunks of about
  // an expert's K, so that its tiles cost about what an expert tile costs;
  // chunk c writes the partial sum h1 + c * L * D (the combine adds the
  // partials in chunk order).  Every other path: kch_d = 1.
  int kch_d;
  int max_tiles;                        // host upper bound on the tile count
  // Q4G64 only: tall tiles (64 rows) for batches with many rows per expert
  int tall;
  // Q4G64, short tiles only: experts with at least tall_min pairs take tall
  // tiles in the same launch (0: none do)
  int tall_min;
  // pairs = L*k (act / slot rows) and n_tok = L (b / a rows): every count read
  // from the workspace is clamped to list_cap and the experts' rows together
  // to pairs; every pair id to [0, pairs) and token to [0, n_tok)
  int64_t pairs, n_tok;
  // error words (sync region) and the call's stamp: an act or slot value that
  // does not fit fp16 flags DG_ERR_RANGE
  uint32_t* sync;
  uint64_t stamp;
};
// Tall tiles pay off from about this many pairs per expert on average
// (measured on the full-size q4 block: at 16 pairs per expert short tiles take
// 0.165 ms per step and tall ones 0.208; at 32, 0.233 vs 0.224; at 48, 0.295
// vs 0.238; at 64, 0.362 vs 0.314).
constexpr int DG_TALL_MIN_ROWS = 32;
// Below that average, an expert with at least this many pairs may still take
// tall tiles in the same launch (one 64-row tile in place of two or more
// 32-row ones); 0 = none do, the default: with only a few such experts their
// tall tiles are too few and too long to fill the GPU (measured on 30 blocks
// whose router sends all 256 positions to the same 8 experts: 116 us per block
// with 32-row tiles only, 125 us with the 8 hot experts on 64-row tiles, and
// no change at canvas 256, where no expert reaches 33 pairs).
constexpr int DG_MIX_TALL_MIN = 0;
hipError_t launch_gate_up(const GemmPhaseArgs& a, hipStream_t st);
hipError_t launch_down(const GemmPhaseArgs& a, hipStream_t st);

// moe = sum_j w[t*k+j] * slots[t*k+j]; then either moe_out = moe, or the post-norms,
// residual and layer_scalar into y (F32 or BF16), with h1 the sum of h1_parts
// partial sums [h1_parts, L, D] added in order.
// Pairs whose expert index is outside [0, E) contribute nothing.
hipError_t launch_combine(const _Float16* slots, const float* h1, int h1_parts, const int32_t* idx,
                          const float* w, const void* x,
                          int x_dtype, int64_t L, int D, int k, int E, float eps, const float* wp1,
                          const float* wp2, const float* wp, float layer_scalar,
                          float* moe_out, void* y, int y_dtype, hipStream_t st);

hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, int fmt, void* codes,
                       uint16_t* scale_bias, hipStream_t st);
hipError_t launch_unpack(const void* codes, const uint16_t* scale_bias, int64_t rows,
                         int64_t cols, int fmt, int out_dtype, void* out, hipStream_t st);

// ---------------------------------------------------------------- canvas head
// The tied embedding table E [V, D] (Q4G64) at both ends of a forward.
//
// Tail: xn = fp16(rms(x) * final_norm) [L, D] (written by the front's norm
// kernel) against E^T.  One tile is up to 256 rows times 256 vocabulary rows;
// for every row it leaves (m, l, s, best) over the tile's columns of
// y = softcap(z) / T: m the largest y, l = sum exp(y - m), s = sum exp(y - m)
// (y - m), best the lowest column holding m (its bits in .w).  The merge then
// gives entropy = ln l - s / l (nats), argmax, and the row's m and l.
constexpr int DG_HEAD_COLS = 256;  // vocabulary rows per tail tile
struct TailArgs {
  const _Float16* xn; int64_t L; int D; int V;
  const uint32_t* codes; const uint32_t* sb;  // the table: codes, (scale | bias << 16) words
  float inv_t;          // 1 / T
  float* logits;        // [L, V] y, or null
  float4* pstat;        // [ceil(V / 256), L]
  float* entropy; int32_t* argmax; float* row_max; float* row_sum;  // [L]; the last two may be null
};
hipError_t launch_tail(const TailArgs& a, hipStream_t st);

// Self-conditioning's soft embedding soft = softmax(y) E sqrt(D), y the
// previous step's logits [L, V] (already divided by T).  The sum over the
// vocabulary is cut into `pieces` ranges of 64-row blocks; per (row, piece)
// the probabilities are kept as p16 = fp16(2^14 exp(y - m_piece)) with
// (m_piece, l_piece = sum exp(y - m_piece)) in pst; each (piece, row tile,
// 256-column block) workgroup sums p16 x E over its range into part; the
// reduce rescales the pieces to the row's max and writes soft.
constexpr int DG_SOFT_ROWS = 256;     // rows per soft-embedding tile
constexpr int DG_SOFT_MAXBLK = 256;   // 64-row blocks per piece at most
constexpr int DG_SOFT_MAXPIECES = 1024;
struct SoftArgs {
  const float* logits; int64_t L; int D; int V;
  const uint32_t* codes; const uint32_t* sb;
  int pieces;
  _Float16* p16;        // [L, V]
  float2* pst;          // [pieces, L]
  float* part;          // [pieces, L, D]
  float* soft;          // [L, D]
  uint32_t* sync; uint64_t stamp;  // the first launch writes the call stamp
};
hipError_t launch_soft_embed(const SoftArgs& a, hipStream_t st);
// Vocabulary pieces of a soft embedding (host): enough workgroups for 256
// CUs, pieces of at most DG_SOFT_MAXBLK blocks.
int soft_pieces(int64_t L, int D, int V);

// The canvas input: out = rms(E[ids] sqrt(D) + sum of h1_parts partials
// [h1_parts, L, D]) without weight (h1 may be null: no self-conditioning
// signal).  An id outside [0, V) reads row 0 and flags DG_ERR_INDEX.  If
// first, the kernel writes the call stamp.
hipError_t launch_sc_out(const int32_t* ids, int64_t L, int D, int V, const uint32_t* codes,
                         const uint32_t* sb, const float* h1, int h1_parts, float eps, float* out,
                         uint32_t* sync, uint64_t stamp, bool first, hipStream_t st);

// ---------------------------------------------------------------- denoise attention
// One layer's canvas attention (attn.hip).  Canvas row t sits at position
// kv_len + t; its keys are the committed positions [s0, kv_len) of the cache
// (n_enc = kv_len - s0 of them) followed by the L canvas rows.
constexpr int DG_ATTN_KT = 32;        // keys per tile
constexpr int DG_ATTN_ROWS = 64;      // query rows (head-major within a KV head) per workgroup
constexpr int DG_ATTN_MAXCHUNKS = 16; // key ranges a row's keys are split into at most
struct AttnArgs {
  const void* q; const void* k; const void* v;  // raw projections [L, H*hd], [L, Hkv*hd] (v null: from k)
  int in_dtype;                                 // DGMOE_F32 or DGMOE_BF16
  int64_t L; int H, Hkv, hd;
  const float* wq; const float* wk;             // QK-norm weights [hd]
  const _Float16* kc; const _Float16* vc;       // committed cache [Hkv, cap, hd]
  int64_t cap, kv_len, s0, n_enc;
  int n_rot, stride;                            // rotated pairs (d, d + stride), d < n_rot
  float theta, den, eps;
  _Float16* qp; _Float16* kp; _Float16* vp;     // prepared q [H, L, hd], k / v [Hkv, L, hd]
  int chunks, tiles_per_chunk;                  // key ranges (tiles of DG_ATTN_KT keys)
  float* opart;                                 // [chunks, H, L, hd] unnormalised partial outputs
  float2* ml;                                   // [chunks, H, L] (running max of log2(e) x score, sum of 2^(. - max))
  void* out; int out_dtype;                     // [L, H*hd], DGMOE_F32 or DGMOE_BF16
};
// Key tiles of a row (host): the committed rows and the canvas rows each
// in tiles of DG_ATTN_KT, the last of each ragged.
int attn_tiles(int64_t n_enc, int64_t L);
// Key ranges (of whole tiles) per row for the workgroups to fill the GPU (host).
int attn_chunks(int64_t L, int H, int Hkv, int hd, int64_t n_tiles);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
