// Internal launchers of libdgmoe (host side).  Each returns the HIP status of
// its launch; the C ABI in dgmoe_api.cpp maps failures to DGMOE_ERR_HIP.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgmoe.h"

// Rows of one GEMM work tile and the column widths of the two GEMM phases.
constexpr int DG_MT = 32;       // rows (token-expert pairs) per tile
constexpr int DG_NGU = 64;      // gate columns per gate_up tile (and 64 matching up columns)
constexpr int DG_NDN = 128;     // output columns per down tile
constexpr int DG_ROUTE_ROWS = 16;

// RMSNorm of x: writes a = fp16(xh*pre_ff_norm), b = fp16(xh*pre_ff_norm_2) and
// u = xh*router_scale*c (fp32); any output pointer may be null.
hipError_t launch_norm(const void* x, int x_dtype, int64_t L, int D, float eps,
                       const float* w_pre, const float* w_pre2, const float* router_scale,
                       _Float16* a, _Float16* b, float* u, hipStream_t st);

// logits[L, E] = u[L, D] . W_r^T (+ bias), fp32.
hipError_t launch_router(const float* u, int64_t L, int D, int E, const dgmoe_matrix* wr,
                         const float* bias, float* logits, hipStream_t st);

// Per row: top-k by (logit desc, index asc), softmax over the k, times pes.
hipError_t launch_topk(const float* logits, int64_t L, int E, int k, const float* pes,
                       int32_t* idx, float* w, hipStream_t st);

// Expert-major permutation of the L*k (token, slot) pairs and the tile tables.
struct PlanOut {
  int32_t* perm;       // [L*k] pair index (t*k + j) for each expert-sorted row
  int32_t* grp_off;    // [E+1] first expert-sorted row of each group (dense: 0)
  int32_t* grp_cnt;    // [E+1] rows of each group (dense: dense_rows)
  int32_t* n_tiles;    // [8]: gate_up {entries, -, first dense entry, -}, down at +4 likewise
  int4* tiles_gu;      // gate_up tiles {group, first row, rows, column tile}
  int4* tiles_dn;      // down tiles, same encoding
};
hipError_t launch_plan(const int32_t* idx, int64_t L, int k, int E, int nt_gu_exp,
                       int nt_gu_dense, int nt_dn, int dense_rows, const PlanOut& out,
                       hipStream_t st);

// Grouped GEMM phases.  Group g < E is expert g (rows = its pairs), group E is
// the dense MLP (rows = positions).
struct GemmPhaseArgs {
  // weights of the experts [E, N_e, K_e] and of the dense MLP [N_d, K_d]
  int wfmt_e, wfmt_d;
  const void* w_e; const uint32_t* sb_e;   // codes (or bf16 values), (scale|bias<<16) pairs
  const void* w_d; const uint32_t* sb_d;
  int n_e, k_e, n_d, k_d;    // matrix rows (out) and cols (in)
  // A operands [rows, K] fp16
  const _Float16* a_e;       // gate_up: b [L, D] gathered via perm; down: act [L*k, I]
  const _Float16* a_d;       // gate_up: a [L, D]; down: act_d [L, I_d]
  // plan
  const int32_t* perm;
  const int4* tiles;       // tile table (device)
  const int32_t* n_tiles;  // [0] entries, [2] first dense entry (device)
  int E, topk;
  // outputs
  _Float16* act_e; _Float16* act_d;    // gate_up outputs [L*k, I], [L, I_d]
  const float* route_w;                 // down: [L*k] weight of each pair
  float* slots; float* h1;              // down outputs [L*k, D], [L, D]
  int max_tiles;                        // host upper bound on the tile count
};
hipError_t launch_gate_up(const GemmPhaseArgs& a, hipStream_t st);
hipError_t launch_down(const GemmPhaseArgs& a, hipStream_t st);

// moe = sum_j slots[t*k+j]; then either moe_out = moe, or the post-norms,
// residual and layer_scalar into y (F32 or BF16).
// Pairs whose expert index is outside [0, E) contribute nothing.
hipError_t launch_combine(const float* slots, const float* h1, const int32_t* idx, const void* x,
                          int x_dtype, int64_t L, int D, int k, int E, float eps, const float* wp1,
                          const float* wp2, const float* wp, float layer_scalar,
                          float* moe_out, void* y, int y_dtype, hipStream_t st);

hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, int fmt, void* codes,
                       uint16_t* scale_bias, hipStream_t st);
hipError_t launch_unpack(const void* codes, const uint16_t* scale_bias, int64_t rows,
                         int64_t cols, int fmt, int out_dtype, void* out, hipStream_t st);
