/*
 * libdgmoe -- the DiffusionGemma parallel dense-MLP + routed-MoE FFN block on
 * one AMD MI355X (gfx950), as a C ABI.
 *
 * What the block computes (per canvas position t, rms(v) = v/sqrt(mean(v^2)+eps)):
 *   xh   = rms(x_t)
 *   z    = ((xh * router_scale) * hidden^-1/2) . W_router^T (+ router_bias)
 *   sel  = the top_k experts by (z desc, expert index asc)
 *   w_j  = softmax over the selected z, times per_expert_scale[sel_j]
 *   h1   = MLP_dense(xh * pre_ff_norm)
 *   moe  = sum_j w_j MLP_{sel_j}(xh * pre_ff_norm_2)
 *   y_t  = layer_scalar * (x_t + rms(rms(h1)*post_ff_norm_1 + rms(moe)*post_ff_norm_2) * post_ff_norm)
 *   MLP(v) = W_down (gelu_tanh(W_gate v) * (W_up v)),  [W_gate ; W_up] stacked in gate_up.
 * Sources: diffgemma "architecture & implemented contract", Part II section 2.1
 * "Forward-pass details" (the Norms and MoE-order bullets) and Part III
 * "Precision policy"; "DiffusionGemma Explained", section "MLP and
 * mixture-of-experts block" (MLP, MOEBlock) and "Complete DiffusionGemma model"
 * (layer_scalar); the mlx-bun DiffusionGemma port dossier, section 2
 * (DecoderLayer, Router, Experts) and section 1 (affine group-64 quantisation).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers unless stated otherwise; the caller
 *    owns every buffer, including the workspace.  The library allocates no
 *    device memory, keeps no state between calls, never synchronises the
 *    stream and never reads results back to the host.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Outputs are valid once the caller has synchronised the stream.
 *  - All arguments are checked on the host BEFORE anything is enqueued; on any
 *    failure nothing is enqueued and no output is touched.  A launch failure
 *    is reported as DGMOE_ERR_HIP; a fault inside a kernel surfaces at the
 *    caller's next synchronisation (HIP semantics).
 *  - L = 0 is a valid no-op.
 *  - Concurrent calls that share a workspace race; give each in-flight call
 *    its own workspace.
 */
#ifndef DGMOE_H
#define DGMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DGMOE_ABI_VERSION 9

typedef enum {
  DGMOE_OK = 0,
  DGMOE_ERR_NULL_ARG = 1,    /* a required pointer is NULL                          */
  DGMOE_ERR_BAD_DIMS = 2,    /* a size is out of range or not a multiple of 64      */
  DGMOE_ERR_BAD_DTYPE = 3,   /* unsupported dtype or format combination             */
  DGMOE_ERR_MISALIGNED = 4,  /* a pointer breaks the alignment rule below           */
  DGMOE_ERR_WORKSPACE = 5,   /* workspace smaller than dgmoe_workspace_size()       */
  DGMOE_ERR_HIP = 6,         /* the HIP runtime refused a launch                    */
  DGMOE_ERR_DEVICE = 7       /* dgmoe_check_workspace: the last call on the
                                workspace flagged a device-side error (flags)       */
} dgmoe_status;

typedef enum {
  DGMOE_F32 = 0,
  DGMOE_BF16 = 1,
  DGMOE_F16 = 2,
  DGMOE_Q4G64 = 3,  /* 4-bit affine, group 64 along the input dim, fp16 scale+bias */
  DGMOE_Q8G64 = 4,  /* 8-bit affine, group 64 along the input dim, fp16 scale+bias */
  DGMOE_Q4G32 = 5,  /* 4-bit affine, group 32 along the input dim, fp16 scale+bias */
  DGMOE_NVFP4 = 6,  /* FP4 E2M1, an E4M3 scale per 16 inputs, an fp32 scale per matrix */
  DGMOE_Q6G32 = 7   /* 6-bit affine, group 32 along the input dim, fp16 scale+bias */
} dgmoe_dtype;

/* Block dimensions.  hidden: a multiple of 64 in [64, 8192]; expert_inter,
 * dense_inter: multiples of 64 in [64, 16384]; 1 <= top_k <= min(n_experts,
 * 32); 1 <= n_experts <= 256; rms_eps finite and >= 0.  L (positions per
 * call) <= 2^20. */
typedef struct {
  int32_t hidden;        /* D                                 */
  int32_t n_experts;     /* E                                 */
  int32_t top_k;         /* k                                 */
  int32_t expert_inter;  /* I    (expert MLP intermediate)    */
  int32_t dense_inter;   /* I_d  (dense MLP intermediate)     */
  float rms_eps;         /* 1e-6 for DiffusionGemma           */
} dgmoe_dims;

/*
 * One matrix [rows, cols] with rows = outputs and cols = inputs (the
 * checkpoint's [out, in] orientation, which the diffgemma contract's "Standing
 * design decisions" keep), or E such matrices back to back for the expert
 * tensors.
 *   F32 / BF16 / F16: `data` holds rows*cols values, row-major; scale_bias NULL.
 *   Q8G64 (row-major): `data` holds rows*cols bytes, one code per input,
 *          row-major; scale_bias holds fp16 (scale, bias) pairs as uint16 at
 *          index (r * (cols/64) + q) * 2 + {0, 1} for group q = c / 64.
 *   Q4G64 (MFMA-tiled; rows % 64 == 0): rows form blocks of 64, G = cols/64.
 *          The code of input c = 64 q + 32 h + 8 g + j (h < 2, g < 4, j < 8)
 *          of row r = 64 b + 16 s + n (s < 4, n < 16) sits in the
 *          little-endian uint32 word
 *              ((((b * G + q) * 4 + g) * 16 + n) * 8 + 2 s + h
 *          at bits [4p + 16t, 4p + 16t + 4) where j = 2p + t; scale_bias holds
 *          the (scale, bias) pair of (r, q) at uint16 index
 *              (((b * G + q) * 16 + n) * 4 + s) * 2 + {0, 1}.
 *          One 64-input group of a 64-row block is thus 2 KB of contiguous
 *          codes and 256 bytes of scale_bias, and the 32 bytes a GEMM lane
 *          (g, n) feeds to the matrix cores for the four strips of the block
 *          (two 32-input halves each) are contiguous, as are its four pairs.
 *   Q4G32 (MFMA-tiled; rows % 64 == 0; the diffgemma contract's section 8
 *          "Quantization (.dgq)": MoE experts as q4 group-32 affine): the codes
 *          exactly as Q4G64; one (scale, bias) pair per 32 inputs, the pair of
 *          row r = 64 b + 16 s + n and inputs 64 q + 32 h .. +31 at uint16
 *          index
 *              ((((b * G + q) * 16 + n) * 4 + s) * 2 + h) * 2 + {0, 1}
 *          (G = cols/64 as for the codes), so the eight pairs a GEMM lane
 *          needs for one 64-input group are 32 contiguous bytes.
 *   NVFP4 (MFMA-tiled; rows % 64 == 0; the diffgemma contract's section 8
 *          nvfp4 expert format, read as NVIDIA's NVFP4): `data` holds 4-bit E2M1
 *          codes (bit 3 the sign; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) in
 *          exactly the words and bit positions of Q4G64; `scale_bias` holds
 *          bytes: the E4M3 scale (bias 7, max 448, no sign) of row
 *          r = 64 b + 16 s + n and inputs 64 q + 16 j .. +15 (j < 4) at byte
 *              (((b * G + q) * 16 + n) * 4 + s) * 4 + j,
 *          then a 64-byte trailer whose first 4 bytes are the matrix's float32
 *          tensor scale gs (the next 4 the packer's amax, the rest zero).
 *          Value: w = e2m1(code) * e4m3(byte) * gs.  The GEMMs feed
 *          e2m1 * e4m3 (exact in fp16) to the matrix cores and multiply the
 *          fp32 sums by gs.
 *   Q6G32 (MFMA-tiled; rows % 64 == 0; the contract's q6 expert format, read
 *          as 6-bit affine with groups of 32): scale_bias exactly as Q4G32;
 *          `data` holds two planes: the low 4 bits of every code in the
 *          rows*cols/8 words of Q4G64, then the high 2 bits in rows*cols/16
 *          words -- the high bits of the code in low-plane word
 *          ((((b * G + q) * 4 + g) * 16 + n) * 8 + 2 s + h, input j = 2p + t of
 *          its eight, sit in high-plane word (((b * G + q) * 4 + g) * 16 + n) * 4 + s
 *          at bits [2 (4h + p) + 16t, +2).
 *   Quantised value (affine formats): w = float(scale) * q + float(bias).  Each expert of a
 *   stacked tensor is laid out on its own (its matrices start at multiples of
 *   rows*cols codes and rows*cols/64 pairs, rows*cols/32 for Q4G32 and Q6G32,
 *   and of rows*cols/16 + 64 scale bytes for NVFP4).
 * Alignment: data and scale_bias must be 64-byte aligned (the diffgemma
 * contract, section 8 "Quantization (.dgq)", makes every tensor offset 64-byte
 * aligned because a misaligned typed read was silently wrong).
 */
typedef struct {
  int32_t dtype;                /* dgmoe_dtype                               */
  const void *data;
  const uint16_t *scale_bias;   /* packed formats only, else NULL           */
} dgmoe_matrix;

/* The block's weights.  Formats: router F32 | BF16 | Q8G64; the experts'
 * pair (expert_gate_up, expert_down) Q4G64 | Q4G32 | Q6G32 | NVFP4 | BF16, one format
 * for the two (the diffgemma contract, section 8.2 "Custom quantization classes",
 * requires experts.gate_up and experts.down to resolve to the same format);
 * the dense MLP's pair (dense_gate_up, dense_down) one of Q4G64 | Q4G32 |
 * Q6G32 | NVFP4 | BF16 | Q8G64, one format for the two, which may differ from the experts'
 * (the contract's section 8 runtime dispatch derives the dense and the expert
 * formats independently; its default pack is Q4G32 experts beside a BF16
 * dense MLP; the OptiQ checkpoint of the mlx-bun dossier, section 1, has Q4G64
 * experts beside an 8-bit group-64 dense MLP and router).  A BF16 or Q8G64
 * dense MLP beside Q4G64, Q4G32, Q6G32 or NVFP4 experts shares the experts' two GEMM
 * launches unless the experts take 64-row tiles (Q4G64 from 32 pairs per
 * expert on average); any other pair of different formats runs as four
 * launches (experts' gate_up, dense gate_up, experts' down, dense down).  The
 * [D] vectors (router_scale and the five norm weights) must be 16-byte
 * aligned; per_expert_scale and router_bias 4. */
typedef struct {
  dgmoe_matrix router;              /* [E, D]                                  */
  const float *router_scale;        /* [D]                                     */
  const float *per_expert_scale;    /* [E]                                     */
  const float *router_bias;         /* [E] added to the logits, or NULL        */
  dgmoe_matrix expert_gate_up;      /* [E, 2I, D]; rows [0,I) gate, [I,2I) up  */
  dgmoe_matrix expert_down;         /* [E, D, I]                               */
  dgmoe_matrix dense_gate_up;       /* [2I_d, D]; rows [0,I_d) gate, then up   */
  dgmoe_matrix dense_down;          /* [D, I_d]                                */
  const float *pre_ff_norm;         /* [D] dense-branch pre-norm weight        */
  const float *pre_ff_norm_2;       /* [D] expert pre-norm weight              */
  const float *post_ff_norm_1;      /* [D] dense-branch post-norm weight       */
  const float *post_ff_norm_2;      /* [D] expert-sum post-norm weight         */
  const float *post_ff_norm;        /* [D] post-norm of the branch sum         */
  float layer_scalar;               /* multiplies the whole block output       */
} dgmoe_block_weights;

/* Bytes of device workspace a call on L positions needs (for any entry point).
 * Returns 0 if the dims are invalid.  Workspace pointers must be 256-byte
 * aligned.  The workspace needs no initialisation: every call clears what it
 * counts with.  It holds, besides scratch, the call stamp and error words that
 * dgmoe_check_workspace reads. */
size_t dgmoe_workspace_size(const dgmoe_dims *dims, int64_t L);

/*
 * Device-side errors.  Some conditions can only be seen on the GPU, after the
 * call has been enqueued.  The kernels record them in the workspace (no host
 * readback happens in the calls themselves); the caller may check them with
 * dgmoe_check_workspace once the call has run.  Flag bits:
 *   DGMOE_FLAG_SYNC_TIMEOUT   a router workgroup gave up its bounded wait (about
 *                             50 ms) for the call's counters to be cleared; its
 *                             16 positions were not routed and the call's
 *                             outputs must not be used.  Not expected in
 *                             normal operation (it means the GPU did not run
 *                             one workgroup of the launch for that long).
 *   DGMOE_FLAG_FP16_RANGE     an intermediate held as fp16 did not fit (|v| >=
 *                             65520: it became inf): an operand x_hat * pre_ff_norm
 *                             or x_hat * pre_ff_norm_2 (|x_hat| <= sqrt(hidden),
 *                             so this needs a norm weight above 65504/sqrt(hidden)),
 *                             a GeGLU output gelu(g) * u of an MLP, or an
 *                             expert's output row (before its routing weight).
 *                             The outputs then hold inf or NaN where affected.
 *   DGMOE_FLAG_ROUTE_OVERFLOW a caller-given routing (dgmoe_moe_ffn, forced
 *                             routing of dgmoe_block_forward) named one expert
 *                             more than L times in total, which only happens if
 *                             a position names an expert twice; the pairs past
 *                             L were dropped.
 * Every index and count the kernels read from the workspace is clamped to its
 * buffer, so none of these conditions makes a kernel access memory out of
 * bounds.
 */
#define DGMOE_FLAG_SYNC_TIMEOUT 1u
#define DGMOE_FLAG_FP16_RANGE 2u
#define DGMOE_FLAG_ROUTE_OVERFLOW 4u
/* DGMOE_FLAG_INDEX: a canvas token id given to dgmoe_sc_input was outside
 * [0, vocab); that position used token 0. */
#define DGMOE_FLAG_INDEX 8u

/* Host, synchronous: waits for `stream`, then reads the flags of the last call
 * (of any entry point) that ran on `ws` (sized for dims and L, as that call
 * was).  Returns DGMOE_OK with *flags = 0, DGMOE_ERR_DEVICE with the flags
 * set, or an argument / DGMOE_ERR_HIP error. */
dgmoe_status dgmoe_check_workspace(const dgmoe_dims *dims, int64_t L, const void *ws,
                                   uint32_t *flags, void *stream);

/*
 * Router only.  x: [L, D] (x_dtype F32 or BF16, 16-byte aligned).
 * Outputs: topk_idx [L, k] int32 ordered by (logit desc, index asc);
 *          topk_w   [L, k] float = softmax over the selected logits *
 *                   per_expert_scale (router-order and sum rule of the
 *                   diffgemma contract's MoE-order bullet);
 *          logits   [L, E] float, the router logits (may be NULL).
 * Logits are computed in fp32 from the fp32 normalised input and the exact
 * dequantised router weights.
 */
dgmoe_status dgmoe_route(const dgmoe_dims *dims, const dgmoe_block_weights *w,
                         const void *x, int32_t x_dtype, int64_t L,
                         int32_t *topk_idx, float *topk_w, float *logits,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Routed experts only, with the routing given (the Experts(x, idx, w) call of
 * the mlx-bun dossier, section 2).  moe_out [L, D] float =
 *   sum_j topk_w[t,j] * MLP_{topk_idx[t,j]}(rms(x_t) * pre_ff_norm_2),
 * before post_ff_norm_2.  Pairs whose index is outside [0, E) contribute 0.
 * An expert may be named at most L times in total (always true when each
 * position names distinct experts); see DGMOE_FLAG_ROUTE_OVERFLOW.
 * The dense branch and the router are not run; the router fields of `w` and
 * the dense/post-norm fields may be NULL.
 */
dgmoe_status dgmoe_moe_ffn(const dgmoe_dims *dims, const dgmoe_block_weights *w,
                           const void *x, int32_t x_dtype, int64_t L,
                           const int32_t *topk_idx, const float *topk_w,
                           float *moe_out, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole block (the diffgemma contract, Part II section 2.1, the MoE-order
 * and Norms bullets; the ML@Berkeley post's MOEBlock and "Complete
 * DiffusionGemma model"; the mlx-bun dossier, section 2 DecoderLayer):
 *   a = rms(x)*pre_ff_norm, b = rms(x)*pre_ff_norm_2, routing of b's row as in
 *   dgmoe_route, h1 = MLP_dense(a), moe = sum_j w_j * MLP_{e_j}(b),
 *   h = rms(h1)*post_ff_norm_1 + rms(moe)*post_ff_norm_2,
 *   y = layer_scalar * (x + rms(h)*post_ff_norm).
 * y: [L, D] in y_dtype (F32, or BF16 = round-to-nearest-even
 * of the F32 result), 16-byte aligned.  If force_idx and force_w are both
 * non-NULL they replace the router's choice (tests inject a routing this way);
 * otherwise the router runs.  topk_idx_out / topk_w_out (each may be NULL)
 * receive the routing that was used.
 */
dgmoe_status dgmoe_block_forward(const dgmoe_dims *dims, const dgmoe_block_weights *w,
                                 const void *x, int32_t x_dtype, int64_t L,
                                 const int32_t *force_idx, const float *force_w,
                                 void *y, int32_t y_dtype,
                                 int32_t *topk_idx_out, float *topk_w_out,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * dgmoe_block_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The library allocates nothing in this
 * call either: the workspace is a static device array of
 * dgmoe_noalloc_max_bytes() bytes (32 MiB, enough for one 256-position canvas
 * at DiffusionGemma's shape, which needs 27.5 MB) that each GPU the library
 * runs on holds until the process ends.  A call whose dgmoe_workspace_size(dims,
 * L) exceeds it returns DGMOE_ERR_WORKSPACE and enqueues nothing.  Every call on
 * one GPU shares that GPU's array (the call stamp and error words included,
 * so dgmoe_check_workspace does not apply): calls that overlap on one GPU --
 * on different streams, or from different threads -- race and must be
 * serialised by the caller.  Everything else as dgmoe_block_forward.
 */
dgmoe_status dgmoe_block_forward_noalloc(const dgmoe_dims *dims, const dgmoe_block_weights *w,
                                         const void *x, int32_t x_dtype, int64_t L,
                                         const int32_t *force_idx, const float *force_w,
                                         void *y, int32_t y_dtype,
                                         int32_t *topk_idx_out, float *topk_w_out, void *stream);

/* Bytes of the static workspace of dgmoe_block_forward_noalloc. */
size_t dgmoe_noalloc_max_bytes(void);

/*
 * dgmoe_block_forward with the router, for per-kernel timing.  `events` holds
 * DGMOE_PROFILE_EVENTS hipEvent_t handles created by the caller; event i is
 * recorded on `stream` just before kernel i of the sequence
 *   0 norm + router + top-k + expert lists, 1 gate_up + GeGLU,
 *   2 down + scatter, 3 combine + post-norms (1 and 2: both launches of the
 *   phase when the dense MLP's format differs from the experts'),
 * and event 4 after the last one.  Everything else as dgmoe_block_forward.
 */
#define DGMOE_PROFILE_EVENTS 5
dgmoe_status dgmoe_block_forward_profiled(const dgmoe_dims *dims, const dgmoe_block_weights *w,
                                          const void *x, int32_t x_dtype, int64_t L,
                                          void *y, int32_t y_dtype, void *ws, size_t ws_bytes,
                                          void *stream, void **events, int32_t n_events);

/* Bytes of the code array of a [rows, cols] matrix in fmt (Q4G64, Q4G32 and
 * NVFP4: rows*cols/2, Q6G32: rows*cols*3/4, Q8G64: rows*cols); 0 if fmt is
 * not a packed format or cols % 64 != 0. */
size_t dgmoe_packed_bytes(int64_t rows, int64_t cols, int32_t fmt);

/*
 * Quantise a float32 [rows, cols] matrix (row-major) on the GPU into fmt
 * (affine, fp16 scale+bias per group of 64 inputs -- the mlx-bun dossier
 * section 1 quantisation -- or of 32 for Q4G32, the diffgemma contract's
 * section 8 expert format, and Q6G32 with 6-bit codes).  The quantiser, per group:
 *   scale = fp16((max - min) / (2^bits - 1)), bias = fp16(min)      (fp32 ops, RNE)
 *   q = clamp(rint((w - bias) / scale), 0, 2^bits - 1), q = 0 if scale == 0
 * with the subtraction and division in fp32.  w must be finite, |w| < 65504.
 * NVFP4, over the whole matrix (one tensor scale), every step in fp32:
 *   amax = max |w|, gs = amax / 2688;  per block of 16: t = bmax / (6 * gs)
 *   (0 if gs == 0), byte = E4M3 of t (round to nearest even, above 448 -> 448),
 *   es = e4m3(byte) * gs;  code = E2M1 of w / es (nearest, ties to the even
 *   code, |x| > 6 -> 6, the sign bit of w / es), code 0 where es == 0.
 * codes: dgmoe_packed_bytes(rows, cols, fmt) bytes; scale_bias: rows*cols/32
 * uint16 (rows*cols/16 for Q4G32 and Q6G32; rows*cols/16 + 64 bytes for
 * NVFP4); both 64-byte aligned; w 16-byte aligned.  cols % 64 == 0, and for
 * every format but Q8G64 rows % 64 == 0.  NVFP4 takes three launches on `stream` (clear
 * the trailer, amax, quantise).
 */
dgmoe_status dgmoe_pack(const float *w, int64_t rows, int64_t cols, int32_t fmt,
                        void *codes, uint16_t *scale_bias, void *stream);

/*
 * Dequantise a packed matrix on the GPU into out [rows, cols], row-major:
 *   out_dtype F32: the exact value float(scale)*q + float(bias) (one fma);
 *                  NVFP4: e2m1 * e4m3 * gs rounded once to fp32;
 *   out_dtype F16: that value rounded once to fp16 -- for Q4G64, Q4G32 and
 *                  Q6G32 exactly the operand the block's GEMM kernels feed to the
 *                  matrix cores; NVFP4: the fp32 value rounded to fp16.
 */
dgmoe_status dgmoe_unpack(const void *codes, const uint16_t *scale_bias, int64_t rows,
                          int64_t cols, int32_t fmt, int32_t out_dtype, void *out, void *stream);

/* ====================================================================== head
 * The tied embedding table at both ends of a denoising forward: the canvas
 * input with self-conditioning before the first decoder layer, and the tail
 * after the last one.  Sources: the diffgemma contract, Part II section 1
 * "Model constants" (vocab 262144, tied embeddings, final softcap 30),
 * section 2.1 (the SC-injection bullet), section 4 "Denoise step" items 1 and
 * 3, section 5 "Self-conditioning (SC)" (the exact chunked path), section 6
 * "Sampler" item 2 (row statistics of the logits divided by T);
 * "DiffusionGemma Explained", "Complete DiffusionGemma model" and "Logit
 * Softcapping"; the mlx-bun port dossier, section 3 "Self-conditioning".
 *
 *   canvas input  e_t  = E[id_t] * sqrt(D)
 *                 soft = softmax(sc_logits_t) @ E * sqrt(D)   (0 without a previous step)
 *                 s_t  = W_down (gelu_tanh(W_gate n) * (W_up n)),  n = rms(soft) * sc_pre_norm
 *                 out_t = rms(e_t + s_t)                       (no weight)
 *   tail          z_t  = (rms(x_t) * final_norm) @ E^T          [V]
 *                 y_t  = 30 tanh(z_t / 30) / T
 *                 entropy_t = -sum p ln p (nats), argmax_t (lowest index on
 *                 ties), row_max_t = max y, row_sum_t = sum exp(y - row_max)
 *                 with p = softmax(y_t); y_t is what the next step's
 *                 self-conditioning reads as sc_logits.
 * E is the [V, D] embedding table, Q4G64 (row = token, the layout above).
 * Precision: MFMA with fp16 operands (x_hat * final_norm, the dequantised
 * table, 2^14 exp(y - m) for the probabilities, n) and fp32 accumulation;
 * softmax statistics, entropy and the norms in fp32.
 */

/* hidden: a multiple of 64 in [64, 8192]; vocab: a multiple of 64 in
 * [64, 2^20]; sc_inter: a multiple of 64 in [64, 16384]; rms_eps finite,
 * >= 0.  L (positions per call) <= 2^20. */
typedef struct {
  int32_t hidden;     /* D                                          */
  int32_t vocab;      /* V                                          */
  int32_t sc_inter;   /* I_sc, the self-conditioning MLP's width     */
  float rms_eps;      /* 1e-6 for DiffusionGemma                    */
} dgmoe_head_dims;

/* Weights of the head.  embed is required by every head entry point; the
 * others only by the entry points that use them (final_norm: dgmoe_tail;
 * sc_gate_up, sc_down, sc_pre_norm: dgmoe_sc_input with sc_logits).  The
 * self-conditioning MLP has the dense MLP's shapes (gate rows first in
 * sc_gate_up).  Vectors 16-byte aligned, matrices 64-byte aligned. */
typedef struct {
  dgmoe_matrix embed;          /* [V, D] Q4G64                  */
  const float *final_norm;     /* [D]                           */
  dgmoe_matrix sc_gate_up;     /* [2 I_sc, D] Q4G64              */
  dgmoe_matrix sc_down;        /* [D, I_sc] Q4G64                */
  const float *sc_pre_norm;    /* [D]                           */
} dgmoe_head_weights;

/* Bytes of device workspace any head entry point needs on L positions (0 if
 * the dims are invalid); the pointer must be 256-byte aligned.  It holds the
 * probabilities of a soft embedding (2 L V bytes) and its partial sums, so it
 * grows with L * V (about 230 MB at L = 256, V = 262144, D = 2816). */
size_t dgmoe_head_workspace_size(const dgmoe_head_dims *h, int64_t L);

/*
 * Forward tail.  x: [L, D] (x_dtype F32 or BF16, 16-byte aligned), the last
 * block's output.  temperature > 0, finite.  Outputs (device, 4-byte aligned):
 *   entropy [L] float, argmax [L] int32 (required);
 *   row_max, row_sum [L] float (each may be NULL);
 *   logits [L, V] float y (16-byte aligned, may be NULL: the full logits are
 *   then never written, only the statistics above).
 * Flags (dgmoe_head_check_workspace): DGMOE_FLAG_FP16_RANGE if an operand
 * x_hat * final_norm does not fit fp16.
 */
dgmoe_status dgmoe_tail(const dgmoe_head_dims *h, const dgmoe_head_weights *w,
                        const void *x, int32_t x_dtype, int64_t L, float temperature,
                        float *entropy, int32_t *argmax, float *row_max, float *row_sum,
                        float *logits, void *ws, size_t ws_bytes, void *stream);

/*
 * The soft embedding alone: soft [L, D] float (16-byte aligned) =
 * softmax(sc_logits_t) @ E * sqrt(D), sc_logits [L, V] float (16-byte
 * aligned, finite), the previous step's logits already divided by T.  The sum
 * over the vocabulary is exact (every entry contributes; no sparse cut).
 */
dgmoe_status dgmoe_soft_embed(const dgmoe_head_dims *h, const dgmoe_head_weights *w,
                              const float *sc_logits, int64_t L, float *soft, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * The canvas input of a denoising step: out [L, D] float (16-byte aligned) as
 * above, from canvas_ids [L] int32 (4-byte aligned) and sc_logits [L, V]
 * (as for dgmoe_soft_embed) or NULL for a step without a previous prediction
 * (then out_t = rms(e_t): the zero signal maps to zero, and the MLP is not
 * run).  Flags: DGMOE_FLAG_INDEX for an id outside [0, V);
 * DGMOE_FLAG_FP16_RANGE if n does not fit fp16.
 */
dgmoe_status dgmoe_sc_input(const dgmoe_head_dims *h, const dgmoe_head_weights *w,
                            const int32_t *canvas_ids, const float *sc_logits, int64_t L,
                            float *out, void *ws, size_t ws_bytes, void *stream);

/* Host, synchronous: the flags of the last head call on ws (sized for h and
 * L); as dgmoe_check_workspace. */
dgmoe_status dgmoe_head_check_workspace(const dgmoe_head_dims *h, int64_t L, const void *ws,
                                        uint32_t *flags, void *stream);

/* ------------------------------------------------------------------------
 * Denoise attention of one decoder layer (the step before the FFN block).
 *
 * Defined by "diffgemma -- architecture & implemented contract", Part II
 * section 2 "Two attention phases" (the Denoise bullet: the canvas attends
 * bidirectionally to itself and to the KV cache; on sliding layers only to
 * the last window committed positions) and section 2.1 (Norms: QK-norm is a
 * per-head RMSNorm with learned weights, V a weightless one; RoPE: split
 * half, theta 1e4 on sliding layers, 1e6 with a partial rotation whose
 * exponent uses the whole head_dim on full layers; no 1/sqrt(d) scale; full
 * layers have no v_proj and take V from the raw K projection), with
 * "DiffusionGemma Explained" (the attention section: rotate() and
 * AttentionBlock.forward) and the mlx-bun port dossier section 2
 * (Attention.__call__, _make_decoder_masks).  For canvas rows t = 0..L-1 at
 * positions kv_len + t and each query head h (KV head n = h / (H / H_kv)):
 *   q = rope(rms(q_raw[t, h]) * q_norm),  k = rope(rms(k_raw[t, n]) * k_norm),
 *   v = rms(v_raw[t, n])   (v_raw = NULL: v = rms(k_raw[t, n]), full layers)
 *   keys: committed positions j in [s0, kv_len) of the cache, s0 =
 *   max(0, kv_len - window) (window 0: s0 = 0), then all L canvas rows;
 *   out[t, h*hd .. +hd) = softmax_j(q . K_j) V_j   (unit scale)
 * rope(x, p): for d < rope_pairs, (x_d, x_{d+rope_stride}) turned by the angle
 * p * rope_theta^(-2 d / rope_den); the other dimensions unchanged.  The
 * pages give two partner strides for the partial rotation of full layers
 * (rotary_dim/2 in the contract; head_dim/2 in the blog's rotate()); either
 * is a value of rope_stride.
 *
 * Precision: the norms, rotation and softmax in fp32 (angles in fp64);
 * q, k, v and the softmax probabilities rounded to fp16 as MFMA operands,
 * fp32 accumulation.
 */
typedef struct dgmoe_attn_dims {
  int32_t n_heads;     /* query heads H (16 in the model) */
  int32_t n_kv_heads;  /* KV heads H_kv (8 sliding, 2 full); H a multiple of H_kv */
  int32_t head_dim;    /* 64, 128, 256 (sliding layers) or 512 (full layers) */
  int32_t window;      /* committed positions a canvas row sees: 1023 on sliding layers, 0 = all */
  int32_t rope_pairs;  /* rotated pairs d = 0 .. rope_pairs-1 (head_dim/2 sliding, head_dim/8 full) */
  int32_t rope_stride; /* partner of d is d + rope_stride; rope_pairs <= rope_stride,
                          rope_pairs + rope_stride <= head_dim */
  float rope_theta;    /* 1e4 sliding, 1e6 full */
  float rope_den;      /* exponent denominator: head_dim on both layer types */
  float rms_eps;       /* 1e-6 */
} dgmoe_attn_dims;

/* Bytes of workspace dgmoe_attn_denoise needs for L canvas rows and kv_len
 * committed positions (0 if the dims are invalid). */
size_t dgmoe_attn_workspace_size(const dgmoe_attn_dims *a, int64_t L, int64_t kv_len);

/* Device, asynchronous on `stream`.
 *   q      [L, H*head_dim]     raw query projection, F32 or BF16 (in_dtype)
 *   k      [L, H_kv*head_dim]  raw key projection, same dtype
 *   v      [L, H_kv*head_dim]  raw value projection, or NULL (full layers)
 *   q_norm, k_norm [head_dim]  fp32 QK-norm weights
 *   k_cache, v_cache [H_kv, cache_rows, head_dim] fp16 (bits): the committed
 *          keys (after k_norm and RoPE at their positions) and values (after
 *          the weightless norm), position j at row j; rows kv_len .. are not read
 *   out    [L, H*head_dim]     F32 or BF16 (out_dtype; BF16 = RNE of the fp32 result)
 * Pointers: q, k, v 4-byte aligned, caches and out 16-byte aligned, ws
 * 256-byte aligned.  Caller owns every buffer; the workspace holds the
 * prepared fp16 q / k / v and the per-key-range partial results of the call.
 * Errors: DGMOE_ERR_NULL_ARG, _BAD_DIMS (dims, L > 2^20, (H / H_kv) * L >
 * 64 * 65535, kv_len outside [0, cache_rows]), _BAD_DTYPE, _MISALIGNED,
 * _WORKSPACE, _HIP.  L = 0 is a
 * no-op.  A QK-norm weight larger than 65504 / sqrt(head_dim) can overflow
 * the fp16 operands; this is not checked. */
dgmoe_status dgmoe_attn_denoise(const dgmoe_attn_dims *a, const void *q, const void *k,
                                const void *v, int32_t in_dtype, int64_t L, const float *q_norm,
                                const float *k_norm, const uint16_t *k_cache,
                                const uint16_t *v_cache, int64_t cache_rows, int64_t kv_len,
                                void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                                void *stream);

const char *dgmoe_status_str(dgmoe_status s);
int dgmoe_abi_version(void);

/* Name of the last HIP error a call on this thread turned into DGMOE_ERR_HIP
 * ("none" if there was none).  Diagnostics only. */
const char *dgmoe_last_hip_error(void);

/* Diagnostics only (tests of the failure path): with spin_limit > 0, the
 * router launches of this thread's later calls never publish their stamp and
 * poll for it at most spin_limit times, so every router workgroup gives up and
 * the call ends with DGMOE_FLAG_SYNC_TIMEOUT (every kernel still exits
 * normally).  0 restores normal operation. */
void dgmoe_debug_force_stamp_timeout(int32_t spin_limit);

/* Tuning and tests (Q4G64 weights): when a batch has fewer than 32 pairs per
 * expert on average, the expert GEMMs use 32-row tiles, except for experts
 * with at least `rows` pairs, which take 64-row tiles in the same launch
 * (each 64-row tile reads its weights once for twice the rows).  Applies to
 * this thread's later calls.  rows = 0: no expert does (the default);
 * rows < 0: the default.  Returns the previous value.  Results agree to the
 * same tolerance whatever the value (the tiles differ only in how the sums
 * are blocked). */
int32_t dgmoe_debug_set_tall_min(int32_t rows);

#ifdef __cplusplus
}
#endif
#endif /* DGMOE_H */
