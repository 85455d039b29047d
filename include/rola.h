/*
 * rola.h -- C ABI of librola: RoLA attention (rotary-positioned low-rank
 * linear attention plus block-sparse softmax attention) on AMD MI355X (gfx950).
 *
 * The operation (pages: "SparkDiffusion: 265x Faster Video Generation on
 * Consumer GPUs via Sparse Attention & Distillation", section "RoLA:
 * Preserving Global Context at Extreme Sparsity"; "SparkDiffusion / SparkWan"
 * news article, section "What's New"): a block-sparse softmax branch keeps the
 * highest-energy query-key blocks, and a low-rank linear-attention branch with
 * rotary positions recovers the global context the sparse branch discards.
 * The keep ratio `topk` (README "AlibabaResearch/SparkDiffusion", inference
 * section: 0.1, 0.05, 0.03 mean 90%, 95%, 97% sparsity) fixes how many key
 * blocks each query block keeps.  fp8 and bf16 are the two precisions the
 * README names (quick-start section).
 *
 * Definitions used by every call (B batch, H heads, D head_dim, N = T*Hg*W
 * tokens of a raster (t,h,w) latent grid, 64-token blocks, nb = ceil(N/64),
 * n_pad = 64*nb, r the low-rank width):
 *  - block energy: Qp[c], Kp[c] = mean of block c's valid tokens (fp32, fixed
 *    binary-tree summation order, times fl32(1/count));
 *  - score s[i][j] = sequential fp32 fma chain over d of Qp[i][d]*Kp[j][d];
 *  - kept blocks: kb = max(1, floor(topk*nb)) (or kb_override) largest scores
 *    per query block i, ties to the lower j, listed in ascending j;
 *  - sparse branch: softmax(q k^T * scale) v over the valid tokens of the kept
 *    key blocks; scale defaults to D^-1/2;
 *  - low-rank branch: a = phi(Wq^T R(q)), b = phi(Wk^T R(k)), phi = elu + 1,
 *    R the 3-D rotary embedding (dims split t/h/w, interleaved pairs, base
 *    theta); S = sum_{n<N} b_n v_n^T, z = sum_{n<N} b_n per (batch, head);
 *    O_lr = (a^T S) / (a^T z).  With config.lowrank_scope =
 *    ROLA_LR_COMPLEMENT the sums of query block i run only over the valid
 *    tokens of the key blocks i does NOT keep (the article's "context the
 *    sparse branch drops" read literally), and O_lr = 0 when i keeps all;
 *  - output O = O_sparse + g * O_lr for rows < N; rows N..n_pad-1 are written 0.
 *    g is the optional learned output gate (README "AlibabaResearch/
 *    SparkDiffusion", sparse-finetune section, names the trainable gate_proj
 *    and gate_bias without their form), read here as g = sigmoid(q . w + b)
 *    per token and head from the unrotated query, fp32 sum of products;
 *    without a gate g = 1.
 *
 * Memory: every pointer is device memory owned by the caller.  Q, K, V and O
 * share one layout: element (b, h, n, d) at b*stride_b + h*stride_h +
 * n*stride_n + d (elements; d contiguous), rows 0..n_pad-1 addressable;
 * input rows >= N are ignored (may hold anything).  Q/K/V are bf16.  O is
 * bf16 or fp32 (config.out_dtype).  Wq, Wk are fp32 [D][r], shared by all
 * heads.  The gate, where given, is fp32 [D+1] (w_0 .. w_{D-1}, then b),
 * shared by all heads, 16-byte aligned.  The workspace (size from rola_plan)
 * is scratch owned by the caller; the library keeps no state in it between
 * calls.
 *
 * Behaviour: every call validates all arguments before launching anything;
 * on error nothing is launched and a status != ROLA_OK is returned.  Launches
 * are asynchronous on `stream` (a hipStream_t; NULL = default stream).  The
 * library never allocates, frees or synchronises device memory.  Calls are
 * thread-safe when they use distinct workspaces.
 */
#ifndef ROLA_H_
#define ROLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROLA_ABI_VERSION 8
#define ROLA_BLOCK 64
#define ROLA_MAX_BLOCKS 4096 /* nb limit: N <= 262144 tokens */

typedef enum rola_status {
  ROLA_OK = 0,
  ROLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, topk outside (0,1], ... */
  ROLA_ERR_UNSUPPORTED = 2, /* D not in {64,128}, r not in {16,32}, nb too large,
                               stride_n above 2^24 elements */
  ROLA_ERR_ALIGNMENT = 3,   /* pointer or row stride not 16-byte aligned */
  ROLA_ERR_WORKSPACE = 4,   /* workspace null or smaller than rola_plan's size */
  ROLA_ERR_DEVICE = 5       /* a HIP launch reported an error */
} rola_status;

enum { ROLA_PREC_BF16 = 0, ROLA_PREC_FP8 = 1 };
enum { ROLA_OUT_BF16 = 0, ROLA_OUT_F32 = 1 };
enum { ROLA_LR_GLOBAL = 0, ROLA_LR_COMPLEMENT = 1 };

typedef struct rola_problem {
  int32_t batch, heads, head_dim;
  int32_t grid_t, grid_h, grid_w;    /* latent token grid; N = grid_t*grid_h*grid_w */
  int64_t stride_b, stride_h, stride_n; /* in elements, shared by Q, K, V, O */
} rola_problem;

typedef struct rola_config {
  float topk;          /* keep ratio in (0, 1] */
  int32_t kb_override; /* > 0: keep exactly this many key blocks (<= nb) */
  int32_t rank;        /* low-rank width r: 16 or 32 */
  int32_t rope_split[3]; /* rotary dims for t, h, w (even, summing to D); all 0: D/4, rest halved */
  float rope_theta;    /* <= 0: 10000 */
  float softmax_scale; /* <= 0: 1/sqrt(D) */
  int32_t precision;   /* ROLA_PREC_BF16 or ROLA_PREC_FP8 (e4m3, per-block absmax scales) */
  int32_t out_dtype;   /* ROLA_OUT_BF16 or ROLA_OUT_F32 */
  int32_t lowrank_scope; /* ROLA_LR_GLOBAL (one state per head) or ROLA_LR_COMPLEMENT */
} rola_config;

typedef struct rola_plan_info {
  int64_t n_tokens; /* N */
  int32_t nb;       /* 64-token blocks */
  int32_t kb;       /* key blocks kept per query block */
  int64_t n_pad;    /* 64*nb rows addressed in every token tensor */
  int64_t workspace_bytes; /* for rola_select_blocks, _sparse_attn, _lowrank_attn, _forward */
  int64_t workspace_bytes_backward; /* for rola_backward (larger) */
} rola_plan_info;

/* ABI version (ROLA_ABI_VERSION) and a static message for a status. */
int32_t rola_abi_version(void);
const char *rola_status_str(int32_t status);

/* Host-only: validate the problem and config and size the workspace.  No device access. */
int32_t rola_plan(const rola_problem *prob, const rola_config *cfg, rola_plan_info *out);

/*
 * Block selection (pages: news article, section "What's New": only a small
 * share of the query-key blocks survives; README "AlibabaResearch/
 * SparkDiffusion", inference section: topk is the keep ratio).  Pools Q and K per
 * block, scores every block pair and writes the kept key blocks of every
 * query block to block_idx (int32 [B][H][nb][kb], ascending).  pooled_scores,
 * if not NULL, receives the fp32 score matrix [B][H][nb][nb].
 */
int32_t rola_select_blocks(const rola_problem *prob, const rola_config *cfg, const void *q,
                           const void *k, int32_t *block_idx, float *pooled_scores,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sparse branch only (pages: section "RoLA: Preserving Global Context at
 * Extreme Sparsity": a block-sparse softmax branch keeps the high-energy
 * query-key interactions).  O = O_sparse (accumulate = 0) or
 * O += O_sparse (accumulate = 1), with block_idx as written by
 * rola_select_blocks (ids must be ascending and < nb).
 */
int32_t rola_sparse_attn(const rola_problem *prob, const rola_config *cfg, const void *q,
                         const void *k, const void *v, const int32_t *block_idx, void *out,
                         int32_t accumulate, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Low-rank branch only (pages: section "RoLA: Preserving Global Context at
 * Extreme Sparsity", which names the RoLA paper, rotary-positioned low-rank
 * linear attention: a linear branch with rotary positions; README
 * "AlibabaResearch/SparkDiffusion", sparse-finetune section: the added
 * query and key projections).
 * O = g * O_lr (accumulate = 0) or O += g * O_lr (accumulate = 1); gate NULL
 * means g = 1.  In the complement scope this call also selects the blocks
 * (as rola_select_blocks does) to know what each query block keeps.
 */
int32_t rola_lowrank_attn(const rola_problem *prob, const rola_config *cfg, const void *q,
                          const void *k, const void *v, const float *wq, const float *wk,
                          const float *gate, void *out, int32_t accumulate, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Fused RoLA forward: O = O_sparse + g * O_lr (gate NULL: g = 1).
 * block_idx_out, if not NULL, receives the block map (int32 [B][H][nb][kb]).
 */
int32_t rola_forward(const rola_problem *prob, const rola_config *cfg, const void *q,
                     const void *k, const void *v, const float *wq, const float *wk,
                     const float *gate, int32_t *block_idx_out, void *out, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * rola_forward with pre-quantised fp8 operands for the sparse branch (the
 * fp8 pipeline of the project page, section "FP8 Quantization & Fused
 * Kernels", with the quantisation done by the caller, e.g. fused into the
 * kernel that produces Q, K and V).  cfg->precision must be ROLA_PREC_FP8.
 * As in the fp8 mode of rola_forward, block selection and the low-rank
 * branch read the bf16 q, k, v, and the sparse branch reads e4m3 codes; here
 * the codes and scales are the caller's and the library quantises nothing:
 *   q8, k8, v8: e4m3 codes [B, H, n_pad, D] with the strides of prob (in
 *     elements, one byte each), 16-byte aligned; rows at or past N are
 *     ignored;
 *   qs, ks, vs: fp32 [B, H, nb] (contiguous), the value of a code being
 *     e4m3(code) * scale of its (batch, head, 64-token block); scales must be
 *     positive and finite.
 * Codes and scales from the library's own rule (scale = fl32(absmax/448),
 * code = RNE-saturating e4m3 of fl32(x * fl32(448/absmax))) give exactly the
 * output of rola_forward in fp8 mode.  Workspace as for rola_forward;
 * errors as for rola_forward, and ROLA_ERR_INVALID_ARG for a bf16 precision.
 */
int32_t rola_forward_e4m3(const rola_problem *prob, const rola_config *cfg, const void *q,
                          const void *k, const void *v, const uint8_t *q8, const uint8_t *k8,
                          const uint8_t *v8, const float *qs, const float *ks, const float *vs,
                          const float *wq, const float *wk, const float *gate, int32_t *block_idx_out,
                          void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * rola_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  The library keeps one scratch array of
 * ROLA_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the first call on
 * that GPU until the process ends; the call allocates and frees nothing.
 * Arguments and behaviour are those of rola_forward; problems whose
 * workspace (rola_plan's workspace_bytes) exceeds the scratch return
 * ROLA_ERR_WORKSPACE and launch nothing.  The scratch belongs to the GPU of
 * `stream`; all calls on one GPU share it, so calls that overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller.
 */
#define ROLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int32_t rola_forward_noalloc(const rola_problem *prob, const rola_config *cfg, const void *q,
                             const void *k, const void *v, const float *wq, const float *wk,
                             const float *gate, int32_t *block_idx_out, void *out, void *stream);

/*
 * Backward of rola_forward (training; the README "AlibabaResearch/
 * SparkDiffusion" fine-tunes and distils this module, sparse-finetune and
 * distillation sections).  Given dout = dL/dO (bf16 or fp32 as
 * config.out_dtype, the layout of O; fp32 values are rounded to bf16, to
 * nearest even, as they enter the products) and the block map the forward used
 * (block_idx, as rola_forward or rola_select_blocks wrote it: ascending ids
 * < nb), writes the gradients of L through O = O_sparse + g * O_lr:
 *   dq, dk, dv: bf16, the layout of Q (rows >= N written as 0);
 *   dwq, dwk:   fp32 [D][rank] (overwritten), the gradients of Wq and Wk;
 *   dgate:      fp32 [D+1] (overwritten), the gate's gradient -- required
 *               exactly when gate is given.
 * The block map is a constant of the backward (the top-k selection has no
 * gradient).  Internally the state S, z, the sparse output and each row's
 * log-sum-exp are recomputed.  Both low-rank scopes are supported: with
 * ROLA_LR_COMPLEMENT the per-query-block states (the sums over the unkept
 * blocks, as the forward forms them) are recomputed too, and each key
 * block's state receives the gradient of the query blocks that do not keep
 * it.  Supported precision: ROLA_PREC_BF16 (ROLA_ERR_UNSUPPORTED for fp8).
 * The workspace must hold plan.workspace_bytes_backward bytes.
 */
int32_t rola_backward(const rola_problem *prob, const rola_config *cfg, const void *q, const void *k,
                      const void *v, const float *wq, const float *wk, const float *gate,
                      const int32_t *block_idx, const void *dout, void *dq, void *dk, void *dv,
                      float *dwq, float *dwk, float *dgate, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * Training pair (same passages as rola_backward): a forward that keeps what
 * the backward would otherwise recompute, and the backward that takes it.
 *
 * rola_forward_train: rola_forward (bf16 precision only; ROLA_ERR_UNSUPPORTED
 * for fp8), and also writes, from the same attention launch,
 *   os:  fp32, the sparse branch's output O_s before the low-rank term is
 *        added, with the element strides of prob (rows >= N written as 0),
 *        16-byte aligned, caller-owned;
 *   lse: fp32 [B*H][n_pad], each valid row's base-2 log-sum-exp of its scaled
 *        logits (s * scale * log2 e), 4-byte aligned, caller-owned; rows >= N
 *        are not written.
 * With bf16 output both come from the fp16-weight form of the forward (its
 * rounding, not the backward's fp32 recompute); with fp32 output they equal
 * what rola_backward recomputes, bit for bit.  Workspace as for rola_forward.
 *
 * rola_backward_saved: rola_backward with os and lse from rola_forward_train
 * on the same inputs, block map and config (both required: NULL is
 * ROLA_ERR_INVALID_ARG); it skips the recompute of the sparse branch and
 * forms only the group schedule of the map.  Workspace as for rola_backward.
 */
int32_t rola_forward_train(const rola_problem *prob, const rola_config *cfg, const void *q,
                           const void *k, const void *v, const float *wq, const float *wk,
                           const float *gate, int32_t *block_idx_out, void *out, float *os, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);
int32_t rola_backward_saved(const rola_problem *prob, const rola_config *cfg, const void *q,
                            const void *k, const void *v, const float *wq, const float *wk,
                            const float *gate, const int32_t *block_idx, const void *dout,
                            const float *os, const float *lse, void *dq, void *dk, void *dv, float *dwq,
                            float *dwk, float *dgate, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Optional kernel timing for measurement.  While enabled, each call records a
 * hipEvent pair around every kernel it launches (on the call's stream).
 * Enabling creates a pool of events on the current device first, so that the
 * timed calls themselves create none while the pool lasts.
 * rola_timing_read synchronises those events and returns, per kernel name,
 * the launch count and total milliseconds (at most `max` entries; returns
 * the number written, or -1 on error).  This is the library's only
 * process-wide state: off by default, and while off a call only reads its
 * flag.  Enabling, reading and the recording are serialised by a lock; the
 * measurement itself is meant for one timing thread (events of concurrent
 * calls on several streams are recorded but interleave in the totals).
 */
typedef struct rola_kernel_time {
  char name[48];
  int32_t launches;
  double total_ms;
} rola_kernel_time;

int32_t rola_timing_enable(int32_t on);
int32_t rola_timing_read(rola_kernel_time *out, int32_t max);

/*
 * w8a8 linear layers: the projections either side of attention in the fp8
 * pipeline (README "AlibabaResearch/SparkDiffusion", highlights: optional
 * weight-activation quantisation; project page, section "FP8 Quantization &
 * Fused Kernels").  Activations are quantised per token (row), weights per
 * output channel (row of W [N, K]), both with the e4m3 absmax rule of the
 * fp8 attention inputs.
 *
 * rola_quant_rows: x bf16 [rows, cols] with row stride ld_x (elements) ->
 * codes e4m3 [rows, cols] with row stride ld_codes (bytes), scale fp32
 * [rows] = fl32(absmax/448) (1 for an all-zero row); code = RNE-saturating
 * e4m3 of fl32(x * fl32(448/absmax)); x must be finite (a row holding an
 * infinity or NaN gets unspecified codes).  Requires cols > 0 and a multiple of
 * 8, ld_x >= cols and ld_codes >= cols both multiples of 8, x and codes
 * 16-byte aligned, scale 4-byte aligned (ROLA_ERR_INVALID_ARG /
 * ROLA_ERR_ALIGNMENT; rows == 0 launches nothing).  No workspace; all
 * buffers are the caller's.
 *
 * rola_gemm_w8a8: out[m, n] = sx[m] * sw[n] * sum_k value(x[m, k]) *
 * value(w[n, k]) + bias[n] for m < M, n < N, accumulated in fp32 on the
 * matrix cores and stored as bf16 (RNE) or fp32 (out_dtype ROLA_OUT_BF16 /
 * ROLA_OUT_F32) with row stride ld_out (elements), so the output may be a
 * column slice of a wider buffer (for example the Q, K or V part of a
 * token-major [T, 3*H*D] tensor).  x e4m3 [M, K] (row stride ld_x bytes),
 * w e4m3 [N, K] (row stride ld_w), sx fp32 [M], sw fp32 [N], bias fp32 [N]
 * or NULL.  Requires M >= 0 (0 launches nothing), N >= 4 and a multiple of 4, K >= 64 and a
 * multiple of 64, ld_x, ld_w in [K, 2^24) and multiples of 16, ld_out >= N
 * and a multiple of 4; x, w, out, sw and bias 16-byte aligned, sx 4-byte
 * aligned.  Other columns of out are not touched.  No workspace.
 */
int32_t rola_quant_rows(const void *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                        int64_t ld_codes, float *scale, void *stream);
int32_t rola_gemm_w8a8(const uint8_t *x, int64_t ld_x, const float *sx, const uint8_t *w,
                       int64_t ld_w, const float *sw, const float *bias, int64_t M, int32_t N,
                       int32_t K, void *out, int64_t ld_out, int32_t out_dtype, void *stream);

/*
 * ---- Diagnostics (not part of RoLA) ----
 * Measurement helper: launches, on `stream`, a kernel
 * that keeps every SIMD's matrix core busy with independent MFMA chains --
 * precision ROLA_PREC_BF16: v_mfma_f32_32x32x16_bf16, ROLA_PREC_FP8:
 * v_mfma_f32_32x32x64_f8f6f4 (e4m3) -- for `iters` steps per chain, and
 * writes the number of floating-point operations it performs to *flop.
 * The caller times it with events on the same stream to obtain the MFMA
 * rate the device sustains, next to its datasheet peak.  The only device
 * memory written is `sink` (device memory of at least 8192 bytes, owned by
 * the caller): one float per workgroup in sink[0..1023], then the ticks of
 * the core clock (s_memtime) and of the constant reference clock
 * (s_memrealtime) that the first wave spent, as floats in sink[1024] and
 * sink[1025]; their ratio times the reference frequency is the shader clock
 * during the run.  Returns ROLA_ERR_INVALID_ARG
 * for a bad precision, iters < 1 or a NULL pointer; launches nothing then.
 */
int32_t rola_mfma_probe(int32_t precision, int32_t iters, double *flop, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROLA_H_ */
