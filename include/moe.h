/*
 * moe.h - C ABI of the MI355X (gfx950) MoE FFN layer forward pass.
 *
 * One call computes, for T tokens, the forward pass of one Mixture-of-Experts
 * FFN layer with block-scaled low-precision expert weights:
 *
 *   1. router logits  l[t,e] = sum_i W_r[e,i] x[t,i] (+ bias[t,e]), in f32
 *      (dragon.c page, "Precision": the router runs in f32);
 *   2. softmax over all E experts and top-k; equal logits go to the lower
 *      index; the k ids of a token are listed in ascending expert id;
 *      weights w = p[ids], divided by their sum when renorm is set;
 *   3. a counting-sort permute that groups the token-slots s = t*k + j by
 *      expert, stable in s (Trochilus README, "Acknowledgements": (token,
 *      expert) pairs sorted by a counting sort);
 *   4. per slot, a SwiGLU expert: g = W_gate x, u = W_up x,
 *      h = bf16(silu(g) * u), y = W_down h, with the weights decoded exactly
 *      from e4m3 codes with 128x128 f32 block scales (dragon.c page,
 *      "Precision" and section 8 Round 3) or from e2m1 codes with one UE8M0
 *      power-of-two scale per 32 inputs (dev.to page, DeepSeek-V4.1-Flash
 *      post, "Bytes per token decide everything");
 *   5. out[t] = sum_j w[t,j] y[t*k+j], j ascending, in f32 (WARP BACKENDS.md,
 *      "Coherent memory": one partial per selected expert, reduced in router
 *      order, is what makes the result reproducible bit for bit).
 *
 * Memory: every pointer passed to moe_forward is HIP device memory owned by
 * the caller.  The library allocates no device memory: all scratch lives in
 * the caller's workspace.  A plan holds host metadata only; once its options
 * are set (moe_plan_set) it is only read by moe_forward, so forwards on
 * different streams with different workspaces may overlap.
 *
 * Errors: every check runs on the host before the first launch, so a call
 * that returns an error has written nothing.  moe_forward is asynchronous on
 * `stream` and never synchronises the host; a fault inside a kernel surfaces
 * at the caller's next synchronisation.  No exception crosses this ABI and
 * the library never aborts.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  MOE_ERR_BAD_SHAPE = 2,    /* a size is out of range (T < 0, T > max_tokens, k > E, ...) */
  MOE_ERR_UNSUPPORTED = 3,  /* dims not divisible by the format's block, E or k too large */
  MOE_ERR_ALIGNMENT = 4,    /* a pointer or stride breaks the alignment stated below */
  MOE_ERR_WORKSPACE = 5,    /* workspace_bytes < moe_workspace_size(plan, T) */
  MOE_ERR_HIP = 6,          /* a HIP call failed; moe_plan_info() names it */
  MOE_ERR_DEVICE = 7        /* no HIP device, or the current device is not gfx950 */
} moe_status;

/* Expert weight formats. */
typedef enum {
  /* OCP E4M3FN codes (1 byte each), one f32 scale per 128x128 block.
   * Requires d_model % 128 == 0 and d_ff % 128 == 0. */
  MOE_W_E4M3_B128 = 0,
  /* OCP E2M1 codes, two per byte, element 2i in the low nibble; one UE8M0
   * byte (scale 2^(b-127)) per 32 contiguous inputs of a row.
   * Requires d_model % 32 == 0 and d_ff % 32 == 0. */
  MOE_W_E2M1_UE8M0_G32 = 1,
  /* NVFP4: OCP E2M1 codes packed as above; one OCP E4M3FN scale byte per 16
   * contiguous inputs of a row (the value is code times scale; no second,
   * per-tensor scale).  dev.to post "Running a 133 GB MoE model on an 8 GB
   * GPU at 11 tokens/s", "The engine" item 4: NVFP4 expert weights.
   * Requires d_model % 32 == 0 and d_ff % 32 == 0. */
  MOE_W_E2M1_E4M3_G16 = 2
} moe_wfmt;

/* Which variant of the one GPU path runs the expert stage. */
typedef enum {
  MOE_PATH_AUTO = 0,     /* decode below a per-plan token threshold, grouped above */
  MOE_PATH_DECODE = 1,   /* HBM-streaming matvec per selected expert */
  MOE_PATH_GROUPED = 2   /* grouped MFMA GEMM over expert tiles */
} moe_path;

/* Precision of the expert inputs.  The dev.to DeepSeek-V4.1-Flash post
 * ("Three bugs on RTX 50xx that never raise an error", item 2) runs its
 * activations through an fp8 quantiser with UE8M0 scales; WARP BACKENDS.md
 * measures what quantised activations cost in accuracy (about 1e-2 relative
 * on logits), so the default keeps them in bf16. */
typedef enum {
  /* bf16 activations, weights decoded exactly to bf16 (the default) */
  MOE_ACT_BF16 = 0,
  /* the token rows x (before gate/up) and h (before down) quantised per
   * 128-input group of a row: scale = the smallest power of two 2^E with
   * max|x| <= 448 * 2^E (UE8M0 byte E + 127; 127 for an all-zero group),
   * codes = e4m3 nearest x / 2^E (ties to even, the sign kept); a row whose
   * length is not a multiple of 128 ends in a shorter group.  The GEMMs run
   * on gfx950's block-scaled fp8/fp4 MFMA with f32 accumulation on the
   * grouped path; on the decode path the quantised values (code * 2^E, exact
   * in bf16) go through the decode kernels.  Weights e4m3 or e2m1 (not
   * NVFP4, whose e4m3 group scales are not powers of two); e2m1 needs
   * d_model % 64 == 0 and d_ff % 64 == 0 and 2-byte aligned scales. */
  MOE_ACT_E4M3_G128 = 1
} moe_act_fmt;

typedef struct {
  int32_t d_model;     /* hidden size d */
  int32_t d_ff;        /* expert FFN width f */
  int32_t n_experts;   /* E, 1..1024 */
  int32_t top_k;       /* k, 1..min(E, 16) */
  int32_t max_tokens;  /* largest T a forward may be called with, >= 1 */
  int32_t wfmt;        /* moe_wfmt */
  int32_t renorm;      /* 1: divide the k weights by their sum; 0: keep softmax probabilities */
  int32_t path;        /* moe_path */
  int32_t act_fmt;     /* moe_act_fmt */
  int32_t shared_expert; /* 1: the layer also has a shared (always-on) expert of the routed
                          * experts' shape and format, run on every token with weight 1
                          * (forwards through moe_forward_block); 0: none.  Not with
                          * n_experts = top_k = 1. */
} moe_desc;

typedef struct moe_plan_s* moe_plan_t;

/* One expert matrix family [E][N][K] (gate and up: N = d_ff, K = d_model;
 * down: N = d_model, K = d_ff).  Rows are K-contiguous.
 *   e4m3: q is uint8 [E][N][K]; scale is f32 [E][N/128][K/128].
 *   e2m1: q is uint8 [E][N][K/2]; scale is uint8 [E][N][K/32].
 *   nvfp4: q is uint8 [E][N][K/2]; scale is uint8 (e4m3 codes) [E][N][K/16].
 * q_expert_stride / s_expert_stride: bytes from expert e to expert e+1, so
 * both one buffer per matrix and one block per expert can be described.
 * Alignment: q and q_expert_stride 16 bytes; e4m3 scale and s_expert_stride
 * 4 bytes; nvfp4 scale and s_expert_stride 2 bytes (a 32-input step reads
 * its two group scales as one 16-bit word); e2m1 scales 1 byte. */
typedef struct {
  const void* q;
  const void* scale;
  int64_t q_expert_stride;
  int64_t s_expert_stride;
} moe_mat;

/* Validate `desc`, check the current HIP device and choose kernel variants.
 * On success *out holds a plan (host memory only).  Shape errors are
 * reported before the device is queried. */
moe_status moe_plan(const moe_desc* desc, moe_plan_t* out);

/* Kernel choices a plan makes from its shape, and the values that override
 * them.  A fresh plan needs none of this; the overrides exist so that every
 * variant a plan can run is reachable by the parity tests (and by tuning
 * sweeps).  Each variant computes the same layer. */
typedef enum {
  /* decode expert stage: 1 = 16-row MFMA tiles (from MOE_OPT_DEC_MFMA_MIN_T
   * tokens, the default), 0 = the wavefront matvec at every T */
  MOE_OPT_DEC_KERNEL = 0,
  /* fewest tokens for the MFMA decode tiles (default 2: one token takes the
   * matvec); >= 1 */
  MOE_OPT_DEC_MFMA_MIN_T = 1,
  /* grouped-GEMM tile shape, 10 * R + C: R wavefront rows (1 or 2) of C
   * 32-token chunks each, so 32 R C tokens x 256 / R weight rows per matrix:
   * 13, 14, 15 (96, 128, 160 tokens x 256 rows), 22, 23, 24 (128, 192, 256
   * tokens x 128 rows); 0 = by the mean slots per expert (the default) */
  MOE_OPT_GROUPED_TILE = 2,
  /* grouped-GEMM tile height of activation-quantised plans: 64, 128 or 192;
   * 0 = by the mean slots per expert (the default) */
  MOE_OPT_Q8_TILE = 3,
  /* top-k and permute in one workgroup up to this many tokens (1..64);
   * 0 = by the expert count (64 with at most 64 experts, else 16) */
  MOE_OPT_SMALL_ROUTE_T = 4
} moe_option;

/* Sets one option of a plan.  MOE_ERR_UNSUPPORTED for an unknown option,
 * MOE_ERR_BAD_SHAPE for a value outside the listed ones.  Call it before the
 * plan's forwards (it changes the plan, so it must not race with them) and
 * query moe_workspace_size afterwards: the workspace layout may change. */
moe_status moe_plan_set(moe_plan_t plan, int32_t option, int32_t value);

/* Bytes of device workspace a forward over n_tokens tokens needs (0 if
 * n_tokens <= 0 or the plan is NULL).  256-byte alignment is required. */
size_t moe_workspace_size(moe_plan_t plan, int32_t n_tokens);

/* The forward pass over T = n_tokens tokens, enqueued on `stream` (a
 * hipStream_t; NULL means the default stream).
 *   x          bf16 bits [T][d], 16-byte aligned
 *   w_router   f32 [E][d], 16-byte aligned
 *   logit_bias f32 [T][E] added to the router logits, or NULL
 *   gate, up, down   expert matrices (see moe_mat)
 *   out        f32 [T][d], 16-byte aligned
 * A plan with a shared expert runs through moe_forward_block instead
 * (MOE_ERR_NULL_ARG here: its matrices are missing).
 * Optional outputs (NULL: kept inside the workspace instead):
 *   topk_ids int32 [T][k] (ascending per token), topk_w f32 [T][k],
 *   counts int32 [E], offsets int32 [E+1] (exclusive scan of counts),
 *   perm int32 [T*k] (sorted position -> slot t*k+j).
 * T = 0 returns MOE_OK and launches nothing. */
moe_status moe_forward(moe_plan_t plan, int32_t n_tokens, const uint16_t* x, const float* w_router,
                       const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                       const moe_mat* down, float* out, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The layer inside a transformer block (dragon.c page, summary and
 * "Precision": the MoE reads the normed hidden state of sub-block 0, a dense
 * per-sub-block branch is quantised like the routed experts, and the MoE
 * output is added to the residual stream at the end of sub-block 1 in the
 * shortcut-connected layout).  As moe_forward, plus:
 *   shared_gate, shared_up, shared_down   the shared expert's matrices (one
 *       expert; expert strides ignored), required exactly when the plan has
 *       shared_expert = 1.  Its rows run inside the routed experts' launches
 *       (the tile lists carry them after the routed experts'), and its output
 *       is added to the combine in f32: out = sum_j w_j y_j + y_shared.
 *   residual, out_bf16   bf16 bits [T][d], 8-byte aligned, both or neither:
 *       out_bf16 = bf16_rne(residual + out), written by the combine (in place
 *       allowed: out_bf16 may be residual).  The plain pre-norm block passes
 *       its hidden rows; the shortcut layout passes a later point of the
 *       stream.
 *   out  f32 [T][d] as in moe_forward, optional when out_bf16 is given.
 * A plan with one expert and top-1 takes no residual (MOE_ERR_UNSUPPORTED). */
moe_status moe_forward_block(moe_plan_t plan, int32_t n_tokens, const uint16_t* x,
                             const float* w_router, const float* logit_bias, const moe_mat* gate,
                             const moe_mat* up, const moe_mat* down, const moe_mat* shared_gate,
                             const moe_mat* shared_up, const moe_mat* shared_down,
                             const uint16_t* residual, uint16_t* out_bf16, float* out,
                             int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* perm, void* workspace, size_t workspace_bytes, void* stream);

/* The same forward for callers that cannot allocate device memory or bring
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments and results as moe_forward, without the
 * workspace: the kernels use instead a scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * (statically, until the process ends; its address is looked up once per
 * device when the first plan is made there).  This call allocates nothing and
 * calls no allocating routine.
 *   - MOE_ERR_WORKSPACE if moe_workspace_size(plan, n_tokens) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES (64 MiB: every decode size of the layers in
 *     this repository, and grouped batches up to a few hundred tokens);
 *   - MOE_ERR_HIP if the scratch address could not be found for the plan's
 *     device.
 * Every call on one device shares that device's scratch and leaves its
 * contents there (the kernels need no cleared scratch): calls that overlap
 * in time on one device, on any streams, race and corrupt each other's
 * results; serialise them (one stream, or events). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(moe_plan_t plan, int32_t n_tokens, const uint16_t* x,
                               const float* w_router, const float* logit_bias,
                               const moe_mat* gate, const moe_mat* up, const moe_mat* down,
                               float* out, int32_t* topk_ids, float* topk_w, int32_t* counts,
                               int32_t* offsets, int32_t* perm, void* stream);

/* MOE_NOALLOC_SCRATCH_BYTES, as a function for bindings that do not read the header. */
size_t moe_noalloc_scratch_bytes(void);

/* Byte offset, inside the workspace of a forward over n_tokens tokens, of
 * the expert hidden activations h: bf16 bits [T*k][d_ff] in sorted-slot
 * order (row p belongs to slot perm[p]).  -1 if the plan is NULL or
 * n_tokens <= 0.  Valid after the forward has completed. */
int64_t moe_workspace_h_offset(moe_plan_t plan, int32_t n_tokens);

/* Which variant a forward over n_tokens tokens runs: MOE_PATH_DECODE or
 * MOE_PATH_GROUPED (-1 for a NULL plan). */
int32_t moe_plan_path(moe_plan_t plan, int32_t n_tokens);

/* Stages of a forward, in launch order (bit i of a timing mask = stage i). */
typedef enum {
  MOE_STAGE_ROUTER = 0,   /* router logits */
  MOE_STAGE_TOPK = 1,     /* softmax + top-k */
  MOE_STAGE_PERMUTE = 2,  /* counting-sort permute */
  MOE_STAGE_GATEUP = 3,   /* gate/up projections + SwiGLU -> h */
  MOE_STAGE_DOWN = 4,     /* down projection -> y */
  MOE_STAGE_COMBINE = 5,  /* fixed-order weighted combine -> out */
  MOE_N_STAGES = 6
} moe_stage;

/* Instrumentation: while enabled, each moe_forward (up to max_forwards of
 * them) records a HIP event before and after every stage whose bit is set in
 * stage_mask, on the forward's stream.  The events are created here (no
 * device memory is allocated).  Timing makes the plan stateful: use it from
 * one host thread and one stream at a time. */
moe_status moe_timing_enable(moe_plan_t plan, uint32_t stage_mask, int32_t max_forwards);

/* Waits for the last recorded event, then writes for each stage the summed
 * GPU time in milliseconds over the recorded forwards (stage_ms[MOE_N_STAGES];
 * 0 for stages not in the mask, and for stages a forward runs fused with the
 * previous one: for T <= 16 (T <= 64 with at most 64 experts) the permute is
 * part of MOE_STAGE_TOPK) and their
 * number, and starts a new count. */
moe_status moe_timing_collect(moe_plan_t plan, float* stage_ms, int32_t* n_forwards);

/* Stops recording and destroys the events. */
moe_status moe_timing_disable(moe_plan_t plan);

/* The steps either side of the layer in a transformer block (dragon.c page,
 * summary and "Precision": the MoE reads the normed hidden state of sub-block
 * 0, norms run in bf16, and the MoE output is added to the residual stream,
 * at the end of sub-block 1 in the shortcut-connected layout).  Neither call
 * needs a plan; both are asynchronous on `stream` (NULL: the default stream)
 * and check every argument before launching.  n_tokens = 0 returns MOE_OK.
 *
 * RMS normalisation of bf16 rows:
 *   xn[t][i] = bf16_rne(x[t][i] * r_t * gamma[i]),  r_t = 1 / sqrt(mean_i x[t][i]^2 + eps),
 * in f32 with one fixed summation order per row.
 *   x, xn  bf16 bits [T][d], gamma bf16 bits [d], all 16-byte aligned; xn may
 *          not overlap x.  Requires d % 8 == 0 and a finite eps >= 0. */
moe_status moe_rmsnorm(int32_t n_tokens, int32_t d, const uint16_t* x, const uint16_t* gamma,
                       float eps, uint16_t* xn, void* stream);

/* Add of the layer output into the residual stream:
 *   out[t][i] = bf16_rne(residual[t][i] + (a[t][i] + b[t][i]))   (b NULL: + a only)
 * in f32, in that order.  a is the routed layer's out, b the dense (shared)
 * branch's out: a plan with one expert and top-1 (renorm) computes that
 * branch exactly, since its routing weight is 1.
 *   residual, out  bf16 bits [T][d], 8-byte aligned (out may be residual);
 *   a, b           f32 [T][d], 16-byte aligned.  Requires d % 4 == 0. */
moe_status moe_residual_add(int32_t n_tokens, int32_t d, const uint16_t* residual, const float* a,
                            const float* b, uint16_t* out, void* stream);

/* The activation quantiser of MOE_ACT_E4M3_G128 on its own (the forward of
 * such a plan runs it on x and on h): each bf16 row of x [rows][K] is cut
 * into groups of 128 inputs (the last group of a row is shorter when
 * K % 128 != 0); a group's scale byte is E + 127 for the smallest power of
 * two 2^E (E >= -127) with max|x| <= 448 * 2^E (127 for an all-zero group),
 * and each input becomes the e4m3 code nearest x / 2^E (ties to the even
 * mantissa, the sign bit kept).  dev.to DeepSeek-V4.1-Flash post, "Three bugs
 * on RTX 50xx that never raise an error", item 2 (fp8 activations with
 * UE8M0 scales).
 *   x       bf16 bits [rows][K], 16-byte aligned
 *   q       e4m3 codes [rows][K], 8-byte aligned
 *   scales  UE8M0 bytes [rows][ceil(K / 128)]
 * Requires K % 8 == 0; rows == 0 is a no-op.  Arguments are checked before
 * the launch. */
moe_status moe_act_quant(int32_t rows, int32_t K, const uint16_t* x, uint8_t* q, uint8_t* scales,
                         void* stream);

void moe_plan_free(moe_plan_t plan);

/* Static string naming a status code. */
const char* moe_status_str(moe_status status);

/* Human-readable description of the plan: device, chosen variants, tiles,
 * and the last HIP error seen by a call on this plan.  Owned by the plan. */
const char* moe_plan_info(moe_plan_t plan);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
