/*
 * moe.h - C ABI of the MI355X (gfx950) routed-expert MoE layer library.
 *
 * The layer computes, for tokens x[T,D], caller-supplied expert ids and
 * scores [T,K], gate|up weights W13[E,2F,D] and down weights W2[E,D,F]:
 *
 *   for every valid route r = t*K + k (0 <= ids[t,k] < E):
 *     h1 = W13[e] x[t] = [g; u]      (gate rows first)
 *     h2 = SiLU(g) * u,  SiLU(z) = z / (1 + e^-z)
 *     h3 = W2[e] h2
 *   y[t] = sum over valid k, ascending, of scores[t,k] * h3(t,k)   (fp32 sum)
 *
 * and its backward (dx, dW13, dW2, dscores).  Sources: the Dist-MoE visual
 * explainer ("Speed-of-light distributed Mixture-of-Experts kernels"),
 * section 01 (the caller-inputs table and the contract that id -1 disables a
 * route, needs score 0, and an all-inactive row returns exact zero; the
 * owner applies the scores and sums the K routes in FP32), section 02 (the
 * expert equation and the MXFP8 formats), sections 03-04 (activation budget,
 * align128 byte accounting, the save/replay inequality, reverse-order
 * backward); and "Mixture of Experts: How Routing Becomes GPU Computation",
 * section 2 (packing rows by expert with a stable sort and exclusive prefix
 * offsets, grouped GEMM C_e = A_e B_e^T and its gradients, SwiGLU backward),
 * section 5 (the combine gradients dH = p dY, dp = <H, dY>).
 *
 * Conventions for every call
 *  - All tensors are contiguous, row-major, in device memory (HBM) unless a
 *    parameter says "host".  Activations and weights are float32 for
 *    MOE_PREC_F32 and bfloat16 for MOE_PREC_BF16 / MOE_PREC_MXFP8 /
 *    MOE_PREC_MXFP4.
 *  - The caller owns every buffer and allocates it with the sizes reported
 *    by moe_plan_sizes; the library never allocates or frees device memory
 *    and keeps no pointer after a call returns.
 *  - Work is enqueued on the caller's stream; nothing but moe_read_status
 *    waits for the device, so a step can be captured in a HIP graph.
 *  - A plan with its workspaces serves one stream at a time (not reentrant);
 *    concurrent layers need separate plans or workspaces.
 *  - Errors detected on the host return a status code before anything is
 *    enqueued.  Errors only the device can see (ids outside [-1, E)) set
 *    sticky bits read by moe_read_status and never trap; such routes are
 *    treated as padding.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null / misaligned pointer, T > t_max, bad layer index */
  MOE_ERR_SHAPE = 2,        /* D, F, E, K outside the supported set */
  MOE_ERR_UNSUPPORTED = 3,  /* combination not built (e.g. backward of an inference plan) */
  MOE_ERR_WORKSPACE = 4,    /* workspace smaller than moe_plan_sizes reported */
  MOE_ERR_HIP = 5           /* a HIP runtime call failed */
} moe_status;

typedef enum moe_prec {
  MOE_PREC_F32 = 0,         /* fp32 operands, fp32 MFMA */
  MOE_PREC_BF16 = 1,        /* bf16 operands, fp32 accumulation */
  MOE_PREC_MXFP8 = 2,       /* E4M3 operands with E8M0 scales per 32 values */
  MOE_PREC_MXFP4 = 3        /* inference only: E2M1 operands (two per byte, low
                               nibble first) with E8M0 scales per 32 values,
                               weights prepared in 1x32 blocks; D and F
                               multiples of 256.  The OCP-MX counterpart of the
                               4-bit inference mode of the Dist-MoE explainer
                               (section 02; section 08's support table: 4-bit
                               is inference-only with prepared weights). */
} moe_prec;

typedef enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1
} moe_dtype;

/* Device status bits (moe_read_status). */
#define MOE_STATUS_BAD_ID     0x1u  /* some id < -1 or >= E: treated as padding */
#define MOE_STATUS_PAD_SCORE  0x2u  /* nonzero score on an id -1 route: ignored */
#define MOE_STATUS_ARENA      0x4u  /* backward of a layer whose forward state is gone */
#define MOE_STATUS_NULL_INPUT 0x8u  /* null x/scores/dy for a call with rows: rows skipped */
#define MOE_STATUS_SYNC_TIMEOUT 0x10u /* fused forward or backward: a record stopped waiting
                                         for the rows it reads */

/* moe_expert_bwd flags */
#define MOE_BWD_ACCUMULATE_DX 0x1u  /* dx += result instead of dx = result */
/* g->dw13 += result and g->dw2 += result instead of =: the in-place
 * accumulation of weight gradients into the caller's parameter-gradient
 * buffers that the explainx.ai post on Dist-MoE lists under Supported modes
 * among the training options (several micro-batches into one dW).  Each value is summed in fp32
 * and rounded once to the dW type; experts with no rows keep their values.
 * dW is then read as well as written. */
#define MOE_BWD_ACCUMULATE_DW 0x2u
/* The fused (Mega) backward of the Dist-MoE explainer, section 05 (and
 * section 0: the MXFP8 path's backward as two fused expert operations, W2
 * then W13, followed by the input-gradient reduction): each projection's
 * DGRAD and WGRAD work records run in one persistent grid, each expert's
 * DGRAD tile range next to its WGRAD range.  Results are bit-identical to
 * the staged backward (the same tiles, summed in the same order).  BF16 and
 * MXFP8 plans.  BF16: the W2 launch's dW2 records wait, bounded, for the h2
 * rows its DGRAD records rebuild; a wait that runs out sets
 * MOE_STATUS_SYNC_TIMEOUT.  MXFP8 records never wait (both records of a
 * projection read operands quantized before the launch). */
#define MOE_BWD_MEGA 0x4u

/* Layer description.  Supported: D % 128 == 0, F % 128 == 0, D and F at
 * most 65,536, 1 <= K <= 16, 1 <= E <= 4096, 0 <= t_max <= 2^24 / K (else
 * MOE_ERR_SHAPE).  K may exceed E: a token may name one expert in several
 * slots, and each such slot is an independent route.  E is bounded by the
 * router, which keeps one counter per expert in on-chip LDS per 256-route
 * chunk (at the pages' expert size, D = 7,168 and F = 2,048, 4,096 BF16
 * experts would already need 360 GB of weights, more than one GPU holds).
 * MXFP4: D % 256 == 0 and F % 256 == 0 (else MOE_ERR_SHAPE), training 0
 * (else MOE_ERR_ARG). */
typedef struct moe_desc {
  int64_t t_max;            /* most tokens any call will pass */
  int32_t d;                /* token width D */
  int32_t f;                /* expert intermediate width F */
  int32_t e;                /* experts E (all local) */
  int32_t k;                /* routes per token K */
  int32_t prec;             /* moe_prec */
  int32_t dw_dtype;         /* moe_dtype of dW13/dW2 (MOE_PREC_F32 needs F32) */
  int32_t training;         /* 1: forward keeps state for moe_expert_bwd */
  int32_t max_layers;       /* layers whose saved state shares one arena (>= 1) */
  int64_t arena_budget;     /* bytes of saved state the arena may hold;
                               0 = enough to save every layer at R = t_max*K */
  float swiglu_limit;       /* 0: plain SwiGLU.  L > 0: clamped SwiGLU (named
                               under Supported modes in the explainx.ai
                               post on Dist-MoE, no formula; read here as h2 = SiLU(min(g, L)) *
                               clamp(u, -L, L), no gradient through a clamped
                               value, the clamps decided on h1 as stored).
                               Negative or non-finite -> MOE_ERR_ARG. */
  int32_t mx_w1x32;         /* MXFP8 inference plans: 1 = weights prepared in
                               1x32 blocks (one E8M0 exponent per 32 values of
                               a weight row along the contraction, the
                               inference preparation of the explainx.ai
                               post's Supported modes); 0 = 32x32
                               blocks (training-compatible).  1 with a
                               training or non-MXFP8 plan -> MOE_ERR_ARG
                               (MXFP4 weights are always 1x32: leave 0). */
  int32_t hot_tiles;        /* BF16 forward tiling of experts with 256 or more
                               rows (their GEMMs reuse each weight tile over
                               hundreds of rows, so they are bound by the
                               matrix cores, not by reading weights):
                               0 = automatic (256 x 256 MFMA tiles when the
                               call could give them at least three work items
                               per four compute units), 1 = always those
                               tiles, 2 = never (every expert on the
                               weight-streaming tiles).  Results agree within
                               rounding either way.  In BF16 and MXFP8
                               training, 0 and 1 also put the bf16 weight
                               gradients of experts with 256 or more rows on
                               256 x 256 tiles (bit-identical to the
                               streaming tiles; not with MOE_BWD_MEGA,
                               MOE_BWD_ACCUMULATE_DW, fp32 dW or widths that
                               are not multiples of 256).  The forward
                               tiling is BF16 only; other values ->
                               MOE_ERR_ARG. */
} moe_desc;

/* Byte sizes of the caller-owned buffers (all 256-byte aligned). */
typedef struct moe_sizes {
  size_t route_ws;          /* per layer: routing metadata + planner record */
  size_t scratch;           /* per call, reused by every layer and both passes */
  size_t h3_slots;          /* per layer: route outputs [t_max*K, D] (act dtype) */
  size_t arena;             /* shared by the layers of one step (header + budget) */
  size_t layer_state_max;   /* one layer's full saved state at R = t_max*K */
  size_t q13, s13, q2, s2;  /* MXFP8 prepared weights (0 otherwise) */
} moe_sizes;

typedef struct moe_plan_s* moe_plan_t;

/* Expert weights of one layer.  w13/w2 are the caller's [E,2F,D] / [E,D,F]
 * tensors; q13/s13/q2/s2 the MXFP8 copies made by moe_prepare_weights
 * (E4M3 bytes with the weight's shape, E8M0 bytes [E,2F/32,D/32] and
 * [E,D/32,F/32]).  Unused members may be null. */
typedef struct moe_weights {
  const void* w13;
  const void* w2;
  const void* q13;
  const void* s13;
  const void* q2;
  const void* s2;
} moe_weights;

/* Gradient outputs of one layer.  dx [T,D] act dtype; dw13 [E,2F,D] and
 * dw2 [E,D,F] in the plan's dw_dtype (fully written: experts with no rows
 * get exact zeros); dscores [T,K] float32 or null (0 for padding routes). */
typedef struct moe_grads {
  void* dx;
  void* dw13;
  void* dw2;
  float* dscores;
} moe_grads;

/* Validate a description and build a host-side plan (no device work).
 * The Dist-MoE explainer's section 08 (public API) and the explainx.ai post's
 * list of key design points describe a context that owns the layer's buffers
 * and is reused sequentially, never reentrantly; on one GPU that context
 * becomes this plan plus caller-owned buffers sized from it.  Section 03
 * (memory planning) gives the sizing rules: one layer's saved state counted
 * with align128 byte terms, one scratch region shared by every call and
 * sized for the largest temporary layout.  desc: host pointer, read only;
 * *out receives a handle owned by the library (free it with
 * moe_plan_destroy).  MOE_ERR_ARG for a null pointer or an option outside
 * its set, MOE_ERR_SHAPE for shapes outside the limits above. */
moe_status moe_plan_create(const moe_desc* desc, moe_plan_t* out);

/* Byte sizes of every caller-owned buffer of a plan (host only; sizes is a
 * host out-parameter).  Explainer section 03: the activation arena holds
 * saved state up to the budget (a soft limit: a layer that does not fit
 * replays), scratch holds the largest single call's temporaries (a hard
 * limit, here guaranteed by sizing it for t_max routes), and each layer's
 * routing metadata and route-output slots are separate.  MOE_ERR_ARG for a
 * null plan or sizes. */
moe_status moe_plan_sizes(moe_plan_t plan, moe_sizes* sizes);

/* Human-readable breakdown of the plan's buffers into buf (host, NUL
 * terminated, truncated to cap bytes).  Cf. plan_memory().explain() of the
 * Dist-MoE API, which likewise runs without touching a device. */
moe_status moe_plan_explain(moe_plan_t plan, char* buf, size_t cap);

void moe_plan_destroy(moe_plan_t plan);

/* MXFP8 weight preparation (explainer section 02: static weights use 32x32
 * blocks so forward and input-gradient GEMMs share the E4M3 values).  Reads
 * w13/w2 (bf16), writes q13/s13/q2/s2.  Done once per weight update; it is
 * not part of a timed step.  With mx_w1x32 (MXFP8) and for MXFP4 plans the
 * weight rows are quantized in 1x32 blocks along the contraction: codes
 * q13 [E, 2F, D] (MXFP4: [E, 2F, D/2] packed E2M1), exponents grouped by
 * stage, s13 [D/G][E*2F][G/32] with G = 128 (MXFP8) or 256 (MXFP4), and
 * likewise q2/s2 over [E*D, F].  Other precisions -> MOE_ERR_UNSUPPORTED. */
moe_status moe_prepare_weights(moe_plan_t plan, const void* w13, const void* w2,
                               void* q13, void* s13, void* q2, void* s2,
                               hipStream_t stream);

/* MXFP8 quantization of bf16 rows src [R, n] of a routed layer (R = the
 * valid routes of route_ws; n % 128 == 0), explainer section 02.  kind 0:
 * 1x32 row blocks -> q [R, n] E4M3 bytes, sc [R, n/32] E8M0 bytes.  kind 1:
 * column bundles, 32x1 blocks down each expert's rows padded to Mp_e =
 * counts[e] rounded up to 32 -> for expert e, q[n*poffsets[e] + c*Mp_e + m]
 * and sc[n*poffsets[e]/32 + c*Mp_e/32 + m/32]; pad rows are +0.  E8M0 byte =
 * e + 127 where e is the smallest integer with amax <= 448 * 2^e (clamped to
 * [-127, 127]); E4M3 values are rounded to nearest even.  kind 2 (MXFP4): 1x32
 * row blocks -> q [R, n/2] E2M1 codes (value 2i in the low nibble of byte i),
 * sc [R, n/32], e the smallest integer with amax <= 6 * 2^e, E2M1 values
 * rounded to nearest even.  Other kinds -> MOE_ERR_ARG. */
moe_status moe_mx_quantize(moe_plan_t plan, void* route_ws, const void* src, int32_t n,
                           int32_t kind, void* q, void* sc, hipStream_t stream);

/* Routing metadata (grouped-GEMM blog section 2 "Packing"): per-expert row
 * counts, exclusive prefix offsets, the stable expert-major order of valid
 * routes (ascending r = t*K + k inside an expert) and its inverse, and the
 * tile schedule of the grouped GEMMs.  ids: device int32 [T,K]; T <= t_max
 * (host value).  Writes route_ws only; clears the status bits. */
moe_status moe_route(moe_plan_t plan, int64_t T, const int32_t* ids, void* route_ws,
                     hipStream_t stream);

/* Expert forward of one layer (explainer section 02, staged form): each
 * expert's rows of x, gathered in expert order by the W13 kernel's loader
 * (x[sorted_route[row] / K]), give h1 = x W13^T with the SwiGLU epilogue,
 * then h3 = h2 W2^T stored bf16 (fp32 for F32 plans) into route slot
 * h3_slots[t*K + k].  Slots of padding routes are not written.  In training
 * the planner decides on the device whether this layer's state is saved in
 * the arena or rebuilt by backward (explainer section 04); layer is the
 * index of this layer in the stack (0 .. max_layers-1) and layer 0 starts
 * a new step (arena cursor 0).  x: [T,D], read again by the backward (keep
 * it until then).  arena may be null for inference.  A null x with routed
 * rows sets MOE_STATUS_NULL_INPUT. */
moe_status moe_expert_fwd(moe_plan_t plan, int32_t layer, void* route_ws, const void* x,
                          const moe_weights* w, void* h3_slots, void* arena, void* scratch,
                          hipStream_t stream);

/* The same expert forward as one fused (Mega) launch (explainer section 05,
 * "Kernel Pipelines: Staged and Mega": the W13 and W2 work records share
 * one persistent grid, and per-chunk counters in HBM let a W2 record start
 * once the h2 rows it reads are complete).  Arguments, outputs, planner
 * behaviour and MOE_STATUS_NULL_INPUT as moe_expert_fwd; h3_slots and the
 * saved or scratch h1 are bit-identical to moe_expert_fwd's where that one
 * runs every expert on the streaming tiles without split-K (the same tiles
 * and epilogues, only scheduled together).  Chunks are experts: each XCD
 * owns a contiguous range of experts and runs their W13 and W2 records
 * from its own queue, so h2 rows are handed over inside one L2.  All experts
 * use the streaming 128 x 128 tiles (no hot-expert tiles, no split-K).
 * Block-scaled plans (MXFP8 32x32 or 1x32 weights, MXFP4) hand over the h2
 * rows as the 1x32 blocks the W13 epilogue quantizes them into, as in the
 * staged forward.  A W2 record that waited too long for its rows (it cannot
 * happen while the grid runs to completion) sets MOE_STATUS_SYNC_TIMEOUT. */
moe_status moe_expert_fwd_mega(moe_plan_t plan, int32_t layer, void* route_ws, const void* x,
                               const moe_weights* w, void* h3_slots, void* arena,
                               void* scratch, hipStream_t stream);

/* Token-owner combine (explainer section 01): y[t] = sum over valid k,
 * ascending, of scores[t,k] * h3_slots[t*K+k] in fp32, plus y_addend[t]
 * (e.g. a shared expert's output, act dtype, nullable), stored in the act
 * dtype.  A token with no valid route gets exactly y_addend (or 0). */
moe_status moe_combine(moe_plan_t plan, void* route_ws, const float* scores,
                       const void* h3_slots, const void* y_addend, void* y,
                       hipStream_t stream);

/* Inference forward with the combine fused into the W2 epilogue: the
 * score-weighted scatter-add of every route's output into its token's row,
 * the combine that "Mixture of Experts: How Routing Becomes GPU Computation"
 * writes as an index_add_ of weighted expert outputs into the original token
 * rows (section 2, selected-expert forward), done inside the W2 kernel
 * instead of as a separate pass.  (The Dist-MoE explainer's own W2 epilogue,
 * section 05, stores each route's result to its return slot and leaves the
 * weighted sum to the token owner; moe_expert_fwd + moe_combine is that
 * form.)  Like moe_expert_fwd followed by moe_combine, but every route's
 * bf16-rounded (F32 plans: fp32)
 * h3, times its score, is added into y32[t] (caller-owned fp32 [T,D]
 * scratch, zeroed by this call) with hardware float atomics, then
 * y = y32 (+ y_addend).  No route slots are written, so the order of the K
 * additions per token is not fixed and y may differ from the slot combine
 * in the last bits; use moe_combine where bit-reproducible outputs matter.
 * Inference plans only (training = 0: nothing is kept for a backward,
 * MOE_ERR_UNSUPPORTED otherwise).  scores: [T,K] fp32; a null scores or y
 * with routed rows sets MOE_STATUS_NULL_INPUT. */
moe_status moe_expert_fwd_fused(moe_plan_t plan, void* route_ws, const void* x,
                                const float* scores, const moe_weights* w, float* y32,
                                const void* y_addend, void* y, void* scratch, hipStream_t stream);

/* Allocation-free variant of moe_expert_fwd_fused, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results minus
 * y32 and scratch: the fused forward's scratch and its fp32 accumulation
 * rows live in a 64 MiB array inside the library, one per GPU, held until the
 * process ends.  The plan must fit it: moe_plan_sizes(plan).scratch and
 * t_max * D * 4 bytes of fp32 rows, each rounded up to 256 bytes, at most
 * 64 MiB together (else MOE_ERR_WORKSPACE, before anything is enqueued; for
 * example the BF16 layer at D = 7,168, F = 2,048, K = 6 fits up to t_max =
 * 655 tokens).  Every call on one GPU shares that array and it keeps the
 * last call's contents (this call clears what must start at zero), so calls
 * that overlap on one GPU - on two streams, or from two threads - race; keep
 * them ordered on one stream.  No hipMalloc, hipFree or allocating library
 * call is made. */
moe_status moe_expert_fwd_fused_noalloc(moe_plan_t plan, void* route_ws, const void* x,
                                        const float* scores, const moe_weights* w,
                                        const void* y_addend, void* y, hipStream_t stream);

/* Backward of one layer (blog section 2 SwiGLU backward, section 5): from
 * dy [T,D] computes dscores, W2 DGRAD with the SwiGLU backward epilogue,
 * W2 and W13 WGRAD, W13 DGRAD and the per-token sum of the K route input
 * gradients into g->dx.  Rebuilds the layer's state first when its forward
 * replayed.  Layers of a step must run in reverse forward order; each
 * backward rewinds the arena cursor to its layer's start. */
/* flags: MOE_BWD_ACCUMULATE_DX | MOE_BWD_ACCUMULATE_DW | MOE_BWD_MEGA; other bits ->
 * MOE_ERR_ARG. */
moe_status moe_expert_bwd(moe_plan_t plan, int32_t layer, void* route_ws, const void* x,
                          const float* scores, const void* dy, const moe_weights* w,
                          const void* h3_slots, void* arena, void* scratch,
                          const moe_grads* g, uint32_t flags, hipStream_t stream);

/* Synchronizes stream and returns the sticky MOE_STATUS_* bits of route_ws
 * (host out-parameter) together with, when not null, the layer's planner
 * decision (*replayed = 1 when its forward chose replay).  The explainx.ai
 * post's list of key design points has invalid ids and overflowing scratch
 * end in a device trap that invalidates the whole context; here the kernels
 * record such conditions as sticky bits and carry on (bad ids act as padding,
 * scratch cannot overflow because it is sized for t_max routes), and this
 * call is the one place that reads them back.  MOE_ERR_ARG for a null
 * route_ws or status, MOE_ERR_HIP if the copy or the wait fails. */
moe_status moe_read_status(void* route_ws, uint32_t* status, int32_t* replayed,
                           hipStream_t stream);

/* Rewind the arena to empty, for a step that was abandoned between its
 * forwards and backwards.  The Dist-MoE explainer's section 06 (pipeline
 * liveness and slot reuse) allows resetting state after an aborted schedule
 * only once no backward still owns it; the caller guarantees that (no
 * pending moe_expert_bwd of this arena).  Enqueued on stream; MOE_ERR_ARG for
 * a null plan or arena. */
moe_status moe_arena_reset(moe_plan_t plan, void* arena, hipStream_t stream);

/* Routing results of route_ws copied to host memory (synchronizes stream):
 * counts [E], offsets [E+1], poffsets [E+1] (counts rounded up to 32),
 * sorted_route [R] and route_to_row [T*K]; any pointer may be null; *R_out
 * receives the number of valid routes. */
moe_status moe_route_readback(moe_plan_t plan, void* route_ws, int32_t* counts,
                              int32_t* offsets, int32_t* poffsets, int32_t* sorted_route,
                              int32_t* route_to_row, int32_t* R_out, hipStream_t stream);

/* Device pointers of the layer's saved tensors inside scratch/arena, for
 * inspection by tests (synchronizes stream): *x_rows is always null (the
 * gathered rows are never materialized: kernels read x through the
 * permutation) and *h1 receives h1 [R,2F] in the act dtype. */
moe_status moe_saved_ptrs(moe_plan_t plan, void* route_ws, void** x_rows, void** h1,
                          hipStream_t stream);

/* Kernel timing, for benchmarks.  While enabled, every kernel launched by a
 * call of this plan is bracketed by two HIP events recorded on that call's
 * stream.  moe_timing_read synchronizes on the recorded events, folds them
 * into per-kernel totals and returns entry idx (0-based; MOE_ERR_ARG past
 * the last): its name (host buffer, NUL terminated), total milliseconds and
 * launch count.  moe_timing_enable(plan, 0) stops recording and clears the
 * totals. */
moe_status moe_timing_enable(moe_plan_t plan, int32_t enable);
/* Benchmark only: while timing is enabled and buf is non-null, every timed
 * kernel is preceded, outside its events, by a write of bytes bytes of buf
 * (caller-owned device memory, 16-byte aligned), so that the kernel reads
 * its inputs from HBM and not from the 256 MiB memory-side Infinity Cache.
 * The Dist-MoE explainer's section 07 times whole steps in steady state; a
 * cold-cache timing of each bandwidth-bound row kernel (routing, gather,
 * combine, combine backward, input-gradient sum) shows whether its rate is
 * an HBM rate.  buf = null turns it off.  MOE_ERR_ARG for a null plan or a
 * misaligned or too small buffer. */
moe_status moe_timing_flush(moe_plan_t plan, void* buf, size_t bytes);
moe_status moe_timing_read(moe_plan_t plan, int32_t idx, char* name, size_t cap,
                           double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
