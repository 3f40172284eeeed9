/*
 * vdn.h -- C ABI of the MI355X (gfx950) forward pass (bf16, fp32 or with an FP8 softmax branch)
 * and backward pass of the Video DeltaNet (VDN) hybrid video-video attention layer.
 *
 * Source of every operation below: "Video DeltaNet: Near-Lossless Hybrid Attention for Video
 * Models" (openvdn.github.io), cited as [VDN] with the section name, and "Faster Than It Plays:
 * Video DeltaNet Generates 14 Seconds of 768p Video in 11 Seconds" (ai-blog.deepmagic.app),
 * cited as [FTP], whose section "Two branches instead of one" prints the frame update in text.
 *
 * The layer, per head h, for video query token i in latent frame t (chunk c = t / C):
 *
 *   softmax branch  ([VDN] "Local Softmax and Long-Range Linear Memory")
 *     o_s = softmax(q_i K^T / sqrt(d)) V over the text keys, the keys of every frame whose chunk is
 *     within one chunk of c (the bidirectional sliding window), and the boundary anchors: frames 0
 *     and T-1 for every query frame, every frame for query frames 0 and T-1.  One normaliser.
 *
 *   linear branch   ([VDN] "Video Delta Attention: A Frame-Wise Solution", [FTP])
 *     per frame f: A_f = sum_u beta_u k_u k_u^T, B_f = sum_u beta_u v_u k_u^T over the frame's N
 *     tokens; the frame update is S <- (S + B_f)(I + A_f)^-1.  The text is written first, as one
 *     joint update from S = 0 with every text weight halved (beta/2), giving S0 for both
 *     directions.  The forward state of query frame t has then absorbed, in increasing order, the
 *     non-boundary frames of chunks <= c-2; the reverse state, in decreasing order, those of
 *     chunks >= c+2.  o_l = (S_fwd + S_rev) q_i; boundary query frames read 2 S0 q_i.
 *
 *   merge           ([VDN] "Gating the Softmax and Linear Branch Outputs")
 *     r = o_l / sqrt(mean(o_l^2) + 1e-6); g_s = sigmoid(q_i Wg[0]); g_l = sigmoid(q_i Wg[1]);
 *     out_i = (g_s * o_s) Wp[0] + (g_l * r) Wp[1].   The residual add is the caller's.
 *
 * With anchors off there are no boundary frames: no anchor keys, and frames 0 and T-1 are
 * written into the states like any other frame.
 *
 * Text and audio tokens ("Video DeltaNet speeds MiniMax H3 video generation 14.5x" (glonce.com),
 * summary and key facts: only video-to-video interactions become hybrid; every interaction with a
 * text or audio token keeps the full softmax attention).  A plan may carry n_audio audio tokens
 * after the n_text text tokens (the n_ctx = n_text + n_audio context tokens): audio keys are
 * global keys of the softmax branch exactly like the text keys, and are never written into the
 * linear memory.  The text and audio query rows (vdn_forward_joint) get one plain softmax over
 * every token, o_c = softmax(q_c K^T / sqrt(d)) V over the context and all T*N video tokens,
 * returned before any projection (the model's own output projection applies to those rows).
 *
 * Layouts (row-major, token-major, head inside the token; every pointer is a DEVICE pointer):
 *   q, k, v, out : [T*N][H][d]         element type = the plan's dtype
 *   beta         : [n_text + T*N][H]    float32, text rows first; beta >= 0
 *   text_kv      : [2][n_ctx][H][d]     keys then values of the context tokens, text rows first,
 *                                       then audio (n_ctx = n_text for plans without audio), plan
 *                                       dtype (may be NULL if n_ctx == 0)
 *   ctx_q, ctx_out : [n_ctx][H][d]      context query rows and their output (vdn_forward_joint)
 *   gate_w       : [2][d][d]            [in][out] (y = x W); [0] softmax gate, [1] linear gate
 *   proj_w       : [2][d][d]            [in][out]; [0] softmax projection, [1] linear projection
 * The weights are shared by all heads.  q, k and text keys are expected L2-normalised per
 * (token, head); the layer does not renormalise.
 *
 * Ownership: the caller owns every tensor; the library reads inputs and writes `out` inside the
 * stream-ordered call and keeps no reference afterwards.  `out` must not alias an input.  The plan
 * owns a device workspace allocated at create time on the device current then (plus one side
 * stream and two events when created with VDN_FLAG_OVERLAP); a plan is used from that device only.  Calls on one plan must not
 * overlap (they share the workspace): serialise them on one stream, or use one plan per stream.
 *
 * Errors: no call aborts or throws.  Argument errors are detected on the host before anything is
 * enqueued.  Faults inside kernels surface at the caller's next synchronisation of `stream`.
 */
#ifndef VDN_H
#define VDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vdn_plan vdn_plan;

typedef enum {
  VDN_OK = 0,
  VDN_ERR_INVALID_ARG = -1,   /* NULL pointer, dimension <= 0, anchors not 0/1, misalignment */
  VDN_ERR_UNSUPPORTED = -2,   /* d not in {16, 32, 64, 128}, unknown dtype, size overflow,
                                 a shape outside a requested variant's limits                 */
  VDN_ERR_OUT_OF_MEMORY = -3, /* workspace allocation failed                                   */
  VDN_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed                    */
  VDN_ERR_TOO_LARGE = -5      /* vdn_forward_noalloc: the shape's workspace exceeds its static
                                 scratch                                                       */
} vdn_status;

typedef enum { VDN_F32 = 0, VDN_BF16 = 1 } vdn_dtype;

/* Build a plan for one layer shape.  T frames of N tokens, chunks of C frames, n_text text tokens
 * (may be 0), H heads of size d, anchors 0/1, element type dtype.  Computes the per-frame key
 * ranges of the softmax branch and the scan order of the linear branch, and allocates the
 * workspace.  Every stage runs in order on the caller's stream.  On success *plan_out owns the
 * plan; on failure *plan_out is set to NULL. */
vdn_status vdn_plan_create(int T, int N, int C, int n_text, int H, int d, int anchors,
                           vdn_dtype dtype, vdn_plan **plan_out);

/* As vdn_plan_create, with flags: VDN_FLAG_GENERIC_KERNELS selects the generic (SIMT) kernel of
 * every stage even where an MFMA kernel exists (used to cross-check the two kernel families);
 * VDN_FLAG_SERIAL requests the default order (every stage one after the other on the caller's
 * stream); VDN_FLAG_OVERLAP instead runs the linear branch on a side stream of the plan, forked
 * from and joined back into the caller's stream, concurrently with the softmax branch (on MI355X
 * this is slower at the 768p shape: the two branches compete for the compute units).  SERIAL and
 * OVERLAP together are an argument error.  Results are identical in every case.
 *
 * VDN_FLAG_FP8_SOFTMAX runs the softmax branch of the video rows and of the context rows in FP8
 * (OCP E4M3) on the matrix cores.  "Video DeltaNet: Near-Lossless Hybrid Attention for Video
 * Models", section "Adapting the Pretrained H3 backbone", reports the production layer with FP8
 * arithmetic but not its roundings; the ones made here are: power-of-two scales 2^(8 - e) (e the
 * binary exponent of the largest magnitude) for the keys and for the values of each head and for
 * each query row taken as c q (c = log2(e)/sqrt(d)); operands rounded to E4M3 (nearest, ties to
 * even); scores x (in log2 units) from the rounded operands in fp32; weights
 * P8 = e4m3(2^(8 + x - m)) with the offset m = c |q| max|k| when that is <= 4, else the row's
 * exact maximum max x; o = sum P8 V8 / (s_v sum P8).  Inputs and outputs are unchanged (bf16); the linear branch and the merge are the
 * bf16 plan's.  Requires VDN_BF16, d = 128 and N a multiple of 16 (else VDN_ERR_UNSUPPORTED);
 * with VDN_FLAG_GENERIC_KERNELS it is an argument error.  vdn_backward and vdn_backward_joint on
 * such a plan return the gradient of the exact (bf16) layer at the same inputs: the roundings,
 * whose derivative is zero almost everywhere, are passed straight through.  The plan computes it
 * with a bf16 plan of the same shape that it creates at its first backward call and keeps (its
 * workspace is not counted by vdn_plan_workspace_bytes); vdn_backward_after_forward rejects FP8
 * plans (VDN_ERR_UNSUPPORTED), since their forward leaves none of the exact intermediates.
 *
 * VDN_FLAG_FP8_EPILOGUE computes the epilogue's four d x d products -- the two sigmoid gates
 * q Wg_m and the two output projections of "Gating the Softmax and Linear Branch Outputs" -- in
 * MXFP8 on the matrix cores (the same page's "Adapting the Pretrained H3 backbone" runs FP8
 * linear layers without fixing their roundings).  The roundings made here: each operand is cut
 * into blocks of 32 consecutive elements along the contraction axis (q and the gated branch
 * outputs per token, each weight column along its input index); a block with largest magnitude
 * f 2^e (f in [0.5, 1)) is scaled by 2^-(e - 8) (X = e - 8 at least -127, 0 for a zero block) and
 * its elements rounded to E4M3 (nearest, ties to even); the products of the dequantised operands
 * accumulate in fp32.  The gated linear-branch output sigmoid(q Wg1) * o_l is quantised before
 * the RMSNorm factor is applied; the readout S q, the RMSNorm, the sigmoids and the gating stay
 * as in the bf16 plan.  Combines with VDN_FLAG_FP8_SOFTMAX.  Requires VDN_BF16 and d = 128 (else
 * VDN_ERR_UNSUPPORTED); with VDN_FLAG_GENERIC_KERNELS it is an argument error.  The backward of
 * such plans is the exact layer's, as for VDN_FLAG_FP8_SOFTMAX. */
enum { VDN_FLAG_GENERIC_KERNELS = 1, VDN_FLAG_SERIAL = 2, VDN_FLAG_OVERLAP = 4, VDN_FLAG_FP8_SOFTMAX = 8,
       VDN_FLAG_FP8_EPILOGUE = 16 };
vdn_status vdn_plan_create_ex(int T, int N, int C, int n_text, int H, int d, int anchors,
                              vdn_dtype dtype, unsigned flags, vdn_plan **plan_out);

/* As vdn_plan_create_ex, for a sequence with n_audio >= 0 audio tokens after the n_text text
 * tokens (see "Text and audio tokens" above).  n_audio = 0 is vdn_plan_create_ex.  Every forward
 * entry point then takes text_kv as [2][n_text + n_audio][H][d]. */
vdn_status vdn_plan_create_joint(int T, int N, int C, int n_text, int n_audio, int H, int d,
                                 int anchors, vdn_dtype dtype, unsigned flags,
                                 vdn_plan **plan_out);

/* Enqueue the whole layer forward on `stream` (a hipStream_t; NULL = the null stream).  Returns
 * after enqueueing.  Every pointer must be 16-byte aligned.  See the layouts above. */
vdn_status vdn_forward(const vdn_plan *plan, const void *q, const void *k, const void *v,
                       const float *beta, const void *text_kv, const void *gate_w,
                       const void *proj_w, void *out, void *stream);

/* As vdn_forward, with the channel-wise decay gate of the linear branch ("Video DeltaNet:
 * Near-Lossless Hybrid Attention for Video Models", section "Video Delta Attention: A Frame-Wise
 * Solution"): before frame f is absorbed, each scan direction's inherited state is scaled per key
 * channel, S <- S Diag(alpha_f), then updated as usual.  alpha is fp32 [T][H][d] (frame-major,
 * d contiguous), device memory owned by the caller and only read; the text initialisation uses
 * no gate, and boundary frames' entries are unused.  alpha = 1 everywhere gives vdn_forward's
 * result.  alpha must be non-NULL, 16-byte aligned and not alias out (else
 * VDN_ERR_INVALID_ARG); values in [0, 1] keep the state non-expansive.  Every other argument and
 * error as vdn_forward. */
vdn_status vdn_forward_decay(const vdn_plan *plan, const void *q, const void *k, const void *v,
                             const float *beta, const void *text_kv, const float *alpha,
                             const void *gate_w, const void *proj_w, void *out, void *stream);

/* The whole joint sequence: vdn_forward (alpha NULL) or vdn_forward_decay (alpha non-NULL) for
 * the video rows, plus, when ctx_q and ctx_out are both non-NULL, the context (text and audio)
 * query rows: ctx_out[j] = softmax over every key of the plan's sequence for query ctx_q[j]
 * ("Video DeltaNet speeds MiniMax H3 video generation 14.5x", summary: text and audio
 * interactions keep the full softmax attention).  ctx_q and ctx_out are [n_ctx][H][d] in the
 * plan's dtype, device memory owned by the caller, 16-byte aligned; ctx_out must not alias any
 * other argument.  ctx_q and ctx_out both NULL computes no context rows; exactly one NULL is
 * VDN_ERR_INVALID_ARG.  With n_ctx = 0 they are ignored.  Other arguments and errors as
 * vdn_forward_decay, except that alpha may be NULL (no decay). */
vdn_status vdn_forward_joint(const vdn_plan *plan, const void *q, const void *k, const void *v,
                             const float *beta, const void *ctx_q, const void *ctx_kv,
                             const float *alpha, const void *gate_w, const void *proj_w,
                             void *out, void *ctx_out, void *stream);

/* Backward pass (reverse mode) of the layer for the output gradient dout ([T*N][H][d], plan dtype):
 * the transposes of every step of the forward definition above -- the merge ("Gating the Softmax
 * and Linear Branch Outputs"), the softmax branch ("Local Softmax and Long-Range Linear Memory") and
 * both frame scans with the text initialisation and, when alpha is given, the decay gate ("Video
 * Delta Attention: A Frame-Wise Solution").  Inputs as vdn_forward / vdn_forward_decay (alpha may
 * be NULL: no decay).  Outputs, all float32 device buffers owned by the caller and overwritten:
 * dq, dk, dv [T*N][H][d]; dbeta [n_text + T*N][H]; dtext_kv [2][n_ctx][H][d] with n_ctx =
 * n_text + n_audio (the gradient of text_kv, whose layout it shares; NULL iff n_ctx == 0);
 * dgate_w, dproj_w [2][d][d]; dalpha [T][H][d] or NULL (requires alpha).  For a plan with audio
 * tokens, text_kv holds the text and audio keys and values as in vdn_forward_joint, and the audio
 * keys' gradients come from the video rows' softmax alone (they are not in the linear memory); the
 * text and audio query rows are not part of this call (see vdn_backward_joint).  The call
 * recomputes the forward quantities it needs on `stream`.  The first call on a plan allocates a
 * backward workspace (about 6 T N H d float32 plus per-frame d x d matrices) that the plan keeps.
 * Errors as vdn_forward, plus VDN_ERR_INVALID_ARG when an output aliases an input. */
vdn_status vdn_backward(vdn_plan *plan, const void *q, const void *k, const void *v,
                        const float *beta, const void *text_kv, const float *alpha,
                        const void *gate_w, const void *proj_w, const void *dout, float *dq,
                        float *dk, float *dv, float *dbeta, float *dtext_kv, float *dgate_w,
                        float *dproj_w, float *dalpha, void *stream);

/* Backward pass of the whole joint sequence, the transpose of vdn_forward_joint: vdn_backward for
 * the video rows plus, when ctx_q, dctx_out and dctx_q are all non-NULL, the text and audio query
 * rows, each one plain softmax over every key of the sequence ("Video DeltaNet speeds MiniMax H3
 * video generation 14.5x", summary), with output gradient dctx_out ([n_ctx][H][d], plan dtype):
 * dctx_q ([n_ctx][H][d] float32) receives their query gradient and their key and value gradients
 * are added to dk, dv and dctx_kv.  All three NULL leaves the context rows out (vdn_backward);
 * one or two NULL is VDN_ERR_INVALID_ARG; with n_ctx = 0 they are ignored.  ctx_kv and dctx_kv are
 * vdn_backward's text_kv and dtext_kv ([2][n_ctx][H][d]).  Ownership, alignment, aliasing and the
 * other arguments and errors as vdn_backward; the context rows' output and normalisers are
 * recomputed on `stream` with the rest. */
vdn_status vdn_backward_joint(vdn_plan *plan, const void *q, const void *k, const void *v,
                              const float *beta, const void *ctx_q, const void *ctx_kv,
                              const float *alpha, const void *gate_w, const void *proj_w,
                              const void *dout, const void *dctx_out, float *dq, float *dk,
                              float *dv, float *dbeta, float *dctx_q, float *dctx_kv,
                              float *dgate_w, float *dproj_w, float *dalpha, void *stream);

/* As vdn_backward, reusing the intermediates the plan's most recent call left in its workspace
 * (linear-branch statistics and states, packed keys, the softmax output and its normalisers)
 * instead of recomputing them: for a training step that runs the forward and then the backward on
 * the same inputs.  Preconditions: the most recent call on this plan was vdn_forward,
 * vdn_forward_decay, vdn_forward_joint, vdn_backward or vdn_backward_joint with exactly these q,
 * k, v, beta, text_kv, alpha and weights, ordered before this call on the stream (the text and
 * audio query rows are not part of this call).  The library checks only that such a
 * call succeeded and that alpha was given to both or to neither (else VDN_ERR_INVALID_ARG); other
 * mismatched inputs give wrong gradients.  Results are identical to vdn_backward's. */
vdn_status vdn_backward_after_forward(vdn_plan *plan, const void *q, const void *k, const void *v,
                                      const float *beta, const void *text_kv, const float *alpha,
                                      const void *gate_w, const void *proj_w, const void *dout,
                                      float *dq, float *dk, float *dv, float *dbeta,
                                      float *dtext_kv, float *dgate_w, float *dproj_w,
                                      float *dalpha, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc): the layer forward of vdn_forward for the plan vdn_plan_create(T, N, C,
 * n_text, H, d, anchors, dtype) would build, without a plan.  The workspace is a static device
 * array of 32 MiB that the library holds on each GPU it runs on until the process ends; the call
 * allocates nothing (no hipMalloc, hipFree or other allocating routine).  A shape whose workspace
 * (vdn_plan_workspace_bytes of that plan) exceeds 32 MiB is rejected with VDN_ERR_TOO_LARGE before
 * anything is enqueued (the 20-frame x 256-token, 4 x 64 workload needs about 15 MiB; the 768p head
 * share needs 0.63 GB and takes a plan).  Arguments, layouts, kernels and results as vdn_forward
 * (the same bits), with the argument errors of vdn_plan_create and vdn_forward.  All calls on one
 * GPU share its array, which keeps the previous call's contents (each call rebuilds what it reads
 * before writing): calls that overlap on one GPU (other streams, other threads) race; serialise
 * them. */
vdn_status vdn_forward_noalloc(int T, int N, int C, int n_text, int H, int d, int anchors, vdn_dtype dtype,
                               const void *q, const void *k, const void *v, const float *beta,
                               const void *text_kv, const void *gate_w, const void *proj_w, void *out,
                               void *stream);

/* Free the plan's workspace, stream and events.  The caller must have synchronised the streams
 * the plan was used on.  NULL is a no-op. */
void vdn_plan_destroy(vdn_plan *plan);

/* Static description of a status code. */
const char *vdn_status_str(vdn_status s);

/* Bytes of device workspace the plan holds (informational). */
size_t vdn_plan_workspace_bytes(const vdn_plan *plan);

/* Host only, no GPU needed.  Key ranges of the softmax branch for query frame t, in the key index
 * space of one head: global (text, then audio) key j is index j; video token j (= f*N + n) is
 * index text_pad + j where text_pad = n_text rounded up to a multiple of 64.  Here n_text counts
 * every global key (n_text + n_audio of a joint plan).  Writes up to max_ranges [start, end) pairs
 * into ranges[2*r], ranges[2*r+1] in ascending order and returns their number, or -1 on an
 * invalid argument.  Empty ranges are omitted. */
int vdn_key_ranges(int T, int N, int C, int n_text, int anchors, int t, int64_t *ranges,
                   int max_ranges);

/* Host only.  Frames absorbed by the forward (dir = 0) or reverse (dir = 1) state of query frame
 * t, in the order they are written; returns their count (<= max_frames written) or -1. */
int vdn_scan_frames(int T, int C, int anchors, int t, int dir, int *frames, int max_frames);

/* Intermediate buffers of the last vdn_forward on this plan, for checking; stream-ordered copy of
 * `bytes` bytes (must equal the buffer's size) into the device buffer dst:
 *   VDN_BUF_OS     o_s     [T*N][H][d]          plan dtype
 *   VDN_BUF_STATES S_fwd, S_rev: [2][Nc+1][H][d][d] float32; slot Nc holds S0 (boundary frames)
 *   VDN_BUF_MINV   M_f = (I + A_f)^-1: [T+1][H][d][d] float32, slot 0 for the text (beta/2),
 *                  slot 1+f for frame f (boundary frames' slots are not written when anchors on)
 *   VDN_BUF_BW     B_f = sum_u beta_u v_u k_u^T: [T+1][H][d][d] float32, same slots as VDN_BUF_MINV
 *   VDN_BUF_K8     FP8 plans: keys e4m3(s_k k) [H][Ls8][d] bytes, Ls8 = round_up(n_ctx, 64) + T*N + 128,
 *                  key j of a head at row j (global keys, then video token j - round_up(n_ctx, 64))
 *   VDN_BUF_V8     FP8 plans: values e4m3(s_v v) transposed, [H][d][Ls8] bytes
 *   VDN_BUF_SCALES8 FP8 plans: [H][2] float32 (s_k, s_v)
 */
enum { VDN_BUF_OS = 0, VDN_BUF_STATES = 1, VDN_BUF_MINV = 2, VDN_BUF_BW = 3, VDN_BUF_K8 = 4, VDN_BUF_V8 = 5,
       VDN_BUF_SCALES8 = 6 };
vdn_status vdn_debug_buffer_bytes(const vdn_plan *plan, int which, size_t *bytes);
vdn_status vdn_debug_copy(const vdn_plan *plan, int which, void *dst, size_t bytes, void *stream);

/* Runs the plan's epilogue alone ("Gating the Softmax and Linear Branch Outputs": readout, RMSNorm,
 * gates, projections; MXFP8 products for VDN_FLAG_FP8_EPILOGUE plans) on a caller-supplied softmax
 * output o_s [T*N][H][d] bf16 and chunk-state buffer in the VDN_BUF_STATES layout
 * ([2][Nc+1][H][d][d] float32: forward slots, then reverse slots; slot Nc is read by the boundary
 * frames), with q, gate_w, proj_w and out as in vdn_forward.  Both are copied into the plan's
 * workspace on `stream` first, so a later vdn_backward_after_forward is rejected until the next
 * forward.  For testing the epilogue in isolation.  MFMA-epilogue plans only (else
 * VDN_ERR_UNSUPPORTED); device pointers, 16-byte aligned; out must not overlap an input
 * (VDN_ERR_INVALID_ARG). */
vdn_status vdn_debug_epilogue(vdn_plan *plan, const void *q, const void *o_s, const float *states,
                              const void *gate_w, const void *proj_w, void *out, void *stream);

/* Kernel timing.  vdn_profile_enable(plan, n) makes the next n forwards record HIP events around
 * each stage on the stream it runs on; vdn_profile_read sums the recorded times (milliseconds,
 * synchronising the events) into ms[VDN_STAGE_*] for n_stages entries and reports the number of
 * forwards recorded.  Stages: */
enum { VDN_STAGE_SOFTMAX = 0, VDN_STAGE_PREP = 1, VDN_STAGE_VDA_STATS = 2, VDN_STAGE_VDA_SCAN = 3,
       VDN_STAGE_EPILOGUE = 4, VDN_STAGE_TOTAL = 5, VDN_STAGE_SOFTMAX_FIRST = 6, VDN_NUM_STAGES = 7 };
/* VDN_STAGE_SOFTMAX covers both launches of the MFMA and FP8 softmax kernels: the fixed-reference
 * launch and the online-maximum launch that redoes the workgroups it flagged.
 * VDN_STAGE_SOFTMAX_FIRST starts with it and ends after the first launch alone (the single launch
 * of the generic kernel). */
vdn_status vdn_profile_enable(vdn_plan *plan, int max_calls);
vdn_status vdn_profile_read(vdn_plan *plan, float *ms, int n_stages, int *calls);

/* Which kernel family a plan selected for each stage (0 = generic SIMT kernel, 1 = MFMA kernel,
 * 2 = FP8 MFMA kernel: the softmax stage of VDN_FLAG_FP8_SOFTMAX plans, the epilogue stage of
 * VDN_FLAG_FP8_EPILOGUE plans). */
vdn_status vdn_plan_kernel_kind(const vdn_plan *plan, int stage, int *kind);

/* On-box reference rates for rooflines (measurement helpers; synchronous, on the current device's
 * null stream; no layer stage uses them).  vdn_measure_mfma_bf16_tflops runs a tight loop of
 * independent v_mfma_f32_32x32x16_bf16 on every compute unit for `iters` iterations and reports
 * dense bf16 TFLOP/s; vdn_measure_copy_gbs copies `bytes` device to device (hipMemcpyAsync) and
 * reports GB/s counting the read and the write.  Both allocate and free their own buffers. */
vdn_status vdn_measure_mfma_bf16_tflops(int iters, double *tflops);
vdn_status vdn_measure_copy_gbs(size_t bytes, double *gbs);

#ifdef __cplusplus
}
#endif

#endif /* VDN_H */
