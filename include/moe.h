/*
 * moe.h - C ABI of the MI355X (gfx950) grouped-expert MoE layer with affine
 * 4-bit expert weights.
 *
 * The layer is the mixture-of-experts block of Qwen3.6-35B-A3B as the pages on
 * Lily (Perplexity's inference engine) describe it:
 *   - every token scores all E routed experts, keeps top_k of them and adds
 *     one always-on shared expert (aimanavo.com page, section "Qwen3.6's 256
 *     experts and two layer types make the MLX-Lily gap");
 *   - routing stays on the GPU with no host synchronisation inside the layer
 *     (same page, section "Lily does not treat prefill and decode as the same
 *     job"; dzen.guru page, section "Where does the speed-up come from?");
 *   - expert weights are MLX affine 4-bit with group size 64 and are restored
 *     inside the grouped matrix product, never written out dequantised (same
 *     sections; aimanavo.com page, section on the single 4-bit checkpoint;
 *     news.mantis.guru page, section "Rust drives the model, Metal does the
 *     compute").
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer (weights, activations, outputs, workspace); the library
 *     allocates nothing, frees nothing, keeps no pointer after returning and
 *     holds no mutable global state, except the static per-device scratch of
 *     moe_layer_no_alloc and its host-side record of each device's address.
 *     Calls only ENQUEUE work on `stream` (stream-ordered: buffers must stay
 *     valid until that work completes); none synchronises the host.
 *   - Every check runs on the host before anything is enqueued.  A status other
 *     than MOE_OK means nothing was enqueued, except MOE_ERR_HIP, which reports
 *     a failed launch (the stream may then hold part of the work).
 *   - Range of the float16 products.  The expert products take float16
 *     operands with float32 accumulation: x, h = silu(gate)*up and, on the
 *     prefill path of moe_layer (T > 4), each expert's unweighted output row
 *     are rounded to float16 (nearest even; bf16 inputs up to 65280 in
 *     magnitude are exact).  A value of magnitude >= 65520 there becomes
 *     +-inf, and every output element computed from it is inf or NaN.  So a
 *     finite output element always meets the layer's accuracy, and a
 *     non-finite one marks a value beyond the float16 range.  The router
 *     (logits, selection, weights) and the decode path's expert outputs are
 *     float32 throughout.
 *   - Device-side preconditions that are documented but not checked: weights
 *     and activations are finite; every topk_idx entry handed to moe_permute lies in [0, E) with top_k distinct
 *     entries per token; offsets/sorted_slot handed to moe_expert_ffn are a
 *     valid permutation such as moe_permute produces.
 *   - Alignment: every pointer must be 16-byte aligned (MOE_ERR_ALIGN).
 *
 * Layouts (row-major; "bf16" = bfloat16 bit patterns in uint16_t)
 *   x          [T][H] bf16 activations
 *   router     [E][H] bf16
 *   logit_bias [E] float32, nullable: added to the router logits before
 *              selection and softmax
 *   moe_qmat   one stack of n matrices of shape [N][K]:
 *                q     [n][N][K/8] uint32, the code of column k in bits
 *                      [4*(k%8), 4*(k%8)+4) of word k/8 (MLX packing);
 *                scale [n][N][K/64], bias [n][N][K/64] (bf16 or float32,
 *                      moe_dims.sb_dtype); weight = scale*code + bias.
 *   experts    gate, up: N=I, K=H; down: N=H, K=I; n=E
 *   shared     gate, up: N=I_shared, K=H; down: N=H, K=I_shared; n=1
 *   slot       s = t*top_k + j for token t and its j-th ranked expert
 */
#ifndef BITMOE_MOE_H
#define BITMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status of every call.  Every argument is validated on the host before any
 * launch, and an unsupported layout is refused with a status instead of being
 * run: the fail-early rule of the engine, which checks the model's
 * architecture and quantisation layout at load and refuses an incompatible
 * checkpoint (news.mantis.guru page, section "Rust drives the model, Metal
 * does the compute"). */
typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* inconsistent or non-positive sizes */
    MOE_ERR_UNSUPPORTED = -3, /* valid in principle, outside this library's limits */
    MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -5,   /* workspace smaller than moe_workspace_size() */
    MOE_ERR_HIP = -6          /* a kernel launch failed */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* Host struct.  Limits (MOE_ERR_UNSUPPORTED beyond them):
 *   group == 64; H % 64 == 0, 64 <= H <= 16384; I % 64 == 0, 64 <= I <= 4096;
 *   I_shared == 0 (no shared expert) or as I; 1 <= top_k <= 8; top_k <= E <= 256;
 *   0 <= T <= 2^22 (T == 0 is a valid empty call that enqueues nothing);
 *   sb_dtype MOE_BF16 or MOE_F32; out_dtype MOE_F32 for moe_layer, MOE_BF16 for
 *   moe_layer_residual (the other calls' outputs are float32 whatever it says). */
typedef struct {
    int32_t T, H, E, top_k, I, I_shared, group;
    int32_t sb_dtype;  /* moe_dtype of expert scales and biases */
    int32_t out_dtype; /* moe_dtype of the layer output */
} moe_dims;

typedef struct {
    const uint32_t *q;
    const void *scale;
    const void *bias;
} moe_qmat;

typedef struct {
    moe_qmat gate, up, down;
} moe_ffn;

typedef struct {
    const uint16_t *router;   /* [E][H] bf16, or NULL when router_q8 is set */
    const float *logit_bias;  /* [E] or NULL */
    moe_ffn experts;          /* E routed experts */
    moe_ffn shared;           /* the shared expert; shared.gate.q == NULL iff I_shared == 0 */
    /* Optional gate of the shared expert, [H] bf16, or NULL.  Not on the pages: a
     * detail of Qwen's mixture-of-experts checkpoints.  When set, the shared
     * expert's output is scaled by sigmoid(sum_h x[t][h] * gate[h]) (float32
     * sum of exact bf16 products) instead of being added with weight 1.  Must
     * be NULL without a shared expert (MOE_ERR_SHAPE). */
    const uint16_t *shared_expert_gate;
    /* Optional 8-bit router in the MLX affine layout, in place of `router`
     * (both set: MOE_ERR_SHAPE; neither: MOE_ERR_NULL).  Not on the pages: a
     * checkpoint may quantise its router too.  router_q8 [E][H/4] holds four
     * codes per word, low byte first; router_scale and router_bias [E][H/64]
     * use dims->sb_dtype; all three 16-byte aligned.  Each layer call first
     * restores the bf16 router into its workspace, w =
     * bf16_nearest_even(fmaf(scale, code, bias)) (see moe_router_dequant), and
     * then scores with it exactly as with `router`. */
    const uint32_t *router_q8;
    const void *router_scale;
    const void *router_bias;
} moe_weights;

/* Bytes of device workspace the calls below need for these dims (host-only,
 * pure; 0 when the dims are invalid: the fail-early validation of
 * news.mantis.guru page, section "Rust drives the model, Metal does the
 * compute", applied before anything is sized).  One workspace serves every entry point.
 * Zero-fill the whole workspace once after allocating it; after that, every
 * call leaves it ready for the next one, whatever the dims of either.  The
 * first 16384 bytes are control words of the decode path: the 32 64-bit words
 * at bytes 2048 + 128 g count the workgroups of a running decode call (low
 * halves, 0 between calls) and the calls made (high halves, uint32 words
 * 513 + 32 g, all equal), and word 255 (bytes 1020..1023) is set to nonzero,
 * and stays so, if a
 * device-side wait of a decode call timed out (that call's output is then
 * invalid).  Calls that share a workspace must not overlap in time (use one
 * workspace per stream). */
size_t moe_workspace_size(const moe_dims *dims /* host */);

/* Router and top-k.  Every token scores all E routed experts and keeps top_k
 * of them (aimanavo.com page, section "Qwen3.6's 256 experts and two layer
 * types make the MLX-Lily gap": 8 of 256), on the GPU with no return to the
 * host (aimanavo.com page, section "Lily does not treat prefill and decode as
 * the same job"; dzen.guru page, section "Where does the speed-up come
 * from?").  The softmax, renormalisation and tie rule are not stated there and
 * are readings.
 * logits l[t][e] = sum_h x[t][h]*router[e][h] (+ logit_bias[e]), float32
 * accumulation of exact bf16 products; the top_k largest logits in rank order
 * (equal logits: lower expert index first); topk_w[t][j] = softmax of the
 * selected logits, i.e. the softmax over all E renormalised over the kept ones.
 * Outputs: topk_idx [T][top_k] int32, topk_w [T][top_k] float32. */
moe_status moe_route(const moe_dims *dims, const uint16_t *x, const uint16_t *router,
                     const float *logit_bias, int32_t *topk_idx, float *topk_w, hipStream_t stream);

/* Permute: the grouping of slots by expert that keeps the routing closed on
 * the GPU, with no host synchronisation per layer (aimanavo.com page, section
 * "Lily does not treat prefill and decode as the same job"; dzen.guru page,
 * section "Where does the speed-up come from?").  A counting sort of the
 * T*top_k slots by expert.  counts [E], offsets [E+1] (exclusive
 * prefix sum of counts), sorted_slot [T*top_k]: the slots of expert e occupy
 * sorted_slot[offsets[e] .. offsets[e+1]), in unspecified order within e.
 * Uses the workspace.  Requires T*top_k <= 2^22 for this call. */
moe_status moe_permute(const moe_dims *dims, const int32_t *topk_idx, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_slot, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* Grouped expert FFN with the 4-bit weights restored inside the grouped
 * products, never written out dequantised (aimanavo.com page, section "Lily
 * does not treat prefill and decode as the same job"; dzen.guru page, section
 * "Where does the speed-up come from?"); the weights are MLX affine 4-bit with
 * group size 64 (aimanavo.com page, section "Only one 4-bit checkpoint at a
 * pinned revision runs"; news.mantis.guru page, section "Rust drives the
 * model, Metal does the compute").  The SwiGLU form is a reading.  For every slot s of expert e,
 * with t = s / top_k:  y_slot[s] = W_down,e (silu(W_gate,e x[t]) * (W_up,e x[t])).
 * y_shared[t] = the shared expert applied to x[t] (skipped when shared or
 * y_shared is NULL).  offsets/sorted_slot as produced by moe_permute.
 * Outputs: y_slot [T*top_k][H] float32 (row = slot), y_shared [T][H] float32. */
moe_status moe_expert_ffn(const moe_dims *dims, const uint16_t *x, const int32_t *offsets,
                          const int32_t *sorted_slot, const moe_ffn *experts /* host */,
                          const moe_ffn *shared /* host, nullable */, float *y_slot,
                          float *y_shared /* nullable */, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* Weighted combine plus the one always-on shared expert (aimanavo.com page,
 * section "Qwen3.6's 256 experts and two layer types make the MLX-Lily gap";
 * the weighting by the routing weights is a reading):
 * out[t] = sum_j topk_w[t][j] * y_slot[t*top_k+j] + y_shared[t] (y_shared nullable).
 * out [T][H] float32. */
moe_status moe_combine(const moe_dims *dims, const float *y_slot, const float *topk_w,
                       const float *y_shared, void *out, hipStream_t stream);

/* Weight of the shared expert under its optional gate (see moe_weights; a
 * checkpoint detail, not on the pages): shared_w[t] = sigmoid(sum_h x[t][h] *
 * gate[h]), float32 sum of exact bf16 products.  x [T][H] bf16, gate [H] bf16,
 * shared_w [T] float32. */
moe_status moe_shared_gate(const moe_dims *dims, const uint16_t *x, const uint16_t *gate, float *shared_w,
                           hipStream_t stream);

/* moe_combine with the shared expert's row scaled per token:
 * out[t] = sum_j topk_w[t][j] * y_slot[t*top_k+j] + shared_w[t] * y_shared[t]
 * (y_shared nullable; shared_w nullable: weight 1, as moe_combine). */
moe_status moe_combine_gated(const moe_dims *dims, const float *y_slot, const float *topk_w,
                             const float *y_shared, const float *shared_w, void *out, hipStream_t stream);

/* The whole layer as one device-side pipeline, shared expert included: the
 * steps above in the pages' order (aimanavo.com page, sections "Qwen3.6's 256
 * experts and two layer types make the MLX-Lily gap" and "Lily does not treat
 * prefill and decode as the same job"; prefill and decode are separate
 * workloads: same section, and news.mantis.guru page, section "Prefill and
 * decode are optimised as different modes").  out [T][H] float32.  Optional copies of the routing: topk_idx_out [T][top_k],
 * topk_w_out [T][top_k], counts_out [E] (each nullable).
 * Prefill (T > 4): route, permute, gate/up with SwiGLU, down storing float16
 * rows per slot, then the weighted combine with the shared expert.  Decode
 * (T <= 4, a bandwidth-bound workload of its own): a single kernel whose router workgroups
 * rank the experts on the device and whose expert workgroups run the SwiGLU
 * experts and combine into out with atomics.  Uses the workspace's decode region
 * and control words (see moe_workspace_size). */
moe_status moe_layer(const moe_dims *dims, const moe_weights *weights /* host */,
                     const uint16_t *x, void *out, int32_t *topk_idx_out, float *topk_w_out,
                     int32_t *counts_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Restores an 8-bit router (the MLX affine layout of moe_weights.router_q8)
 * to bf16: router_out[e][h] = bf16_nearest_even(fmaf(scale[e][h/64],
 * code[e][h], bias[e][h/64])), code[e][h] = byte h%4 (low byte first) of word
 * router_q8[e][h/4]; scale and bias use dims->sb_dtype.  Not on the pages: a
 * checkpoint detail.  The output [E][H] feeds moe_route.  Device pointers,
 * all 16-byte aligned (MOE_ERR_ALIGN); NULL pointers: MOE_ERR_NULL. */
moe_status moe_router_dequant(const moe_dims *dims, const uint32_t *router_q8, const void *scale, const void *bias,
                              uint16_t *router_out, hipStream_t stream);

/* moe_layer writing into a bf16 residual stream (not on the pages: how a
 * decoder consumes the layer, a real-checkpoint detail):
 * out[t][h] = bf16(residual[t][h] + layer(x)[t][h]), the layer computed as in
 * moe_layer (float32), the residual added in float32, then one
 * round-to-nearest-even to bf16.  residual [T][H] bf16 is nullable (then 0)
 * and may be the same buffer as out (an in-place update of the stream).
 * Requires dims->out_dtype == MOE_BF16 (else MOE_ERR_UNSUPPORTED).  Decode
 * (T <= 4) adds one small kernel after the layer kernel. */
moe_status moe_layer_residual(const moe_dims *dims, const moe_weights *weights /* host */, const uint16_t *x,
                              const uint16_t *residual, uint16_t *out, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Bytes from one layer's copy of a tensor to the next layer's, for stacks of
 * layers (moe_decode_stack).  Each stride is a multiple of 16 (logit_bias: of
 * 4) and may be 0 (every layer shares the tensor). */
typedef struct {
    int64_t q, scale, bias;
} moe_qmat_stride;

typedef struct {
    moe_qmat_stride gate, up, down;
} moe_ffn_stride;

typedef struct {
    int64_t router, logit_bias, norm_weight;
    moe_ffn_stride experts, shared;
} moe_layer_strides;

/* A decode step of one token through a stack of n_layers MoE layers of a
 * pre-norm decoder in ONE kernel launch.  Each layer reads the root-mean-square
 * normalisation of the bf16 residual stream and adds its output to it:
 *     n(l)   = bf16(x(l) / sqrt(mean(x(l)^2) + 1e-6) * gamma_l)
 *     x(l+1) = bf16(x(l) + layer_l(n(l)))   (float32 sum, one round to nearest even)
 * with x(0) = x_in and x_out = x(n_layers); layer_l is moe_layer's layer with
 * layer l's weights, gamma_l layer l's norm_weight (1 when NULL).  The
 * normalisation is not on the pages: it is how a decoder feeds its MoE blocks,
 * and without it the stream grows by orders of magnitude per layer.  Pages: a
 * decode step is one chain of dependent stages that the engine overlaps
 * instead of running its kernels one after the other (aimanavo.com page,
 * section "Lily does not treat prefill and decode as the same job"), and its
 * routing stays on the GPU (same section; dzen.guru page, section "Where does
 * the speed-up come from?").  The kernel reads each layer's router and shared
 * expert ahead, while the layer before runs, and hands values between its
 * workgroups through the workspace's fixed-offset decode region (word 255 is
 * set if a device-side wait timed out; the outputs of that call are then
 * invalid).
 *   weights, norm_weight: layer 0's tensors (norm_weight [H] bf16, nullable);
 *     layer l's are at + l * strides (host struct; strides NULL: each tensor
 *     of a layer directly follows the previous layer's, i.e. stacked
 *     [n_layers][...] tensors).  router must be the bf16 matrix (router_q8 and
 *     shared_expert_gate: MOE_ERR_UNSUPPORTED).
 *   x_in [H] bf16; x_out [H] bf16 (may be x_in: an in-place update).
 *   Optional records (nullable), [n_layers][...]: layer_x [H] bf16, the stream
 *     entering each layer; layer_in [H] bf16, its normalisation; layer_out [H]
 *     float32, each layer's output; topk_idx_out, topk_w_out [top_k], the
 *     routing in rank order.
 * The layer is spread over the device's 8 XCDs: XCD x computes routed slot x
 * (rank order) and the shared expert's intermediate rows [x I / 8,
 * (x + 1) I / 8).  Each element of a layer's output is the float32 sum, in XCD
 * order, of the XCDs' partials w_x y_x + (the shared expert's part), so
 * outputs are the same bit for bit on every call.  Limits
 * (MOE_ERR_UNSUPPORTED): T == 1 (T == 0: nothing to do); H <= 2048; I a power
 * of two in [64, 512]; top_k <= 8; dims->out_dtype == MOE_BF16; n_layers >= 1
 * (else MOE_ERR_SHAPE); the device must hold 256 workgroups of 512 threads at
 * once (all of them run together and wait on each other; launch nothing else
 * on the device concurrently), spread evenly over 8 XCDs (a workgroup on an
 * XCD numbered 8 or more sets word 255). */
moe_status moe_decode_stack(const moe_dims *dims, const moe_weights *weights /* host */,
                            const uint16_t *norm_weight, const moe_layer_strides *strides /* host, nullable */,
                            int32_t n_layers, const uint16_t *x_in, uint16_t *x_out, uint16_t *layer_x,
                            uint16_t *layer_in, float *layer_out, int32_t *topk_idx_out, float *topk_w_out,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the device scratch that moe_layer_no_alloc uses in place of a
 * workspace (32 MiB per device; enough for every T up to 512 at H=2048, E=256,
 * top_k=8, I=512). */
#define MOE_NO_ALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* moe_layer for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same work and outputs as moe_layer, on the current
 * device (hipGetDevice; `stream` must belong to it), with the workspace taken
 * from a static device array of MOE_NO_ALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends.  Nothing is
 * allocated or freed.  Dims whose moe_workspace_size() exceeds that:
 * MOE_ERR_WORKSPACE; dims->out_dtype must be MOE_F32 (else
 * MOE_ERR_UNSUPPORTED).  Every argument is checked before anything is
 * enqueued.  The scratch keeps what the last call left; until a call outside
 * graph capture has run on a device, each call first clears the decode region
 * of the scratch with a small kernel on `stream` (captured, that kernel runs
 * on every replay).  All calls on one device share the one scratch: calls that
 * overlap in time on one device (on different streams, or from different
 * threads without ordering) race and give undefined results. */
moe_status moe_layer_no_alloc(const moe_dims *dims, const moe_weights *weights /* host */, const uint16_t *x,
                              void *out, int32_t *topk_idx_out, float *topk_w_out, int32_t *counts_out,
                              hipStream_t stream);

/* Instrumentation variant of moe_layer: the same work, plus HIP events recorded
 * on `stream` around its kernels.  events (host array) holds
 * moe_layer_stage_count(dims) + 1 caller-created events: events[0] is recorded
 * before the first kernel and events[i] right after kernel i (i >= 1).  Fewer
 * events than that: MOE_ERR_SHAPE.  Adds one event record per kernel. */
moe_status moe_layer_events(const moe_dims *dims, const moe_weights *weights /* host */,
                            const uint16_t *x, void *out, int32_t *topk_idx_out, float *topk_w_out,
                            int32_t *counts_out, void *ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t *events /* host */, int32_t n_events);

/* Decode attention of a full-attention layer with grouped-query KV sharing:
 * the layer next to the MoE block in the same decode step.  The model's
 * full-attention layers have 16 query heads over 2 KV heads (aimanavo.com
 * page, section "Qwen3.6's 256 experts and two layer types make the MLX-Lily
 * gap"), and the decode kernel packs the query heads of a KV head so that each
 * K and V row is read once for all of them (aimanavo.com page, section "Lily
 * does not treat prefill and decode as the same job"; dzen.guru page, section
 * "Where does the speed-up come from?").  The formula is not on the pages; the
 * plain one is computed.  For sequence b with n = seq_len[b] cached rows
 * (clamped to [0, max_seq]) and query head h, whose KV head is
 * g = h / (n_q_heads / n_kv_heads):
 *     s_j = scale * sum_d q[b][h][d] * k_cache[b][g][j][d]       (j < n)
 *     out[b][h][d] = sum_j softmax(s)_j * v_cache[b][g][j][d]
 * float32 accumulation of exact bf16 products; the probabilities enter the
 * second product rounded to bf16, and the normaliser sums those rounded values,
 * so |error| <= 2^-8 * max_j |v_j| per element, far less on average.  n == 0
 * gives zeros.  Rows j >= n are never read.
 * Host struct; limits (MOE_ERR_UNSUPPORTED beyond them): head_dim 64, 128 or
 * 256; n_q_heads / n_kv_heads <= 16; B and n_kv_heads <= 65535; max_seq <=
 * 2^24.  n_q_heads a multiple of n_kv_heads, all sizes positive (B >= 0):
 * else MOE_ERR_SHAPE. */
typedef struct {
    int32_t B;          /* sequences, one query token each; 0: nothing to do */
    int32_t n_q_heads;  /* Hq */
    int32_t n_kv_heads; /* Hkv */
    int32_t head_dim;   /* D */
    int32_t max_seq;    /* rows per (sequence, KV head) in the cache */
} moe_gqa_dims;

/* Bytes of device workspace moe_gqa_decode needs (host-only, pure; 0 when the
 * dims are invalid): B * n_kv_heads * ceil(max_seq / R) partials of
 * 128 + 6 * G * head_dim bytes (R = 256 rows, 128 at head_dim 256), rounded
 * up to 256 bytes, then 256 bytes of control words per (sequence, KV head),
 * then 256
 * bytes whose first word is set to nonzero, and stays so, if a device-side
 * wait of a call timed out (that call's output is then invalid).  Zero-fill it
 * once after allocating it; every call leaves it ready for the next, for any
 * dims that fit.  Its own contract, separate from moe_workspace_size's; calls
 * that share one must not overlap in time. */
size_t moe_gqa_workspace_size(const moe_gqa_dims *dims /* host */);

/* q [B][Hq][D] bf16; k_cache, v_cache [B][Hkv][max_seq][D] bf16 (16-byte
 * aligned, each head's rows contiguous); seq_len [B] int32 (4-byte aligned);
 * out [B][Hq][D] float32; scale finite (1/sqrt(D) is the usual one; NaN or
 * infinite: MOE_ERR_SHAPE); ws of moe_gqa_workspace_size bytes, 256-byte
 * aligned (MOE_ERR_WORKSPACE when smaller).  One kernel on `stream` when the
 * device holds all B * n_kv_heads * ceil(max_seq / R) of its workgroups at
 * once (they then wait on each other to merge their partials: launch nothing
 * else on the device concurrently), two kernels otherwise. */
moe_status moe_gqa_decode(const moe_gqa_dims *dims /* host */, const uint16_t *q, const uint16_t *k_cache,
                          const uint16_t *v_cache, const int32_t *seq_len, float scale, float *out, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* Number of kernels a moe_gqa_decode call with these dims launches on the
 * current device: 1 when all its workgroups fit on the device at once (the
 * merge of the partials then runs in the same launch), else 2; 0 when the dims
 * are invalid or B == 0 (host-only). */
int32_t moe_gqa_decode_kernels(const moe_gqa_dims *dims /* host */);

/* moe_gqa_decode plus HIP events, for instrumentation: events[0] is recorded
 * on `stream` before its first kernel (the per-run partials), events[1] after
 * it and events[2] after the merge (with the merge in the same kernel,
 * events[1] and events[2] both follow that kernel).
 * events NULL: MOE_ERR_NULL; n_events < 3: MOE_ERR_SHAPE.  B == 0 records
 * nothing. */
moe_status moe_gqa_decode_events(const moe_gqa_dims *dims /* host */, const uint16_t *q, const uint16_t *k_cache,
                                 const uint16_t *v_cache, const int32_t *seq_len, float scale, float *out, void *ws,
                                 size_t ws_bytes, hipStream_t stream, hipEvent_t *events /* host */,
                                 int32_t n_events);

/* Number of kernels moe_layer launches for these dims (host-only, pure; 0 when
 * the dims are invalid or T == 0). */
int32_t moe_layer_stage_count(const moe_dims *dims /* host */);

/* Static name of kernel i (0-based) of moe_layer for these dims, or NULL. */
const char *moe_layer_stage_name(const moe_dims *dims /* host */, int32_t i);

/* Static English text for a status code (host): the refusal message of the
 * fail-early validation (news.mantis.guru page, section "Rust drives the
 * model, Metal does the compute"). */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* BITMOE_MOE_H */
