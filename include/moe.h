/*
 * moe.h - C ABI of libmoe: the routed Mixture-of-Experts FFN layer with
 * group-quantised experts, on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (the pages, cited by title and section):
 *   - "I ran a 7B Mixture-of-Experts LLM in a language I built" (dev.to),
 *     section "Mixture-of-Experts": each token runs only its top-k experts
 *     (OLMoE: top 8 of 64 per layer), chosen by a softmax router.
 *   - "Show HN: Getting GLM-5.2 running on my slow computer" (note.crab.center),
 *     section "What's implemented": a sigmoid router of the DeepSeek-V3 kind
 *     (noaux_tc selection, a routed scaling factor) and a shared expert; int8
 *     and packed int4 weights dequantised on use; batches take integer dot
 *     products on int8 activations quantised the Q8_0 way, while a single
 *     row keeps f32 activations; batch-union MoE, where a batch loads every
 *     expert it selects one time, for all of the positions that chose it.
 *   - "mtlm-7m-base" (huggingface.co), section "Files": int8 weights with a
 *     scale per group of 32; "What is and is not machin": SwiGLU with SiLU.
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are HIP device memory owned by the caller; the
 *     library allocates nothing, keeps no state between calls and never
 *     frees caller memory. Host pointers (the parameter structs) are read
 *     during the call only.
 *   - Every call enqueues work on `stream` (NULL = the null stream) and
 *     returns without waiting for the GPU. Calls on one stream run in order.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid or unsupported argument returns an error and enqueues nothing
 *     (no silent fallback). A failed launch returns MOE_ERR_HIP.
 *     moe_last_error_detail() gives a text for the last error of the
 *     calling thread.
 *   - T = 0 tokens is a valid no-op.
 *   - Activations and outputs are row-major and contiguous. d = d_model,
 *     I = d_ff, E = routed experts, k = top_k, G_d = d / 32, G_I = I / 32.
 *   - Weight formats (symmetric): MOE_W_INT8_G32 stores int8 codes in
 *     [-127, 127]; MOE_W_INT4_G32 stores codes in [-7, 7] as 4-bit two's
 *     complement, eight to a little-endian dword, the lower k in the lower
 *     nibble; MOE_W_INT2_G32 stores codes in [-1, 1] as 2-bit two's
 *     complement, eight to a little-endian 16-bit word, the lower k in the
 *     lower bits. All carry one fp32 scale per group of 32 along each
 *     matrix's input axis, and a group's weights are scale * code.
 *     MOE_W_INT8_ROW, MOE_W_INT4_ROW and MOE_W_INT2_ROW store the same codes
 *     in the same layout with one fp32 scale per matrix row (output) instead
 *     ("Show HN: Getting GLM-5.2 running on my slow computer", section
 *     "What's implemented": packed int2, per-row scales), row n's weights
 *     being scale[n] * code; their scales are N floats per matrix in row
 *     order. The int2 formats need K % 128 == 0.
 *   - Weight layout ("lane-tiled"; written by moe_quantize_weights, read by
 *     every expert kernel). A matrix of N rows (outputs) and K columns
 *     (inputs), N % 32 == 0, K % 64 == 0, is cut into NT = N/32 tiles of 32
 *     rows, tile t holding rows 32t .. 32t+31. Inside a tile, "lane"
 *     l = nl + 16h (0 <= nl < 16, 0 <= h < 4) owns, for each group g, the
 *     codes of k = 32g + 8h .. 32g + 8h + 7 of rows 32t + nl and
 *     32t + 16 + nl. With G = K/32, P = K/64 and r = row % 32:
 *       int8 codes   byte ((g*NT + t)*64 + l)*16 + 8*(r >= 16) + (k % 8)
 *                    (K*N bytes in all);
 *       int4 codes   dword ((g/2*NT + t)*64 + l)*4 + 2*(g % 2) + (r >= 16),
 *                    nibble k % 8 (K*N/2 bytes in all);
 *       int2 codes   16-bit word ((g/4*NT + t)*64 + l)*8 + 2*(g % 4) + (r >= 16),
 *                    bits 2*(k % 8), +1 (K*N/4 bytes in all);
 *       scales fp32  float (t*P + g/2)*64 + 4*nl + 2*(g % 2) + (r >= 16)
 *                    (K*N/32 floats in all; per-row formats: float n of
 *                    row n, N floats in all).
 *     Codes are group-major, so the waves that stream the tiles of a matrix
 *     side by side read neighbouring kilobytes; scales are tile-major, so one
 *     16-byte load per lane brings a wave the scales of four group pairs. A
 *     wave reads 1 KB of operands per 16-byte load.
 *   - Results are deterministic: the same inputs give bitwise equal outputs
 *     (no floating-point atomics anywhere).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shapes */
    MOE_ERR_UNSUPPORTED = -2,   /* a valid request the library does not support */
    MOE_ERR_WORKSPACE = -3,     /* workspace missing or smaller than moe_workspace_size() */
    MOE_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} moe_status;

typedef enum {
    MOE_ROUTER_SOFTMAX_TOPK = 0,     /* softmax over logits, top-k by logit */
    MOE_ROUTER_SIGMOID_NOAUX_TC = 1  /* sigmoid, group-limited top-k on sigmoid + bias */
} moe_router_mode;

typedef enum {
    MOE_W_INT8_G32 = 0,   /* int8 codes, fp32 scale per group of 32 */
    MOE_W_INT4_G32 = 1,   /* packed int4 codes, fp32 scale per group of 32 */
    MOE_W_INT8_ROW = 2,   /* int8 codes, fp32 scale per matrix row */
    MOE_W_INT4_ROW = 3,   /* packed int4 codes, fp32 scale per matrix row */
    MOE_W_INT2_G32 = 4,   /* packed int2 codes, fp32 scale per group of 32 */
    MOE_W_INT2_ROW = 5    /* packed int2 codes, fp32 scale per matrix row */
} moe_weight_format;

typedef enum {
    MOE_ACT_F32 = 0,   /* fp32 activations x dequantised weights (decode GEMV path) */
    MOE_ACT_Q8_0 = 1   /* Q8_0 int8 activations, exact integer dots on the matrix cores (prefill / verify path) */
} moe_act_mode;

/* Timed stages of moe_layer_forward_timed. */
typedef enum {
    MOE_STAGE_ROUTE = 0,     /* router logits + hidden-state preparation (Q8_0 codes or f32 parts), one
                                launch; T > 16: + top-k */
    MOE_STAGE_DISPATCH = 1,  /* (T <= 16: top-k +) counts, offsets, permutation, work lists */
    MOE_STAGE_QUANT_X = 2,   /* not recorded by the layer calls (their router launch prepares the hidden
                                states): its two events are left untouched */
    MOE_STAGE_GATEUP = 3,    /* gate and up projections + SwiGLU (all experts) */
    MOE_STAGE_DOWN = 4,      /* down projections (all experts) */
    MOE_STAGE_COMBINE = 5,   /* weighted gather-sum + shared expert */
    MOE_STAGE_COUNT = 6
} moe_stage;

/* Router parameters.
 *   n_experts   E, 1 <= E <= 1024.
 *   top_k       k, 1 <= k <= E.
 *   mode        moe_router_mode.
 *   renormalize softmax mode: nonzero divides the selected probabilities by
 *               their sum; zero keeps the plain softmax probabilities.
 *               Ignored by noaux_tc (which always normalises).
 *   n_group, topk_group   noaux_tc: E splits into n_group contiguous groups
 *               (E % n_group == 0, n_group <= 64); only the topk_group groups
 *               with the largest sum of their two best scores stay eligible.
 *               k <= topk_group * E / n_group. Ignored by softmax mode.
 *   routed_scaling_factor noaux_tc: multiplies the normalised weights.
 *   score_bias  noaux_tc: device fp32 [E] added to the sigmoid scores for
 *               selection only (NULL = zero). Ignored by softmax mode.
 *   top_p       adaptive expert top-p ("Show HN: Getting GLM-5.2 running on
 *               my slow computer", section "Useful knobs"), both modes. With S
 *               the sum of a token's k weights, slot j is kept when j == 0 or
 *               the weights of slots 0 .. j-1 sum to less than top_p * S; the
 *               kept weights are rescaled to sum to S, and a dropped slot
 *               gets expert -1 and weight 0 (dropped slots are always the
 *               last ones). 0, or any value >= 1, keeps all k slots; a
 *               negative or NaN value is MOE_ERR_INVALID_ARG. The keep
 *               decisions are taken in fp32.
 *   shared_gate device fp32 [d], or NULL: gates the shared expert. When a
 *               shared expert is passed to moe_layer_forward(_timed) or
 *               moe_block_forward, its output for token t is multiplied by
 *               sigmoid(x[t] . shared_gate), x[t] being the layer's input row
 *               (after the RMSNorm of moe_block_forward), the dot taken in
 *               fp32. The pages name no such gate; it is an option for model
 *               families that have one (off when NULL). Ignored without a
 *               shared expert, and by moe_route.
 */
typedef struct {
    int32_t n_experts;
    int32_t top_k;
    int32_t mode;
    int32_t renormalize;
    int32_t n_group;
    int32_t topk_group;
    float routed_scaling_factor;
    const float* score_bias;
    float top_p;
    const float* shared_gate;
} moe_router_params;

/* A stack of n_experts quantised SwiGLU experts (device pointers), each
 * matrix in the lane-tiled layout above, experts back to back:
 *   gate_q, up_q : per expert an [I x d] matrix: I*d bytes (int8), I*d/2 (int4) or I*d/4 (int2)
 *   gate_s, up_s : per expert I*d/32 fp32 (per-row formats: I fp32)
 *   down_q       : per expert a [d x I] matrix: d*I bytes (int8), d*I/2 (int4) or d*I/4 (int2)
 *   down_s       : per expert d*I/32 fp32 (per-row formats: d fp32)
 * Expert e computes  y = (silu(x Wg^T) * (x Wu^T)) Wd^T  with W = scale*code.
 * d % 64 == 0 and I % 64 == 0 are required, d % 128 == 0 and I % 128 == 0
 * for the int2 formats (MOE_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
    int32_t n_experts;
    int32_t d_model;
    int32_t d_ff;
    int32_t format;       /* moe_weight_format */
    const void* gate_q;
    const float* gate_s;
    const void* up_q;
    const float* up_s;
    const void* down_q;
    const float* down_s;
} moe_experts;

/* Bytes of device workspace the calls below need for this problem size.
 * has_shared: nonzero when a shared expert is passed to moe_layer_forward.
 * The same size serves moe_route, moe_dispatch, moe_expert_ffn and
 * moe_layer_forward for the same (T, k, E, d, I, act_mode, has_shared).
 * Returns 0 for invalid sizes. Any 256-byte-aligned device buffer works.
 */
size_t moe_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d, int32_t d_ff,
                          int32_t act_mode, int32_t has_shared);

/* Symmetric weight quantiser ("mtlm-7m-base", section "Files": group 32;
 * "Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": int8 / packed int4,
 * per-row scales).
 *   w      device fp32 [rows, cols] row-major, cols % 64 == 0: a stack of
 *          rows / matrix_rows matrices of matrix_rows rows each
 *          (matrix_rows % 32 == 0, rows % matrix_rows == 0), each written
 *          in the layout above, one after the other
 *   format MOE_W_INT8_G32 / MOE_W_INT8_ROW -> q holds rows*cols bytes;
 *          MOE_W_INT4_G32 / MOE_W_INT4_ROW -> q holds rows*cols/2 bytes;
 *          MOE_W_INT2_G32 / MOE_W_INT2_ROW -> q holds rows*cols/4 bytes
 *          (cols % 128 == 0)
 *   s      device fp32: rows*cols/32 floats (group formats) or rows floats
 *          (per-row formats, s[i] the scale of row i of w)
 *   q and s are written in the lane-tiled layout described at the top.
 * Per group (per row for the per-row formats): s = amax/qmax (qmax 127, 7
 * or 1, fp32 divide), code = clamp(round_half_even(w/s), -qmax, qmax) (fp32
 * divide); amax == 0 gives s = 0 and codes 0.
 */
moe_status moe_quantize_weights(const float* w, int64_t rows, int32_t cols, int32_t matrix_rows,
                                int32_t format, void* q, float* s, hipStream_t stream);

/* Q8_0-style activation quantiser ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
 * implemented": Q8_0-style int8 activations).
 *   x [rows, cols] device fp32, cols % 32 == 0 -> q int8 [rows, cols],
 *   d fp32 [rows, cols/32]. Per group, in fp32: d = amax/127,
 *   inv = (d == 0) ? 0 : 1/d, q = clamp(round_half_even(x*inv), -127, 127).
 */
moe_status moe_quantize_q8_0(const float* x, int64_t rows, int32_t cols,
                             int8_t* q, float* d, hipStream_t stream);

/* Router ("I ran a 7B Mixture-of-Experts LLM...", section
 * "Mixture-of-Experts": softmax top-k; "Show HN: Getting GLM-5.2 running on my slow computer", section "What's
 * implemented": sigmoid noaux_tc with routed_scaling_factor).
 *   x        device fp32 [T, d];  gate_w device fp32 [E, d]
 *   topk_idx device int32 [T, k]: selected experts, larger selection key
 *            first (logit in softmax mode, sigmoid + bias in noaux_tc mode),
 *            equal keys to the lower expert id.
 *   topk_w   device fp32 [T, k]: the weight of each selected expert.
 *            With top_p, dropped slots hold -1 and 0.
 *   ws       device workspace, 16-byte aligned: moe_workspace_size with this
 *            T, k, E and d (d rounded up to a multiple of 32 where it is not
 *            one) is enough. It holds the logits' slice sums first, then for
 *            T > 16 the f16 operand parts of the matrix-core router.
 * Logits are fp32 on the GPU; a selection whose margin lies within fp32
 * rounding of the logits may differ from an exact-arithmetic ranking.
 */
moe_status moe_route(const float* x, int32_t T, int32_t d, const float* gate_w,
                     const moe_router_params* p, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch for batch-union ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
 * implemented": each distinct expert is read once for all of its positions).
 *   topk_idx device int32 [T, k], values in [0, E), or -1 for a slot
 *            dropped by top_p.
 *   counts   device int32 [E]      assignments per expert
 *   offsets  device int32 [E + 1]  exclusive prefix sum of counts
 *   perm     device int32 [T*k]    flat assignments f = t*k + j, stably
 *                                  sorted by expert (so by f within one);
 *                                  entries past offsets[E] are -1
 *   inv_perm device int32 [T*k]    inv_perm[perm[p]] = p; -1 for a slot
 *                                  that is not dispatched
 * A -1 entry is a dropped slot (not counted). Other entries outside [0, E)
 * are skipped the same way; they never cause an out-of-bounds access.
 *   ws, ws_bytes  optional scratch (device, 16-byte aligned, or NULL): with
 *            T*k > 2048 and at least moe_workspace_size(T, k, E, 64, 64,
 *            MOE_ACT_Q8_0, 0) bytes the dispatch spreads over many blocks;
 *            otherwise it runs in one block. The result is the same.
 */
moe_status moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* Batch-union expert FFN: every expert with rows runs once over all of them.
 *   x       device fp32 [T, d]
 *   ex      the routed experts (ex->n_experts = E, ex->d_model = d)
 *   counts, offsets, perm   as produced by moe_dispatch for (T, k, E)
 *   act_mode MOE_ACT_F32: fp32 activations times dequantised weights, fp32
 *            accumulation. MOE_ACT_Q8_0: x is Q8_0-quantised per token, each
 *            32-group gives an exact integer dot (int8 x int8 or int4 codes,
 *            summed exactly on the matrix cores),
 *            rescaled by both group scales; H = silu(G)*U is Q8_0-quantised
 *            again before the down projection.
 *   y_perm  device fp32 [T*k, d]: row p is expert e's output for token
 *           perm[p] / k, un-weighted, in permuted order.
 */
moe_status moe_expert_ffn(const float* x, int32_t T, int32_t k, const moe_experts* ex,
                          const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          int32_t act_mode, float* y_perm, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Combine: out[t] = sum_{j<k} topk_w[t, j] * y_perm[inv_perm[t*k + j]] + shared_y[t],
 * summed in slot order j = 0..k-1, then the shared term; no atomics.
 *   y_perm device fp32 [T*k, d]; topk_w device fp32 [T, k];
 *   inv_perm device int32 [T*k]; shared_y device fp32 [T, d] or NULL;
 *   out device fp32 [T, d].
 * A gated shared expert is the caller's to scale here: pass shared_y
 * already multiplied by its gate.
 */
moe_status moe_combine(const float* y_perm, const float* topk_w, const int32_t* inv_perm,
                       const float* shared_y, int32_t T, int32_t k, int32_t d, float* out,
                       hipStream_t stream);

/* The whole layer: route -> dispatch -> batch-union experts -> combine.
 *   x      device fp32 [T, d];  gate_w device fp32 [E, d]
 *   routed E routed experts; shared NULL or one expert (n_experts == 1) of
 *          the same d, format and d_ff, applied to every token with weight 1
 *          ("Show HN: Getting GLM-5.2 running on my slow computer": shared expert).
 *   out    device fp32 [T, d]
 *   ws     device workspace of moe_workspace_size(T, k, E, d, d_ff,
 *          act_mode, shared != NULL) bytes.
 */
moe_status moe_layer_forward(const float* x, int32_t T, const float* gate_w,
                             const moe_router_params* p, const moe_experts* routed,
                             const moe_experts* shared, int32_t act_mode, float* out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine): its scratch is an
 * array of MOE_NOALLOC_SCRATCH_BYTES bytes in the library's device code, one
 * per GPU, held from the library's load until the process ends; the first
 * call on a device looks up that device's copy.
 *   Everything else as moe_layer_forward (the caller still passes x, the
 *   weights and out).
 *   A call whose moe_workspace_size(T, k, E, d, d_ff, act_mode, shared !=
 *   NULL) exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_UNSUPPORTED
 *   before anything is enqueued (decode and verification batches fit; large
 *   prefills need moe_layer_forward and a workspace).
 *   Every call on one GPU shares that GPU's array: calls that can overlap on
 *   one GPU (several streams, or several host threads) race and must be
 *   serialised by the caller. Calls on one stream run in order. Nothing in
 *   the array needs to start at any value (every kernel writes what it
 *   reads), so the contents a previous call left are harmless.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_forward_noalloc(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                                     const moe_experts* routed, const moe_experts* shared, int32_t act_mode,
                                     float* out, hipStream_t stream);

/* moe_layer_forward that also records stage_events[2*s] before and
 * stage_events[2*s+1] after stage s (moe_stage) on `stream`. stage_events
 * is a host array of 2*MOE_STAGE_COUNT hipEvent_t created by the caller;
 * NULL entries are skipped. Stages that do not run are not recorded.
 * The gate/up and down stages are one kernel each: their two events (both
 * must be given) are attached to that kernel's dispatch (hipExtLaunchKernel),
 * so the interval is the kernel's own execution time. The other stages are
 * bracketed by event records.
 */
moe_status moe_layer_forward_timed(const float* x, int32_t T, const float* gate_w,
                                   const moe_router_params* p, const moe_experts* routed,
                                   const moe_experts* shared, int32_t act_mode, float* out,
                                   void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                                   hipStream_t stream);

/* The layer between its neighbours in a transformer block:
 *   out = x + moe_layer_forward(RMSNorm(x))
 * with RMSNorm(x)[t] = x[t] / sqrt(mean_c(x[t][c]^2) + eps) * norm_w, the
 * normalisation the layer's input has been through ("mtlm-7m-base",
 * section "What is and is not machin": RMSNorm, SwiGLU) and the residual
 * connection around it.
 *   x        device fp32 [T, d], the block's hidden states before the norm.
 *   norm_w   device fp32 [d], the norm's gain; NULL skips the normalisation
 *            (out = x + layer(x)).
 *   eps      finite, >= 0.
 *   out      device fp32 [T, d]; may be the same buffer as x (each element
 *            of x is read before the same element of out is written).
 *   stage_events  as moe_layer_forward_timed, or NULL. The normalisation is
 *            part of the route stage.
 * Up to 16 tokens the normalisation happens inside the router's logits
 * kernel (no extra pass over x); above that, once into the workspace.
 * Everything else as moe_layer_forward (same workspace size).
 */
moe_status moe_block_forward(const float* x, int32_t T, const float* norm_w, float eps,
                             const float* gate_w, const moe_router_params* p,
                             const moe_experts* routed, const moe_experts* shared,
                             int32_t act_mode, float* out, void* ws, size_t ws_bytes,
                             const hipEvent_t* stage_events, hipStream_t stream);

/* Test hook for the Q8_0 path: runs the kernels moe_expert_ffn(act_mode =
 * MOE_ACT_Q8_0) runs for the same T (the small-batch GEMV up to 16 tokens,
 * the tiled matrix-core GEMM above that) and also writes their exact int32
 * per-group dots and the Q8_0 codes of H. With R = T*k rows in permuted
 * order:
 *   dots_gate, dots_up  device int32 [R, I, d/32]  sum over a 32-group of
 *                       xq * wq for gate and up
 *   hq, hd              device int8 [R, I], fp32 [R, I/32]  Q8_0 of H
 *   dots_down           device int32 [R, d, I/32]  sum over a 32-group of
 *                       hq * wq for down
 *   y_perm              device fp32 [R, d] as moe_expert_ffn
 * Meant for small shapes; the dot arrays grow as R * I * d / 32.
 */
moe_status moe_debug_q8_expert_ffn(const float* x, int32_t T, int32_t k, const moe_experts* ex,
                                   const int32_t* counts, const int32_t* offsets,
                                   const int32_t* perm, int32_t* dots_gate, int32_t* dots_up,
                                   int8_t* hq, float* hd, int32_t* dots_down, float* y_perm,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Test hook: where moe_layer_forward, moe_layer_forward_timed and
 * moe_block_forward leave their intermediate results inside the workspace
 * (a buffer of moe_workspace_size(T, k, E, d, d_ff, act_mode, has_shared)
 * bytes), so that a test can read them back after the call. offsets_out
 * (host, MOE_WS_SECTION_COUNT entries) receives byte offsets from the start
 * of the workspace:
 *   MOE_WS_TOPK_IDX   int32 [T, k]    the router's selection (as moe_route)
 *   MOE_WS_TOPK_W     fp32  [T, k]    its weights
 *   MOE_WS_COUNTS     int32 [E]       as moe_dispatch
 *   MOE_WS_OFFSETS    int32 [E + 1]
 *   MOE_WS_PERM       int32 [T*k]
 *   MOE_WS_INV_PERM   int32 [T*k]
 *   MOE_WS_H_CODES    Q8_0 mode: H's codes as fp16 [R, d_ff] (R = T*k, plus T
 *                     rows of the shared expert after them), row p of the
 *                     permuted order; inside each 8-wide slice of a row the
 *                     codes sit in the operand order of the weight format (for
 *                     int8: k offsets 0, 2, 1, 3, 4, 6, 5, 7; int4: 0, 4, 1, 5,
 *                     2, 6, 3, 7; int2: 0 .. 7). -1 in F32 mode.
 *   MOE_WS_H_SCALES   Q8_0 mode: fp32 [R, d_ff/32], H's Q8_0 scales. -1 in
 *                     F32 mode.
 * Returns MOE_ERR_INVALID_ARG for sizes moe_workspace_size rejects.
 */
typedef enum {
    MOE_WS_TOPK_IDX = 0,
    MOE_WS_TOPK_W = 1,
    MOE_WS_COUNTS = 2,
    MOE_WS_OFFSETS = 3,
    MOE_WS_PERM = 4,
    MOE_WS_INV_PERM = 5,
    MOE_WS_H_CODES = 6,
    MOE_WS_H_SCALES = 7,
    MOE_WS_SECTION_COUNT = 8
} moe_ws_section;

moe_status moe_debug_workspace_sections(int32_t T, int32_t k, int32_t E, int32_t d, int32_t d_ff, int32_t act_mode,
                                        int32_t has_shared, int64_t* offsets_out);

/* Static text for a status code. */
const char* moe_status_string(moe_status st);

/* Detail text for the last error returned to the calling thread ("" if none). */
const char* moe_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
