// Internal launchers of the libmoe kernels. Each enqueues on `st` and returns
// the launch status; shapes are validated by the callers in abi.hip.
#pragma once

#include "common.h"

namespace moe {

hipError_t launch_quantize_weights(const float* w, int64_t rows, int cols, int matrix_rows, int format, void* q,
                                   float* s, hipStream_t st);
hipError_t launch_quantize_q8_0(const float* x, int64_t rows, int cols, int8_t* q, float* d, hipStream_t st);

// Hidden-state preparation for the expert kernels, done inside the router's
// logits launch (or, for moe_expert_ffn, by a kernel of its own).
enum { XPREP_NONE = 0, XPREP_SPLIT = 1, XPREP_Q8_0 = 2 };
struct XPrep {
    int mode = XPREP_NONE;
    int fmt = MOE_W_INT8_G32;      // the weight format (operand-slot order of the f16 outputs)
    _Float16* hi = nullptr;        // XPREP_SPLIT: [T, d] f16 parts and one power of
    _Float16* lo = nullptr;        //   two per 32-group over all rows, [d/32]
    float* pow = nullptr;
    _Float16* q = nullptr;         // XPREP_Q8_0: [T, d] codes as f16 in slot order, [T, d/32] scales
    float* qd = nullptr;
    // RMSNorm applied on the way in (the small-T router kernel only): the
    // prepared value of x[t][c] is x[t][c] * gamma[c] * inv_rms[t]
    const float* gamma = nullptr;  // [d] or null (no normalisation)
    const float* inv_rms = nullptr;
};

// rp: the operand parts' memory (router_parts_at) when router_splits(T, E, d)
// > 0, else unused (may be null)
hipError_t launch_router(const float* x, int T, int d, const float* wg, const moe_router_params& p, float* logits,
                         const RouterParts* rp, int* idx, float* w, hipStream_t st);
// The logits launches also do xp: waves of the small-T kernels, or the
// operand preparation kernel of larger T (router_splits(T, E, d) > 0, which
// needs rp). norm_w (router_splits(T, E, d) == 0 only, else null): the
// logits and xp see RMSNorm(x) with gain norm_w and eps.
// The logits leave as S = router_slices(T, E, d, norm_w != null) slice sums
// [S, T, E]; sg (or null): the shared-expert gate vector, whose logit x . sg
// goes to sgl as slice sums [S, T].
hipError_t launch_router_logits(const float* x, int T, int d, const float* wg, int E, float* logits,
                                const XPrep& xp, const float* norm_w, float eps, const float* sg, float* sgl,
                                const RouterParts* rp, hipStream_t st);
// RMSNorm of T rows into xn [T, d] (the larger-T path)
hipError_t launch_rmsnorm(const float* x, int T, int d, const float* norm_w, float eps, float* xn, hipStream_t st);
hipError_t launch_router_topk(const float* logits, int T, int S, const moe_router_params& p, int* idx, float* w,
                              hipStream_t st);
hipError_t launch_xprep(const float* x, int T, int d, const XPrep& xp, hipStream_t st);

// Top-k and dispatch in one block for small batches (T <= kFusedRouteT):
// routing results never leave LDS between the two.
constexpr int kFusedRouteT = 16;
size_t route_dispatch_lds_bytes(int T, int k, int E, int mode);
hipError_t launch_route_dispatch(const float* logits, int T, int S, const moe_router_params& p, int* idx, float* w,
                                 int* counts, int* offsets, int* perm, int* inv_perm, int has_shared,
                                 int* row_token, int* slots, int* tiles, int* meta, hipStream_t st);

size_t dispatch_lds_bytes(int E);
// chunks of the multi-block dispatch for n assignments (its scratch: a
// histogram [chunks, E] and a flag per chunk, ints)
int dispatch_chunks(int64_t n);
// chunk_hist / chunk_bad null: the single-block dispatch for any size
hipError_t launch_dispatch(const int* idx, int T, int k, int E, int* counts, int* offsets, int* perm,
                           int* inv_perm, int has_shared, int* row_token, int* slots, int* tiles, int* meta,
                           int* chunk_hist, int* chunk_bad, hipStream_t st);
hipError_t launch_plan(const int* counts, const int* offsets, const int* perm, int T, int k, int E, int has_shared,
                       int* row_token, int* slots, int* tiles, int* meta, hipStream_t st);

// Decode path (fp32 activations). gate/up: A = the token rows' f16 parts
// [T, d] (read through row_token) with one power of two per 32-group, [d/32];
// it writes H's parts [R, I] with one power of two per (row, 32-group),
// [R, I/32]. down: A = H's parts -> Y fp32 [R, d].
// q8 (small-batch Q8_0 path): A = Q8_0 codes as f16 in slot order with
// per-row scales in apow ([rows, K/32]); gate/up writes H's Q8_0 codes to hhi
// and its per-row scales to hpow; alo and hlo are unused. Every slot must
// hold at most 16 rows for the weights to be read once (T <= 16). The dbg
// pointers (q8 only; all or none) receive the exact group dots, [R, N, K/32]
// (gate/up: gate to dbg0, up to dbg1; down: dbg0), and H's int8 codes in
// natural order [R, N] (gate/up).
constexpr int kGemvMaxT = 16;   // the Q8_0 path takes the GEMV up to this many tokens
hipError_t launch_gemv(const moe_experts& routed, const moe_experts* shared, bool gateup, bool q8, const _Float16* ahi,
                       const _Float16* alo, const float* apow, const int* row_token, int a_rows, int R,
                       const int* slots, const int* meta, int max_slots, _Float16* hhi, _Float16* hlo, float* hpow,
                       float* y, hipStream_t st, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                       int32_t* dbg0 = nullptr, int32_t* dbg1 = nullptr, int8_t* dbg_hq = nullptr);

// Prefill path (Q8_0 activations). gate/up: A = the token rows' Q8_0 codes
// as f16 in slot order [a_rows = T, d] (read through row_token) + scales
// [T, d/32]; it writes H's Q8_0 codes the same way, [R, I] + [R, I/32].
// down: A = those (a_rows = R) -> Y fp32 [R, d]. The dbg pointers (all or
// none) receive the exact group dots and H's int8 codes in natural order.
hipError_t launch_q8_mfma(const moe_experts& routed, const moe_experts* shared, bool gateup, const _Float16* a_q,
                          const float* a_s, int a_rows, const int* row_token, const int* tiles, const int* meta,
                          int max_tiles, _Float16* hq, float* hd, float* y, int32_t* dbg0, int32_t* dbg1,
                          int8_t* dbg_hq,
                          hipStream_t st, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// residual: [T, d] added last, or null
hipError_t launch_combine(const float* y, const float* w, const int* inv_perm, const float* shared_y,
                          const float* sgl, int sgl_slices, const float* residual, int T, int k, int d, float* out,
                          hipStream_t st);

}  // namespace moe
