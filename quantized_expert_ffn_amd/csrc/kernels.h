// Internal launchers of the libmoe kernels. Each enqueues on `st` and returns
// the launch status; shapes are validated by the callers in abi.hip.
#pragma once

#include "common.h"

namespace moe {

hipError_t launch_quantize_weights(const float* w, int64_t rows, int cols, int bits, void* q, float* s,
                                   hipStream_t st);
hipError_t launch_quantize_q8_0(const float* x, int64_t rows, int cols, int8_t* q, float* d, hipStream_t st);

hipError_t launch_router(const float* x, int T, int d, const float* wg, const moe_router_params& p, float* logits,
                         int* idx, float* w, hipStream_t st);

size_t dispatch_lds_bytes(int E);
hipError_t launch_dispatch(const int* idx, int T, int k, int E, int* counts, int* offsets, int* perm,
                           int* inv_perm, int has_shared, int* row_token, int* slots, int* tiles, int* meta,
                           hipStream_t st);
hipError_t launch_plan(const int* counts, const int* offsets, const int* perm, int T, int k, int E, int has_shared,
                       int* row_token, int* slots, int* tiles, int* meta, hipStream_t st);

// Decode path (fp32 activations). prep writes the activations of every
// permuted row as exact f16 hi/lo parts + a power of two per (16-row tile of
// a slot, 32-group);
// the GEMV runs gate/up (x parts -> H parts) or down (H parts -> Y fp32).
hipError_t launch_prep_act(int fmt, const float* x, const int* row_token, const int* slots, const int* meta,
                           int max_slots, int R, int K, _Float16* ahi, _Float16* alo, float* apow, hipStream_t st);
hipError_t launch_gemv(const moe_experts& routed, const moe_experts* shared, bool gateup, const _Float16* ahi,
                       const _Float16* alo, const float* apow, int R, const int* slots, const int* meta, int max_slots,
                       _Float16* hhi, _Float16* hlo, float* hpow, float* y, hipStream_t st,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_q8_mfma(const moe_experts& routed, const moe_experts* shared, bool gateup, const int8_t* a_q,
                          const float* a_s, const int* row_token, const int* tiles, const int* meta, int max_tiles,
                          int8_t* hq, float* hd, float* y, int32_t* dbg0, int32_t* dbg1, hipStream_t st,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_combine(const float* y, const float* w, const int* inv_perm, const float* shared_y, int T, int k,
                          int d, float* out, hipStream_t st);

}  // namespace moe
