// The C ABI of libmoe (declared in include/moe.h): argument validation,
// workspace carving and kernel sequencing. Every check runs on the host
// before anything is enqueued, so a rejected call leaves the stream untouched
// ("Show HN: Getting GLM-5.2 running on my slow computer", section "OpenAI-compatible API": a request the
// server cannot honour gets an error back; section "Experimental resident
// CUDA backend": a path that cannot run reports it, with no quiet fallback).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"

// The scratch of moe_layer_forward_noalloc: one array per GPU, part of the
// library's device code object, so it exists on every device the library is
// loaded on and lives until the process ends. Host code never uses this name
// as an address (it is a host-side stand-in there): it asks the runtime for
// the current device's copy (scratch_for_current_device).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_detail;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    return st;
}

moe_status ok() {
    g_detail.clear();
    return MOE_OK;
}

moe_status hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_REQUIRE(cond, status, ...) \
    do {                               \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define MOE_HIP(expr, what)                           \
    do {                                              \
        hipError_t _e = (expr);                       \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

moe_status check_router(const moe_router_params* p, int E_expected) {
    MOE_REQUIRE(p != nullptr, MOE_ERR_INVALID_ARG, "router params is NULL");
    const int E = p->n_experts, k = p->top_k;
    MOE_REQUIRE(E >= 1, MOE_ERR_INVALID_ARG, "n_experts = %d must be >= 1", E);
    MOE_REQUIRE(E_expected < 0 || E == E_expected, MOE_ERR_INVALID_ARG,
                "router n_experts %d != experts n_experts %d", E, E_expected);
    MOE_REQUIRE(E <= moe::kMaxExperts, MOE_ERR_UNSUPPORTED, "n_experts = %d > %d", E, moe::kMaxExperts);
    MOE_REQUIRE(k >= 1 && k <= E, MOE_ERR_INVALID_ARG, "top_k = %d outside [1, n_experts = %d]", k, E);
    MOE_REQUIRE(k <= 64, MOE_ERR_UNSUPPORTED, "top_k = %d > 64", k);
    MOE_REQUIRE(p->top_p >= 0.0f, MOE_ERR_INVALID_ARG, "top_p = %g must be >= 0 (0 keeps every slot)",
                (double)p->top_p);   // also rejects NaN
    if (p->mode == MOE_ROUTER_SOFTMAX_TOPK) return MOE_OK;
    MOE_REQUIRE(p->mode == MOE_ROUTER_SIGMOID_NOAUX_TC, MOE_ERR_INVALID_ARG, "unknown router mode %d", p->mode);
    MOE_REQUIRE(p->n_group >= 1, MOE_ERR_INVALID_ARG, "n_group = %d must be >= 1", p->n_group);
    MOE_REQUIRE(p->n_group <= moe::kMaxGroups, MOE_ERR_UNSUPPORTED, "n_group = %d > %d", p->n_group,
                moe::kMaxGroups);
    MOE_REQUIRE(E % p->n_group == 0, MOE_ERR_INVALID_ARG, "n_experts %d not divisible by n_group %d", E,
                p->n_group);
    MOE_REQUIRE(p->topk_group >= 1 && p->topk_group <= p->n_group, MOE_ERR_INVALID_ARG,
                "topk_group = %d outside [1, n_group = %d]", p->topk_group, p->n_group);
    MOE_REQUIRE(k <= p->topk_group * (E / p->n_group), MOE_ERR_INVALID_ARG,
                "top_k = %d exceeds the %d experts of the kept groups", k, p->topk_group * (E / p->n_group));
    MOE_REQUIRE(std::isfinite(p->routed_scaling_factor), MOE_ERR_INVALID_ARG, "routed_scaling_factor not finite");
    return MOE_OK;
}

// T: the call's token count (the GEMV paths bound the reduction length)
moe_status check_experts(const moe_experts* ex, const char* name, int act_mode, int T) {
    MOE_REQUIRE(ex != nullptr, MOE_ERR_INVALID_ARG, "%s experts is NULL", name);
    MOE_REQUIRE(ex->n_experts >= 1, MOE_ERR_INVALID_ARG, "%s n_experts = %d", name, ex->n_experts);
    MOE_REQUIRE(ex->d_model > 0 && ex->d_ff > 0, MOE_ERR_INVALID_ARG, "%s d_model %d / d_ff %d must be > 0", name,
                ex->d_model, ex->d_ff);
    MOE_REQUIRE(ex->d_model % (2 * moe::kGroup) == 0 && ex->d_ff % (2 * moe::kGroup) == 0, MOE_ERR_UNSUPPORTED,
                "%s d_model %d and d_ff %d must be multiples of 64 (pairs of groups)", name, ex->d_model, ex->d_ff);
    MOE_REQUIRE(moe::fmt_valid(ex->format), MOE_ERR_INVALID_ARG, "%s unknown weight format %d", name, ex->format);
    const int km = moe::fmt_k_multiple(ex->format);
    MOE_REQUIRE(ex->d_model % km == 0 && ex->d_ff % km == 0, MOE_ERR_UNSUPPORTED,
                "%s d_model %d and d_ff %d must be multiples of %d for weight format %d", name, ex->d_model,
                ex->d_ff, km, ex->format);
    MOE_REQUIRE(ex->gate_q && ex->gate_s && ex->up_q && ex->up_s && ex->down_q && ex->down_s, MOE_ERR_INVALID_ARG,
                "%s has a NULL weight or scale pointer", name);
    MOE_REQUIRE(aligned16(ex->gate_q) && aligned16(ex->up_q) && aligned16(ex->down_q), MOE_ERR_INVALID_ARG,
                "%s weight codes must be 16-byte aligned", name);
    MOE_REQUIRE(aligned16(ex->gate_s) && aligned16(ex->up_s) && aligned16(ex->down_s), MOE_ERR_INVALID_ARG,
                "%s scales must be 16-byte aligned", name);
    // the decode GEMV (f32 activations, or Q8_0 up to kGemvMaxT tokens) keeps
    // one activation scale per group in LDS: K / 32 <= 256 groups
    if (act_mode == MOE_ACT_F32 || T <= moe::kGemvMaxT)
        MOE_REQUIRE(ex->d_model <= 8192 && ex->d_ff <= 8192, MOE_ERR_UNSUPPORTED,
                    "%s: the f32 path, and the Q8_0 path up to %d tokens, support d_model and d_ff up to 8192", name,
                    moe::kGemvMaxT);
    return MOE_OK;
}

moe_status check_act_mode(int act_mode) {
    MOE_REQUIRE(act_mode == MOE_ACT_F32 || act_mode == MOE_ACT_Q8_0, MOE_ERR_INVALID_ARG, "unknown act_mode %d",
                act_mode);
    return MOE_OK;
}

// The f32 path addresses its activation parts ([R, max(d, I)] f16, R = T*k
// rows plus T for a shared expert) with 32-bit offsets.
// The expert kernels address their f16 activation rows with 32-bit byte
// offsets: R rows of max(d, d_ff) values, 2 bytes each (both modes).
moe_status check_rows(int T, int k, int has_shared, const moe_experts* ex) {
    const int64_t R = (int64_t)T * k + (has_shared ? T : 0);
    const int64_t K = ex->d_model > ex->d_ff ? ex->d_model : ex->d_ff;
    MOE_REQUIRE(R * K * 2 < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
                "up to 2^30 routed activation values (T*k rows of max(d, d_ff)) per call");
    return MOE_OK;
}

template <class T>
T* ws_at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

void record(const hipEvent_t* ev, int idx, hipStream_t st) {
    if (ev && ev[idx]) (void)hipEventRecord(ev[idx], st);
}

hipEvent_t stage_ev(const hipEvent_t* ev, int idx) { return ev ? ev[idx] : nullptr; }

// Where the prepared hidden states go in the workspace (f32 parts or Q8_0).
moe::XPrep xprep_for(int act_mode, int fmt, const moe::WsLayout& L, void* ws) {
    moe::XPrep xp;
    xp.fmt = moe::fmt_codes(fmt);
    if (act_mode == MOE_ACT_F32) {
        xp.mode = moe::XPREP_SPLIT;
        xp.hi = ws_at<_Float16>(ws, L.xq);
        xp.lo = ws_at<_Float16>(ws, L.xd);
        xp.pow = ws_at<float>(ws, L.xp);
    } else {
        xp.mode = moe::XPREP_Q8_0;
        xp.q = ws_at<_Float16>(ws, L.xq);
        xp.qd = ws_at<float>(ws, L.xd);
    }
    return xp;
}

// The expert FFN over a prepared work list (slots / tiles / row_token in ws)
// and prepared hidden states (xprep_for).
moe_status run_experts(int T, int k, const moe_experts& routed, const moe_experts* shared, int act_mode,
                       const moe::WsLayout& L, void* ws, float* y, int32_t* dots_gate, int32_t* dots_up,
                       int8_t* hq_out, float* hd_out, int32_t* dots_down, const hipEvent_t* ev, hipStream_t st) {
    const int E = routed.n_experts;
    const int n = T * k;
    const int has_shared = shared != nullptr;
    const int* row_token = ws_at<int>(ws, L.row_token);
    const int* slots = ws_at<int>(ws, L.slots);
    const int* tiles = ws_at<int>(ws, L.tiles);
    const int* meta = ws_at<int>(ws, L.meta);
    const int max_slots = (E < n ? E : n) + has_shared;
    const int R = n + (has_shared ? T : 0);
    if (act_mode == MOE_ACT_F32) {
        const _Float16* ahi = ws_at<_Float16>(ws, L.xq);
        const _Float16* alo = ws_at<_Float16>(ws, L.xd);
        const float* apow = ws_at<float>(ws, L.xp);
        _Float16* hhi = ws_at<_Float16>(ws, L.h);
        _Float16* hlo = ws_at<_Float16>(ws, L.hd);
        float* hpow = ws_at<float>(ws, L.hp);
        MOE_HIP(moe::launch_gemv(routed, shared, true, false, ahi, alo, apow, row_token, T, R, slots, meta, max_slots,
                                 hhi, hlo, hpow, nullptr, st, stage_ev(ev, 2 * MOE_STAGE_GATEUP),
                                 stage_ev(ev, 2 * MOE_STAGE_GATEUP + 1)),
                "gate/up GEMV");
        MOE_HIP(moe::launch_gemv(routed, shared, false, false, hhi, hlo, hpow, nullptr, R, R, slots, meta, max_slots,
                                 nullptr, nullptr, nullptr, y, st, stage_ev(ev, 2 * MOE_STAGE_DOWN),
                                 stage_ev(ev, 2 * MOE_STAGE_DOWN + 1)),
                "down GEMV");
        return MOE_OK;
    }
    if (T <= moe::kGemvMaxT) {
        // Q8_0 with a handful of tokens (verification): every slot holds at
        // most T <= 16 rows, so the GEMV reads each weight once, with the
        // same exact integer group dots as the tiled kernel (the test hook's
        // dots come from these same kernels)
        _Float16* xq = ws_at<_Float16>(ws, L.xq);
        float* xd = ws_at<float>(ws, L.xd);
        _Float16* hq = ws_at<_Float16>(ws, L.h);
        float* hd = hd_out ? hd_out : ws_at<float>(ws, L.hd);
        MOE_HIP(moe::launch_gemv(routed, shared, true, true, xq, nullptr, xd, row_token, T, R, slots, meta, max_slots,
                                 hq, nullptr, hd, nullptr, st, stage_ev(ev, 2 * MOE_STAGE_GATEUP),
                                 stage_ev(ev, 2 * MOE_STAGE_GATEUP + 1), dots_gate, dots_up, hq_out),
                "gate/up GEMV (Q8_0)");
        MOE_HIP(moe::launch_gemv(routed, shared, false, true, hq, nullptr, hd, nullptr, R, R, slots, meta, max_slots,
                                 nullptr, nullptr, nullptr, y, st, stage_ev(ev, 2 * MOE_STAGE_DOWN),
                                 stage_ev(ev, 2 * MOE_STAGE_DOWN + 1), dots_down, dots_down, nullptr),
                "down GEMV (Q8_0)");
        return MOE_OK;
    }
    const _Float16* xq = ws_at<_Float16>(ws, L.xq);
    const float* xd = ws_at<float>(ws, L.xd);
    _Float16* hq = ws_at<_Float16>(ws, L.h);
    float* hd = hd_out ? hd_out : ws_at<float>(ws, L.hd);
    MOE_HIP(moe::launch_q8_mfma(routed, shared, true, xq, xd, T, row_token, tiles, meta, L.max_tiles, hq, hd, nullptr,
                                dots_gate, dots_up, hq_out, st, stage_ev(ev, 2 * MOE_STAGE_GATEUP),
                                stage_ev(ev, 2 * MOE_STAGE_GATEUP + 1)),
            "gate/up matrix-core GEMM");
    MOE_HIP(moe::launch_q8_mfma(routed, shared, false, hq, hd, R, nullptr, tiles, meta, L.max_tiles, nullptr, nullptr, y,
                                dots_down, nullptr, nullptr, st, stage_ev(ev, 2 * MOE_STAGE_DOWN),
                                stage_ev(ev, 2 * MOE_STAGE_DOWN + 1)),
            "down matrix-core GEMM");
    return MOE_OK;
}

moe_status expert_ffn_impl(const float* x, int32_t T, int32_t k, const moe_experts* ex, const int32_t* counts,
                           const int32_t* offsets, const int32_t* perm, int32_t act_mode, float* y_perm,
                           int32_t* dots_gate, int32_t* dots_up, int8_t* hq, float* hd, int32_t* dots_down,
                           void* ws, size_t ws_bytes, hipStream_t st) {
    moe_status s;
    if ((s = check_act_mode(act_mode)) != MOE_OK) return s;
    if ((s = check_experts(ex, "routed", act_mode, T)) != MOE_OK) return s;
    MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T = %d < 0", T);
    MOE_REQUIRE(k >= 1 && k <= ex->n_experts, MOE_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, ex->n_experts);
    MOE_REQUIRE(ex->n_experts <= moe::kMaxExperts, MOE_ERR_UNSUPPORTED, "n_experts = %d > %d", ex->n_experts,
                moe::kMaxExperts);
    if (T == 0) return ok();
    if ((s = check_rows(T, k, 0, ex)) != MOE_OK) return s;
    MOE_REQUIRE(x && counts && offsets && perm && y_perm, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(x) && aligned16(y_perm), MOE_ERR_INVALID_ARG, "x and y_perm must be 16-byte aligned");
    const moe::WsLayout L = moe::ws_layout(T, k, ex->n_experts, ex->d_model, ex->d_ff, act_mode, 0);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
                ws ? ws_bytes : 0, L.total);
    MOE_REQUIRE(aligned16(ws), MOE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    MOE_HIP(moe::launch_plan(counts, offsets, perm, T, k, ex->n_experts, 0, ws_at<int>(ws, L.row_token),
                             ws_at<int>(ws, L.slots), ws_at<int>(ws, L.tiles), ws_at<int>(ws, L.meta), st),
            "work-list kernel");
    MOE_HIP(moe::launch_xprep(x, T, ex->d_model, xprep_for(act_mode, ex->format, L, ws), st), "hidden states");
    if ((s = run_experts(T, k, *ex, nullptr, act_mode, L, ws, y_perm, dots_gate, dots_up, hq, hd, dots_down, nullptr,
                         st)) != MOE_OK)
        return s;
    return ok();
}

// The layer; with `block`, between its neighbours: out = x + layer(RMSNorm(x))
// (norm_w null: no normalisation, the residual is still added).
// Every check of the layer's arguments except the workspace's (host only).
moe_status check_layer(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                       const moe_experts* routed, const moe_experts* shared, int32_t act_mode, const float* out,
                       const float* norm_w, float eps) {
    moe_status s;
    if ((s = check_act_mode(act_mode)) != MOE_OK) return s;
    if ((s = check_experts(routed, "routed", act_mode, T)) != MOE_OK) return s;
    if ((s = check_router(p, routed->n_experts)) != MOE_OK) return s;
    if (shared) {
        if ((s = check_experts(shared, "shared", act_mode, T)) != MOE_OK) return s;
        MOE_REQUIRE(shared->n_experts == 1, MOE_ERR_INVALID_ARG, "shared expert set must hold 1 expert, not %d",
                    shared->n_experts);
        MOE_REQUIRE(shared->d_model == routed->d_model && shared->d_ff == routed->d_ff &&
                        shared->format == routed->format,
                    MOE_ERR_UNSUPPORTED, "shared expert must match the routed d_model, d_ff and format");
        MOE_REQUIRE(p->shared_gate == nullptr || aligned16(p->shared_gate), MOE_ERR_INVALID_ARG,
                    "shared_gate must be 16-byte aligned");
    }
    MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T = %d < 0", T);
    if (T == 0) return ok();
    if ((s = check_rows(T, p->top_k, shared != nullptr, routed)) != MOE_OK) return s;
    MOE_REQUIRE(x && gate_w && out, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(x) && aligned16(gate_w) && aligned16(out), MOE_ERR_INVALID_ARG,
                "x, gate_w and out must be 16-byte aligned");
    MOE_REQUIRE(norm_w == nullptr || aligned16(norm_w), MOE_ERR_INVALID_ARG, "norm_w must be 16-byte aligned");
    MOE_REQUIRE(std::isfinite(eps) && eps >= 0.0f, MOE_ERR_INVALID_ARG, "eps = %g must be finite and >= 0",
                (double)eps);
    return MOE_OK;
}

moe_status layer_forward_impl(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                              const moe_experts* routed, const moe_experts* shared, int32_t act_mode, float* out,
                              void* ws, size_t ws_bytes, const hipEvent_t* ev, hipStream_t st, bool block = false,
                              const float* norm_w = nullptr, float eps = 0.0f) {
    moe_status s;
    if ((s = check_layer(x, T, gate_w, p, routed, shared, act_mode, out, norm_w, eps)) != MOE_OK) return s;
    if (T == 0) return ok();
    const int E = routed->n_experts, k = p->top_k, d = routed->d_model;
    const int has_shared = shared != nullptr;
    const moe::WsLayout L = moe::ws_layout(T, k, E, d, routed->d_ff, act_mode, has_shared);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
                ws ? ws_bytes : 0, L.total);
    MOE_REQUIRE(aligned16(ws), MOE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    int* idx = ws_at<int>(ws, L.idx);
    float* w = ws_at<float>(ws, L.wts);
    int* inv_perm = ws_at<int>(ws, L.inv_perm);
    float* logits = ws_at<float>(ws, L.logits);
    const moe::XPrep xp = xprep_for(act_mode, routed->format, L, ws);
    // the logits launch also prepares the hidden states; small T: top-k +
    // dispatch are one block, larger T: kernels of their own
    const bool small = moe::router_splits(T, E, d) == 0;
    const bool fused = T <= moe::kFusedRouteT;
    const bool norm = block && norm_w != nullptr;
    const int S = moe::router_slices(T, E, d, norm && small);   // logits slices
    // the layer's input: x, or RMSNorm(x) (inside the router kernel for small
    // T; larger T normalises once into the workspace)
    const float* xl = x;
    record(ev, 2 * MOE_STAGE_ROUTE, st);
    if (norm && !small) {
        float* xn = ws_at<float>(ws, L.xn);
        MOE_HIP(moe::launch_rmsnorm(x, T, d, norm_w, eps, xn, st), "RMSNorm");
        xl = xn;
    }
    // the shared expert's gate logit rides along as one more router row
    const float* sg = has_shared ? p->shared_gate : nullptr;
    float* sgl = sg ? ws_at<float>(ws, L.sgl) : nullptr;
    const moe::RouterParts rp = small ? moe::RouterParts{} : moe::router_parts_at(ws_at<char>(ws, L.rparts), T, E, d);
    MOE_HIP(moe::launch_router_logits(xl, T, d, gate_w, E, logits, xp, (norm && small) ? norm_w : nullptr, eps, sg,
                                      sgl, &rp, st),
            "router logits");
    if (!fused) MOE_HIP(moe::launch_router_topk(logits, T, S, *p, idx, w, st), "router top-k");
    record(ev, 2 * MOE_STAGE_ROUTE + 1, st);

    record(ev, 2 * MOE_STAGE_DISPATCH, st);
    if (fused)
        MOE_HIP(moe::launch_route_dispatch(logits, T, S, *p, idx, w, ws_at<int>(ws, L.counts),
                                           ws_at<int>(ws, L.offsets), ws_at<int>(ws, L.perm), inv_perm, has_shared,
                                           ws_at<int>(ws, L.row_token), ws_at<int>(ws, L.slots),
                                           ws_at<int>(ws, L.tiles), ws_at<int>(ws, L.meta), st),
                "router top-k + dispatch");
    else
        MOE_HIP(moe::launch_dispatch(idx, T, k, E, ws_at<int>(ws, L.counts), ws_at<int>(ws, L.offsets),
                                     ws_at<int>(ws, L.perm), inv_perm, has_shared, ws_at<int>(ws, L.row_token),
                                     ws_at<int>(ws, L.slots), ws_at<int>(ws, L.tiles), ws_at<int>(ws, L.meta),
                                     L.dhist ? ws_at<int>(ws, L.dhist) : nullptr, L.dbad ? ws_at<int>(ws, L.dbad) : nullptr, st),
                "dispatch");
    record(ev, 2 * MOE_STAGE_DISPATCH + 1, st);
    float* y = ws_at<float>(ws, L.y);
    if ((s = run_experts(T, k, *routed, shared, act_mode, L, ws, y, nullptr, nullptr, nullptr, nullptr, nullptr, ev,
                         st)) != MOE_OK)
        return s;
    record(ev, 2 * MOE_STAGE_COMBINE, st);
    MOE_HIP(moe::launch_combine(y, w, inv_perm, has_shared ? y + (size_t)T * k * d : nullptr, sgl, S,
                                block ? x : nullptr, T, k, d, out, st),
            "combine");
    record(ev, 2 * MOE_STAGE_COMBINE + 1, st);
    return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of this device's scratch array, looked up once per device
// (with that device current) and kept.
moe_status scratch_for_current_device(void** out) {
    int dev = 0;
    MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
    MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks",
                dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        MOE_REQUIRE(p != nullptr, MOE_ERR_HIP, "no scratch address for device %d", dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d, int32_t d_ff, int32_t act_mode,
                          int32_t has_shared) {
    if (T < 0 || k < 1 || E < 1 || k > E || d <= 0 || d_ff <= 0 || d % moe::kGroup || d_ff % moe::kGroup) return 0;
    if (act_mode != MOE_ACT_F32 && act_mode != MOE_ACT_Q8_0) return 0;
    return moe::ws_layout(T, k, E, d, d_ff, act_mode, has_shared ? 1 : 0).total;
}

moe_status moe_quantize_weights(const float* w, int64_t rows, int32_t cols, int32_t matrix_rows, int32_t format,
                                void* q, float* s, hipStream_t stream) {
    MOE_REQUIRE(rows >= 0 && cols > 0, MOE_ERR_INVALID_ARG, "bad shape [%lld, %d]", (long long)rows, cols);
    MOE_REQUIRE(matrix_rows > 0 && rows % matrix_rows == 0, MOE_ERR_INVALID_ARG,
                "rows = %lld is not a whole number of matrices of %d rows", (long long)rows, matrix_rows);
    MOE_REQUIRE(cols % (2 * moe::kGroup) == 0, MOE_ERR_UNSUPPORTED,
                "cols = %d is not a multiple of 64 (pairs of groups)", cols);
    MOE_REQUIRE(matrix_rows % moe::kTile == 0, MOE_ERR_UNSUPPORTED,
                "matrix_rows = %d is not a multiple of 32 (tiled layout)", matrix_rows);
    MOE_REQUIRE(moe::fmt_valid(format), MOE_ERR_INVALID_ARG, "unknown format %d", format);
    MOE_REQUIRE(cols % moe::fmt_k_multiple(format) == 0, MOE_ERR_UNSUPPORTED,
                "cols = %d is not a multiple of %d (whole code blocks of format %d)", cols,
                moe::fmt_k_multiple(format), format);
    if (rows == 0) return ok();
    MOE_REQUIRE(w && q && s, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(w) && aligned16(q), MOE_ERR_INVALID_ARG, "w and q must be 16-byte aligned");
    MOE_HIP(moe::launch_quantize_weights(w, rows, cols, matrix_rows, format, q, s, stream), "weight quantiser");
    return ok();
}

moe_status moe_quantize_q8_0(const float* x, int64_t rows, int32_t cols, int8_t* q, float* d, hipStream_t stream) {
    MOE_REQUIRE(rows >= 0 && cols > 0, MOE_ERR_INVALID_ARG, "bad shape [%lld, %d]", (long long)rows, cols);
    MOE_REQUIRE(cols % moe::kGroup == 0, MOE_ERR_UNSUPPORTED, "cols = %d is not a multiple of 32", cols);
    if (rows == 0) return ok();
    MOE_REQUIRE(x && q && d, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(x) && aligned16(q), MOE_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
    MOE_HIP(moe::launch_quantize_q8_0(x, rows, cols, q, d, stream), "Q8_0 quantiser");
    return ok();
}

moe_status moe_route(const float* x, int32_t T, int32_t d, const float* gate_w, const moe_router_params* p,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status s;
    if ((s = check_router(p, -1)) != MOE_OK) return s;
    MOE_REQUIRE(T >= 0 && d > 0, MOE_ERR_INVALID_ARG, "bad shape T = %d, d = %d", T, d);
    MOE_REQUIRE(d % 4 == 0, MOE_ERR_UNSUPPORTED, "d = %d is not a multiple of 4", d);
    if (T == 0) return ok();
    MOE_REQUIRE(x && gate_w && topk_idx && topk_w, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(x) && aligned16(gate_w), MOE_ERR_INVALID_ARG, "x and gate_w must be 16-byte aligned");
    // the logits' slices, then the matrix-core router's operands (larger T)
    const int E = p->n_experts;
    const size_t lbytes = moe::align256((size_t)moe::router_slices(T, E, d, false) * T * E * sizeof(float));
    const size_t need = lbytes + moe::router_parts_bytes(T, E, d);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
                ws ? ws_bytes : 0, need);
    MOE_REQUIRE(aligned16(ws), MOE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const moe::RouterParts rp = moe::router_parts_at(static_cast<char*>(ws) + lbytes, T, E, d);
    MOE_HIP(moe::launch_router(x, T, d, gate_w, *p, static_cast<float*>(ws), &rp, topk_idx, topk_w, stream),
            "router");
    return ok();
}

moe_status moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && k >= 1 && E >= 1 && k <= E, MOE_ERR_INVALID_ARG, "bad sizes T = %d, k = %d, E = %d", T,
                k, E);
    MOE_REQUIRE(E <= moe::kMaxExperts, MOE_ERR_UNSUPPORTED, "E = %d > %d", E, moe::kMaxExperts);
    MOE_REQUIRE((int64_t)T * k <= (int64_t)1 << 30, MOE_ERR_UNSUPPORTED, "T*k too large");
    MOE_REQUIRE(counts && offsets, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    if (T > 0) MOE_REQUIRE(topk_idx && perm && inv_perm, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    // scratch for the multi-block dispatch when the caller's workspace holds it
    const int64_t n = (int64_t)T * k;
    int* chunk_hist = nullptr;
    int* chunk_bad = nullptr;
    if (n > moe::kDispatchWaveMax && ws && aligned16(ws)) {
        const size_t nch = (size_t)moe::dispatch_chunk_count(n);
        const size_t hb = moe::align256(nch * E * sizeof(int));
        if (ws_bytes >= hb + nch * sizeof(int)) {
            chunk_hist = static_cast<int*>(ws);
            chunk_bad = ws_at<int>(ws, hb);
        }
    }
    MOE_HIP(moe::launch_dispatch(topk_idx, T, k, E, counts, offsets, perm, inv_perm, 0, nullptr, nullptr, nullptr,
                                 nullptr, chunk_hist, chunk_bad, stream),
            "dispatch");
    return ok();
}

moe_status moe_expert_ffn(const float* x, int32_t T, int32_t k, const moe_experts* ex, const int32_t* counts,
                          const int32_t* offsets, const int32_t* perm, int32_t act_mode, float* y_perm, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    return expert_ffn_impl(x, T, k, ex, counts, offsets, perm, act_mode, y_perm, nullptr, nullptr, nullptr, nullptr,
                           nullptr, ws, ws_bytes, stream);
}

moe_status moe_debug_q8_expert_ffn(const float* x, int32_t T, int32_t k, const moe_experts* ex,
                                   const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                   int32_t* dots_gate, int32_t* dots_up, int8_t* hq, float* hd, int32_t* dots_down,
                                   float* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_REQUIRE(dots_gate && dots_up && hq && hd && dots_down, MOE_ERR_INVALID_ARG, "NULL debug output");
    return expert_ffn_impl(x, T, k, ex, counts, offsets, perm, MOE_ACT_Q8_0, y_perm, dots_gate, dots_up, hq, hd,
                           dots_down, ws, ws_bytes, stream);
}

moe_status moe_combine(const float* y_perm, const float* topk_w, const int32_t* inv_perm, const float* shared_y,
                       int32_t T, int32_t k, int32_t d, float* out, hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && k >= 1 && d > 0, MOE_ERR_INVALID_ARG, "bad sizes T = %d, k = %d, d = %d", T, k, d);
    MOE_REQUIRE(d % 4 == 0, MOE_ERR_UNSUPPORTED, "d = %d is not a multiple of 4", d);
    if (T == 0) return ok();
    MOE_REQUIRE(y_perm && topk_w && inv_perm && out, MOE_ERR_INVALID_ARG, "NULL tensor argument");
    MOE_REQUIRE(aligned16(y_perm) && aligned16(out) && (shared_y == nullptr || aligned16(shared_y)),
                MOE_ERR_INVALID_ARG, "y_perm, shared_y and out must be 16-byte aligned");
    MOE_HIP(moe::launch_combine(y_perm, topk_w, inv_perm, shared_y, nullptr, 0, nullptr, T, k, d, out, stream),
            "combine");
    return ok();
}

moe_status moe_layer_forward(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                             const moe_experts* routed, const moe_experts* shared, int32_t act_mode, float* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
    return layer_forward_impl(x, T, gate_w, p, routed, shared, act_mode, out, ws, ws_bytes, nullptr, stream);
}

moe_status moe_layer_forward_noalloc(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                                     const moe_experts* routed, const moe_experts* shared, int32_t act_mode, float* out,
                                     hipStream_t stream) {
    moe_status s;
    if ((s = check_layer(x, T, gate_w, p, routed, shared, act_mode, out, nullptr, 0.0f)) != MOE_OK) return s;
    if (T == 0) return ok();
    const size_t need = moe_workspace_size(T, p->top_k, routed->n_experts, routed->d_model, routed->d_ff, act_mode,
                                           shared != nullptr);
    MOE_REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch, more than the %zu the allocation-free entry point holds "
                "(moe_layer_forward takes a workspace of any size)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((s = scratch_for_current_device(&ws)) != MOE_OK) return s;
    return layer_forward_impl(x, T, gate_w, p, routed, shared, act_mode, out, ws, MOE_NOALLOC_SCRATCH_BYTES, nullptr,
                              stream);
}

moe_status moe_layer_forward_timed(const float* x, int32_t T, const float* gate_w, const moe_router_params* p,
                                   const moe_experts* routed, const moe_experts* shared, int32_t act_mode, float* out,
                                   void* ws, size_t ws_bytes, const hipEvent_t* stage_events, hipStream_t stream) {
    return layer_forward_impl(x, T, gate_w, p, routed, shared, act_mode, out, ws, ws_bytes, stage_events, stream);
}

moe_status moe_block_forward(const float* x, int32_t T, const float* norm_w, float eps, const float* gate_w,
                             const moe_router_params* p, const moe_experts* routed, const moe_experts* shared,
                             int32_t act_mode, float* out, void* ws, size_t ws_bytes,
                             const hipEvent_t* stage_events, hipStream_t stream) {
    return layer_forward_impl(x, T, gate_w, p, routed, shared, act_mode, out, ws, ws_bytes, stage_events, stream, true,
                              norm_w, eps);
}

moe_status moe_debug_workspace_sections(int32_t T, int32_t k, int32_t E, int32_t d, int32_t d_ff, int32_t act_mode,
                                        int32_t has_shared, int64_t* offsets_out) {
    MOE_REQUIRE(offsets_out != nullptr, MOE_ERR_INVALID_ARG, "offsets_out is NULL");
    MOE_REQUIRE(moe_workspace_size(T, k, E, d, d_ff, act_mode, has_shared) > 0, MOE_ERR_INVALID_ARG,
                "invalid sizes T = %d, k = %d, E = %d, d = %d, d_ff = %d, act_mode = %d", T, k, E, d, d_ff, act_mode);
    const moe::WsLayout L = moe::ws_layout(T, k, E, d, d_ff, act_mode, has_shared ? 1 : 0);
    offsets_out[MOE_WS_TOPK_IDX] = (int64_t)L.idx;
    offsets_out[MOE_WS_TOPK_W] = (int64_t)L.wts;
    offsets_out[MOE_WS_COUNTS] = (int64_t)L.counts;
    offsets_out[MOE_WS_OFFSETS] = (int64_t)L.offsets;
    offsets_out[MOE_WS_PERM] = (int64_t)L.perm;
    offsets_out[MOE_WS_INV_PERM] = (int64_t)L.inv_perm;
    offsets_out[MOE_WS_H_CODES] = act_mode == MOE_ACT_Q8_0 ? (int64_t)L.h : -1;
    offsets_out[MOE_WS_H_SCALES] = act_mode == MOE_ACT_Q8_0 ? (int64_t)L.hd : -1;
    return ok();
}

const char* moe_status_string(moe_status st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported request";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    }
    return "unknown moe_status";
}

const char* moe_last_error_detail(void) { return g_detail.c_str(); }

}  // extern "C"
