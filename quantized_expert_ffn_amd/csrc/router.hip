// Router: logits L = X Wg^T (fp32) and per-token top-k selection.
//
// Softmax top-k: "I ran a 7B Mixture-of-Experts LLM in a language I built"
// (dev.to), section "Mixture-of-Experts" (OLMoE routes each token to its top 8
// of 64 experts). Sigmoid noaux_tc: "Show HN: Getting GLM-5.2 running on my slow computer", section "What's
// implemented" (DeepSeek-V3-style sigmoid router, noaux_tc,
// routed_scaling_factor); its steps are the DeepSeek-V3 ones: sigmoid scores,
// selection on score + bias, groups ranked by the sum of their two best
// scores, top-k among the kept groups, weights = scores normalised and scaled.
//
// Ranking is by key descending, ties to the lower expert (group) id.
//
// Logits are written as S partial sums over contiguous slices of d
// ([S, T, E]); the top-k kernel adds them in slice order, so the result is
// deterministic whatever S the launcher picks for the shape.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Full-wave sum, result in every lane (DPP inside rows of 16, then the four
// row totals read back as uniform values and added in row order).
__device__ __forceinline__ float wave_sum_all(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max_all(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// (key, id) ranking: larger key first, then lower id. id = INT_MAX means "none".
__device__ __forceinline__ bool ranks_before(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& k, int& id) {
    const float ok = dppf<CTRL>(k);
    const int oi = dppi<CTRL>(id);
    if (ranks_before(ok, oi, k, id)) { k = ok; id = oi; }
}

// Wave argmax over (key, id); every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& k, int& id) {
    argmax_step<0xB1>(k, id);
    argmax_step<0x4E>(k, id);
    argmax_step<0x141>(k, id);
    argmax_step<0x140>(k, id);
    float bk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), 0));
    int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float rk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), r));
        const int ri = __builtin_amdgcn_readlane(id, r);
        if (ranks_before(rk, ri, bk, bi)) { bk = rk; bi = ri; }
    }
    k = bk;
    id = bi;
}

// ---------------------------------------------------------------------------
// Logits, small T (decode): one block per expert; the 256 threads split d,
// each keeps T partial sums, then a wave reduction and a fixed-order sum of
// the four wave partials.
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void router_logits_gemv_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wg, int T, int d,
                                                                 int E, float* __restrict__ L) {
    __shared__ float part[4][TB];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x;
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
    const float4* wr = reinterpret_cast<const float4*>(wg + (size_t)e * d);
    const int n4 = d >> 2;
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 w4 = wr[i];
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < T) {
                const float4 x4 = reinterpret_cast<const float4*>(x + (size_t)t * d)[i];
                acc[t] = fmaf(x4.x, w4.x, acc[t]);
                acc[t] = fmaf(x4.y, w4.y, acc[t]);
                acc[t] = fmaf(x4.z, w4.z, acc[t]);
                acc[t] = fmaf(x4.w, w4.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const float s = wave_sum_all(acc[t]);
        if (lane == 0) part[wave][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        L[(size_t)t * E + e] = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
    }
}

// ---------------------------------------------------------------------------
// Logits, larger T: fp32 matrix cores (v_mfma_f32_32x32x2_f32), split over d.
// Block: 64 tokens x 64 experts, four waves of 32 x 32; blockIdx.z = slice.
// Each lane loads 4 consecutive k of its token row and its expert row; the
// four MFMAs of a step each take one of them (the two lane halves cover
// k..k+3 and k+4..k+7), so every (token, expert, k) product enters once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wg, int T, int d,
                                                                 int E, int kslice, float* __restrict__ L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = blockIdx.y * 64 + (wave & 1) * 32;
    const int e0 = blockIdx.x * 64 + (wave >> 1) * 32;
    const int ks = blockIdx.z;
    const int kbeg = ks * kslice, kend = min(d, kbeg + kslice);
    const int row = lane & 31, h = lane >> 5;
    const bool tok_ok = t0 + row < T, exp_ok = e0 + row < E;
    const float* xr = x + (size_t)(tok_ok ? t0 + row : 0) * d;
    const float* wr = wg + (size_t)(exp_ok ? e0 + row : 0) * d;
    v16f acc = {};
    for (int k = kbeg; k < kend; k += 8) {
        const int kk = k + 4 * h;
        const bool kok = kk < kend;
        const float4 a = (tok_ok && kok) ? *reinterpret_cast<const float4*>(xr + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 b = (exp_ok && kok) ? *reinterpret_cast<const float4*>(wr + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
    }
    float* out = L + (size_t)ks * T * E;
    const int e = e0 + row;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (t < T && e < E) out[(size_t)t * E + e] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token. Lane l owns experts [l*EPL, l*EPL + EPL).
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ L, int S, int T, int E, int k,
                                                          int mode, int renorm, int n_group, int topk_group,
                                                          float rsf, const float* __restrict__ bias,
                                                          int* __restrict__ idx_out, float* __restrict__ w_out) {
    __shared__ float keybuf[4][kMaxExperts];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    const bool active = t < T;
    constexpr float NEG_INF = -INFINITY;

    float key[EPL], val[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        float l = NEG_INF;
        if (active && e < E) {
            l = L[(size_t)t * E + e];
            for (int s = 1; s < S; ++s) l += L[((size_t)s * T + t) * E + e];
        }
        if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
            key[i] = l;
            val[i] = l;
        } else {
            const float sg = (e < E) ? 1.0f / (1.0f + expf(-l)) : 0.0f;
            val[i] = sg;
            key[i] = (e < E) ? sg + (bias ? bias[e] : 0.0f) : NEG_INF;
        }
    }

    float lmax = 0.0f, denom = 1.0f;
    if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
        float m = NEG_INF;
#pragma unroll
        for (int i = 0; i < EPL; ++i) m = fmaxf(m, val[i]);
        lmax = wave_max_all(m);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) s += expf(val[i] - lmax);
        denom = wave_sum_all(s);
    } else {
        // group-limited selection: group score = sum of the two best keys
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) keybuf[wave][lane * EPL + i] = key[i];
        __syncthreads();
        const int gs = E / n_group;
        float gscore = NEG_INF;
        if (lane < n_group) {
            float m1 = NEG_INF, m2 = NEG_INF;
            for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
                const float c = keybuf[wave][e];
                if (c > m1) { m2 = m1; m1 = c; }
                else if (c > m2) { m2 = c; }
            }
            gscore = gs >= 2 ? m1 + m2 : m1;
        }
        uint64_t kept = 0;
        for (int r = 0; r < topk_group; ++r) {
            const bool taken = lane < n_group && ((kept >> lane) & 1ull);
            float kk = (lane < n_group && !taken) ? gscore : NEG_INF;
            int id = (lane < n_group && !taken) ? lane : INT_MAX;
            wave_argmax(kk, id);
            if (id != INT_MAX) kept |= 1ull << id;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (e < E && !((kept >> (e / gs)) & 1ull)) key[i] = NEG_INF;
        }
    }

    // k rounds of wave argmax; lane j keeps slot j's expert and value
    uint32_t taken = 0;
    int my_e = -1;
    float my_v = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bk = NEG_INF;
        int be = INT_MAX;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            const bool cand = e < E && !((taken >> i) & 1u) && key[i] != NEG_INF;
            if (cand && ranks_before(key[i], e, bk, be)) { bk = key[i]; be = e; }
        }
        wave_argmax(bk, be);
        if (be == INT_MAX) break;                 // cannot happen for validated k
        float v = 0.0f;
        const int owner = be / EPL;
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == be - owner * EPL) { v = val[i]; taken |= 1u << i; }
        }
        v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), owner));
        if (lane == j) { my_e = be; my_v = v; }
    }

    float wj = 0.0f;
    if (lane < k) {
        if (mode == MOE_ROUTER_SOFTMAX_TOPK) wj = expf(my_v - lmax) / denom;
        else wj = my_v;
    }
    if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
        if (renorm) {
            const float tot = wave_sum_all(lane < k ? wj : 0.0f);
            wj = wj / tot;
        }
    } else {
        const float tot = wave_sum_all(lane < k ? wj : 0.0f);
        wj = wj / tot * rsf;
    }
    if (active && lane < k) {
        idx_out[(size_t)t * k + lane] = my_e;
        w_out[(size_t)t * k + lane] = wj;
    }
}

hipError_t launch_router(const float* x, int T, int d, const float* wg, const moe_router_params& p,
                         float* logits, int* idx, float* w, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int E = p.n_experts;
    const int S = router_splits(T, E, d);
    if (S == 0) {
        const dim3 grid(E);
        if (T == 1) hipLaunchKernelGGL(router_logits_gemv_kernel<1>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 2) hipLaunchKernelGGL(router_logits_gemv_kernel<2>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 4) hipLaunchKernelGGL(router_logits_gemv_kernel<4>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 8) hipLaunchKernelGGL(router_logits_gemv_kernel<8>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else hipLaunchKernelGGL(router_logits_gemv_kernel<16>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
    } else {
        const int kslice = router_kslice(d, S);
        const dim3 grid((E + 63) / 64, (T + 63) / 64, S);
        hipLaunchKernelGGL(router_logits_mfma_kernel, grid, dim3(256), 0, st, x, wg, T, d, E, kslice, logits);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int Ssum = S == 0 ? 1 : S;
    const dim3 grid((T + 3) / 4);
    const float rsf = p.routed_scaling_factor;
#define MOE_TOPK(EPL)                                                                                          \
    hipLaunchKernelGGL(router_topk_kernel<EPL>, grid, dim3(256), 0, st, logits, Ssum, T, E, p.top_k, p.mode,  \
                       p.renormalize, p.n_group, p.topk_group, rsf, p.score_bias, idx, w)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace moe
