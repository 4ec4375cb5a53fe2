// Router: logits L = X Wg^T (fp32) and per-token top-k selection.
//
// Softmax top-k: "I ran a 7B Mixture-of-Experts LLM in a language I built"
// (dev.to), section "Mixture-of-Experts" (OLMoE routes each token to its top 8
// of 64 experts). Sigmoid noaux_tc: "Show HN: colibri", section "What's
// implemented" (DeepSeek-V3-style sigmoid router, noaux_tc,
// routed_scaling_factor); its steps are the DeepSeek-V3 ones: sigmoid scores,
// selection on score + bias, groups ranked by the sum of their two best
// scores, top-k among the kept groups, weights = scores normalised and scaled.
//
// Ranking is by key descending, ties to the lower expert (group) id.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Logits, small T: one wave per expert row, the T token rows read through the
// cache; each lane strides over d in float4 steps, then a wave reduction.
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void router_logits_gemv_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wg, int T, int d,
                                                                 int E, float* __restrict__ L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
    const float4* wr = reinterpret_cast<const float4*>(wg + (size_t)e * d);
    const int n4 = d >> 2;
    for (int i = lane; i < n4; i += kWave) {
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
    for (int t = 0; t < TB; ++t) acc[t] = wave_sum(acc[t]);
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < TB; ++t)
            if (t < T) L[(size_t)t * E + e] = acc[t];
    }
}

// ---------------------------------------------------------------------------
// Logits, large T: LDS-tiled fp32 GEMM, 64 tokens x 64 experts per block,
// 4x4 outputs per thread, k in steps of 32. Each output sums k in order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_gemm_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wg, int T, int d,
                                                                 int E, float* __restrict__ L) {
    constexpr int BT = 64, BE = 64, BK = 32;
    __shared__ float xs[BK][BT + 4];
    __shared__ float ws[BK][BE + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int t0 = blockIdx.y * BT, e0 = blockIdx.x * BE;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += BK) {
        // each thread loads 2 float4 of X and 2 of Wg: 64 rows x 32 k
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int li = tid + r * 256;        // 0..511
            const int row = li >> 3, kc = (li & 7) * 4;
            float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = xv;
            if (t0 + row < T && k0 + kc < d)
                xv = *reinterpret_cast<const float4*>(x + (size_t)(t0 + row) * d + k0 + kc);
            if (e0 + row < E && k0 + kc < d)
                wv = *reinterpret_cast<const float4*>(wg + (size_t)(e0 + row) * d + k0 + kc);
            xs[kc + 0][row] = xv.x; xs[kc + 1][row] = xv.y; xs[kc + 2][row] = xv.z; xs[kc + 3][row] = xv.w;
            ws[kc + 0][row] = wv.x; ws[kc + 1][row] = wv.y; ws[kc + 2][row] = wv.z; ws[kc + 3][row] = wv.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) L[(size_t)t * E + e] = acc[i][j];
        }
    }
}

// (key, id) ranking: larger key first, then lower id. id = INT_MAX means "none".
__device__ __forceinline__ bool ranks_before(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ void wave_argmax(float& k, int& id) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ok = __shfl_xor(k, off, kWave);
        const int oi = __shfl_xor(id, off, kWave);
        if (ranks_before(ok, oi, k, id)) { k = ok; id = oi; }
    }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token. Lane l owns experts [l*EPL, l*EPL + EPL).
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ L, int T, int E, int k,
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
        const float l = (active && e < E) ? L[(size_t)t * E + e] : NEG_INF;
        if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
            key[i] = l;
            val[i] = l;
        } else {
            const float s = (e < E) ? 1.0f / (1.0f + expf(-l)) : 0.0f;
            val[i] = s;
            key[i] = (e < E) ? s + (bias ? bias[e] : 0.0f) : NEG_INF;
        }
    }

    float lmax = 0.0f, denom = 1.0f;
    if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
        float m = NEG_INF;
#pragma unroll
        for (int i = 0; i < EPL; ++i) m = fmaxf(m, val[i]);
        lmax = wave_max(m);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) s += expf(val[i] - lmax);
        denom = wave_sum(s);
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
        v = __shfl(v, owner, kWave);
        if (lane == j) { my_e = be; my_v = v; }
    }

    float wj = 0.0f;
    if (lane < k) {
        if (mode == MOE_ROUTER_SOFTMAX_TOPK) wj = expf(my_v - lmax) / denom;
        else wj = my_v;
    }
    if (mode == MOE_ROUTER_SOFTMAX_TOPK) {
        if (renorm) {
            const float tot = wave_sum(lane < k ? wj : 0.0f);
            wj = wj / tot;
        }
    } else {
        const float tot = wave_sum(lane < k ? wj : 0.0f);
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
    if (T <= 16) {
        const dim3 grid((E + 3) / 4);
        if (T == 1) hipLaunchKernelGGL(router_logits_gemv_kernel<1>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 2) hipLaunchKernelGGL(router_logits_gemv_kernel<2>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 4) hipLaunchKernelGGL(router_logits_gemv_kernel<4>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else if (T <= 8) hipLaunchKernelGGL(router_logits_gemv_kernel<8>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
        else hipLaunchKernelGGL(router_logits_gemv_kernel<16>, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
    } else {
        const dim3 grid((E + 63) / 64, (T + 63) / 64);
        hipLaunchKernelGGL(router_logits_gemm_kernel, grid, dim3(256), 0, st, x, wg, T, d, E, logits);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid((T + 3) / 4);
    const float rsf = p.routed_scaling_factor;
#define MOE_TOPK(EPL)                                                                                          \
    hipLaunchKernelGGL(router_topk_kernel<EPL>, grid, dim3(256), 0, st, logits, T, E, p.top_k, p.mode,        \
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
