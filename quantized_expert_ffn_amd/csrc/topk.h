// Wave-level reductions and the per-token top-k selection of the router.
//
// Softmax top-k: "I ran a 7B Mixture-of-Experts LLM in a language I built"
// (dev.to), section "Mixture-of-Experts" (each token goes to its top 8 of 64
// experts). Sigmoid noaux_tc: "Show HN: Getting GLM-5.2 running on my slow
// computer", section "What's implemented" (a sigmoid router of the
// DeepSeek-V3 kind: noaux_tc selection and a routed scaling factor); its
// steps are the DeepSeek-V3 ones:
// sigmoid scores, selection on score + bias, groups ranked by the sum of
// their two best keys, top-k among the kept groups, weights = the chosen
// scores normalised to sum 1 and scaled.
//
// Ranking is by key descending, ties to the lower expert (group) id; the
// output slot order is the selection order.
#pragma once

#include <float.h>

#include "common.h"

namespace moe {

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
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

// Wave argmax over (key, id); every lane gets the winner. Lanes hold
// increasing ids (a lane's candidate being its own best, ties to its lower
// id), so the first lane that holds the largest key holds the winner: one
// wave max, one ballot and one read, instead of a compare-exchange per step.
__device__ __forceinline__ void wave_argmax(float& k, int& id) {
    const float m = wave_max_all(k);
    const uint64_t b = __ballot(k == m);
    const int src = b ? __builtin_ctzll(b) : 0;   // no lane equal: only NaN keys
    id = __builtin_amdgcn_readlane(id, src);
    k = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(m)));
    id = __builtin_amdgcn_readfirstlane(id);
}

struct TopkArgs {
    const float* L;      // logits as S partial sums [S, T, E]
    int S, T, E, k;
    int mode, renorm, n_group, topk_group;
    float rsf;
    const float* bias;   // [E] or null
    float top_p;         // adaptive expert top-p in (0, 1), or 0 = off
};

// S: the number of partial-sum slices the logits kernel wrote (router_slices)
TopkArgs topk_args(const float* logits, int T, int S, const moe_router_params& p);

// Top-k of token t by one wave (lane l owns experts l*EPL .. l*EPL+EPL-1).
// Lane j < k returns slot j's expert and weight. keybuf: E floats of LDS
// private to this wave (noaux_tc only). A wave with nothing to do (active
// false) returns at once; no block-wide barrier is involved.
template <int EPL>
__device__ __forceinline__ void topk_token(const TopkArgs& a, int t, bool active, float* keybuf, int* out_e, float* out_w) {
    const int lane = threadIdx.x & 63;
    *out_e = -1;
    *out_w = 0.0f;
    if (!active) return;
    const int E = a.E, k = a.k;
    constexpr float NEG_INF = -INFINITY;

    // every load goes out at once (clamped indices, masked afterwards): a load
    // under its own condition would wait for the one before it
    const int tc = active ? t : 0;
    float lv[EPL], bv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int ec = min(lane * EPL + i, E - 1);
        lv[i] = 0.0f;
        bv[i] = a.bias ? a.bias[ec] : 0.0f;
    }
    // the slices' partial sums, added in slice order; a batch of slices is
    // loaded before any of it is added, so the loads overlap
    constexpr int SB = EPL >= 16 ? 2 : EPL >= 8 ? 4 : 8;
    // a lane's EPL experts are consecutive: 16-byte loads when every lane's
    // run lies inside the row (E == 64 EPL, so the rows are 16-byte aligned
    // too). The condition is the same for the whole wave, and each path has
    // its own loop: with one loop, the compiler merged the two paths into
    // 4-byte loads.
    auto add_slices = [&](auto load_row) __attribute__((always_inline)) {
        for (int s0 = 0; s0 < a.S; s0 += SB) {
            float pv[SB][EPL];
#pragma unroll
            for (int u = 0; u < SB; ++u) load_row(a.L + ((size_t)min(s0 + u, a.S - 1) * a.T + tc) * E, pv[u]);
#pragma unroll
            for (int u = 0; u < SB; ++u)
                if (s0 + u < a.S)
#pragma unroll
                    for (int i = 0; i < EPL; ++i) lv[i] = u == 0 && s0 == 0 ? pv[0][i] : lv[i] + pv[u][i];
        }
    };
    if (EPL % 4 == 0 && E == kWave * EPL) {
        add_slices([&](const float* row, float (&v)[EPL]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const float4 q = *reinterpret_cast<const float4*>(row + lane * EPL + (i & ~3));
                v[i] = q.x;
                v[(i + 1) % EPL] = q.y;
                v[(i + 2) % EPL] = q.z;
                v[(i + 3) % EPL] = q.w;
            }
        });
    } else {
        add_slices([&](const float* row, float (&v)[EPL]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = row[min(lane * EPL + i, E - 1)];
        });
    }

    float key[EPL], val[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        const float l = (active && e < E) ? lv[i] : NEG_INF;
        if (a.mode == MOE_ROUTER_SOFTMAX_TOPK) {
            key[i] = l;
            val[i] = l;
        } else {
            const float sg = (e < E) ? 1.0f / (1.0f + expf(-l)) : 0.0f;
            val[i] = sg;
            key[i] = (e < E) ? sg + bv[i] : NEG_INF;
        }
    }

    float lmax = 0.0f, denom = 1.0f;
    if (a.mode == MOE_ROUTER_SOFTMAX_TOPK) {
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
            if (lane * EPL + i < E) keybuf[lane * EPL + i] = key[i];
        // the keys are this wave's own: a wave-level barrier orders them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int gs = E / a.n_group;
        float gscore = NEG_INF;
        if (lane < a.n_group) {
            // the two largest keys of the group, branch-free (m1 >= m2)
            float m1 = NEG_INF, m2 = NEG_INF;
            auto take = [&](float c) {
                m2 = fmaxf(m2, fminf(m1, c));
                m1 = fmaxf(m1, c);
            };
            const float* grp = keybuf + lane * gs;
            int e = 0;
            if ((gs & 3) == 0)
                for (; e < gs; e += 4) {
                    const float4 c = *reinterpret_cast<const float4*>(grp + e);
                    take(c.x);
                    take(c.y);
                    take(c.z);
                    take(c.w);
                }
            for (; e < gs; ++e) take(grp[e]);
            gscore = gs >= 2 ? m1 + m2 : m1;
        }
        uint64_t kept = 0;
        for (int r = 0; r < a.topk_group; ++r) {
            const bool taken = lane < a.n_group && ((kept >> lane) & 1ull);
            float kk = (lane < a.n_group && !taken) ? gscore : NEG_INF;
            int id = (lane < a.n_group && !taken) ? lane : INT_MAX;
            wave_argmax(kk, id);
            if (id != INT_MAX) kept |= 1ull << id;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (e < E && !((kept >> (e / gs)) & 1ull)) key[i] = NEG_INF;
        }
    }

    // Each lane sorts its EPL (key, id) pairs by rank (Batcher's odd-even
    // merge sort, a fixed network), so a lane's best candidate is its head.
    // Then k rounds: the wave argmax of the heads (a lane's ids are all below
    // the next lane's, so the first lane holding the largest head key holds
    // the winner, ties to the lower id), and the winning lane drops its head.
    // Lane j keeps slot j's expert and key.
    int id[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) id[i] = lane * EPL + i;
#pragma unroll
    for (int p = 1; p < EPL; p <<= 1)
#pragma unroll
        for (int q = p; q >= 1; q >>= 1)
#pragma unroll
            for (int j = q % p; j + q < EPL; j += 2 * q)
#pragma unroll
                for (int i = 0; i < q; ++i) {
                    const int u = i + j, v = i + j + q;
                    if (v < EPL && u / (2 * p) == v / (2 * p) && ranks_before(key[v], id[v], key[u], id[u])) {
                        const float tk = key[u];
                        key[u] = key[v];
                        key[v] = tk;
                        const int ti = id[u];
                        id[u] = id[v];
                        id[v] = ti;
                    }
                }
    if (a.mode != MOE_ROUTER_SOFTMAX_TOPK) {
        // the selected experts' sigmoid scores, looked up by expert after the
        // rounds (the group scores above read keybuf before these writes, and
        // a wave executes its LDS operations in order)
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) keybuf[lane * EPL + i] = val[i];
    }
    int my_e = -1;
    float my_v = 0.0f;
    for (int j = 0; j < k; ++j) {
        const float m = wave_max_all(key[0]);
        if (!(m > NEG_INF)) break;               // no candidate left: cannot happen for validated k
        const uint64_t b = __ballot(key[0] == m);
        const int src = b ? __builtin_ctzll(b) : 0;
        const int be = __builtin_amdgcn_readlane(id[0], src);
        if (lane == j) { my_e = be; my_v = m; }
        if (lane == src) {
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) {
                key[i] = key[i + 1];
                id[i] = id[i + 1];
            }
            key[EPL - 1] = NEG_INF;
        }
    }
    if (a.mode != MOE_ROUTER_SOFTMAX_TOPK) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        my_v = my_e >= 0 ? keybuf[my_e] : 0.0f;
    }

    float wj = 0.0f;
    if (lane < k) {
        if (a.mode == MOE_ROUTER_SOFTMAX_TOPK) wj = expf(my_v - lmax) / denom;
        else wj = my_v;
    }
    if (a.mode == MOE_ROUTER_SOFTMAX_TOPK) {
        if (a.renorm) {
            const float tot = wave_sum_all(lane < k ? wj : 0.0f);
            wj = wj / tot;
        }
    } else {
        const float tot = wave_sum_all(lane < k ? wj : 0.0f);
        wj = wj / tot * a.rsf;
    }
    if (a.top_p > 0.0f) {
        // adaptive expert top-p: keep slot j while the slots before it hold
        // less than top_p of the total, then rescale the kept ones to the total
        const float w_in = lane < k ? wj : 0.0f;
        float incl = w_in;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += o;
        }
        const float tot = __shfl(incl, kWave - 1, kWave);
        const bool keep = lane < k && (lane == 0 || incl - w_in < a.top_p * tot);
        const float kept = wave_sum_all(keep ? wj : 0.0f);
        wj = keep ? wj * (tot / kept) : 0.0f;
        if (!keep) my_e = -1;
    }
    *out_e = my_e;
    *out_w = wj;
}

// experts per lane for the top-k wave: the smallest power of two with 64*EPL >= E
inline int topk_epl(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

}  // namespace moe
