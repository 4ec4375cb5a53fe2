// Combine: out[t] = sum_j w[t, j] * Y[inv_perm[t*k + j]] + g[t] * S[t], over
// the dispatched slots (inv_perm >= 0; a slot dropped by top-p adds nothing),
// plus the block's residual when the layer runs between its neighbours.
// g[t] = 1, or for a gated shared expert sigmoid of the gate logit, whose
// slice sums the router left in sgl [slices, T] (added here in slice order).
//
// The weighted sum of a token's k expert outputs plus the shared expert
// ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": shared expert). Each
// token gathers its own k rows in slot order, so no two threads ever add into
// the same output and the result does not depend on scheduling (no atomics).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef float v4f_t __attribute__((ext_vector_type(4)));

// Grid (column blocks of 256 floats, tokens); one wave per block, one float4
// column per lane. The token's weights and row indices are uniform loads.
// Slots go in batches of 16 whose rows are all loaded before the first is
// added (a slot past k or dropped by top-p loads nothing; every such test is
// the same for the whole wave), so the loads overlap; the sum still runs in
// slot order.
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                     const int* __restrict__ inv_perm,
                                                     const float* __restrict__ shared_y,
                                                     const float* __restrict__ sgl, int sgl_slices,
                                                     const float* __restrict__ residual, int T, int k, int d,
                                                     float* __restrict__ out) {
    const int t = blockIdx.y;
    const int c0 = blockIdx.x * 64 + threadIdx.x;
    if (t >= T) return;
    // lanes past the row's end take part in the slot loads (all 64 lanes are
    // needed there) and store nothing
    const bool col_in = c0 < (d >> 2);
    const int c = col_in ? c0 : 0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int kB = 16;
    // lane u < kB fetches slot j0 + u's row and weight (clamped index), then
    // every lane reads them from lane u: one load each for a batch
    auto slot_loads = [&](int j0, int& rl, float& wl) __attribute__((always_inline)) {
        const int jl = min(j0 + (int)(threadIdx.x % kB), k - 1);
        rl = inv_perm[(size_t)t * k + jl];   // -1: dropped by top-p
        wl = w[(size_t)t * k + jl];
    };
    auto batch = [&](int j0, int rl, float wl) __attribute__((always_inline)) {
        float4 v[kB];
        float wv[kB];
        bool use[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int row = __builtin_amdgcn_readlane(rl, u);
            use[u] = j0 + u < k && row >= 0;
            wv[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
            v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (use[u]) {
                // expert outputs are read once: non-temporal loads
                const v4f_t nv = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(y + (size_t)row * d) + c);
                v[u] = make_float4(nv[0], nv[1], nv[2], nv[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (!use[u]) continue;   // uniform across the block
            acc.x = fmaf(wv[u], v[u].x, acc.x);
            acc.y = fmaf(wv[u], v[u].y, acc.y);
            acc.z = fmaf(wv[u], v[u].z, acc.z);
            acc.w = fmaf(wv[u], v[u].w, acc.w);
        }
    };
    // one batch covers the usual k (no loop for the compiler to wait at);
    // the shared expert's row goes out right after its indices
    int rl;
    float wl;
    slot_loads(0, rl, wl);
    // (without a shared expert the load reads Y's first row and is unused:
    // an unconditional load keeps the count of loads in flight the same on
    // every path, so that the wait for the indices does not also wait for it)
    const float4 s = reinterpret_cast<const float4*>(shared_y ? shared_y + (size_t)t * d : y)[c];
    batch(0, rl, wl);
    for (int j0 = kB; j0 < k; j0 += kB) {
        slot_loads(j0, rl, wl);
        batch(j0, rl, wl);
    }
    if (shared_y) {
        if (sgl) {
            float z = 0.0f;
            for (int i = 0; i < sgl_slices; ++i) z += sgl[(size_t)i * T + t];
            const float g = 1.0f / (1.0f + __expf(-z));
            acc.x = fmaf(g, s.x, acc.x);
            acc.y = fmaf(g, s.y, acc.y);
            acc.z = fmaf(g, s.z, acc.z);
            acc.w = fmaf(g, s.w, acc.w);
        } else {
            acc.x += s.x;
            acc.y += s.y;
            acc.z += s.z;
            acc.w += s.w;
        }
    }
    if (residual) {
        // read before the store of the same element: out may alias residual
        const float4 r = reinterpret_cast<const float4*>(residual + (size_t)t * d)[c];
        acc.x += r.x;
        acc.y += r.y;
        acc.z += r.z;
        acc.w += r.w;
    }
    if (col_in) reinterpret_cast<float4*>(out + (size_t)t * d)[c] = acc;
}

hipError_t launch_combine(const float* y, const float* w, const int* inv_perm, const float* shared_y,
                          const float* sgl, int sgl_slices, const float* residual, int T, int k, int d, float* out,
                          hipStream_t st) {
    if (T == 0) return hipSuccess;
    const dim3 grid((d / 4 + 63) / 64, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(64), 0, st, y, w, inv_perm, shared_y, sgl, sgl_slices, residual, T,
                       k, d, out);
    return hipGetLastError();
}

}  // namespace moe
