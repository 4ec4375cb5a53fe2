// Router: logits L = X Wg^T (fp32) and per-token top-k selection (topk.h
// gives the selection rules and their sources).
//
// Logits are written as S partial sums over contiguous slices of d
// ([S, T, E]); the top-k adds them in slice order, so the result is
// deterministic whatever S the launcher picks for the shape.
//
// The small-T logits kernel also prepares the hidden states for the expert
// kernels while it has them in hand: the exact f16 hi/lo split of the f32
// path, or the Q8_0 codes of the int8 path ("Show HN: Getting GLM-5.2 running
// on my slow computer", section "What's implemented": Q8_0-style int8
// activations in batch, a single row in f32).
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Hidden-state preparation
// ---------------------------------------------------------------------------
// 8 consecutive values x[r][c .. c+7], normalised when xp carries an RMSNorm
__device__ __forceinline__ void load8(const float* __restrict__ x, int r, int d, int c, const XPrep& xp, float4& a,
                                      float4& b) {
    const float4* src = reinterpret_cast<const float4*>(x + (size_t)r * d + c);
    a = src[0];
    b = src[1];
    if (xp.gamma) {
        const float s = xp.inv_rms[r];
        const float4 ga = *reinterpret_cast<const float4*>(xp.gamma + c);
        const float4 gb = *reinterpret_cast<const float4*>(xp.gamma + c + 4);
        a = make_float4(a.x * ga.x * s, a.y * ga.y * s, a.z * ga.z * s, a.w * ga.w * s);
        b = make_float4(b.x * gb.x * s, b.y * gb.y * s, b.z * gb.z * s, b.w * gb.w * s);
    }
}

// f32 path, group g of every row, one wave: p = 2^(e-15) with max|x| < 2^e
// over the T rows' 32 values, x/p split into f16 hi + lo in operand-slot order.
template <int FMT>
__device__ __forceinline__ void split_group(const float* __restrict__ x, int T, int d, int g, const XPrep& xp) {
    const int lane = threadIdx.x & 63;
    const int rsub = lane >> 2, q = lane & 3;   // 16 rows per pass, 8 values per lane
    float amax = 0.0f;
    for (int r0 = 0; r0 < T; r0 += 16) {
        const int r = min(r0 + rsub, T - 1);
        float4 a, b;
        load8(x, r, d, g * kGroup + 8 * q, xp, a, b);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    }
    amax = wave_max_all(amax);
    const int ex = pow2_exponent(amax);
    const float up = ldexpf(1.0f, 15 - ex);
    for (int r0 = 0; r0 < T; r0 += 16) {
        const int r = r0 + rsub;
        if (r >= T) break;
        float4 a, b;
        load8(x, r, d, g * kGroup + 8 * q, xp, a, b);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        v8h hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float sv = v[slot_k(FMT, j)] * up;
            const _Float16 hv = (_Float16)sv;
            hi[j] = hv;
            lo[j] = (_Float16)(sv - (float)hv);
        }
        const size_t off = (size_t)r * d + g * kGroup + 8 * q;
        *reinterpret_cast<v8h*>(xp.hi + off) = hi;
        *reinterpret_cast<v8h*>(xp.lo + off) = lo;
    }
    if (lane == 0) xp.pow[g] = ldexpf(1.0f, ex - 15);
}

// Q8_0 of one group of one row by 4 lanes (one 8-wide slice each), in the
// fp32 steps of quantize_q8_0_kernel: d = amax / 127, inv = 1 / d,
// q = rne(x * inv). The codes leave as f16 (exact) in operand-slot order,
// ready to be a matrix-core operand.
// v: the lane's 8 values, off: their position in [T, d], item = t * G + g;
// the group's four lanes are neighbours (lane / 4 the same).
template <int FMT>
__device__ __forceinline__ void q8_store(const float (&v)[8], size_t off, int item, const XPrep& xp) {
    const int sub = threadIdx.x & 3;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    const float dd = __fdiv_rn(amax, 127.0f);
    const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
    v8h q;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float r = rintf(__fmul_rn(v[slot_k(FMT, j)], inv));
        q[j] = (_Float16)fminf(fmaxf(r, -127.0f), 127.0f);
    }
    *reinterpret_cast<v8h*>(xp.q + off) = q;
    if (sub == 0) xp.qd[item] = dd;
}

template <int FMT>
__device__ __forceinline__ void q8_item(const float* __restrict__ x, int d, int G, int item, const XPrep& xp) {
    const int sub = threadIdx.x & 3;
    const int t = item / G, g = item - t * G;
    float4 a, b;
    load8(x, t, d, g * kGroup + 8 * sub, xp, a, b);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    q8_store<FMT>(v, (size_t)t * d + g * kGroup + 8 * sub, item, xp);
}

// the preparation job, spread over every wave of the grid
__device__ __forceinline__ void xprep_waves(const float* __restrict__ x, int T, int d, const XPrep& xp, int gw, int nw) {
    const int G = d / kGroup;
    if (xp.mode == XPREP_SPLIT) {
        for (int g = gw; g < G; g += nw) {
            if (xp.fmt == MOE_W_INT8_G32) split_group<MOE_W_INT8_G32>(x, T, d, g, xp);
            else if (xp.fmt == MOE_W_INT4_G32) split_group<MOE_W_INT4_G32>(x, T, d, g, xp);
            else split_group<MOE_W_INT2_G32>(x, T, d, g, xp);
        }
    } else if (xp.mode == XPREP_Q8_0) {
        const int items = T * G;
        for (int base = gw * 16; base < items; base += nw * 16) {
            const int item = base + ((threadIdx.x & 63) >> 2);
            if (item >= items) continue;
            if (xp.fmt == MOE_W_INT8_G32) q8_item<MOE_W_INT8_G32>(x, d, G, item, xp);
            else if (xp.fmt == MOE_W_INT4_G32) q8_item<MOE_W_INT4_G32>(x, d, G, item, xp);
            else q8_item<MOE_W_INT2_G32>(x, d, G, item, xp);
        }
    }
}

// waves for one pass over the preparation job: one per group column (the
// split), one per 16 (token, group) items (Q8_0)
inline int xprep_waves_wanted(int T, int d, const XPrep& xp) {
    const int G = d / kGroup;
    return xp.mode == XPREP_SPLIT ? G : xp.mode == XPREP_Q8_0 ? (T * G + 15) / 16 : 0;
}

__global__ __launch_bounds__(256) void xprep_kernel(const float* __restrict__ x, int T, int d, const XPrep xp) {
    xprep_waves(x, T, d, xp, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

// ---------------------------------------------------------------------------
// Logits, small T (decode): one block per expert; the 256 threads split d,
// each keeps T partial sums, then a wave reduction and a fixed-order sum of
// the four wave partials. The block's waves then take their share of the
// hidden-state preparation. With a shared-expert gate vector sg, block E
// computes x . sg the same way into sgl [T].
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void router_logits_gemv_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wg, int T, int d,
                                                                 int E, float* __restrict__ L, XPrep xp,
                                                                 const float* __restrict__ gamma, float eps,
                                                                 const float* __restrict__ sg,
                                                                 float* __restrict__ sgl) {
    __shared__ float part[4][TB];
    __shared__ float sq[4][TB];
    __shared__ float inv_rms[TB];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x;
    float acc[TB], ss[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = ss[t] = 0.0f;
    const float4* wr = reinterpret_cast<const float4*>(e < E ? wg + (size_t)e * d : sg);
    const int n4 = d >> 2;
    for (int i = threadIdx.x; i < n4; i += 256) {
        float4 w4 = wr[i];
        if (gamma) {
            // RMSNorm(x) . w = inv_rms * sum x (gamma w); the sums of squares
            // come from the same loads
            const float4 g4 = reinterpret_cast<const float4*>(gamma)[i];
            w4 = make_float4(w4.x * g4.x, w4.y * g4.y, w4.z * g4.z, w4.w * g4.w);
        }
        // rows past T repeat the last row (unused sums): loads without
        // conditions all go out together instead of one at a time
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const float4 x4 = reinterpret_cast<const float4*>(x + (size_t)min(t, T - 1) * d)[i];
            acc[t] = fmaf(x4.x, w4.x, acc[t]);
            acc[t] = fmaf(x4.y, w4.y, acc[t]);
            acc[t] = fmaf(x4.z, w4.z, acc[t]);
            acc[t] = fmaf(x4.w, w4.w, acc[t]);
            if (gamma) {
                ss[t] = fmaf(x4.x, x4.x, ss[t]);
                ss[t] = fmaf(x4.y, x4.y, ss[t]);
                ss[t] = fmaf(x4.z, x4.z, ss[t]);
                ss[t] = fmaf(x4.w, x4.w, ss[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const float s = wave_sum_all(acc[t]);
        if (lane == 0) part[wave][t] = s;
        if (gamma) {
            const float q = wave_sum_all(ss[t]);
            if (lane == 0) sq[wave][t] = q;
        }
    }
    __syncthreads();
    if (gamma && threadIdx.x < TB) {
        const int t = threadIdx.x;
        const float tot = (sq[0][t] + sq[1][t]) + (sq[2][t] + sq[3][t]);
        inv_rms[t] = 1.0f / sqrtf(tot / (float)d + eps);
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        const float l = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
        const float v = gamma ? l * inv_rms[t] : l;
        if (e < E) L[(size_t)t * E + e] = v;
        else sgl[t] = v;
    }
    if (gamma) {
        xp.gamma = gamma;
        xp.inv_rms = inv_rms;
    }
    xprep_waves(x, T, d, xp, blockIdx.x * 4 + wave, gridDim.x * 4);
}

// ---------------------------------------------------------------------------
// Logits, small T without a fused norm: fp32 matrix-core products
// (v_mfma_f32_16x16x4_f32), d cut into slices of PU * kSmallUnit values.
// Block (r, s) computes router rows 16 r .. 16 r + 15 (the experts, then the
// shared-expert gate as row E) for every token of slice s: no block reads
// more of X and of the router weights than its slice. Wave w takes a quarter
// of the slice in steps of 16 values; in a step lane l (m = l % 16,
// q = l / 16) holds the four values k = 4 q .. 4 q + 3 of token m (the A
// operand) and of router row 16 r + m (B), and four products take one value
// each, so A and B use the same k in every lane. The next four steps' loads
// are in flight during a group's products. Output lane l, register i: token
// 4 q + i, row 16 r + m. The four waves' tiles are added in wave order
// through LDS. With a hidden-state preparation job, nprep more blocks do that
// job alone, alongside the products (grid: nrb * S product blocks, block b
// taking rows 16 (b % nrb) .. of slice b / nrb, then the nprep).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_small_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ wg, int T, int d, int E,
                                                                  int PU, int nrb, int S, float* __restrict__ L,
                                                                  XPrep xp, const float* __restrict__ sg,
                                                                  float* __restrict__ sgl) {
    __shared__ float part[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = blockIdx.x;
    if (b >= nrb * S) {
        const int pb = b - nrb * S;
        xprep_waves(x, T, d, xp, pb * 4 + wave, (gridDim.x - nrb * S) * 4);
        return;
    }
    const int m = lane & 15, q = lane >> 4;
    const int r0 = (b % nrb) * 16, slice = b / nrb;
    const int row = r0 + m;
    const float* wrow = row < E ? wg + (size_t)row * d : (row == E ? sg : nullptr);
    const float* xrow = x + (size_t)min(m, T - 1) * d;   // rows past T repeat the last (unused)
    const int steps = 4 * PU;                             // steps of 16 values per wave
    const int k0 = (slice * 4 + wave) * 16 * steps + 4 * q;
    auto load4 = [&](int j0, float4 (&xa)[4], float4 (&wb)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + 16 * (j0 + j);
            const bool in = j0 + j < steps && k < d;   // d % 4 == 0: a float4 is wholly in or out
            xa[j] = in ? *reinterpret_cast<const float4*>(xrow + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            wb[j] = (in && wrow) ? *reinterpret_cast<const float4*>(wrow + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto mfma4 = [&](const float4 (&xa)[4], const float4 (&wb)[4], v4f acc) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[j].x, wb[j].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[j].y, wb[j].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[j].z, wb[j].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[j].w, wb[j].w, acc, 0, 0, 0);
        }
        return acc;
    };
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    float4 xa[4], wb[4], xb[4], wc[4];
    load4(0, xa, wb);
    for (int j = 0; j < steps; j += 8) {
        load4(j + 4, xb, wc);   // zeros past the slice
        acc = mfma4(xa, wb, acc);
        if (j + 8 < steps) load4(j + 8, xa, wb);
        if (j + 4 < steps) acc = mfma4(xb, wc, acc);
    }
    *reinterpret_cast<float4*>(&part[wave][lane * 4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    {
        // thread o: lane o / 4 of the tiles, register o % 4
        const int o = threadIdx.x, ol = o >> 2;
        const int t = 4 * (ol >> 4) + (o & 3), n = r0 + (ol & 15);
        const float v = (part[0][o] + part[1][o]) + (part[2][o] + part[3][o]);
        if (t < T) {
            if (n < E) L[((size_t)slice * T + t) * E + n] = v;
            else if (n == E && sg) sgl[(size_t)slice * T + t] = v;
        }
    }
}

// RMSNorm of one row per block (the larger-T path writes the normalised rows
// once; every later stage reads them)
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int d,
                                                      const float* __restrict__ gamma, float eps,
                                                      float* __restrict__ xn) {
    __shared__ float part[4];
    const int t = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * d);
    float ss = 0.0f;
    for (int i = threadIdx.x; i < (d >> 2); i += 256) {
        const float4 v = xr[i];
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum_all(ss);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)d + eps);
    float4* dst = reinterpret_cast<float4*>(xn + (size_t)t * d);
    for (int i = threadIdx.x; i < (d >> 2); i += 256) {
        const float4 v = xr[i], g = reinterpret_cast<const float4*>(gamma)[i];
        dst[i] = make_float4(v.x * g.x * inv, v.y * g.y * inv, v.z * g.z * inv, v.w * g.w * inv);
    }
}

// ---------------------------------------------------------------------------
// Logits, larger T: fp32-level products on the f16 matrix cores
// (v_mfma_f32_16x16x32_f16), split over d, in two kernels.
//
// router_prep_kernel, one wave per row of X and of the gate matrix: with
// p = 2^(e-15) where e is the smallest exponent such that the row's largest
// |v| < 2^e, each value splits as v/p = hi + lo, hi = f16(v/p) and
// lo = f16(v/p - hi), both rounded to nearest even (the scaling by a power of
// two and the difference are exact; |v/p| < 2^15 keeps hi finite). Then
// |v/p - hi - lo| <= 2^-22 |v/p| while lo is a normal f16, else <= 2^-25 (an
// absolute bound, 2^-39 of the row's largest value). A product of two parts
// is exact in fp32; hi*hi + hi*lo + lo*hi leaves out lo*lo (<= 2^-22 of
// |x w|), so each product x*w carries a relative error of about 2^-21, below
// the rounding of the fp32 sums it enters. X's waves also take the rest of
// the preparation while they hold the row: the Q8_0 codes of the expert
// kernels, and the shared-expert gate's logit x . sg (fp32 sums in a fixed
// order) into slice 0 of sgl [S, T] with zeros in the other slices. With the
// f32 path's preparation (a power per 32-column group over all rows), waves
// past the rows do that job.
//
// router_logits_f16_kernel<RBN>: block = kRBM tokens x RBN experts (64, or
// 128 where E > 64), RBN / 16 waves of 64 tokens x 32 experts (4 x 2
// products of 16 x 16 per part pair);
// blockIdx.z = slice. The slice goes through LDS kRKC = 32 k (one product) at
// a time, the next chunk's loads in flight while the current one is
// multiplied; the products of the parts are added small ones first, and the
// sum is scaled by the two rows' powers (exact). Rows past T or E read a
// valid row and are never stored.
// ---------------------------------------------------------------------------
constexpr int kRBM = 128, kRKC = 32;

// one row (X row t, or gate row e) by one wave: 8 values per lane and pass
// of 512. NP > 0: the row has at most NP passes and stays in registers (all
// its loads go out together); NP == 0: any length, read twice (the second
// read comes from the cache).
template <int NP>
__device__ __forceinline__ void prep_row(const float* __restrict__ src, int d, int dp, _Float16* __restrict__ hi_out,
                                         _Float16* __restrict__ lo_out, float* __restrict__ pow_out, int t,
                                         const XPrep& xp, bool q8, const float* __restrict__ sg,
                                         float* __restrict__ sgl, int T, int S) {
    constexpr int kPass = 8 * kWave;
    const int lane = threadIdx.x & 63;
    auto load = [&](const float* __restrict__ p, int c, float (&v)[8]) __attribute__((always_inline)) {
        // d % 4 == 0: a float4 is wholly in or out; zeros pad to dp
        const float4 a = c + 4 <= d ? *reinterpret_cast<const float4*>(p + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 b = c + 8 <= d ? *reinterpret_cast<const float4*>(p + c + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
    auto scan = [&](const float (&v)[8], int c, float& amax, float& dot) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
        if (sg) {
            float w[8];
            load(sg, c, w);
#pragma unroll
            for (int j = 0; j < 8; ++j) dot = fmaf(v[j], w[j], dot);
        }
    };
    auto emit = [&](const float (&v)[8], int c, float up) __attribute__((always_inline)) {
        v8h h, l;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float sv = v[j] * up;
            const _Float16 hv = (_Float16)sv;
            h[j] = hv;
            l[j] = (_Float16)(sv - (float)hv);
        }
        *reinterpret_cast<v8h*>(hi_out + c) = h;
        *reinterpret_cast<v8h*>(lo_out + c) = l;
        if (q8 && c < d) {
            // the layer path has d % 32 == 0: the group's four lanes are all here
            const int G = d / kGroup, g = c / kGroup;
            const size_t off = (size_t)t * d + c;
            if (xp.fmt == MOE_W_INT8_G32) q8_store<MOE_W_INT8_G32>(v, off, t * G + g, xp);
            else if (xp.fmt == MOE_W_INT4_G32) q8_store<MOE_W_INT4_G32>(v, off, t * G + g, xp);
            else q8_store<MOE_W_INT2_G32>(v, off, t * G + g, xp);
        }
    };
    float amax = 0.0f, dot = 0.0f;
    int ex;
    if constexpr (NP > 0) {
        float v[NP][8];
#pragma unroll
        for (int p = 0; p < NP; ++p) load(src, p * kPass + 8 * lane, v[p]);
#pragma unroll
        for (int p = 0; p < NP; ++p) scan(v[p], p * kPass + 8 * lane, amax, dot);
        amax = wave_max_all(amax);
        ex = pow2_exponent(amax);
        const float up = ldexpf(1.0f, 15 - ex);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (p * kPass + 8 * lane < dp) emit(v[p], p * kPass + 8 * lane, up);
    } else {
        for (int c = 8 * lane; c < dp; c += kPass) {
            float v[8];
            load(src, c, v);
            scan(v, c, amax, dot);
        }
        amax = wave_max_all(amax);
        ex = pow2_exponent(amax);
        const float up = ldexpf(1.0f, 15 - ex);
        for (int c = 8 * lane; c < dp; c += kPass) {
            float v[8];
            load(src, c, v);
            emit(v, c, up);
        }
    }
    if (sg) dot = wave_sum_all(dot);
    if (lane == 0) pow_out[t] = ldexpf(1.0f, ex - 15);
    if (sg)
        for (int s = lane; s < S; s += kWave) sgl[(size_t)s * T + t] = s == 0 ? dot : 0.0f;
}

// waves 0 .. T-1: rows of X; T .. T+E-1: gate rows; then the f32 path's
// preparation job (XPREP_SPLIT), if any
template <int NP>
__global__ __launch_bounds__(256) void router_prep_kernel(const float* __restrict__ x, int T, int d,
                                                          const float* __restrict__ wg, int E,
                                                          const RouterParts rp, const XPrep xp,
                                                          const float* __restrict__ sg, float* __restrict__ sgl,
                                                          int S) {
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw < T) {
        prep_row<NP>(x + (size_t)gw * d, d, rp.dp, rp.xh + (size_t)gw * rp.dp, rp.xl + (size_t)gw * rp.dp, rp.xp,
                     gw, xp, xp.mode == XPREP_Q8_0, sg, sgl, T, S);
    } else if (gw < T + E) {
        const int e = gw - T;
        prep_row<NP>(wg + (size_t)e * d, d, rp.dp, rp.wh + (size_t)e * rp.dp, rp.wl + (size_t)e * rp.dp, rp.wp, e,
                     xp, false, nullptr, nullptr, T, S);
    } else if (xp.mode == XPREP_SPLIT) {
        xprep_waves(x, T, d, xp, gw - T - E, gridDim.x * 4 - T - E);
    }
}

template <int RBN>
__global__ __launch_bounds__(4 * RBN) void router_logits_f16_kernel(const RouterParts rp, int T, int E, int kslice,
                                                                    float* __restrict__ L) {
    // [part][16-row tile][64 lanes][8 halves], parts hi, lo: lane l = r + 16 h
    // of a tile holds row r, k 8 h .. 8 h + 7 (the matrix-core operand as it
    // is read: every 16-byte read and write of a wave covers 1 KB without bank
    // conflicts)
    // two buffers: chunk c + 1 is stored into one while chunk c is multiplied
    // out of the other, one barrier per chunk
    __shared__ __attribute__((aligned(16))) _Float16 xsb[2][2 * kRBM * kRKC];
    __shared__ __attribute__((aligned(16))) _Float16 wsb[2][2 * RBN * kRKC];
    constexpr int kThreads = 4 * RBN;           // RBN / 16 waves
    constexpr int kXR = kRBM * 4 / kThreads;    // token rows per thread (one expert row each)
    static_assert(kRBM == 128 && (RBN == 64 || RBN == 128), "tile shapes");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave & 1, wn = wave >> 1;
    // XCD-aware order (blocks go to the 8 XCDs in turn by linear id): every
    // (expert tile, slice) block of one token tile runs on the same XCD, so
    // the token rows come into that XCD's L2 once. The grid's token-tile
    // count is padded to a multiple of 8; padding tiles exit here.
    const int ncol = gridDim.x * gridDim.z;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int sl = lin >> 3, col = sl % ncol;
    const int tb = ((sl / ncol) * 8 + (lin & 7)) * kRBM;
    if (tb >= T) return;
    const int eb = (col % gridDim.x) * RBN;
    const int ks = col / gridDim.x;
    const int dp = rp.dp;
    const int kbeg = ks * kslice, kend = min(dp, kbeg + kslice);
    // loads: token rows lr + (kThreads / 4) j and expert row lr, halves
    // 8 lq .. 8 lq + 7 of each 32-wide chunk (four neighbouring lanes read one
    // row's 64 bytes); dp % 32 == 0 and kslice % 64 == 0: every chunk is
    // whole; rows past T or E read the last valid row (never stored)
    const int lr = tid >> 2, lq = (tid & 3) * 8;
    size_t xr[kXR];
#pragma unroll
    for (int j = 0; j < kXR; ++j) xr[j] = (size_t)min(tb + lr + (kThreads / 4) * j, T - 1) * dp + lq;
    const size_t wrow = (size_t)min(eb + lr, E - 1) * dp + lq;
    uint4 xh[kXR], xl[kXR], wh0, wl0;
    // LDS position (16-byte units) of row r % 16 of a tile, halves 8 h ..:
    // slot r + 16 h with r XOR (4 h ^ (h & 2)). Each 8 (and 16) lanes of a
    // write (two (four) rows x four quads) and of a read (eight (sixteen)
    // rows, one quad) then land in 8 (16) different 16-byte bank groups.
    auto pos = [](int r, int h) { return ((r & 15) ^ (4 * h ^ (h & 2))) + 16 * h; };
    const int hq = tid & 3;
    auto ld16 = [](const _Float16* p) { return *reinterpret_cast<const uint4*>(p); };
    auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            xh[j] = ld16(rp.xh + xr[j] + k0);
            xl[j] = ld16(rp.xl + xr[j] + k0);
        }
        wh0 = ld16(rp.wh + wrow + k0);
        wl0 = ld16(rp.wl + wrow + k0);
    };
    // operand rows of this lane: tokens 64 wm + 16 i + (lane % 16), experts
    // 32 wn + 16 j + (lane % 16); k 8 (lane / 16) .. + 7 of the chunk, at
    // position rl of each tile
    const int orow = lane & 15, rl = pos(orow, lane >> 4);
    v4f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    auto stage = [&](_Float16* xs, _Float16* wsh) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            const int rr = lr + (kThreads / 4) * j;
            *reinterpret_cast<uint4*>(&xs[((rr >> 4) * 64 + pos(rr, hq)) * 8]) = xh[j];
            *reinterpret_cast<uint4*>(&xs[(((kRBM >> 4) + (rr >> 4)) * 64 + pos(rr, hq)) * 8]) = xl[j];
        }
        *reinterpret_cast<uint4*>(&wsh[((lr >> 4) * 64 + pos(lr, hq)) * 8]) = wh0;
        *reinterpret_cast<uint4*>(&wsh[(((RBN >> 4) + (lr >> 4)) * 64 + pos(lr, hq)) * 8]) = wl0;
    };
    auto multiply = [&](const _Float16* xs, const _Float16* wsh) __attribute__((always_inline)) {
        v8h b[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                b[j][p] = *reinterpret_cast<const v8h*>(&wsh[((p * (RBN >> 4) + 2 * wn + j) * 64 + rl) * 8]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v8h a[2];
#pragma unroll
            for (int p = 0; p < 2; ++p)
                a[p] = *reinterpret_cast<const v8h*>(&xs[((p * (kRBM >> 4) + 4 * wm + i) * 64 + rl) * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // the small terms first
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[j][0], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[j][1], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[j][0], acc[i][j], 0, 0, 0);
            }
        }
    };
    // chunk c lives in buffer c % 2; at step c the registers hold chunk c + 1,
    // which goes into the other buffer (read last at step c - 1, before the
    // barrier that ended it) while chunk c is multiplied; then the loads of
    // chunk c + 2 go out
    const int nchunk = kend > kbeg ? (kend - kbeg) / kRKC : 0;
    if (nchunk > 0) {
        gload(kbeg);
        stage(xsb[0], wsb[0]);
        if (nchunk > 1) gload(kbeg + kRKC);
        __syncthreads();
    }
    for (int c = 0; c < nchunk; ++c) {
        const int cur = c & 1;
        if (c + 1 < nchunk) {
            stage(xsb[cur ^ 1], wsb[cur ^ 1]);
            if (c + 2 < nchunk) gload(kbeg + (c + 2) * kRKC);
        }
        multiply(xsb[cur], wsb[cur]);
        __syncthreads();
    }
    // output lane l, register r: token 4 (l / 16) + r, expert l % 16 of the
    // tile pair; the rows' powers first (all loads out together), then the
    // stores
    float* out = L + (size_t)ks * T * E;
    float pe[2], pt[4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) pe[j] = rp.wp[min(eb + 32 * wn + 16 * j + orow, E - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) pt[i][r] = rp.xp[min(tb + 64 * wm + 16 * i + 4 * (lane >> 4) + r, T - 1)];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = eb + 32 * wn + 16 * j + orow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tb + 64 * wm + 16 * i + 4 * (lane >> 4) + r;
                if (t < T && e < E) out[(size_t)t * E + e] = (acc[i][j][r] * pt[i][r]) * pe[j];
            }
    }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const TopkArgs a, int* __restrict__ idx_out,
                                                          float* __restrict__ w_out) {
    __shared__ __attribute__((aligned(16))) float keybuf[4][kMaxExperts];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    const bool active = t < a.T;
    int my_e;
    float my_w;
    topk_token<EPL>(a, t, active, keybuf[wave], &my_e, &my_w);
    if (active && lane < a.k) {
        idx_out[(size_t)t * a.k + lane] = my_e;
        w_out[(size_t)t * a.k + lane] = my_w;
    }
}

TopkArgs topk_args(const float* logits, int T, int S, const moe_router_params& p) {
    TopkArgs a;
    a.L = logits;
    a.S = S;
    a.T = T;
    a.E = p.n_experts;
    a.k = p.top_k;
    a.mode = p.mode;
    a.renorm = p.renormalize;
    a.n_group = p.n_group;
    a.topk_group = p.topk_group;
    a.rsf = p.routed_scaling_factor;
    a.bias = p.score_bias;
    a.top_p = (p.top_p > 0.0f && p.top_p < 1.0f) ? p.top_p : 0.0f;
    return a;
}

hipError_t launch_router_logits(const float* x, int T, int d, const float* wg, int E, float* logits,
                                const XPrep& xp, const float* norm_w, float eps, const float* sg, float* sgl,
                                const RouterParts* rp, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int S = router_splits(T, E, d);
    const int rows = E + (sg ? 1 : 0);   // experts, then the shared-expert gate
    if (S == 0 && !norm_w && T > kSmallSplitMinT) {
        const int nrb = (rows + 15) / 16, SS = router_slices(T, E, d, false);
        // preparation blocks: enough waves for one pass over the job
        const int nprep = (xprep_waves_wanted(T, d, xp) + 3) / 4;
        hipLaunchKernelGGL(router_logits_small_kernel, dim3(nrb * SS + nprep), dim3(256), 0, st, x, wg, T, d, E,
                           router_small_units(d), nrb, SS, logits, xp, sg, sgl);
        return hipGetLastError();
    }
    if (S == 0) {
        const dim3 grid(rows);
#define MOE_RL(TB)                                                                                            \
    hipLaunchKernelGGL(router_logits_gemv_kernel<TB>, grid, dim3(256), 0, st, x, wg, T, d, E, logits, xp, norm_w, \
                       eps, sg, sgl)
        if (T == 1) MOE_RL(1);
        else if (T <= 2) MOE_RL(2);
        else if (T <= 4) MOE_RL(4);
        else if (T <= 8) MOE_RL(8);
        else MOE_RL(16);
#undef MOE_RL
        return hipGetLastError();
    }
    // larger T: the operand parts (and the rest of the preparation), then
    // the products
    if (rp == nullptr || rp->dp != router_row_pad(d)) return hipErrorInvalidValue;
    const int split_waves = xp.mode == XPREP_SPLIT ? xprep_waves_wanted(T, d, xp) : 0;
    const dim3 pgrid((T + E + split_waves + 3) / 4);
    const int passes = (rp->dp + 8 * kWave - 1) / (8 * kWave);
#define MOE_PREP(NP) hipLaunchKernelGGL(router_prep_kernel<NP>, pgrid, dim3(256), 0, st, x, T, d, wg, E, *rp, xp, sg, sgl, S)
    if (passes <= 1) MOE_PREP(1);
    else if (passes <= 2) MOE_PREP(2);
    else if (passes <= 4) MOE_PREP(4);
    else MOE_PREP(0);
#undef MOE_PREP
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int gy = ((T + kRBM - 1) / kRBM + 7) / 8 * 8, kslice = router_kslice(d, S);
    if (E > 64)
        hipLaunchKernelGGL(router_logits_f16_kernel<128>, dim3((E + 127) / 128, gy, S), dim3(512), 0, st, *rp, T, E,
                           kslice, logits);
    else
        hipLaunchKernelGGL(router_logits_f16_kernel<64>, dim3(1, gy, S), dim3(256), 0, st, *rp, T, E, kslice, logits);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int T, int d, const float* norm_w, float eps, float* xn, hipStream_t st) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, st, x, d, norm_w, eps, xn);
    return hipGetLastError();
}

hipError_t launch_xprep(const float* x, int T, int d, const XPrep& xp, hipStream_t st) {
    const int waves = xprep_waves_wanted(T, d, xp);
    if (T == 0 || waves == 0) return hipSuccess;
    hipLaunchKernelGGL(xprep_kernel, dim3((waves + 3) / 4), dim3(256), 0, st, x, T, d, xp);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int T, int S, const moe_router_params& p, int* idx, float* w,
                              hipStream_t st) {
    if (T == 0) return hipSuccess;
    const TopkArgs a = topk_args(logits, T, S, p);
    const dim3 grid((T + 3) / 4);
#define MOE_TOPK(EPL) hipLaunchKernelGGL(router_topk_kernel<EPL>, grid, dim3(256), 0, st, a, idx, w)
    switch (topk_epl(p.n_experts)) {
        case 1: MOE_TOPK(1); break;
        case 2: MOE_TOPK(2); break;
        case 4: MOE_TOPK(4); break;
        case 8: MOE_TOPK(8); break;
        default: MOE_TOPK(16); break;
    }
#undef MOE_TOPK
    return hipGetLastError();
}

hipError_t launch_router(const float* x, int T, int d, const float* wg, const moe_router_params& p,
                         float* logits, const RouterParts* rp, int* idx, float* w, hipStream_t st) {
    hipError_t err =
        launch_router_logits(x, T, d, wg, p.n_experts, logits, XPrep{}, nullptr, 0.0f, nullptr, nullptr, rp, st);
    if (err != hipSuccess) return err;
    return launch_router_topk(logits, T, router_slices(T, p.n_experts, d, false), p, idx, w, st);
}

}  // namespace moe
