// Decode path: batch-union grouped GEMV with group-32 weights dequantised on
// load ("Show HN: colibri", section "What's implemented": int8 / packed int4
// weights dequantised on use; a single row stays in f32 rather than going
// through int8 activations).
//
// Grid: blockIdx.y = slot (an expert with rows, or the shared expert),
// blockIdx.x = a block of output rows of that expert's matrix. Each expert's
// weights are therefore streamed from HBM once, whatever number of tokens it
// serves (batch-union); the tokens' activations sit in registers.
//
// Layout of the work inside a wave: LPR lanes cover one output row, lane
// `sub` owning groups sub, sub + LPR, ... (NCH of them). A group is 32
// consecutive weights: one 16-byte load of packed int4 or two of int8, plus
// one fp32 scale. Each lane keeps the 32*NCH activations of its groups for
// BT tokens in registers, so each weight byte loaded is used BT times.
//
// Dequantisation without a sign extension: XOR with 0x80 (int8) or 0x8
// (int4 nibble) turns a code q into q + 128 (q + 8) as an unsigned byte,
// which converts to float in one instruction; the constant offset times the
// group's activation sum is subtracted once per group:
//   sum_k x_k q_k = sum_k x_k (q_k + c) - c * sum_k x_k.
#include "common.h"
#include "kernels.h"

namespace moe {

struct GemvMat {
    const uint8_t* q;   // expert 0's codes
    const float* s;     // expert 0's scales
    int64_t q_stride;   // bytes per expert
    int64_t s_stride;   // floats per expert
};

struct GemvArgs {
    const float* x;         // activation rows, row length K
    const int* row_token;   // permuted row -> activation row (nullptr: identity)
    const int4* slots;      // (expert, row_begin, n_rows, 0)
    const int* meta;        // meta[0] = number of slots
    GemvMat routed[2];      // gate, up (gate/up kernel) or down (down kernel)
    GemvMat shared[2];
    int E;                  // a slot with expert == E uses the shared weights
    int K, N;               // reduction length; output rows of each matrix
    int lpr;                // lanes per output row (power of two <= 64)
    int rows_per_wave;      // a multiple of 64 / lpr
    float* out;             // [rows, N]
};

template <int CTRL>
__device__ __forceinline__ float dpp_src(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned segment of `lpr` lanes; the total lands in the
// segment's first lane (other lanes hold partial sums). DPP steps inside a
// row of 16 lanes, a swizzle across 16, a lane read across 32.
__device__ __forceinline__ float segment_reduce(float v, int lpr) {
    if (lpr >= 2) v += dpp_src<0xB1>(v);    // quad_perm [1,0,3,2]
    if (lpr >= 4) v += dpp_src<0x4E>(v);    // quad_perm [2,3,0,1]
    if (lpr >= 8) v += dpp_src<0x141>(v);   // row_half_mirror
    if (lpr >= 16) v += dpp_src<0x140>(v);  // row_mirror
    if (lpr >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // xor 16
    if (lpr >= 64) v += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return v;
}

// Weight-stationary batch-union GEMV. A wave owns NP passes of rpp = 64/lpr
// output rows; it issues the loads of all of them (NMAT matrices, NCH groups
// per lane) at once, keeps the codes in registers, and then runs the slot's
// tokens past them BT at a time, so each weight byte leaves HBM once per
// slot whatever the number of tokens.
// Hides a register's value from the optimiser, so the decode of the codes
// stays inside the token loop instead of being hoisted as 4x more floats.
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Passes per wave: enough rows that about 64 dwords of codes are in flight.
__host__ __device__ constexpr int gemv_passes(int fmt, int nch, int nmat) {
    return (64 / (nmat * nch * (fmt == MOE_W_INT8_G32 ? 8 : 4))) < 1 ? 1
           : (64 / (nmat * nch * (fmt == MOE_W_INT8_G32 ? 8 : 4))) > 8 ? 8
           : 64 / (nmat * nch * (fmt == MOE_W_INT8_G32 ? 8 : 4));
}

template <int FMT, int NCH, int BT, int NMAT>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvArgs a) {
    constexpr int kDw = FMT == MOE_W_INT8_G32 ? 8 : 4;   // dwords per group
    constexpr int NP = gemv_passes(FMT, NCH, NMAT);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = blockIdx.y;
    if (slot >= a.meta[0]) return;
    const int4 sl = a.slots[slot];
    const int e = sl.x, row_begin = sl.y, n_rows = sl.z;
    const bool is_shared = e == a.E;
    const GemvMat* M = is_shared ? a.shared : a.routed;
    const int64_t eo = is_shared ? 0 : e;

    const int G = a.K / kGroup;
    const int lpr = a.lpr;
    const int rpp = kWave / lpr;
    const int sub = lane & (lpr - 1);
    const int rsub = lane / lpr;
    const int n_base = (blockIdx.x * 4 + wave) * NP * rpp + rsub;
    const int row_bytes = FMT == MOE_W_INT8_G32 ? a.K : a.K / 2;

    // ---- all weight loads of this wave, up front ----
    uint32_t wd[NP][NMAT][NCH][kDw];
    float sc[NP][NMAT][NCH];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int n = n_base + p * rpp;
        const bool vn = n < a.N;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint8_t* rowp = M[m].q + eo * M[m].q_stride + (size_t)(vn ? n : 0) * row_bytes;
            const float* srow = M[m].s + eo * M[m].s_stride + (size_t)(vn ? n : 0) * G;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int gi = c * lpr + sub;
                const bool v = vn && gi < G;
                const uint4* src = reinterpret_cast<const uint4*>(rowp + (size_t)(v ? gi : 0) * (kDw * 4));
#pragma unroll
                for (int h = 0; h < kDw / 4; ++h) {
                    const uint4 u = v ? src[h] : make_uint4(0, 0, 0, 0);
                    wd[p][m][c][4 * h + 0] = u.x;
                    wd[p][m][c][4 * h + 1] = u.y;
                    wd[p][m][c][4 * h + 2] = u.z;
                    wd[p][m][c][4 * h + 3] = u.w;
                }
                sc[p][m][c] = v ? srow[gi] : 0.0f;
            }
        }
    }

    for (int tb = 0; tb < n_rows; tb += BT) {
        // activations of BT tokens for this lane's groups
        float xr[BT][NCH][kGroup];
        float xs[BT][NCH];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const int r = tb + b;
            const bool vr = r < n_rows;
            const int xrow = vr ? (a.row_token ? a.row_token[row_begin + r] : row_begin + r) : 0;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int gi = c * lpr + sub;
                const bool vg = vr && gi < G;
                const float4* src =
                    reinterpret_cast<const float4*>(a.x + (size_t)xrow * a.K + (size_t)(vg ? gi : 0) * kGroup);
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < kGroup / 4; ++q) {
                    const float4 f = vg ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
                    xr[b][c][4 * q + 0] = f.x;
                    xr[b][c][4 * q + 1] = f.y;
                    xr[b][c][4 * q + 2] = f.z;
                    xr[b][c][4 * q + 3] = f.w;
                    s += (f.x + f.y) + (f.z + f.w);
                }
                xs[b][c] = s;
            }
        }

#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float acc[NMAT][BT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
#pragma unroll
                for (int b = 0; b < BT; ++b) acc[m][b] = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    float dot[BT];
#pragma unroll
                    for (int b = 0; b < BT; ++b) dot[b] = 0.0f;
                    if constexpr (FMT == MOE_W_INT8_G32) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            uint32_t raw = wd[p][m][c][j];
                            opaque(raw);
                            const uint32_t u = raw ^ 0x80808080u;
                            const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
                            const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
#pragma unroll
                            for (int b = 0; b < BT; ++b) {
                                dot[b] = fmaf(xr[b][c][4 * j + 0], f0, dot[b]);
                                dot[b] = fmaf(xr[b][c][4 * j + 1], f1, dot[b]);
                                dot[b] = fmaf(xr[b][c][4 * j + 2], f2, dot[b]);
                                dot[b] = fmaf(xr[b][c][4 * j + 3], f3, dot[b]);
                            }
                        }
#pragma unroll
                        for (int b = 0; b < BT; ++b)
                            acc[m][b] = fmaf(sc[p][m][c], fmaf(-128.0f, xs[b][c], dot[b]), acc[m][b]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            uint32_t raw = wd[p][m][c][j];
                            opaque(raw);
                            const uint32_t u = raw ^ 0x88888888u;
                            const uint32_t lo = u & 0x0f0f0f0fu, hi = (u >> 4) & 0x0f0f0f0fu;
                            float f[8];
                            f[0] = (float)(lo & 0xffu);
                            f[1] = (float)(hi & 0xffu);
                            f[2] = (float)((lo >> 8) & 0xffu);
                            f[3] = (float)((hi >> 8) & 0xffu);
                            f[4] = (float)((lo >> 16) & 0xffu);
                            f[5] = (float)((hi >> 16) & 0xffu);
                            f[6] = (float)(lo >> 24);
                            f[7] = (float)(hi >> 24);
#pragma unroll
                            for (int b = 0; b < BT; ++b)
#pragma unroll
                                for (int i = 0; i < 8; ++i) dot[b] = fmaf(xr[b][c][8 * j + i], f[i], dot[b]);
                        }
#pragma unroll
                        for (int b = 0; b < BT; ++b)
                            acc[m][b] = fmaf(sc[p][m][c], fmaf(-8.0f, xs[b][c], dot[b]), acc[m][b]);
                    }
                }
#pragma unroll
                for (int b = 0; b < BT; ++b) acc[m][b] = segment_reduce(acc[m][b], lpr);
            }
            const int n = n_base + p * rpp;
            if (sub == 0 && n < a.N) {
#pragma unroll
                for (int b = 0; b < BT; ++b) {
                    if (tb + b < n_rows) {
                        float v;
                        if constexpr (NMAT == 2) v = silu(acc[0][b]) * acc[1][b];
                        else v = acc[0][b];
                        a.out[(size_t)(row_begin + tb + b) * a.N + n] = v;
                    }
                }
            }
        }
    }
}

static int lanes_per_row(int K) {
    const int G = K / kGroup;
    int lpr = 1;
    while (lpr < G && lpr < kWave) lpr <<= 1;
    return lpr;
}

template <int FMT, int NMAT>
static hipError_t launch_gemv_fmt(GemvArgs a, int max_slots, int bt_hint, hipStream_t st) {
    const int G = a.K / kGroup;
    const int nch = (G + a.lpr - 1) / a.lpr;
    const int rpp = kWave / a.lpr;
    a.rows_per_wave = gemv_passes(FMT, nch, NMAT) * rpp;
    const dim3 grid((a.N + 4 * a.rows_per_wave - 1) / (4 * a.rows_per_wave), max_slots);
    // tokens per register batch: a slot serves at most bt_hint tokens
    const int bt = nch >= 3 ? 1 : (bt_hint >= 2 ? 2 : 1);
#define MOE_GEMV(NCH, BT) hipLaunchKernelGGL((gemv_kernel<FMT, NCH, BT, NMAT>), grid, dim3(256), 0, st, a)
    switch (nch) {
        case 1:
            if (bt == 2) MOE_GEMV(1, 2);
            else MOE_GEMV(1, 1);
            break;
        case 2:
            if (bt == 2) MOE_GEMV(2, 2);
            else MOE_GEMV(2, 1);
            break;
        case 3: MOE_GEMV(3, 1); break;
        case 4: MOE_GEMV(4, 1); break;
        default: return hipErrorInvalidValue;
    }
#undef MOE_GEMV
    return hipGetLastError();
}

hipError_t launch_gemv(const ExpertsView& routed, const ExpertsView* shared, bool gateup, const float* x,
                       const int* row_token, const int* slots, const int* meta, int max_slots, int bt_hint,
                       float* out, hipStream_t st) {
    GemvArgs a{};
    a.x = x;
    a.row_token = row_token;
    a.slots = reinterpret_cast<const int4*>(slots);
    a.meta = meta;
    a.E = routed.n_experts;
    const int d = routed.d_model, I = routed.d_ff;
    a.K = gateup ? d : I;
    a.N = gateup ? I : d;
    a.lpr = lanes_per_row(a.K);
    a.out = out;
    auto fill = [&](GemvMat* dst, const ExpertsView& ev) {
        const int64_t rowb = ev.format == MOE_W_INT8_G32 ? a.K : a.K / 2;
        const int64_t qs = (int64_t)a.N * rowb, ss = (int64_t)a.N * (a.K / kGroup);
        if (gateup) {
            dst[0] = GemvMat{(const uint8_t*)ev.gate_q, ev.gate_s, qs, ss};
            dst[1] = GemvMat{(const uint8_t*)ev.up_q, ev.up_s, qs, ss};
        } else {
            dst[0] = GemvMat{(const uint8_t*)ev.down_q, ev.down_s, qs, ss};
            dst[1] = dst[0];
        }
    };
    fill(a.routed, routed);
    if (shared) fill(a.shared, *shared);
    else fill(a.shared, routed);
    if (max_slots == 0) return hipSuccess;
    if (routed.format == MOE_W_INT8_G32)
        return gateup ? launch_gemv_fmt<MOE_W_INT8_G32, 2>(a, max_slots, bt_hint, st)
                      : launch_gemv_fmt<MOE_W_INT8_G32, 1>(a, max_slots, bt_hint, st);
    return gateup ? launch_gemv_fmt<MOE_W_INT4_G32, 2>(a, max_slots, bt_hint, st)
                  : launch_gemv_fmt<MOE_W_INT4_G32, 1>(a, max_slots, bt_hint, st);
}

}  // namespace moe
