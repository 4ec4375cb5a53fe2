// Decode path (fp32 activations): batch-union grouped GEMV on the f16 matrix
// cores, weights dequantised on use ("Show HN: colibri", section "What's
// implemented": int8 / packed int4 weights dequantised on use; batch-union
// over the positions routed to one expert; a single row stays in f32).
//
// Exact fp32-level activations on f16 matrix cores. For every tile of up to 16
// activation rows of one expert and group of 32, a power of two p = 2^(e-15)
// with max|x| < 2^e is chosen and x/p (exact) is split into hi = f16(x/p) and
// lo = f16(x/p - hi): together 22 significant bits. Weight codes are small integers, exact in f16. So
//     sum_k x_k q_k = p * (MFMA(hi, q) + MFMA(lo, q))
// with exact products and fp32 accumulation (v_mfma_f32_16x16x32_f16, K = 32
// = one quantisation group); the group's weight scale and p are applied once
// per output per group.
//
// Three kernels:
//   prep:    the activations of every permuted row (token of each routed
//            assignment, then the shared expert's tokens) as hi/lo, with one
//            p per (16-row tile of a slot, group).
//   gate/up: per (expert, 32 weight rows): G and U for the expert's tokens,
//            H = silu(G) * U written straight back as hi/lo + p per 32.
//   down:    Y = H Wd^T, fp32, rows in permuted order.
// Weight codes come straight from HBM into operand registers: in the 32-row
// tiled layout, 16 rows x one group are 512 (int8) or 256 (int4) contiguous
// bytes, which a wave reads as one load. Activation fragments come from L2;
// token rows past an expert's count are masked, so they cost no traffic.
//
// Codes to f16 without a conversion instruction: an unsigned byte u ORed
// into 0x6400 is the f16 number 1024 + u; a packed f16 subtract of 1152
// (int8 after XOR 0x80) or 1032 (int4 after XOR 0x8) leaves the signed code.
// That pairs bytes (0,2),(1,3) of an int8 dword and nibbles (0,4),(1,5),
// (2,6),(3,7) of an int4 dword; activations are stored in the same k order
// inside every 8-wide slice, and a dot product ignores the order of terms.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// k offset (0..7) inside an 8-wide slice for operand slot j
__host__ __device__ constexpr int slot_k(int fmt, int j) {
    return fmt == MOE_W_INT8_G32 ? ((j & 4) | ((j & 1) << 1) | ((j >> 1) & 1)) : (((j & 1) << 2) | (j >> 1));
}

// operand slot holding k offset kin (0..7) of an 8-wide slice
__host__ __device__ constexpr int k_slot(int fmt, int kin) {
    return fmt == MOE_W_INT8_G32 ? ((kin & 4) | ((kin & 2) >> 1) | ((kin & 1) << 1)) : (((kin & 3) << 1) | (kin >> 2));
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// 8 codes of one lane slice -> 8 f16 in slot order
template <int FMT>
__device__ __forceinline__ v8h codes_to_f16(uint32_t w0, uint32_t w1) {
    union {
        uint32_t u[4];
        v8h h;
    } r;
    v2h off;
    if constexpr (FMT == MOE_W_INT8_G32) {
        const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
        r.u[0] = and_or(a, 0x00ff00ffu, 0x64006400u);
        r.u[1] = and_or(a >> 8, 0x00ff00ffu, 0x64006400u);
        r.u[2] = and_or(b, 0x00ff00ffu, 0x64006400u);
        r.u[3] = and_or(b >> 8, 0x00ff00ffu, 0x64006400u);
        off = v2h{(_Float16)-1152.0f, (_Float16)-1152.0f};
    } else {
        const uint32_t a = w0 ^ 0x88888888u;
        r.u[0] = and_or(a, 0x000f000fu, 0x64006400u);
        r.u[1] = and_or(a >> 4, 0x000f000fu, 0x64006400u);
        r.u[2] = and_or(a >> 8, 0x000f000fu, 0x64006400u);
        r.u[3] = and_or(a >> 12, 0x000f000fu, 0x64006400u);
        off = v2h{(_Float16)-1032.0f, (_Float16)-1032.0f};
        (void)w1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r.u[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, r.u[i]) + off);
    return r.h;
}

// exponent e with |x| < 2^e for x = amax (0 -> 0), clamped so 2^(15-e) stays finite
__device__ __forceinline__ int pow2_exponent(float amax) {
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);
    return min(max(ex, -100), 120);
}

// ---------------------------------------------------------------------------
// prep: block (slot, 8 groups); each wave takes 2 groups of every 16-row tile
// of the slot: lane -> (row r = lane % 16, group of the pair, half of 32)
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void prep_act_kernel(const float* __restrict__ x, const int* __restrict__ row_token,
                                                       const int4* __restrict__ slots, const int* __restrict__ meta,
                                                       int R, int K, _Float16* __restrict__ ahi,
                                                       _Float16* __restrict__ alo, float* __restrict__ apow) {
    const int slot = blockIdx.y;
    if (slot >= meta[0]) return;
    const int4 sl = slots[slot];
    const int row_begin = sl.y, n_rows = sl.z;
    const int G = K / kGroup;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, gsel = (lane >> 4) & 1, half = lane >> 5;
    const int g = blockIdx.x * 8 + wave * 2 + gsel;
    const bool g_ok = g < G;
    for (int mt = 0; mt < n_rows; mt += 16) {
        const bool ok = g_ok && r < n_rows - mt;
        const int p = row_begin + mt + r;
        float v[16];
        const float4* src = reinterpret_cast<const float4*>(x + (size_t)(ok ? row_token[p] : 0) * K +
                                                            (size_t)(g_ok ? g : 0) * kGroup + 16 * half);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = ok ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
        // max over the 16 rows (a DPP row) and the two halves (lanes l, l ^ 32)
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1, 0xF, 0xF, true)));
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E, 0xF, 0xF, true)));
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x141, 0xF, 0xF, true)));
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x140, 0xF, 0xF, true)));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int ex = pow2_exponent(amax);
        const float up = ldexpf(1.0f, 15 - ex);
        if (ok) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                v8h hi, lo;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sv = v[8 * s2 + slot_k(FMT, j)] * up;
                    const _Float16 hv = (_Float16)sv;
                    hi[j] = hv;
                    lo[j] = (_Float16)(sv - (float)hv);
                }
                const size_t off = (size_t)p * K + (size_t)g * kGroup + 16 * half + 8 * s2;
                *reinterpret_cast<v8h*>(ahi + off) = hi;
                *reinterpret_cast<v8h*>(alo + off) = lo;
            }
        }
        if (g_ok && r == 0 && half == 0) apow[(size_t)g * R + row_begin + mt] = ldexpf(1.0f, ex - 15);
    }
}

struct GemvArgs {
    const _Float16* ahi;    // activation parts [R, K] in slot order
    const _Float16* alo;
    const float* apow;      // [K/32, R], at the first row of each 16-row tile
    const int4* slots;      // (expert, row_begin, n_rows, 0)
    const int* meta;        // meta[0] = number of slots
    const uint8_t* q[2];    // routed codes: gate, up (gate/up) or down, down
    const float* s[2];
    const uint8_t* sq[2];   // shared expert
    const float* ss[2];
    int64_t q_stride, s_stride;   // per expert (bytes, floats)
    int E, K, N, R;
    // gate/up output: H as parts + powers of two for the down kernel
    _Float16* hhi;
    _Float16* hlo;
    float* hpow;            // [N/32, R], at the first row of each 16-row tile
    // down output
    float* y;               // [R, N]
};

// Operands in flight per wave: NB groups ahead, weight codes (HBM) and
// activation fragments (L2) alike. Loads retire in order, so a shallower
// activation ring would make every wait cover the deeper weight loads too.
__host__ __device__ constexpr int gemv_nb(int fmt, int nmat) { return (fmt == MOE_W_INT8_G32 && nmat == 2) ? 4 : 6; }

// Block: 2 x KS waves. Wave (wn, ks): weight rows 32 * tile + 16 wn .. + 16,
// groups ks, ks + KS, ... of the reduction axis.
template <int FMT, int NMAT, int KS>
__global__ __launch_bounds__(128 * KS) void gemv_kernel(const GemvArgs a) {
    constexpr int kDw = FMT == MOE_W_INT8_G32 ? 2 : 1;      // code dwords per lane per group
    constexpr int kBpg = FMT == MOE_W_INT8_G32 ? 32 : 16;   // code bytes per row per group
    constexpr int NB = gemv_nb(FMT, NMAT);
    constexpr int kNA = NB;
    __shared__ float red[KS > 1 ? 2 * KS : 1][NMAT][64][4];
    __shared__ float hmax[2];

    const int slot = blockIdx.y;
    if (slot >= a.meta[0]) return;
    const int4 sl = a.slots[slot];
    const int e = sl.x, row_begin = sl.y, n_rows = sl.z;
    const bool is_shared = e == a.E;
    const int64_t eo = is_shared ? 0 : e;
    // the wave index is uniform across the wave; say so, so that group offsets
    // stay in scalar registers
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave & 1, ks = wave >> 1;
    const int K = a.K, N = a.N, G = K / kGroup, R = a.R;
    const int h = lane >> 4, nl = lane & 15;
    const int tile = blockIdx.x;                       // 32-row tile of every matrix
    const int n = tile * kTile + wn * 16 + nl;         // this lane's weight row (B operand column)
    // operands through buffer resources: one lane offset per stream, the group
    // step in a uniform register; offsets past a resource's end read as 0
    __amdgpu_buffer_rsrc_t rq[NMAT], rs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint8_t* qbase = (is_shared ? a.sq[m] : a.q[m]) + eo * a.q_stride;
        const float* sbase = (is_shared ? a.ss[m] : a.s[m]) + eo * a.s_stride;
        rq[m] = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, 0, (int)a.q_stride, 0x00020000);
        rs[m] = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, (int)(a.s_stride * 4), 0x00020000);
    }
    const int q_voff = tile * G * (kTile * kBpg) + (wn * 16 + nl) * kBpg + (kBpg / 4) * h;
    const int s_voff = (tile * G * kTile + wn * 16 + nl) * 4;
    const __amdgpu_buffer_rsrc_t rah = __builtin_amdgcn_make_buffer_rsrc((void*)a.ahi, 0, R * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t ral = __builtin_amdgcn_make_buffer_rsrc((void*)a.alo, 0, R * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rpw = __builtin_amdgcn_make_buffer_rsrc((void*)a.apow, 0, R * G * 4, 0x00020000);
    const int n_my = (G - ks + KS - 1) / KS;           // groups of this wave: ks + KS * j

    for (int mt = 0; mt < n_rows; mt += 16) {
        const int rows_here = min(16, n_rows - mt);
        const bool a_ok = nl < rows_here;
        // rows past the expert's count read past the resource: zeros, no traffic
        const int a_voff = a_ok ? ((row_begin + mt + nl) * K + 8 * h) * 2 : 0x7ffffff0;
        const int pw_off = (row_begin + mt) * 4;      // apow[g][row_begin + mt]: one per group for the tile
        const int prow = row_begin + mt + 4 * h;        // output rows (tokens) 4h .. 4h + 3 of the tile

        v4f acc[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};

        uint32_t wc[NB][NMAT][kDw];
        float wsc[NB][NMAT];
        v8h xh[kNA], xl[kNA];
        float xpw[kNA];
        auto load_b = [&](int sp, int j) {
            const int g = ks + KS * (j < n_my ? j : 0);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                if constexpr (kDw == 2) {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rq[m], q_voff, g * (kTile * kBpg), 0);
                    wc[sp][m][0] = v[0];
                    wc[sp][m][1] = v[1];
                } else {
                    wc[sp][m][0] = __builtin_amdgcn_raw_buffer_load_b32(rq[m], q_voff, g * (kTile * kBpg), 0);
                }
                wsc[sp][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs[m], s_voff, g * kTile * 4, 0));
            }
        };
        auto load_a = [&](int sp, int j) {
            const int g = ks + KS * (j < n_my ? j : 0);
            xh[sp] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rah, a_voff, g * kGroup * 2, 0));
            xl[sp] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(ral, a_voff, g * kGroup * 2, 0));
            xpw[sp] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rpw, pw_off, g * R * 4, 0));
        };
#pragma unroll
        for (int j = 0; j < kNA; ++j) load_a(j, j);
#pragma unroll
        for (int j = 0; j < NB; ++j) load_b(j, j);
        for (int j0 = 0; j0 < n_my; j0 += NB) {
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                const int j = j0 + jj;
                if (j >= n_my) break;
                const float pw = xpw[jj % kNA];
                const v8h ahi = xh[jj % kNA], alo = xl[jj % kNA];
                load_a(jj % kNA, j + kNA);
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const v8h b = codes_to_f16<FMT>(wc[jj][m][0], wc[jj][m][kDw - 1]);
                    v4f d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b, d, 0, 0, 0);
                    const float f = wsc[jj][m] * pw;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[m][i] = fmaf(d[i], f, acc[m][i]);
                }
                load_b(jj, j + NB);
            }
        }

        // reduce the KS partial sums of each output, in slice order
        if constexpr (KS > 1) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][m][lane][i] = acc[m][i];
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s = red[wn][m][lane][i];
#pragma unroll
                        for (int k2 = 1; k2 < KS; ++k2) s += red[wn + 2 * k2][m][lane][i];
                        acc[m][i] = s;
                    }
            }
        }

        if constexpr (NMAT == 2) {
            // H = silu(G) * U for tokens 4h + i and column n. This block holds
            // the tile's 16 tokens x 32 columns, one group of the down
            // projection's reduction axis: one power of two for all of it.
            float hv[4], am = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[i] = (4 * h + i < rows_here) ? silu(acc[0][i]) * acc[1][i] : 0.0f;
                am = fmaxf(am, fabsf(hv[i]));
            }
            am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0xB1, 0xF, 0xF, true)));
            am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x4E, 0xF, 0xF, true)));
            am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x141, 0xF, 0xF, true)));
            am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x140, 0xF, 0xF, true)));
            {
                const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 0));
                const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 16));
                const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 32));
                const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 48));
                am = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
            }
            if (ks == 0 && lane == 0) hmax[wn] = am;
            __syncthreads();
            if (ks == 0) {
                const int ex = pow2_exponent(fmaxf(hmax[0], hmax[1]));
                const float up = ldexpf(1.0f, 15 - ex);
                const int kk = wn * 16 + nl;                      // k of column n inside the group
                const int pos = 8 * (kk >> 3) + k_slot(FMT, kk & 7);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (4 * h + i < rows_here) {
                        const float sv = hv[i] * up;
                        const _Float16 hh = (_Float16)sv;
                        const size_t off = (size_t)(prow + i) * N + (size_t)tile * kGroup + pos;
                        a.hhi[off] = hh;
                        a.hlo[off] = (_Float16)(sv - (float)hh);
                    }
                }
                if (wn == 0 && lane == 0) a.hpow[(size_t)tile * R + row_begin + mt] = ldexpf(1.0f, ex - 15);
            }
            __syncthreads();
        } else {
            if (ks == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * h + i < rows_here) a.y[(size_t)(prow + i) * N + n] = acc[0][i];
            }
            if constexpr (KS > 1) __syncthreads();
        }
    }
}

// K-split per block: enough waves to keep ~16 per CU busy, at least 4 groups per wave
static int choose_ks(int slots, int tiles, int G) {
    int ks = 1;
    while (ks < 4 && (long)slots * tiles * 2 * ks < 4096 && G / (2 * ks) >= 4) ks *= 2;
    return ks;
}

hipError_t launch_prep_act(int fmt, const float* x, const int* row_token, const int* slots, const int* meta,
                           int max_slots, int R, int K, _Float16* ahi, _Float16* alo, float* apow, hipStream_t st) {
    if (max_slots == 0) return hipSuccess;
    const dim3 grid((K / kGroup + 7) / 8, max_slots);
    const int4* sl = reinterpret_cast<const int4*>(slots);
    if (fmt == MOE_W_INT8_G32)
        hipLaunchKernelGGL(prep_act_kernel<MOE_W_INT8_G32>, grid, dim3(256), 0, st, x, row_token, sl, meta, R, K, ahi,
                           alo, apow);
    else
        hipLaunchKernelGGL(prep_act_kernel<MOE_W_INT4_G32>, grid, dim3(256), 0, st, x, row_token, sl, meta, R, K, ahi,
                           alo, apow);
    return hipGetLastError();
}

hipError_t launch_gemv(const moe_experts& routed, const moe_experts* shared, bool gateup, const _Float16* ahi,
                       const _Float16* alo, const float* apow, int R, const int* slots, const int* meta, int max_slots,
                       _Float16* hhi, _Float16* hlo, float* hpow, float* y, hipStream_t st) {
    if (max_slots == 0) return hipSuccess;
    GemvArgs a{};
    a.ahi = ahi;
    a.alo = alo;
    a.apow = apow;
    a.slots = reinterpret_cast<const int4*>(slots);
    a.meta = meta;
    a.E = routed.n_experts;
    const int d = routed.d_model, I = routed.d_ff;
    a.K = gateup ? d : I;
    a.N = gateup ? I : d;
    a.R = R;
    const int G = a.K / kGroup;
    const int64_t bpg = routed.format == MOE_W_INT8_G32 ? 32 : 16;
    a.q_stride = (int64_t)a.N * G * bpg;
    a.s_stride = (int64_t)a.N * G;
    const moe_experts& sh = shared ? *shared : routed;
    if (gateup) {
        a.q[0] = (const uint8_t*)routed.gate_q; a.s[0] = routed.gate_s;
        a.q[1] = (const uint8_t*)routed.up_q;   a.s[1] = routed.up_s;
        a.sq[0] = (const uint8_t*)sh.gate_q;    a.ss[0] = sh.gate_s;
        a.sq[1] = (const uint8_t*)sh.up_q;      a.ss[1] = sh.up_s;
    } else {
        a.q[0] = a.q[1] = (const uint8_t*)routed.down_q; a.s[0] = a.s[1] = routed.down_s;
        a.sq[0] = a.sq[1] = (const uint8_t*)sh.down_q;   a.ss[0] = a.ss[1] = sh.down_s;
    }
    a.hhi = hhi;
    a.hlo = hlo;
    a.hpow = hpow;
    a.y = y;
    const int tiles = a.N / kTile;
    const int ks = choose_ks(max_slots, tiles, G);
    const dim3 grid(tiles, max_slots);
#define MOE_GEMV(FMT, NM, KSV) hipLaunchKernelGGL((gemv_kernel<FMT, NM, KSV>), grid, dim3(128 * KSV), 0, st, a)
#define MOE_GEMV_KS(FMT, NM)                \
    if (ks == 1) MOE_GEMV(FMT, NM, 1);      \
    else if (ks == 2) MOE_GEMV(FMT, NM, 2); \
    else MOE_GEMV(FMT, NM, 4);
    if (routed.format == MOE_W_INT8_G32) {
        if (gateup) { MOE_GEMV_KS(MOE_W_INT8_G32, 2) } else { MOE_GEMV_KS(MOE_W_INT8_G32, 1) }
    } else {
        if (gateup) { MOE_GEMV_KS(MOE_W_INT4_G32, 2) } else { MOE_GEMV_KS(MOE_W_INT4_G32, 1) }
    }
#undef MOE_GEMV_KS
#undef MOE_GEMV
    return hipGetLastError();
}

}  // namespace moe
