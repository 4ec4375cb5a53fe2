// One LDS stage of the prefill grouped GEMM (mfma_gemm.hip): the layout of
// the stage buffer and the products and scaling of one group pair for one
// wave. Shared by the GEMM and by the calibration kernel that measures this
// instruction mix on its own (calib.hip).
//
// The wave owns one 32-row weight tile (two 16-row halves) and multiplies it
// by LIVE 16-token tiles of activation codes, for the two groups of the
// stage: 2 LIVE steps of two v_mfma_f32_16x16x32_f16 each (weights as the A
// operand, tokens as B: output rows are weight rows, columns tokens), and per
// output and group
//     acc += I_g * (sw * sx)        (group scales: two VALU operations)
//     acc += I_g * sx               (a scale per weight row: one)
// where I_g, the matrix core's result, is the exact integer group dot.
#pragma once

#include "common.h"
#include "f16codes.h"

namespace moe {

constexpr int kBM = kTileRows;       // 128 token rows per block
constexpr int kM16 = kBM / 16;       // 16-token tiles per block
constexpr int kGemmWaves = 8;        // waves per block, one 32-row weight tile each

// One LDS stage (bytes), filled by direct global -> LDS loads (each wave
// load writes 64 lanes x 16 (or 4) bytes contiguously):
//   TOK [2 groups][8 tiles][64 lanes][16 B]  f16 activation codes; block
//       (g, i) is the B operand of 16-token tile i: lane l = r + 16 h holds
//       token 16 i + r, slice h (k 8h .. 8h+7 in operand-slot order)
//   W   int8: [8 tiles][2 groups][1 KB]  weight blocks exactly as in HBM
//       int4: [8 tiles][1 KB]            (one block holds the pair)
//       int2: [8 tiles][2 groups][256 B] the pair's dwords of each lane (a
//                                        block holds two pairs)
//   SX  [8 tiles][2 groups][16 r] fp32    activation scales of token 16 i + r
//       (the 16 tokens a read serves lie in 16 different banks)
//   SW  [8 tiles][64] fp32                the tiles' scale blocks of the pair
//                                         (group-scale formats only)
constexpr int kLdsTok = 2 * kM16 * 1024;           // 16384
constexpr int kLdsSX = 2 * kBM * 4;                // 1024
constexpr int kLdsSW = kGemmWaves * 64 * 4;        // 2048
template <int FMT>
constexpr int lds_w_bytes() {
    return kGemmWaves * (FMT == MOE_W_INT8_G32 ? 2 * 1024 : FMT == MOE_W_INT4_G32 ? 1024 : 2 * 256);
}
// byte offset of wave w's weight block(s) inside W
template <int FMT>
constexpr int lds_w_wave(int w) {
    return w * (FMT == MOE_W_INT8_G32 ? 2 * 1024 : FMT == MOE_W_INT4_G32 ? 1024 : 2 * 256);
}
template <int FMT>
constexpr int lds_stage_bytes() { return kLdsTok + lds_w_bytes<FMT>() + kLdsSX + kLdsSW; }
// After the K loop the gate/up kernel's up waves hand U (up to 16 KB per
// wave: eight 16-token tiles x two halves x 64 lanes x 16 B) to the gate
// waves through the two stage buffers, two waves per buffer: each buffer
// holds at least a stage and 32 KB.
constexpr int kHandoverBytes = kM16 * 2 * 64 * 16;
template <int FMT>
constexpr int lds_gemm_buffer_bytes() {
    return lds_stage_bytes<FMT>() > 2 * kHandoverBytes ? lds_stage_bytes<FMT>() : 2 * kHandoverBytes;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) uint8_t lds_byte;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16-byte LDS read of any 16-byte type
template <typename T>
__device__ __forceinline__ T lds_read(const lds_byte* p) {
    static_assert(sizeof(T) == 16, "16-byte reads only");
    const v4u v = *reinterpret_cast<const __attribute__((address_space(3))) v4u*>(p);
    return __builtin_bit_cast(T, v);
}

typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v2f lds_read_f2(const lds_byte* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) v2f*>(p);
}

__device__ __forceinline__ uint32_t lds_read_u32(const lds_byte* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(p);
}

// Per-lane byte offsets of a wave's operands inside a stage buffer.
struct StageOffsets {
    int tok;   // TOK + lane * 16
    int w;     // W + this wave's weight block(s) + lane share
    int sx;    // SX + token nl of the lane
    int sw;    // SW + this wave's scale block + rows 4 rq ..
};

// One stage (one group pair) of one wave. acc[i][hh][r]: weight row
// 16 hh + 4 rq + r of the wave's tile, token 16 i + nl (lane = nl + 16 rq).
// on_dot(step, hh, d) sees every product (step = group * LIVE + token tile),
// for the test hook's exact dots; a no-op otherwise.
//
// 2 LIVE steps, each two products and their scaling, software pipelined by
// hand: the products of step s + 1 are issued before the scaling of step s
// (so the matrix core runs while the VALU scales), the token operand and
// activation scale of step s + 2 are read from LDS meanwhile, and a
// scheduling barrier closes every step, which keeps the live registers to a
// few steps' worth.
template <int FMT, bool ROW, int LIVE, class OnDot>
__device__ __forceinline__ void q8_stage(const lds_byte* base, const StageOffsets& o, v4f (&acc)[LIVE][2],
                                         OnDot&& on_dot) {
    constexpr int NS = 2 * LIVE;
    // the weight codes of both halves and groups
    uint4 cw[2] = {};
    uint32_t cw2[2] = {};
    if constexpr (FMT == MOE_W_INT4_G32) {
        cw[0] = lds_read<uint4>(base + o.w);
    } else if constexpr (FMT == MOE_W_INT8_G32) {
        cw[0] = lds_read<uint4>(base + o.w);
        cw[1] = lds_read<uint4>(base + o.w + 1024);
    } else {
        cw2[0] = lds_read_u32(base + o.w);
        cw2[1] = lds_read_u32(base + o.w + 256);
    }
    // weight scales of the lane's rows 4 rq + r for the current group g:
    // swg[r] = {half 0, half 1} (the block holds {g0 h0, g0 h1, g1 h0, g1 h1}
    // per row); one group at a time keeps eight registers, not sixteen
    v2f swg[4];
    auto load_sw = [&](int g) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) swg[r] = lds_read_f2(base + o.sw + r * 16 + g * 8);
    };
    if constexpr (!ROW) load_sw(0);
    // step s: group g = s / LIVE, token tile i = s % LIVE
    auto tok = [&](int st) __attribute__((always_inline)) {
        return lds_read<v8h>(base + o.tok + ((st / LIVE) * kM16 + st % LIVE) * 1024);
    };
    auto sxs = [&](int st) __attribute__((always_inline)) {
        return *reinterpret_cast<const __attribute__((address_space(3))) float*>(
            base + o.sx + ((st % LIVE) * 2 + st / LIVE) * 64);
    };
    // both halves of group g as f16 A operands
    auto weights = [&](int g, v8h* wa) __attribute__((always_inline)) {
        if constexpr (FMT == MOE_W_INT8_G32) {
            wa[0] = codes_to_f16<FMT>(cw[g].x, cw[g].y);
            wa[1] = codes_to_f16<FMT>(cw[g].z, cw[g].w);
        } else if constexpr (FMT == MOE_W_INT2_G32) {
            wa[0] = int2_codes_to_f16<0>(cw2[g]);
            wa[1] = int2_codes_to_f16<1>(cw2[g]);
        } else {
            wa[0] = codes_to_f16<FMT>(g ? cw[0].z : cw[0].x, 0u);
            wa[1] = codes_to_f16<FMT>(g ? cw[0].w : cw[0].y, 0u);
        }
    };
    v8h wa0[2], wa1[2];
    v8h tb[NS];
    float sx[NS];
    v4f d[NS][2];
    tb[0] = tok(0);
    sx[0] = sxs(0);
    if (NS > 1) {
        tb[1] = tok(1);
        sx[1] = sxs(1);
    }
    weights(0, wa0);
    d[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa0[0], tb[0], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    d[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa0[1], tb[0], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st + 2 < NS) {
            tb[st + 2] = tok(st + 2);
            sx[st + 2] = sxs(st + 2);
        }
        if (st + 1 < NS) {
            const int g1 = (st + 1) / LIVE;
            if ((st + 1) % LIVE == 0) weights(1, wa1);
            const v8h* wa = g1 ? wa1 : wa0;
            d[st + 1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[0], tb[st + 1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            d[st + 1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[1], tb[st + 1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
        const int i = st % LIVE;
        if constexpr (!ROW)
            if (st == LIVE) load_sw(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if constexpr (ROW) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][hh][r] = fmaf(d[st][hh][r], sx[st], acc[i][hh][r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sw = hh ? swg[r].y : swg[r].x;
                    acc[i][hh][r] = fmaf(d[st][hh][r], sw * sx[st], acc[i][hh][r]);
                }
            }
            on_dot(st, hh, d[st][hh]);
            // the step's accumulators are final here: without this pin,
            // earlier passes sink the scaling past the stage barrier, where
            // every product of the stage would stay live at once
            asm volatile("" : "+v"(acc[i][hh]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace moe
