// Prefill / verification path: batch-union grouped GEMM with Q8_0
// activations and exact integer group dots ("Show HN: Getting GLM-5.2
// running on my slow computer", section "What's implemented": batches take
// integer dot products on int8 activations quantised the Q8_0 way, and in
// prefill as in multi-token verification every selected expert is read once
// per batch).
//
// Each 32-deep quantisation group is one v_mfma_f32_16x16x32_f16 per 16 x 16
// output tile, fed with the integer codes themselves: activation and weight
// codes are exact in f16, their products are exact, and the group's sum
// (|sum| <= 32 * 127 * 127 < 2^24) is exact in the fp32 result, so the matrix
// core returns the exact integer group dot I_g, already as a float. The
// group's two fp32 scales (activation row, weight row) are then applied
// before it joins the fp32 accumulator:
//     acc[m][n] += I_g[m, n] * (sx[m, g] * sw[n, g])
// which is two VALU operations per output and group (an int8 matrix-core
// product would need a third, the int -> float conversion, and the VALU work
// is what bounds this kernel). With one scale per weight row (the per-row
// formats) the group's factor is sx alone, one VALU operation per output and
// group, and the row's scale multiplies the finished sum:
//     acc[m][n] = sw[n] * sum_g I_g[m, n] * sx[m, g]
//
// Block tile: 128 rows (tokens of one expert) x 128 weight rows (four 32-row
// tiles), staged through LDS one group pair (64 k) at a time, double
// buffered, by direct global -> LDS loads: no staging registers; weight
// blocks land exactly as they are stored. Four waves in 2 x 2; each wave owns
// 64 rows (four 16-row tiles) and two weight tiles (four 16-row halves), 16
// matrix-core products per group. 16-row tiles past the tile's row count
// are neither loaded nor multiplied (wave-uniform), so a short tile costs
// little more than its rows.
//   gate/up kernel: the wave's two weight tiles are gate and up of the same 32
//     outputs, so SwiGLU and the Q8_0 quantisation of H (32 outputs = one
//     group) happen in registers; H leaves as f16 codes in operand-slot
//     order + one fp32 scale per 32, ready to be the down kernel's A operand.
//   down kernel: two adjacent 32-row weight tiles; Y leaves fp32.
// Work list: one tile per (expert, 128-row block) from the dispatch kernel;
// blocks past the live tile count exit at once (no host read-back).
#include <type_traits>

#include "common.h"
#include "f16codes.h"
#include "kernels.h"

namespace moe {

constexpr int kBM = kTileRows;       // 128 token rows per block
constexpr int kSG = 2;               // groups per LDS stage (one pair, 64 k)
constexpr int kM16 = kBM / 16;       // 16-row tiles per block

// One LDS stage (bytes), filled by direct global -> LDS loads (each wave
// load writes 64 lanes x 16 (or 4) bytes contiguously):
//   A  [kSG groups][kM16 tiles][64 lanes][16 B]  f16 activation codes; block
//      (g, i) is the MFMA A operand of 16-row tile i, lane l = r + 16 h
//      holding row 16 i + r, slice h (k 8h .. 8h+7 in slot order): one
//      contiguous 1 KB read per operand
//   B  int8: [4 tiles][kSG groups][1 KB]  weight blocks exactly as in HBM
//      int4: [4 tiles][1 KB]              (one block holds the pair)
//      int2: [4 tiles][kSG groups][256 B] the pair's dwords of each lane (a
//                                         block holds two pairs)
//   SX [kSG groups][kBM rows] fp32        activation scales
//   SW [4 tiles][64] fp32                 the tiles' scale blocks of the pair
//                                         (group-scale formats only)
constexpr int kLdsA = kSG * kM16 * 1024;   // 16384
constexpr int kLdsSX = kSG * kBM * 4;      // 1024
constexpr int kLdsSW = 4 * 64 * 4;         // 1024
template <int FMT>
constexpr int lds_b_bytes() {
    return FMT == MOE_W_INT8_G32 ? 4 * kSG * 1024 : FMT == MOE_W_INT4_G32 ? 4 * 1024 : 4 * kSG * 256;
}
template <int FMT>
constexpr int lds_stage_bytes() { return kLdsA + lds_b_bytes<FMT>() + kLdsSX + kLdsSW; }

struct MfmaMat {
    const uint8_t* q;
    const float* s;
    int64_t q_stride;   // bytes per expert
    int64_t s_stride;   // floats per expert
};

struct MfmaArgs {
    const _Float16* a_q;    // activation codes as f16, rows of K, slot order
    const float* a_s;       // activation scales, rows of K/32
    uint32_t a_bytes;       // sizes of the two (rows * K * 2, rows * K/32 * 4)
    uint32_t s_bytes;
    const int* row_token;   // permuted row -> activation row (nullptr: identity)
    const int4* tiles;      // (expert, row_begin, row_end, 0)
    const int* meta;        // meta[1] = live tile count
    MfmaMat routed[2];      // gate, up (or down, down)
    MfmaMat shared[2];
    int E, K, N;
    _Float16* hq;           // gate/up output codes  [R, N], f16, slot order
    float* hd;              // gate/up output scales [R, N/32]
    float* y;               // down output           [R, N]
    int32_t* dbg0;          // optional exact group dots [R, N, K/32]
    int32_t* dbg1;
    int8_t* dbg_hq;         // optional int8 H codes [R, N], natural order
};

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

// one wave's direct load of 64 x BYTES from per-lane global addresses into
// LDS at `dst` (wave-uniform), lane L at dst + L * BYTES
template <int BYTES>
__device__ __forceinline__ void wave_load_lds(const void* src, lds_byte* dst) {
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
}

// the same through a buffer resource: lane L reads BYTES at voff + soff
template <int BYTES>
__device__ __forceinline__ void buffer_load_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, lds_byte* dst) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, so, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, so, 0, 0);
}

__device__ __forceinline__ uint32_t lds_read_u32(const lds_byte* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(p);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// max over the 16 lanes of a DPP row, result in every lane of the row
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));   // row_mirror
    return v;
}

template <int FMT, bool GATEUP, bool DBG, bool ROW>
__global__ __launch_bounds__(256) void q8_mfma_kernel(const MfmaArgs a) {
    constexpr int kStage = lds_stage_bytes<FMT>();
    // the two stage buffers are separate objects, so the compiler can tell
    // that reading one does not wait for the direct loads into the other
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    // XCD-aware order: the hardware deals blocks to the 8 XCDs in turn by
    // linear id, so linear id L runs on XCD L % 8. Block L takes column block
    // (L / 8) % ncol of row tile ((L / 8) / ncol) * 8 + L % 8: all column
    // blocks of one row tile share an XCD, and its activation rows are
    // fetched into that XCD's L2 once (the grid's tile count is a multiple
    // of 8, so this is a bijection).
    const int ncol = gridDim.x;
    const int lin = blockIdx.y * ncol + blockIdx.x;
    const int xcd = lin & 7, sl = lin >> 3;
    const int col_blk = sl % ncol;
    const int tile_id = (sl / ncol) * 8 + xcd;
    if (tile_id >= a.meta[1]) return;
    const int4 td = a.tiles[tile_id];
    const int e = td.x, row_begin = td.y, rows = td.z - td.y;
    const bool is_shared = e == a.E;
    const MfmaMat* M = is_shared ? a.shared : a.routed;
    const int64_t eo = is_shared ? 0 : e;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int K = a.K, N = a.N, G = K / kGroup, P = G / 2, NT = N / kTile;
    const int T0 = col_blk * (GATEUP ? 2 : 4);         // first 32-row weight tile of the block
    const int m16_live = (rows + 15) >> 4;               // 16-row tiles holding rows (1 .. 8)
    const int my_live = min(max(m16_live - 4 * wm, 0), 4);

    // block weight tile j (0..3) -> matrix and tile index (clamped to the
    // matrix: loads stay inside it; results of a clamped tile are not stored)
    auto tile_of = [&](int j) { return min(T0 + (GATEUP ? (j & 1) : j), NT - 1); };
    auto mat_of = [&](int j) { return GATEUP ? (j >> 1) : 0; };
    const uint8_t* wq[2];
    const float* wsb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        wq[m] = M[m].q + eo * M[m].q_stride;
        wsb[m] = M[m].s + eo * M[m].s_stride;
    }
    // activation row of a block row (clamped to the tile's rows: rows past it
    // are loaded only inside a live 16-row tile and never stored)
    auto src_row = [&](int r) {
        const int pr = row_begin + min(r, rows - 1);
        return a.row_token ? a.row_token[pr] : pr;
    };
    // this wave's stage jobs are fixed (job index % 4 == wave): A tiles
    // i = wave and wave + 4 of both groups, and the scale job of (group
    // wave / 2, rows 64 * (wave % 2) ..). Activation rows, their scales and
    // the weight codes are read through buffer resources: the per-lane byte
    // offset stays in a register for the whole kernel and the stage's offset
    // goes in a scalar register, so issuing a stage costs no vector ALU work
    // (and a read past a resource's end returns zeros).
    uint32_t a_off[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        a_off[s] = ((uint32_t)src_row(16 * (wave + 4 * s) + (lane & 15)) * K + 8 * (lane >> 4)) * 2;
    const uint32_t s_off = (uint32_t)src_row(64 * (wave & 1) + lane) * G * 4;
    const uint32_t l_off = lane * 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.a_q, 0, a.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc((void*)a.a_s, 0, a.s_bytes, 0x00020000);
    __amdgpu_buffer_rsrc_t rw[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        rw[m] = __builtin_amdgcn_make_buffer_rsrc((void*)wq[m], 0, (int)M[m].q_stride, 0x00020000);

    auto issue_stage = [&](int st, lds_byte* base) __attribute__((always_inline)) {
        lds_byte* A = base;
        lds_byte* B = base + kLdsA;
        lds_byte* SX = B + lds_b_bytes<FMT>();
        lds_byte* SW = SX + kLdsSX;
        const int pc = min(st, P - 1);
        constexpr int nA = kSG * kM16;
        constexpr int nB = FMT == MOE_W_INT4_G32 ? 4 : 4 * kSG;
        constexpr int nSX = kSG * 2;
        constexpr int nJobs = nA + nB + nSX + (ROW ? 0 : 1);
        static_assert((nA + nB) % 4 == 0, "scale jobs must start on wave 0");
#pragma unroll
        for (int job = 0; job < nJobs; ++job) {
            if (job % 4 != (wave & 3)) continue;   // wave-uniform
            if (job < nA) {
                const int g = job / kM16, i = job % kM16;
                if (i < m16_live) buffer_load_lds<16>(ra, a_off[i >= 4], (2 * pc + g) * kGroup * 2, A + (g * kM16 + i) * 1024);
            } else if (job < nA + nB) {
                const int b = job - nA;
                if constexpr (FMT == MOE_W_INT8_G32) {
                    const int j = b / kSG, g = b % kSG;
                    buffer_load_lds<16>(rw[mat_of(j)], l_off, ((2 * pc + g) * NT + tile_of(j)) * 1024,
                                        B + (j * kSG + g) * 1024);
                } else if constexpr (FMT == MOE_W_INT2_G32) {
                    // dword 2 (pc % 2) + g of each lane's 16 bytes in the quad block
                    const int j = b / kSG, g = b % kSG;
                    buffer_load_lds<4>(rw[mat_of(j)], l_off, ((pc >> 1) * NT + tile_of(j)) * 1024 + (2 * (pc & 1) + g) * 4,
                                       B + (j * kSG + g) * 256);
                } else {
                    const int j = b;
                    buffer_load_lds<16>(rw[mat_of(j)], l_off, (pc * NT + tile_of(j)) * 1024, B + j * 1024);
                }
            } else if (job < nA + nB + nSX) {
                // job q = wave: group q / 2, rows 64 * (q % 2) + lane
                const int q = job - nA - nB;
                buffer_load_lds<4>(rsx, s_off, (2 * pc + (q >> 1)) * 4, SX + ((q >> 1) * kBM + 64 * (q & 1)) * 4);
            } else {
                // the four tiles' scale blocks of pair pc, 256 B each
                const int j = lane >> 4;
                wave_load_lds<16>(wsb[mat_of(j)] + ((size_t)tile_of(j) * P + pc) * 64 + (lane & 15) * 4, SW);
            }
        }
    };

    // output (i, n, r): row 64 wm + 16 i + 4 (lane / 16) + r of the block,
    // weight row 16 (n % 2) + lane % 16 of the wave's weight tile n / 2
    const int nl = lane & 15, rq = lane >> 4;
    const int jt0 = GATEUP ? wn : 2 * wn;       // block weight tiles of the wave
    const int jt1 = GATEUP ? 2 + wn : 2 * wn + 1;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = v4f{0.f, 0.f, 0.f, 0.f};

    // Per-lane LDS byte offsets of the operands inside a stage buffer, kept
    // opaque to the optimiser: every LDS read is then the buffer plus one
    // offset plus a constant. The compiler proves that a read of one buffer
    // does not alias the direct loads into the other only for addresses it
    // can trace back to the buffer in a few steps; a longer chain makes it
    // wait for every load in flight.
    auto opaque = [](int v) __attribute__((always_inline)) {
        asm volatile("" : "+v"(v));
        return v;
    };
    const int oA = opaque((4 * wm * 64 + lane) * 16);
    const int oB0 = opaque(kLdsA + (FMT == MOE_W_INT2_G32 ? jt0 * kSG * 256 + lane * 4
                                                          : (FMT == MOE_W_INT8_G32 ? jt0 * kSG : jt0) * 1024 + lane * 16));
    const int oB1 = opaque(kLdsA + (FMT == MOE_W_INT2_G32 ? jt1 * kSG * 256 + lane * 4
                                                          : (FMT == MOE_W_INT8_G32 ? jt1 * kSG : jt1) * 1024 + lane * 16));
    const int oSX = opaque(kLdsA + lds_b_bytes<FMT>() + (64 * wm + 4 * rq) * 4);
    const int oSW0 = opaque(kLdsA + lds_b_bytes<FMT>() + kLdsSX + (jt0 * 64 + nl * 4) * 4);
    const int oSW1 = opaque(kLdsA + lds_b_bytes<FMT>() + kLdsSX + (jt1 * 64 + nl * 4) * 4);

    // ROW: the scales of the wave's four 16-row weight halves, lane row nl
    float srow[4];
    if constexpr (ROW) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int jt = n < 2 ? jt0 : jt1;
            srow[n] = wsb[mat_of(jt)][tile_of(jt) * kTile + 16 * (n & 1) + nl];
        }
    }

    auto compute = [&](const lds_byte* base, int st) __attribute__((always_inline)) {
        // [row nl, g0][row 16+nl, g0][row nl, g1][row 16+nl, g1] of each tile
        // (zero for the padding stage past the last pair)
        const bool real = st < P;
        float4 sw0 = make_float4(0.f, 0.f, 0.f, 0.f), sw1 = sw0;
        if constexpr (!ROW) {
            sw0 = lds_read<float4>(base + oSW0);
            sw1 = lds_read<float4>(base + oSW1);
            if (!real) sw0 = sw1 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        uint4 c4[2];
        if constexpr (FMT == MOE_W_INT4_G32) {
            c4[0] = lds_read<uint4>(base + oB0);
            c4[1] = lds_read<uint4>(base + oB1);
        }
        // One group for a wave with LIVE live 16-row tiles. The count is a
        // compile-time constant inside, so no branch separates a product from
        // the instructions that read it (the compiler's wait-state insertion
        // does not cover a matrix-core result read across a branch).
        auto group = [&](auto live_c, int g) __attribute__((always_inline)) {
            constexpr int LIVE = decltype(live_c)::value;
            v8h af[LIVE];
            float4 sx[LIVE];
#pragma unroll
            for (int i = 0; i < LIVE; ++i) {
                af[i] = lds_read<v8h>(base + oA + (g * kM16 + i) * 1024);
                sx[i] = lds_read<float4>(base + oSX + (g * kBM + 16 * i) * 4);
            }
            // one weight half-tile (16 rows) at a time: convert its codes,
            // then its products with every live 16-row tile
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int t = n >> 1, hh = n & 1;
                v8h bf;
                if constexpr (FMT == MOE_W_INT8_G32) {
                    const uint4 c = lds_read<uint4>(base + (t ? oB1 : oB0) + g * 1024);
                    bf = hh ? codes_to_f16<FMT>(c.z, c.w) : codes_to_f16<FMT>(c.x, c.y);
                } else if constexpr (FMT == MOE_W_INT2_G32) {
                    const uint32_t c = lds_read_u32(base + (t ? oB1 : oB0) + g * 256);
                    bf = hh ? int2_codes_to_f16<1>(c) : int2_codes_to_f16<0>(c);
                } else {
                    const uint4 c = c4[t];
                    bf = codes_to_f16<FMT>(g ? (hh ? c.w : c.z) : (hh ? c.y : c.x), 0u);
                }
                const float4 swt = t ? sw1 : sw0;
                const float sw = g ? (hh ? swt.w : swt.z) : (hh ? swt.y : swt.x);
#pragma unroll
                for (int i = 0; i < LIVE; ++i) {
                    const v4f d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (ROW) {
                        acc[i][n][0] = fmaf(d[0], sx[i].x, acc[i][n][0]);
                        acc[i][n][1] = fmaf(d[1], sx[i].y, acc[i][n][1]);
                        acc[i][n][2] = fmaf(d[2], sx[i].z, acc[i][n][2]);
                        acc[i][n][3] = fmaf(d[3], sx[i].w, acc[i][n][3]);
                    } else {
                        acc[i][n][0] = fmaf(d[0], sx[i].x * sw, acc[i][n][0]);
                        acc[i][n][1] = fmaf(d[1], sx[i].y * sw, acc[i][n][1]);
                        acc[i][n][2] = fmaf(d[2], sx[i].z * sw, acc[i][n][2]);
                        acc[i][n][3] = fmaf(d[3], sx[i].w * sw, acc[i][n][3]);
                    }
                    if constexpr (DBG) {
                        const int jt = t ? jt1 : jt0;
                        const int wt = T0 + (GATEUP ? (jt & 1) : jt);
                        const int col = wt * kTile + 16 * hh + nl;
                        int32_t* dst = (GATEUP && t) ? a.dbg1 : a.dbg0;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = 64 * wm + 16 * i + 4 * rq + r;
                            if (row < rows && wt < NT && real)
                                dst[((size_t)(row_begin + row) * N + col) * G + 2 * st + g] = (int32_t)d[r];
                        }
                    }
                }
            }
        };
#pragma unroll
        for (int g = 0; g < kSG; ++g) {
            // wave-uniform: a wave with 2 or 3 live tiles computes all four
            // (the rows of a dead tile are never stored)
            if (my_live >= 2) group(std::integral_constant<int, 4>{}, g);
            else if (my_live == 1) group(std::integral_constant<int, 1>{}, g);
        }
    };

    lds_byte* const buf0 = (lds_byte*)lds0;
    lds_byte* const buf1 = (lds_byte*)lds1;
    issue_stage(0, buf0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Stages alternate between the buffers; each stage's direct loads for the
    // next one are in flight while it is multiplied. An odd stage count runs
    // one more stage whose weight scales are taken as zero (its loads repeat
    // the last pair), so the loop body has no exit in its middle.
    const int P2 = (P + 1) & ~1;
    for (int st = 0; st < P2; st += 2) {
        issue_stage(st + 1, buf1);
        compute(buf0, st);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (st + 2 < P2) issue_stage(st + 2, buf0);
        // per-row formats have no weight scale to zero: they skip the
        // padding stage's products
        if (!ROW || st + 1 < P) compute(buf1, st + 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue ----
    if constexpr (ROW) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][n][r] *= srow[n];
    }
    if constexpr (GATEUP) {
        const int t = T0 + wn;                  // weight tile = group of H's columns
        const int GN = N / kGroup;
        // H column 32 t + kk sits at slot position (kk & ~7) + k_slot(kk & 7)
        const int pos0 = (nl & 8) + k_slot(FMT, nl & 7);
        const int pos1 = 16 + pos0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= my_live) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float h0 = silu(acc[i][0][r]) * acc[i][2][r];   // H column 32 t + nl
                const float h1 = silu(acc[i][1][r]) * acc[i][3][r];   // H column 32 t + 16 + nl
                const float amax = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
                const float dd = __fdiv_rn(amax, 127.0f);
                const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
                const float q0 = fminf(fmaxf(rintf(__fmul_rn(h0, inv)), -127.0f), 127.0f);
                const float q1 = fminf(fmaxf(rintf(__fmul_rn(h1, inv)), -127.0f), 127.0f);
                const int row = 64 * wm + 16 * i + 4 * rq + r;
                if (row < rows) {
                    const size_t R = (size_t)(row_begin + row);
                    _Float16* hrow = a.hq + R * N + t * kTile;
                    hrow[pos0] = (_Float16)q0;
                    hrow[pos1] = (_Float16)q1;
                    if (nl == 0) a.hd[R * GN + t] = dd;
                    if constexpr (DBG) {
                        a.dbg_hq[R * N + t * kTile + nl] = (int8_t)(int)q0;
                        a.dbg_hq[R * N + t * kTile + 16 + nl] = (int8_t)(int)q1;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int t = T0 + (n < 2 ? jt0 : jt1);
            if (t >= NT) continue;
            const int col = t * kTile + 16 * (n & 1) + nl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= my_live) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 64 * wm + 16 * i + 4 * rq + r;
                    if (row < rows) a.y[(size_t)(row_begin + row) * N + col] = acc[i][n][r];
                }
            }
        }
    }
}

hipError_t launch_q8_mfma(const moe_experts& routed, const moe_experts* shared, bool gateup, const _Float16* a_q,
                          const float* a_s, int a_rows, const int* row_token, const int* tiles, const int* meta,
                          int max_tiles, _Float16* hq, float* hd, float* y, int32_t* dbg0, int32_t* dbg1, int8_t* dbg_hq,
                          hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (max_tiles == 0) return hipSuccess;
    MfmaArgs a{};
    a.a_q = a_q;
    a.a_s = a_s;
    a.row_token = row_token;
    a.tiles = reinterpret_cast<const int4*>(tiles);
    a.meta = meta;
    a.E = routed.n_experts;
    const int d = routed.d_model, I = routed.d_ff;
    a.K = gateup ? d : I;
    a.N = gateup ? I : d;
    a.a_bytes = (uint32_t)((size_t)a_rows * a.K * 2);
    a.s_bytes = (uint32_t)((size_t)a_rows * (a.K / kGroup) * 4);
    a.hq = hq;
    a.hd = hd;
    a.y = y;
    a.dbg0 = dbg0;
    a.dbg1 = dbg1;
    a.dbg_hq = dbg_hq;
    auto fill = [&](MfmaMat* dst, const moe_experts& ev) {
        const int64_t qs = fmt_code_bytes(ev.format, a.N, a.K), ss = fmt_scale_floats(ev.format, a.N, a.K);
        if (gateup) {
            dst[0] = MfmaMat{(const uint8_t*)ev.gate_q, ev.gate_s, qs, ss};
            dst[1] = MfmaMat{(const uint8_t*)ev.up_q, ev.up_s, qs, ss};
        } else {
            dst[0] = MfmaMat{(const uint8_t*)ev.down_q, ev.down_s, qs, ss};
            dst[1] = dst[0];
        }
    };
    fill(a.routed, routed);
    fill(a.shared, shared ? *shared : routed);
    const int bn = gateup ? 2 * kTile : 4 * kTile;   // output columns per block
    const dim3 grid((a.N + bn - 1) / bn, (max_tiles + 7) / 8 * 8);   // tile count padded for the XCD order
    const bool dbg = dbg0 != nullptr;
#define MOE_Q8(FMT, GU, DB, RW) launch_timed(q8_mfma_kernel<FMT, GU, DB, RW>, grid, dim3(256), st, ev0, ev1, a)
#define MOE_Q8_GU(FMT, RW)                                                              \
    if (gateup) { if (dbg) MOE_Q8(FMT, true, true, RW); else MOE_Q8(FMT, true, false, RW); } \
    else { if (dbg) MOE_Q8(FMT, false, true, RW); else MOE_Q8(FMT, false, false, RW); }
    switch (routed.format) {
        case MOE_W_INT8_G32: MOE_Q8_GU(MOE_W_INT8_G32, false) break;
        case MOE_W_INT4_G32: MOE_Q8_GU(MOE_W_INT4_G32, false) break;
        case MOE_W_INT2_G32: MOE_Q8_GU(MOE_W_INT2_G32, false) break;
        case MOE_W_INT8_ROW: MOE_Q8_GU(MOE_W_INT8_G32, true) break;
        case MOE_W_INT4_ROW: MOE_Q8_GU(MOE_W_INT4_G32, true) break;
        default: MOE_Q8_GU(MOE_W_INT2_G32, true) break;
    }
#undef MOE_Q8_GU
#undef MOE_Q8
    return hipGetLastError();
}

}  // namespace moe
