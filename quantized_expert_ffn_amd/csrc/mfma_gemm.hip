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
// group's two fp32 scales (weight row, activation row) are then applied
// before it joins the fp32 accumulator:
//     acc[n][m] += I_g[n, m] * (sw[n, g] * sx[m, g])
// which is two VALU operations per output and group (an int8 matrix-core
// product would need a third, the int -> float conversion). The VALU work
// bounds this kernel, so the layout is chosen to spend as little of it as
// possible besides those two operations: with one scale per weight row (the
// per-row formats) the group's factor is sx alone, one operation per output
// and group, and the row's scale multiplies the finished sum.
//
// Block tile: 128 token rows (one work-list tile: rows of one expert) x eight
// 32-row weight tiles; eight waves, each owning ONE weight tile (gate/up: four
// gate tiles and the same four up tiles; down: eight adjacent tiles) for ALL
// of the block's token rows. The eight waves share each staged token tile,
// and two blocks (four waves per SIMD) fit a CU. The weights are the matrix
// core's A operand (output rows = weight rows) and the token codes its B
// operand (output columns = tokens), so
//   - a wave converts each weight code to f16 once and uses it for every
//     live 16-token tile (up to eight products per conversion);
//   - a lane's outputs share one token per 16-token tile: its activation
//     scale is one float per tile and group, its weight scales four floats
//     per 16-row half and group, read one group at a time.
// Operands are staged through LDS one group pair (64 k) at a time, double
// buffered, by direct global -> LDS loads (no staging registers; weight
// blocks land exactly as they are stored in HBM). 16-token tiles past the
// tile's row count are neither loaded nor multiplied: the live count (1, 2,
// 4 or 8 tiles) is a compile-time constant of the whole K loop, chosen once
// per block, so no branch ever separates a product from its use.
//   gate/up kernel: the up waves hand U to the gate waves through LDS (the
//     stage buffers, free after the K loop), and the gate waves form
//     H = silu(G) * U and quantise it (Q8_0, one group = the 32 outputs of a
//     weight tile) in registers; H leaves as f16 codes in operand-slot order
//     + one fp32 scale per 32, ready to be the down kernel's B operand.
//   down kernel: Y leaves fp32, four consecutive outputs per 16-byte store.
// Work list: one tile per (expert, 128-row block) from the dispatch kernel;
// blocks past the live tile count exit at once (no host read-back).
#include <type_traits>

#include "common.h"
#include "f16codes.h"
#include "kernels.h"
#include "q8_stage.h"

namespace moe {

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

// one wave's load of 64 x BYTES through a buffer resource into LDS at `dst`
// (wave-uniform), lane L at dst + L * BYTES: lane L reads BYTES at
// voff + soff (soff wave-uniform); a read past the resource's end gives zeros
template <int BYTES>
__device__ __forceinline__ void buffer_load_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, lds_byte* dst) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, so, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, so, 0, 0);
}

// live 16-token tiles -> the compile-time count the K loop runs with
__device__ __forceinline__ int live_bucket(int m16) { return m16 <= 1 ? 1 : m16 <= 2 ? 2 : m16 <= 4 ? 4 : 8; }

// Everything a block needs besides its K loop's live-tile count.
struct TileCtx {
    int e, row_begin, rows, m16_live;
    int tt;                         // this wave's weight tile (may be >= NT: loads clamped, nothing stored)
    int T0;
    bool is_shared;
    int K, N, G, P, NT;
    int lane, wave, nl, rq;
    const float* wsb;               // this wave's matrix scales (expert base)
    __amdgpu_buffer_rsrc_t ra, rsx, rw, rsw;
    uint32_t tok_off;               // per-lane source offset of this wave's token-tile loads
    uint32_t sx_off;                // per-lane source offset of this wave's scale load
};

template <int FMT, bool GATEUP, bool DBG, bool ROW, int LIVE>
__device__ __forceinline__ void gemm_tile(const MfmaArgs& a, const TileCtx& c, lds_byte* const buf0,
                                          lds_byte* const buf1) {
    constexpr int kW = lds_w_bytes<FMT>();
    const int lane = c.lane, wave = c.wave, nl = c.nl, rq = c.rq;
    const int P = c.P, NT = c.NT;
    // this wave's weight tile (tt may be >= NT: loads clamped to ttl,
    // nothing stored) and its scale-block resource
    const int tt = c.tt;
    const int ttl = min(tt, NT - 1);
    const __amdgpu_buffer_rsrc_t rsw = c.rsw;

    // Stage jobs, each a wave-wide direct load (wave-uniform): token tile
    // i = wave of both groups (live tiles only), this wave's weight
    // block(s) of tile tl, a quarter of the activation scales (waves 0 .. 3),
    // and this wave's weight scale block (through rs).
    auto issue_stage = [&](int pc, lds_byte* base, int tl, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
        lds_byte* TOK = base;
        lds_byte* W = base + kLdsTok;
        lds_byte* SX = W + kW;
        lds_byte* SW = SX + kLdsSX;
        if (wave < LIVE) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
                buffer_load_lds<16>(c.ra, c.tok_off, (2 * pc + g) * kGroup * 2, TOK + (g * kM16 + wave) * 1024);
        }
        if constexpr (FMT == MOE_W_INT8_G32) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
                buffer_load_lds<16>(c.rw, lane * 16, ((2 * pc + g) * NT + tl) * 1024,
                                    W + lds_w_wave<FMT>(wave) + g * 1024);
        } else if constexpr (FMT == MOE_W_INT2_G32) {
            // dwords 2 (pc % 2) + g of each lane's 16 bytes in the quad block
#pragma unroll
            for (int g = 0; g < 2; ++g)
                buffer_load_lds<4>(c.rw, lane * 16, ((pc >> 1) * NT + tl) * 1024 + (2 * (pc & 1) + g) * 4,
                                   W + lds_w_wave<FMT>(wave) + g * 256);
        } else {
            buffer_load_lds<16>(c.rw, lane * 16, (pc * NT + tl) * 1024, W + lds_w_wave<FMT>(wave));
        }
        if (wave < 4) buffer_load_lds<4>(c.rsx, c.sx_off, 2 * pc * 4, SX + wave * 256);
        if constexpr (!ROW) buffer_load_lds<4>(rs, lane * 4, pc * 256, SW + wave * 256);
    };

    // per-lane LDS byte offsets of the operands inside a stage buffer, kept
    // opaque to the optimiser: every LDS read is then the buffer plus one
    // offset plus a constant, which the compiler can tell apart from the
    // direct loads in flight into the other buffer (a longer address chain
    // made it wait for every load before each read)
    auto opaque = [](int v) __attribute__((always_inline)) {
        asm volatile("" : "+v"(v));
        return v;
    };
    const int oTok = opaque(lane * 16);
    const int oW = opaque(kLdsTok + lds_w_wave<FMT>(wave) + (FMT == MOE_W_INT2_G32 ? lane * 4 : lane * 16));
    const int oSX = opaque(kLdsTok + kW + nl * 4);
    const int oSW = opaque(kLdsTok + kW + kLdsSX + wave * 256 + rq * 64);

    // acc[i][hh][r]: weight row 16 hh + 4 rq + r of the wave's tile, token
    // 16 i + nl of the block
    v4f acc[LIVE][2];
#pragma unroll
    for (int i = 0; i < LIVE; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) acc[i][hh] = v4f{0.f, 0.f, 0.f, 0.f};

    const StageOffsets so{oTok, oW, oSX, oSW};
    auto compute = [&](const lds_byte* base, int pc) __attribute__((always_inline)) {
        q8_stage<FMT, ROW, LIVE>(base, so, acc, [&](int st, int hh, const v4f& d) __attribute__((always_inline)) {
            if constexpr (DBG) {
                const int g = st / LIVE, i = st % LIVE;
                const int col = tt * kTile + 16 * hh + 4 * rq;     // weight rows col .. col + 3
                const int row = 16 * i + nl;                       // token row of the block
                int32_t* dst = (GATEUP && (wave >> 2)) ? a.dbg1 : a.dbg0;
                if (row < c.rows && tt < NT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dst[((size_t)(c.row_begin + row) * c.N + col + r) * c.G + 2 * pc + g] = (int32_t)d[r];
                }
            }
        });
    };

    // Stages alternate between the two buffers (separate LDS objects, so a
    // read of one is never held up by the direct loads into the other); each
    // stage's loads for the next one are in flight while it is multiplied.
    issue_stage(0, buf0, ttl, rsw);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int pc = 0; pc < P; pc += 2) {
        if (pc + 1 < P) issue_stage(pc + 1, buf1, ttl, rsw);
        compute(buf0, pc);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (pc + 1 < P) {
            if (pc + 2 < P) issue_stage(pc + 2, buf0, ttl, rsw);
            compute(buf1, pc + 1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }

    if constexpr (ROW) {
        // the lane's rows' scales (a tile past the matrix reads row NT*32-1's; not stored)
        const float* srow = c.wsb + ttl * kTile + 4 * rq;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float4 sr = *reinterpret_cast<const float4*>(srow + 16 * hh);
#pragma unroll
            for (int i = 0; i < LIVE; ++i) {
                acc[i][hh][0] *= sr.x;
                acc[i][hh][1] *= sr.y;
                acc[i][hh][2] *= sr.z;
                acc[i][hh][3] *= sr.w;
            }
        }
    }
    if constexpr (!GATEUP) {
        // ---- down epilogue: Y, four consecutive outputs per 16-byte store ----
        if (tt >= NT) return;
#pragma unroll
        for (int i = 0; i < LIVE; ++i) {
            const int row = 16 * i + nl;
            if (row >= c.rows) continue;
            float* yrow = a.y + (size_t)(c.row_begin + row) * c.N + tt * kTile + 4 * rq;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *reinterpret_cast<float4*>(yrow + 16 * hh) =
                    make_float4(acc[i][hh][0], acc[i][hh][1], acc[i][hh][2], acc[i][hh][3]);
        }
        return;
    }

    // ---- gate/up epilogue ----
    if constexpr (GATEUP) {
        // up waves (4 .. 7) hand U to the gate waves (0 .. 3) of the same
        // tile through the stage buffers (free after the loop's last
        // barrier): waves 4, 5 -> 0, 1 in the two halves of buf0, waves 6, 7
        // -> 2, 3 in those of buf1; lane-major float4s, 16 KB per wave
        lds_byte* xb = ((wave >> 1) & 1 ? buf1 : buf0) + (wave & 1) * kHandoverBytes;
        if (wave >= 4) {
#pragma unroll
            for (int i = 0; i < LIVE; ++i)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    *reinterpret_cast<__attribute__((address_space(3))) v4f*>(xb + ((i * 2 + hh) * 64 + lane) * 16) =
                        acc[i][hh];
        }
        __syncthreads();
        if (wave >= 4) return;
        const int GN = c.N / kGroup;
#pragma unroll
        for (int i = 0; i < LIVE; ++i) {
            const v4f u0 = *reinterpret_cast<const __attribute__((address_space(3))) v4f*>(xb + ((i * 2) * 64 + lane) * 16);
            const v4f u1 =
                *reinterpret_cast<const __attribute__((address_space(3))) v4f*>(xb + ((i * 2 + 1) * 64 + lane) * 16);
            float h[2][4];
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                h[0][r] = silu(acc[i][0][r]) * u0[r];   // output 32 tt + 4 rq + r
                h[1][r] = silu(acc[i][1][r]) * u1[r];   // output 32 tt + 16 + 4 rq + r
                amax = fmaxf(amax, fmaxf(fabsf(h[0][r]), fabsf(h[1][r])));
            }
            // the token's 32 outputs sit in lanes nl, nl + 16, nl + 32, nl + 48
            amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
            const float dd = __fdiv_rn(amax, 127.0f);
            const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
            const int row = 16 * i + nl;
            if (row < c.rows && tt < NT) {
                const size_t R = (size_t)(c.row_begin + row);
                _Float16* hrow = a.hq + R * c.N + tt * kTile;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = 16 * hh + 4 * rq + r;     // H column inside the group
                        const float q = fminf(fmaxf(rintf(__fmul_rn(h[hh][r], inv)), -127.0f), 127.0f);
                        hrow[(kk & ~7) + k_slot(FMT, kk & 7)] = (_Float16)q;
                        if constexpr (DBG) a.dbg_hq[R * c.N + tt * kTile + kk] = (int8_t)(int)q;
                    }
                if (rq == 0) a.hd[R * GN + tt] = dd;
            }
        }
    }
}

template <int FMT, bool GATEUP, bool DBG, bool ROW>
__device__ __forceinline__ void q8_mfma_body(const MfmaArgs& a) {
    constexpr int kStage = lds_gemm_buffer_bytes<FMT>();
    // the two stage buffers are separate objects, so the compiler can tell
    // that reading one does not wait for the direct loads into the other
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    // XCD-aware order: the hardware deals blocks to the 8 XCDs in turn by
    // linear id, so linear id L runs on XCD L % 8. Block L takes column block
    // (L / 8) % ncol of row tile ((L / 8) / ncol) * 8 + L % 8: all column
    // blocks of one row tile share an XCD, and its token rows are fetched
    // into that XCD's L2 once (the grid's tile count is a multiple of 8, so
    // this is a bijection).
    const int ncol = gridDim.x;
    const int lin = blockIdx.y * ncol + blockIdx.x;
    const int xcd = lin & 7, sl = lin >> 3;
    const int col_blk = sl % ncol;
    const int tile_id = (sl / ncol) * 8 + xcd;
    if (tile_id >= a.meta[1]) return;
    const int4 td = a.tiles[tile_id];
    if (td.z <= td.y) return;   // an empty tile (evens the full tiles out over the XCDs)

    TileCtx c;
    c.e = td.x;
    c.row_begin = td.y;
    c.rows = td.z - td.y;
    c.m16_live = (c.rows + 15) >> 4;
    c.is_shared = c.e == a.E;
    c.K = a.K;
    c.N = a.N;
    c.G = a.K / kGroup;
    c.P = c.G / 2;
    c.NT = a.N / kTile;
    c.lane = threadIdx.x & 63;
    c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.nl = c.lane & 15;
    c.rq = c.lane >> 4;
    c.T0 = col_blk * (GATEUP ? kGemmWaves / 2 : kGemmWaves);
    c.tt = c.T0 + (GATEUP ? (c.wave & (kGemmWaves / 2 - 1)) : c.wave);
    const int mat = GATEUP ? (c.wave >> 2) : 0;
    const MfmaMat& M = (c.is_shared ? a.shared : a.routed)[mat];
    const int64_t eo = c.is_shared ? 0 : c.e;
    const uint8_t* wq = M.q + eo * M.q_stride;
    c.wsb = M.s + eo * M.s_stride;
    c.ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.a_q, 0, a.a_bytes, 0x00020000);
    c.rsx = __builtin_amdgcn_make_buffer_rsrc((void*)a.a_s, 0, a.s_bytes, 0x00020000);
    c.rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, 0, (int)M.q_stride, 0x00020000);
    // this wave's scale block of each pair: (tile, pair) blocks of 64 floats, tile-major
    const int ttl = min(c.tt, c.NT - 1);
    c.rsw = __builtin_amdgcn_make_buffer_rsrc((void*)(c.wsb + (size_t)ttl * c.P * 64), 0, c.P * 256, 0x00020000);
    // activation row of a block row (clamped to the tile's rows: rows past it
    // are loaded only inside a live 16-token tile and never stored)
    auto src_row = [&](int r) {
        const int pr = c.row_begin + min(r, c.rows - 1);
        return a.row_token ? a.row_token[pr] : pr;
    };
    // token tile i = wave: lane l = r + 16 h reads token 16 i + r, slice h
    c.tok_off = ((uint32_t)src_row(16 * c.wave + c.nl) * c.K + 8 * c.rq) * 2;
    // scale job of waves 0 .. 3: floats 64 wave + lane of the SX layout
    // [8 tiles][2 groups][16 r]: token 16 i + r, group g of the pair
    {
        const int f = 64 * (c.wave & 3) + c.lane;
        const int i = f >> 5, g = (f >> 4) & 1, r = f & 15;
        c.sx_off = ((uint32_t)src_row(16 * i + r) * c.G + g) * 4;
    }

    lds_byte* const buf0 = (lds_byte*)lds0;
    lds_byte* const buf1 = (lds_byte*)lds1;
    switch (live_bucket(c.m16_live)) {   // block-uniform
        case 1: gemm_tile<FMT, GATEUP, DBG, ROW, 1>(a, c, buf0, buf1); break;
        case 2: gemm_tile<FMT, GATEUP, DBG, ROW, 2>(a, c, buf0, buf1); break;
        case 4: gemm_tile<FMT, GATEUP, DBG, ROW, 4>(a, c, buf0, buf1); break;
        default: gemm_tile<FMT, GATEUP, DBG, ROW, 8>(a, c, buf0, buf1); break;
    }
}

// Two blocks of eight waves share a CU (LDS), so the kernel is held to the
// registers of four waves per SIMD.
template <int FMT, bool GATEUP, bool ROW>
__global__ __launch_bounds__(64 * kGemmWaves) __attribute__((amdgpu_waves_per_eu(4, 4))) void q8_mfma_kernel(
    const MfmaArgs a) {
    q8_mfma_body<FMT, GATEUP, false, ROW>(a);
}

// The test hook's variant (every group dot and H code written out): the
// same body without the register limit.
template <int FMT, bool GATEUP, bool ROW>
__global__ __launch_bounds__(64 * kGemmWaves) void q8_mfma_dbg_kernel(const MfmaArgs a) {
    q8_mfma_body<FMT, GATEUP, true, ROW>(a);
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
    const int bn = (gateup ? kGemmWaves / 2 : kGemmWaves) * kTile;   // output columns per block
    const dim3 grid((a.N + bn - 1) / bn, (max_tiles + 7) / 8 * 8);   // tile count padded for the XCD order
    const bool dbg = dbg0 != nullptr;
#define MOE_Q8(FMT, GU, DB, RW)                                                                          \
    do {                                                                                                  \
        if (DB) launch_timed(q8_mfma_dbg_kernel<FMT, GU, RW>, grid, dim3(64 * kGemmWaves), st, ev0, ev1, a); \
        else launch_timed(q8_mfma_kernel<FMT, GU, RW>, grid, dim3(64 * kGemmWaves), st, ev0, ev1, a);        \
    } while (0)
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
