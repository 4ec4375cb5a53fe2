// Prefill / verification path: batch-union grouped GEMM on the int8 matrix
// cores ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": integer-dot
// kernels with Q8_0-style int8 activations, used in batch; batch-union MoE in
// prefill and MTP verification).
//
// Each 32-deep quantisation group is one v_mfma_i32_32x32x32_i8, whose int32
// result is exact; the group's two fp32 scales (activation row, weight
// column) are applied to it before it joins the fp32 accumulator:
//     acc[m][n] += sx[m, g] * sw[n, g] * I_g[m, n].
// Packed int4 weights are widened to int8 bytes holding 16*q (the nibble in
// the high half of the byte), so the matrix core sees int8 codes; the factor
// 16 is removed exactly by folding 1/16 into the weight scale.
//
// Block tile: 64 rows (tokens of one expert) x 128 weight rows, staged
// through LDS in steps of 4 groups (128 k), double buffered. Four waves in
// 2 x 2; each wave owns 32 rows and two 32-column MFMA tiles.
//   gate/up kernel: the two tiles are gate and up of the same 32 outputs, so
//     SwiGLU and the Q8_0 quantisation of H (32 outputs = one group) happen
//     in registers; H leaves as int8 codes + one fp32 scale per 32.
//   down kernel: two adjacent 32-column tiles of the output; Y leaves fp32.
// Work list: one tile per (expert, 64-row block) from the dispatch kernel;
// blocks past the live tile count exit at once (no host read-back).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = kTileRows;       // 64 rows per tile
constexpr int kBRows = 128;          // weight rows per block
constexpr int kGroupsPerStage = 4;   // 128 k per LDS stage
constexpr int kStageK = kGroupsPerStage * kGroup;
constexpr int kLdsRow = kStageK + 16;              // padded row pitch in bytes
constexpr int kLdsA = kBM * kLdsRow;               // 9216
constexpr int kLdsB = kBRows * kLdsRow;            // 18432
constexpr int kLdsSA = kBM * kGroupsPerStage * 4;  // 1024
constexpr int kLdsSB = kBRows * kGroupsPerStage * 4;
constexpr int kLdsStage = kLdsA + kLdsB + kLdsSA + kLdsSB;

struct MfmaMat {
    const uint8_t* q;
    const float* s;
    int64_t q_stride;   // bytes per expert
    int64_t s_stride;   // floats per expert
};

struct MfmaArgs {
    const int8_t* a_q;      // activation codes, rows of K
    const float* a_s;       // activation scales, rows of K/32
    const int* row_token;   // permuted row -> activation row (nullptr: identity)
    const int4* tiles;      // (expert, row_begin, row_end, 0)
    const int* meta;        // meta[1] = live tile count
    MfmaMat routed[2];      // gate, up (or down, down)
    MfmaMat shared[2];
    int E, K, N;
    int8_t* hq;             // gate/up output codes  [R, N]
    float* hd;              // gate/up output scales [R, N/32]
    float* y;               // down output           [R, N]
    int32_t* dbg0;          // optional exact group dots [R, N, K/32]
    int32_t* dbg1;
};

// Widen 8 packed int4 codes (one dword) to 8 bytes of 16*q, natural order.
__device__ __forceinline__ void widen_int4x8(uint32_t p, uint32_t& out_lo, uint32_t& out_hi) {
    const uint32_t even = (p << 4) & 0xf0f0f0f0u;   // elements 0,2,4,6 as 16*q
    const uint32_t odd = p & 0xf0f0f0f0u;           // elements 1,3,5,7 as 16*q
    // byte i of the 8-byte {odd:even} pair: 0..3 -> even, 4..7 -> odd
    out_lo = __builtin_amdgcn_perm(odd, even, 0x05010400u);
    out_hi = __builtin_amdgcn_perm(odd, even, 0x07030602u);
}

template <int FMT, bool GATEUP, bool DBG>
__global__ __launch_bounds__(256) void q8_mfma_kernel(const MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kLdsStage];
    const int tile = blockIdx.y;
    if (tile >= a.meta[1]) return;
    const int4 td = a.tiles[tile];
    const int e = td.x, row_begin = td.y, rows = td.z - td.y;
    const bool is_shared = e == a.E;
    const MfmaMat* M = is_shared ? a.shared : a.routed;
    const int64_t eo = is_shared ? 0 : e;
    const uint8_t* wq0 = M[0].q + eo * M[0].q_stride;
    const uint8_t* wq1 = M[1].q + eo * M[1].q_stride;
    const float* ws0 = M[0].s + eo * M[0].s_stride;
    const float* ws1 = M[1].s + eo * M[1].s_stride;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int K = a.K, N = a.N, G = K / kGroup, NT = N / kTile;
    const int n0 = blockIdx.x * (GATEUP ? kBRows / 2 : kBRows);
    const int row_bytes = FMT == MOE_W_INT8_G32 ? K : K / 2;
    constexpr float kWScale = FMT == MOE_W_INT8_G32 ? 1.0f : 0.0625f;

    // ---- per-thread global load assignments (fixed over the K loop) ----
    // A codes: 2 x 16 B per thread: row = li / 8, chunk = li % 8
    int a_row_src[2];
    bool a_row_ok[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int li = tid + 256 * r;
        const int row = li >> 3;
        a_row_ok[r] = row < rows;
        const int prow = row_begin + (a_row_ok[r] ? row : 0);
        a_row_src[r] = a.row_token ? a.row_token[prow] : prow;
    }
    // A scales: thread -> (row = tid / 4, group = tid % 4)
    const int sa_row = tid >> 2, sa_g = tid & 3;
    const bool sa_ok = sa_row < rows;
    const int sa_src = a.row_token ? a.row_token[row_begin + (sa_ok ? sa_row : 0)] : row_begin + (sa_ok ? sa_row : 0);
    // B: 4 tiles of 32 weight rows per block (gate/up: 2 gate + 2 up tiles;
    // down: 4 down tiles). Tile bt of the block -> matrix codes/scales + tile row.
    auto b_tile = [&](int bt, const uint8_t*& q, const float*& s, int& tile) {
        if (GATEUP) {
            const bool up = bt >= 2;
            q = up ? wq1 : wq0;
            s = up ? ws1 : ws0;
            tile = n0 / kTile + (up ? bt - 2 : bt);
        } else {
            q = wq0;
            s = ws0;
            tile = n0 / kTile + bt;
        }
    };
    constexpr int kBLoads = FMT == MOE_W_INT8_G32 ? 4 : 2;
    uint4 ra[2];
    uint4 rb[kBLoads];
    float rsa;
    float rsb[2];

    auto load_stage = [&](int stage) {
        const int k0 = stage * kStageK;
        const int g0 = stage * kGroupsPerStage;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int li = tid + 256 * r;
            const int chunk = li & 7;
            const bool ok = a_row_ok[r] && (k0 + chunk * 16) < K;
            ra[r] = ok ? *reinterpret_cast<const uint4*>(a.a_q + (size_t)a_row_src[r] * K + k0 + chunk * 16)
                       : make_uint4(0, 0, 0, 0);
        }
        rsa = (sa_ok && g0 + sa_g < G) ? a.a_s[(size_t)sa_src * G + g0 + sa_g] : 0.0f;
        // a 1 KB block of codes (int8: one tile x group, int4: one tile x
        // pair of groups) is contiguous: a wave reads it whole
#pragma unroll
        for (int r = 0; r < kBLoads; ++r) {
            const int li = tid + 256 * r;
            const int blk = li >> 6, j = li & 63;
            const uint8_t* q;
            const float* sp;
            int tile;
            if constexpr (FMT == MOE_W_INT8_G32) {
                const int bt = blk >> 2, g = blk & 3;
                b_tile(bt, q, sp, tile);
                const bool ok = tile * kTile < N && g0 + g < G;
                rb[r] = ok ? *reinterpret_cast<const uint4*>(q + ((size_t)(g0 + g) * NT + tile) * 1024 + j * 16)
                           : make_uint4(0, 0, 0, 0);
            } else {
                const int bt = blk >> 1, pr = g0 / 2 + (blk & 1);
                b_tile(bt, q, sp, tile);
                const bool ok = tile * kTile < N && pr < G / 2;
                rb[r] = ok ? *reinterpret_cast<const uint4*>(q + ((size_t)pr * NT + tile) * 1024 + j * 16)
                           : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int li = tid + 256 * r;
            const int blk = li >> 5, r32 = li & 31;
            const int bt = blk >> 2, g = g0 + (blk & 3);
            const uint8_t* q;
            const float* sp;
            int tile;
            b_tile(bt, q, sp, tile);
            const bool ok = tile * kTile < N && g < G;
            rsb[r] = ok ? sp[((size_t)tile * (G / 2) + g / 2) * 64 + (r32 & 15) * 4 + (g & 1) * 2 + (r32 >> 4)] *
                              kWScale
                        : 0.0f;
        }
    };

    auto store_stage = [&](int buf) {
        uint8_t* base = lds + buf * kLdsStage;
        uint8_t* A = base;
        uint8_t* B = base + kLdsA;
        float* SA = reinterpret_cast<float*>(base + kLdsA + kLdsB);
        float* SB = reinterpret_cast<float*>(base + kLdsA + kLdsB + kLdsSA);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int li = tid + 256 * r;
            *reinterpret_cast<uint4*>(A + (li >> 3) * kLdsRow + (li & 7) * 16) = ra[r];
        }
        SA[sa_row * kGroupsPerStage + sa_g] = rsa;
        // lane j = nl + 16 h of a block holds k 8h .. 8h+7 of rows nl and 16 + nl
        if constexpr (FMT == MOE_W_INT8_G32) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int li = tid + 256 * r;
                const int blk = li >> 6, j = li & 63;
                const int brow = (blk >> 2) * kTile + (j & 15), g = blk & 3, h = j >> 4;
                uint8_t* dst = B + brow * kLdsRow + g * kGroup + 8 * h;
                *reinterpret_cast<uint2*>(dst) = make_uint2(rb[r].x, rb[r].y);
                *reinterpret_cast<uint2*>(dst + 16 * kLdsRow) = make_uint2(rb[r].z, rb[r].w);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int li = tid + 256 * r;
                const int blk = li >> 6, j = li & 63;
                const int brow = (blk >> 1) * kTile + (j & 15), g = 2 * (blk & 1), h = j >> 4;
                const uint32_t words[4] = {rb[r].x, rb[r].y, rb[r].z, rb[r].w};
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    uint2 w;
                    widen_int4x8(words[qd], w.x, w.y);
                    uint8_t* dst = B + (brow + 16 * (qd & 1)) * kLdsRow + (g + (qd >> 1)) * kGroup + 8 * h;
                    *reinterpret_cast<uint2*>(dst) = w;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int li = tid + 256 * r;
            const int blk = li >> 5, r32 = li & 31;
            SB[((blk >> 2) * kTile + r32) * kGroupsPerStage + (blk & 3)] = rsb[r];
        }
    };

    // wave's operand rows inside the block tile
    const int a_lrow = wm * 32 + (lane & 31);
    const int b_lrow0 = GATEUP ? wn * 32 + (lane & 31) : wn * 64 + (lane & 31);
    const int b_lrow1 = GATEUP ? kBRows / 2 + wn * 32 + (lane & 31) : wn * 64 + 32 + (lane & 31);
    const int khalf = (lane >> 5) * 16;
    // output row of accumulator register i: 8*(i/4) + 4*(lane/32) + i%4
    int m_of[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m_of[i] = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);

    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc0[i] = 0.0f; acc1[i] = 0.0f; }

    const int n_stages = (G + kGroupsPerStage - 1) / kGroupsPerStage;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < n_stages; ++st) {
        if (st + 1 < n_stages) load_stage(st + 1);
        const uint8_t* base = lds + (st & 1) * kLdsStage;
        const uint8_t* A = base;
        const uint8_t* B = base + kLdsA;
        const float* SA = reinterpret_cast<const float*>(base + kLdsA + kLdsB);
        const float* SB = reinterpret_cast<const float*>(base + kLdsA + kLdsB + kLdsSA);
        const int g_here = min(kGroupsPerStage, G - st * kGroupsPerStage);
        for (int g = 0; g < g_here; ++g) {
            const v4i af = *reinterpret_cast<const v4i*>(A + a_lrow * kLdsRow + g * kGroup + khalf);
            const v4i bf0 = *reinterpret_cast<const v4i*>(B + b_lrow0 * kLdsRow + g * kGroup + khalf);
            const v4i bf1 = *reinterpret_cast<const v4i*>(B + b_lrow1 * kLdsRow + g * kGroup + khalf);
            const v16i zero = {};
            const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf0, zero, 0, 0, 0);
            const v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf1, zero, 0, 0, 0);
            const float sw0 = SB[b_lrow0 * kGroupsPerStage + g];
            const float sw1 = SB[b_lrow1 * kGroupsPerStage + g];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float sx = SA[(wm * 32 + m_of[i]) * kGroupsPerStage + g];
                acc0[i] = fmaf((float)d0[i] * sw0, sx, acc0[i]);
                acc1[i] = fmaf((float)d1[i] * sw1, sx, acc1[i]);
            }
            if constexpr (DBG) {
                const int gg = st * kGroupsPerStage + g;
                const int c0 = GATEUP ? n0 + wn * 32 + (lane & 31) : n0 + wn * 64 + (lane & 31);
                const int c1 = GATEUP ? c0 : c0 + 32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = wm * 32 + m_of[i];
                    if (row >= rows) continue;
                    const size_t r = (size_t)(row_begin + row);
                    const int v0 = FMT == MOE_W_INT8_G32 ? d0[i] : (d0[i] >> 4);
                    const int v1 = FMT == MOE_W_INT8_G32 ? d1[i] : (d1[i] >> 4);
                    if (c0 < N) a.dbg0[(r * N + c0) * G + gg] = v0;
                    if (c1 < N) (GATEUP ? a.dbg1 : a.dbg0)[(r * N + c1) * G + gg] = v1;
                }
            }
        }
        if (st + 1 < n_stages) store_stage((st + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue ----
    if constexpr (GATEUP) {
        const int col = n0 + wn * 32 + (lane & 31);
        const bool col_ok = n0 + wn * 32 < N;
        const int GN = N / kGroup;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float h = silu(acc0[i]) * acc1[i];
            float amax = fabsf(h);
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
            const float dd = __fdiv_rn(amax, 127.0f);
            const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
            float q = rintf(__fmul_rn(h, inv));
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            const int row = wm * 32 + m_of[i];
            if (row < rows && col_ok) {
                const size_t r = (size_t)(row_begin + row);
                a.hq[r * N + col] = (int8_t)(int)q;
                if ((lane & 31) == 0) a.hd[r * GN + (n0 + wn * 32) / kGroup] = dd;
            }
        }
    } else {
        const int c0 = n0 + wn * 64 + (lane & 31);
        const int c1 = c0 + 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = wm * 32 + m_of[i];
            if (row >= rows) continue;
            const size_t r = (size_t)(row_begin + row);
            if (c0 < N) a.y[r * N + c0] = acc0[i];
            if (c1 < N) a.y[r * N + c1] = acc1[i];
        }
    }
}

hipError_t launch_q8_mfma(const moe_experts& routed, const moe_experts* shared, bool gateup, const int8_t* a_q,
                          const float* a_s, const int* row_token, const int* tiles, const int* meta, int max_tiles,
                          int8_t* hq, float* hd, float* y, int32_t* dbg0, int32_t* dbg1, hipStream_t st,
                          hipEvent_t ev0, hipEvent_t ev1) {
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
    a.hq = hq;
    a.hd = hd;
    a.y = y;
    a.dbg0 = dbg0;
    a.dbg1 = dbg1;
    auto fill = [&](MfmaMat* dst, const moe_experts& ev) {
        const int64_t rowb = ev.format == MOE_W_INT8_G32 ? a.K : a.K / 2;
        const int64_t qs = (int64_t)a.N * rowb, ss = (int64_t)a.N * (a.K / kGroup);
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
    const int bn = gateup ? kBRows / 2 : kBRows;
    const dim3 grid((a.N + bn - 1) / bn, max_tiles);
    const bool dbg = dbg0 != nullptr;
#define MOE_Q8(FMT, GU, DB) launch_timed(q8_mfma_kernel<FMT, GU, DB>, grid, dim3(256), st, ev0, ev1, a)
    if (routed.format == MOE_W_INT8_G32) {
        if (gateup) { if (dbg) MOE_Q8(MOE_W_INT8_G32, true, true); else MOE_Q8(MOE_W_INT8_G32, true, false); }
        else { if (dbg) MOE_Q8(MOE_W_INT8_G32, false, true); else MOE_Q8(MOE_W_INT8_G32, false, false); }
    } else {
        if (gateup) { if (dbg) MOE_Q8(MOE_W_INT4_G32, true, true); else MOE_Q8(MOE_W_INT4_G32, true, false); }
        else { if (dbg) MOE_Q8(MOE_W_INT4_G32, false, true); else MOE_Q8(MOE_W_INT4_G32, false, false); }
    }
#undef MOE_Q8
    return hipGetLastError();
}

}  // namespace moe
