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
// Block tile: 64 rows (tokens of one expert) x 128 weight rows (four 32-row
// tiles), staged through LDS in steps of 4 groups (128 k), double buffered,
// by direct global -> LDS loads: no staging registers, the weight blocks land
// exactly as they are stored. Four waves in 2 x 2; each wave owns 32 rows
// and two 32-column MFMA tiles.
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

constexpr int kBM = kTileRows;       // 64 token rows per block
constexpr int kSG = 4;               // groups per LDS stage (128 k)

// One LDS stage (bytes), filled by direct global -> LDS loads (each wave
// load writes 64 lanes x 16 (or 4) bytes contiguously):
//   A  [kSG groups][2 halves][64 rows][16 B]   activation codes; a wave's
//      MFMA A operand (row l%32, k 16(l/32) .. +15) is one conflict-free read
//   B  int8: [4 tiles][kSG groups][1 KB]  weight blocks exactly as in HBM
//      int4: [4 tiles][kSG/2 pairs][1 KB]
//   SX [kSG groups][64 rows] fp32   activation scales (4 rows per 16-byte read)
//   SW [4 tiles][kSG/2 pairs][64] fp32  weight scale blocks as in HBM
constexpr int kLdsA = kSG * 2 * kBM * 16;        // 8192
constexpr int kLdsSX = kSG * kBM * 4;            // 1024
constexpr int kLdsSW = 4 * (kSG / 2) * 64 * 4;   // 2048
template <int FMT>
constexpr int lds_b_bytes() { return FMT == MOE_W_INT8_G32 ? 4 * kSG * 1024 : 4 * (kSG / 2) * 1024; }
template <int FMT>
constexpr int lds_stage_bytes() { return kLdsA + lds_b_bytes<FMT>() + kLdsSX + kLdsSW; }

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// one wave's direct load of 64 x BYTES from per-lane global addresses into
// LDS at `dst` (wave-uniform), lane L at dst + L * BYTES
template <int BYTES>
__device__ __forceinline__ void wave_load_lds(const void* src, uint8_t* dst) {
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
}

template <int FMT, bool GATEUP, bool DBG>
__global__ __launch_bounds__(256) void q8_mfma_kernel(const MfmaArgs a) {
    constexpr int kStage = lds_stage_bytes<FMT>();
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage];
    const int tile_id = blockIdx.y;
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
    const int T0 = blockIdx.x * (GATEUP ? 2 : 4);      // first 32-row weight tile of the block
    constexpr float kWScale = FMT == MOE_W_INT8_G32 ? 1.0f : 0.0625f;

    // block tile j (0..3) -> matrix and tile index (clamped to the matrix:
    // loads stay inside it; results of a clamped tile are not stored)
    auto tile_of = [&](int j) { return min(T0 + (GATEUP ? (j & 1) : j), NT - 1); };
    auto mat_of = [&](int j) { return GATEUP ? (j >> 1) : 0; };
    const uint8_t* wq[2];
    const float* wsb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        wq[m] = M[m].q + eo * M[m].q_stride;
        wsb[m] = M[m].s + eo * M[m].s_stride;
    }
    // this lane's activation row for the stage loads (row L of the tile,
    // clamped to the tile's rows: rows past it are computed, never stored)
    const int arow = row_begin + min(lane, rows - 1);
    const int asrc = a.row_token ? a.row_token[arow] : arow;
    const int8_t* arow_ptr = a.a_q + (size_t)asrc * K;
    const float* srow_ptr = a.a_s + (size_t)asrc * G;

    // stage loads: every wave takes every fourth job
    auto issue_stage = [&](int st, int buf) {
        uint8_t* base = lds + buf * kStage;
        uint8_t* A = base;
        uint8_t* B = base + kLdsA;
        uint8_t* SX = B + lds_b_bytes<FMT>();
        uint8_t* SW = SX + kLdsSX;
        const int g0 = st * kSG;
        constexpr int nA = kSG * 2;
        constexpr int nB = FMT == MOE_W_INT8_G32 ? 4 * kSG : 4 * (kSG / 2);
        constexpr int nSX = kSG;
        constexpr int nSW = 2;
        constexpr int nJobs = nA + nB + nSX + nSW;
#pragma unroll
        for (int job = wave; job < nJobs; job += 4) {
            if (job < nA) {
                const int g = job >> 1, half = job & 1;
                const int gc = min(g0 + g, G - 1);
                wave_load_lds<16>(arow_ptr + gc * kGroup + half * 16, A + (g * 2 + half) * kBM * 16);
            } else if (job < nA + nB) {
                const int b = job - nA;
                if constexpr (FMT == MOE_W_INT8_G32) {
                    const int j = b / kSG, g = b % kSG;
                    const int gc = min(g0 + g, G - 1);
                    wave_load_lds<16>(wq[mat_of(j)] + ((size_t)gc * NT + tile_of(j)) * 1024 + lane * 16,
                                      B + (j * kSG + g) * 1024);
                } else {
                    const int j = b / (kSG / 2), pp = b % (kSG / 2);
                    const int pc = min(g0 / 2 + pp, P - 1);
                    wave_load_lds<16>(wq[mat_of(j)] + ((size_t)pc * NT + tile_of(j)) * 1024 + lane * 16,
                                      B + (j * (kSG / 2) + pp) * 1024);
                }
            } else if (job < nA + nB + nSX) {
                const int g = job - nA - nB;
                wave_load_lds<4>(srow_ptr + min(g0 + g, G - 1), SX + g * kBM * 4);
            } else {
                // two tiles' scale blocks for this stage's two pairs, 512 B each
                const int q = job - nA - nB - nSX;
                const int j = 2 * q + (lane >> 5);
                const int pc = min(g0 / 2 + ((lane & 31) >> 4), P - 1);
                wave_load_lds<16>(wsb[mat_of(j)] + ((size_t)tile_of(j) * P + pc) * 64 + (lane & 15) * 4,
                                  SW + q * 1024);
            }
        }
    };

    // output rows of accumulator register i: 8*(i/4) + 4*(lane/32) + i%4
    const int khalf = lane >> 5, ncol = lane & 31;
    // wave's two MFMA tiles (block tile index j)
    const int jt0 = GATEUP ? wn : 2 * wn;
    const int jt1 = GATEUP ? 2 + wn : 2 * wn + 1;

    float acc[2][16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc[0][i] = 0.0f; acc[1][i] = 0.0f; }

    const int n_stages = (G + kSG - 1) / kSG;
    issue_stage(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < n_stages; ++st) {
        if (st + 1 < n_stages) issue_stage(st + 1, (st + 1) & 1);
        const uint8_t* base = lds + (st & 1) * kStage;
        const uint8_t* A = base;
        const uint8_t* B = base + kLdsA;
        const float* SX = reinterpret_cast<const float*>(B + lds_b_bytes<FMT>());
        const float* SW = SX + kSG * kBM;
        const int g_here = min(kSG, G - st * kSG);
#pragma unroll
        for (int g = 0; g < kSG; ++g) {
            if (g >= g_here) break;
            const v4i af = *reinterpret_cast<const v4i*>(A + ((g * 2 + khalf) * kBM + wm * 32 + ncol) * 16);
            float sx[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(SX + g * kBM + wm * 32 + 8 * q + 4 * khalf);
                sx[4 * q] = v.x;
                sx[4 * q + 1] = v.y;
                sx[4 * q + 2] = v.z;
                sx[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int j = tt ? jt1 : jt0;
                v4i bf;
                if constexpr (FMT == MOE_W_INT8_G32) {
                    // row ncol, k 16 khalf .. +15: lanes (ncol%16) + 32 khalf (+16) of the block
                    const uint8_t* blk = B + (j * kSG + g) * 1024 + ((ncol & 15) + 32 * khalf) * 16 + (ncol >> 4) * 8;
                    const uint2 p0 = *reinterpret_cast<const uint2*>(blk);
                    const uint2 p1 = *reinterpret_cast<const uint2*>(blk + 256);
                    bf = v4i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y};
                } else {
                    const uint8_t* blk = B + (j * (kSG / 2) + (g >> 1)) * 1024 + ((ncol & 15) + 32 * khalf) * 16 +
                                         ((g & 1) * 2 + (ncol >> 4)) * 4;
                    const uint32_t d0 = *reinterpret_cast<const uint32_t*>(blk);
                    const uint32_t d1 = *reinterpret_cast<const uint32_t*>(blk + 256);
                    uint32_t w0, w1, w2, w3;
                    widen_int4x8(d0, w0, w1);
                    widen_int4x8(d1, w2, w3);
                    bf = v4i{(int)w0, (int)w1, (int)w2, (int)w3};
                }
                const v16i zero = {};
                const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, zero, 0, 0, 0);
                const float sw = SW[(j * (kSG / 2) + (g >> 1)) * 64 + (ncol & 15) * 4 + (g & 1) * 2 + (ncol >> 4)] *
                                 kWScale;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[tt][i] = fmaf((float)d[i] * sw, sx[i], acc[tt][i]);
                if constexpr (DBG) {
                    const int gg = st * kSG + g;
                    const int col = GATEUP ? T0 * kTile + 32 * wn + ncol : (T0 + j) * kTile + ncol;
                    int32_t* dst = (GATEUP && tt == 1) ? a.dbg1 : a.dbg0;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int row = wm * 32 + 8 * (i >> 2) + 4 * khalf + (i & 3);
                        if (row >= rows || col >= N) continue;
                        const int v = FMT == MOE_W_INT8_G32 ? d[i] : (d[i] >> 4);
                        dst[((size_t)(row_begin + row) * N + col) * G + gg] = v;
                    }
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue ----
    if constexpr (GATEUP) {
        const int col = T0 * kTile + 32 * wn + ncol;
        const bool col_ok = T0 + wn < NT;
        const int GN = N / kGroup;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float h = silu(acc[0][i]) * acc[1][i];
            float amax = fabsf(h);
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
            const float dd = __fdiv_rn(amax, 127.0f);
            const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
            float q = rintf(__fmul_rn(h, inv));
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            const int row = wm * 32 + 8 * (i >> 2) + 4 * khalf + (i & 3);
            if (row < rows && col_ok) {
                const size_t r = (size_t)(row_begin + row);
                a.hq[r * N + col] = (int8_t)(int)q;
                if (ncol == 0) a.hd[r * GN + T0 + wn] = dd;
            }
        }
    } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = T0 + (tt ? jt1 : jt0);
            if (t >= NT) continue;
            const int col = t * kTile + ncol;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = wm * 32 + 8 * (i >> 2) + 4 * khalf + (i & 3);
                if (row < rows) a.y[(size_t)(row_begin + row) * N + col] = acc[tt][i];
            }
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
    const int bn = gateup ? 2 * kTile : 4 * kTile;   // output columns per block
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
