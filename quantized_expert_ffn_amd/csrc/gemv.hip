// Decode path (fp32 activations): batch-union grouped GEMV on the f16 matrix
// cores, weights dequantised on use ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
// implemented": int8 / packed int4 weights dequantised on use; batch-union
// over the positions routed to one expert; a single row stays in f32).
//
// Exact fp32-level activations on f16 matrix cores. For every group of 32
// along the reduction axis, a power of two p = 2^(e-15) with max|x| < 2^e over
// the values that share it (the whole batch for X, one row for H) is chosen
// and x/p (exact) is split into hi = f16(x/p) and lo = f16(x/p - hi):
// together 22 significant bits. Weight codes are small integers, exact in f16
// (f16codes.h). So
//     sum_k x_k q_k = p * (MFMA(hi, q) + MFMA(lo, q))
// with exact products and fp32 accumulation (v_mfma_f32_16x16x32_f16, K = 32
// = one quantisation group); the group's weight scale and p are applied once
// per output per group.
//
// Two kernels (the hidden states' f16 parts come from the router, one power
// of two per 32-group over the batch):
//   gate/up: per (expert, 32 weight rows): G and U for the expert's tokens,
//            H = silu(G) * U written straight back as hi/lo + p per (row,
//            32 columns), so the down kernel reads it as it is.
//   down:    Y = H Wd^T, fp32, rows in permuted order.
// Weight codes come straight from HBM into operand registers: in the
// lane-tiled layout one 16-byte load per lane brings a wave the B operands of
// both 16-row halves of a 32-row tile for one group (int8) or two groups
// (int4), and one more brings the scales of four group pairs of the tile.
// Every vector memory instruction costs the CU's address unit about the same
// time whatever its width, so the kernel issues few, wide ones: per pair of
// groups and 32-row tile of two matrices, 4 (int8) or 2 (int4) code loads,
// half a scale load and 4 activation loads (hi/lo of two groups), the
// activations serving 64 weight rows. Activation fragments come from L2;
// token rows past an expert's count read as zeros.
#include "common.h"
#include "f16codes.h"
#include "kernels.h"

namespace moe {

struct GemvArgs {
    // f32 path: activation parts in slot order (gate/up [T, K] token rows,
    // down [R, K]) and powers of two (gate/up [K/32]; down [R, K/32], one per
    // row and group). Q8_0 path: ahi holds the Q8_0 codes as
    // f16 in slot order, alo is unused and apow holds the per-row scales
    // [rows, K/32].
    const _Float16* ahi;
    const _Float16* alo;
    const float* apow;
    const int* row_token;   // gate/up: permuted row -> token row of ahi / alo
    int a_rows;             // rows of ahi / alo
    const int4* slots;      // (expert, row_begin, n_rows, 0)
    const int* meta;        // meta[0] = number of slots
    const uint8_t* q[2];    // routed codes: gate, up (gate/up) or down, down
    const float* s[2];
    const uint8_t* sq[2];   // shared expert
    const float* ss[2];
    int64_t q_stride, s_stride;   // per expert (bytes, floats)
    int E, K, N, R;
    // gate/up output, as the down kernel reads it: f32 path H as parts +
    // powers of two ([R, N/32], one per row and group); Q8_0
    // path H's codes as f16 in hhi and its per-row scales in hpow [R, N/32]
    _Float16* hhi;
    _Float16* hlo;
    float* hpow;
    // down output
    float* y;               // [R, N]
    // debug (Q8_0 path only, all or none): the exact group dots [R, N, K/32]
    // of the first and second matrix (gate, up; down: both tiles to dbg0),
    // and H's int8 codes in natural order [R, N]
    int32_t* dbg0;
    int32_t* dbg1;
    int8_t* dbg_hq;
};

constexpr int kMaxGemvGroups = 256;   // K <= 8192

// Block: KS waves splitting the group pairs of the reduction axis into
// contiguous runs. Each wave covers two 32-row matrix tiles: gate and up of
// tile blockIdx.x (GATEUP), or down tiles 2 blockIdx.x and +1. Two pairs of
// groups are in flight per wave, weight codes (HBM) and activation
// fragments (L2) alike; loads retire in order, so both streams keep the same
// depth. Scales come four pairs per load and reach their lanes through
// ds_bpermute.
//
// Q8 (Q8_0 activations, the small-batch verification case): the activation
// operand is the codes themselves, exact in f16 like the weight codes, so one
// product per group gives the exact integer group dot and no lo part is
// needed; both group scales are applied to it per output (the activation
// scale varies by row, from an LDS table of the tile's 16 rows).
//
// ROW (a scale per weight row): no scale loads in the loop; only the
// activation side's per-group factor joins each group's product, and the
// row's scale multiplies the finished sum once.
//
// DBG (Q8 only, the test hook): also writes every exact group dot and H's
// int8 codes, from the same products the outputs are made of.
template <int FMT, bool GATEUP, int KS, bool Q8, bool ROW, bool DBG = false>
__global__ __launch_bounds__(64 * KS) void gemv_kernel(const GemvArgs a) {
    static_assert(Q8 || !DBG, "group dots exist on the Q8_0 path only");
    // 16-byte code loads per tile per pair (int2: one per two pairs)
    constexpr int kCL = FMT == MOE_W_INT8_G32 ? 2 : 1;
    // cache policy of the code loads: non-temporal where it measured faster
    // (one wave per tile, or Q8_0 activations: OLMoE int8 / int4 at 16 tokens
    // and GLM verification gained 5-10%); the f32 path's K-split waves at one
    // token measured ~3% slower with it, so they keep the default policy
    constexpr int kCodePolicy = (Q8 || KS == 1) ? kStreamed : 0;
    constexpr bool I2 = FMT == MOE_W_INT2_G32;
    // the activation side's per-group factors: one per group over the batch
    // (f32 gate/up), or one per group and row of the 16-row tile, [group][16]
    // (Q8: the rows' Q8_0 scales; f32 down: H's powers of two per row)
    constexpr bool kRowFactors = Q8 || !GATEUP;
    __shared__ float pwtab[kRowFactors ? 16 * kMaxGemvGroups : kMaxGemvGroups];
    __shared__ float red[KS > 1 ? KS - 1 : 1][2][2][4][64];

    const int slot = blockIdx.y;
    if (slot >= a.meta[0]) return;
    const int4 sl = a.slots[slot];
    const int e = sl.x, row_begin = sl.y, n_rows = sl.z;
    const bool is_shared = e == a.E;
    const int64_t eo = is_shared ? 0 : e;
    const int lane = threadIdx.x & 63, ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 4, nl = lane & 15;
    const int K = a.K, N = a.N, G = K / kGroup, P = G / 2, R = a.R;
    const int n_tiles = N / kTile;
    int tile[2];
    tile[0] = GATEUP ? blockIdx.x : 2 * blockIdx.x;
    // down with an odd tile count: tile[1] of the last block is n_tiles, a
    // phantom whose code loads land on real bytes but whose scales read as
    // zeros (past the scale resource), so it adds zeros and is not stored
    tile[1] = GATEUP ? blockIdx.x : 2 * blockIdx.x + 1;

    // operands through buffer resources: a lane offset per stream, the pair
    // step in a uniform register; offsets past a resource's end read as 0
    // (rq0: the same codes with no records, every read a zero)
    __amdgpu_buffer_rsrc_t rq[2], rq0[2], rs[2];
    int q_voff[2], s_voff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int m = GATEUP ? t : 0;
        const uint8_t* qbase = (is_shared ? a.sq[m] : a.q[m]) + eo * a.q_stride;
        const float* sbase = (is_shared ? a.ss[m] : a.s[m]) + eo * a.s_stride;
        rq[t] = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, 0, (int)a.q_stride, 0x00020000);
        rq0[t] = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, 0, 0, 0x00020000);
        rs[t] = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, (int)(a.s_stride * 4), 0x00020000);
        q_voff[t] = tile[t] * 1024 + lane * 16;
        // four consecutive pairs' scale blocks are 1 KB: lane nl + 16q reads
        // pair q's 16 bytes for rows nl, 16 + nl
        s_voff[t] = tile[t] * P * 256 + lane * 16;
    }
    // ROW: the scales of this lane's output rows (a tile past the matrix
    // reads zeros)
    float srow[2][2];
    if constexpr (ROW) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                srow[t][r] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rs[t], (tile[t] * kTile + 16 * r + nl) * 4, 0, 0));
    }
    const int a_bytes = a.a_rows * K * 2;
    const __amdgpu_buffer_rsrc_t rah = __builtin_amdgcn_make_buffer_rsrc((void*)a.ahi, 0, a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ral = __builtin_amdgcn_make_buffer_rsrc((void*)a.alo, 0, a_bytes, 0x00020000);
    // wave ks takes a contiguous run of pairs [c0, c0 + n_my) (int2: whole
    // quads of groups, as its code blocks hold them)
    int c0, n_my;
    if constexpr (I2) {
        const int Q = P / 2;
        c0 = 2 * (ks * Q / KS);
        n_my = 2 * ((ks + 1) * Q / KS) - c0;
    } else {
        c0 = ks * P / KS;
        n_my = (ks + 1) * P / KS - c0;
    }
    if constexpr (GATEUP && !Q8) {
        for (int i = threadIdx.x; i < G; i += 64 * KS) pwtab[i] = a.apow[i];
    }

    for (int mt = 0; mt < n_rows; mt += 16) {
        const int rows_here = min(16, n_rows - mt);
        // this lane's operand row: a token (gate/up) or a permuted row (down);
        // rows past the expert's count read past the resource: zeros
        int a_voff = 0x7ffffff0;
        if (nl < rows_here) {
            const int ar = GATEUP ? a.row_token[row_begin + mt + nl] : row_begin + mt + nl;
            a_voff = (ar * K + 8 * h) * 2;
        }
        const int prow = row_begin + mt + 4 * h;   // output rows 4h .. 4h+3 of the tile

        __syncthreads();   // pwtab is written; the previous tile's readers of red are done
        if constexpr (kRowFactors) {
            for (int i = threadIdx.x; i < 16 * G; i += 64 * KS) {
                const int g = i >> 4, rr = i & 15;
                float v = 0.0f;
                if (rr < rows_here) {
                    const int ar = GATEUP ? a.row_token[row_begin + mt + rr] : row_begin + mt + rr;
                    v = a.apow[(size_t)ar * G + g];
                }
                pwtab[i] = v;
            }
            __syncthreads();
        }

        v4f acc[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 2; ++r) acc[t][r] = v4f{0.f, 0.f, 0.f, 0.f};

        // ring of NB = 2 pairs (codes, activation parts) and of two scale
        // quads (four pairs each: the current one and the next). int2: the
        // code ring holds two quads of groups, slot (j / 2) % 2, each loaded
        // by its even pair for itself and the odd one after it.
        uint4 wq[2][2][kCL];
        v8h xh[2][2], xl[2][2];
        uint4 sq_cur[2] = {}, sq_next[2] = {};
        // pair j of the run into ring slot sp; rr = j % 4 (a constant at every
        // call: runs start on an even pair and rounds hold four)
        auto load = [&](int sp, int j, int rr) {
            // past the end of the run every step still issues the same loads,
            // so that waits stay counted: the activations of the last pair
            // again (L2-resident), and code loads through a resource with no
            // records, which return zeros without touching memory (codes
            // streamed with the non-temporal policy would otherwise be read
            // from HBM again)
            const bool past = j >= n_my;
            const int p = c0 + (past ? n_my - 1 : j);
            if constexpr (I2) {
                if ((rr & 1) == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        wq[(rr >> 1) & 1][t][0] = __builtin_bit_cast(
                            uint4, __builtin_amdgcn_raw_buffer_load_b128(past ? rq0[t] : rq[t], q_voff[t],
                                                                         (p >> 1) * n_tiles * 1024, kCodePolicy));
                }
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int c = 0; c < kCL; ++c)
                        wq[sp][t][c] = __builtin_bit_cast(
                            uint4, __builtin_amdgcn_raw_buffer_load_b128(past ? rq0[t] : rq[t], q_voff[t],
                                                                         (kCL * p + c) * n_tiles * 1024, kCodePolicy));
            }
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                xh[sp][gi] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rah, a_voff, (2 * p + gi) * 64, 0));
                if constexpr (!Q8)
                    xl[sp][gi] =
                        __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(ral, a_voff, (2 * p + gi) * 64, 0));
            }
        };
        // scales of pairs c0 + 4q .. + 3 (those past the run are read but unused)
        auto load_quad = [&](int q) {
            if constexpr (ROW) return;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                sq_next[t] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rs[t], s_voff[t], (c0 + 4 * q) * 256, 0));
        };
        // pair j of the run, from ring slot jj; its scales sit in lane row r
        // (= j % 4) of the current quad
        auto step = [&](int jj, int j, int r) {
            const int p = c0 + j;
            float pw0 = 0.0f, pw1 = 0.0f;
            float4 sx[2];
            if constexpr (kRowFactors) {
                // activation factors of the lane's rows 4h .. 4h+3, both groups
                sx[0] = *reinterpret_cast<const float4*>(&pwtab[(2 * p) * 16 + 4 * h]);
                sx[1] = *reinterpret_cast<const float4*>(&pwtab[(2 * p + 1) * 16 + 4 * h]);
            } else {
                pw0 = pwtab[2 * p];
                pw1 = pwtab[2 * p + 1];
            }
            const int src = (nl + 16 * r) * 4;
            float sc[2][4] = {};
            if constexpr (!ROW) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sc[t][0] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, (int)sq_cur[t].x));
                    sc[t][1] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, (int)sq_cur[t].y));
                    sc[t][2] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, (int)sq_cur[t].z));
                    sc[t][3] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, (int)sq_cur[t].w));
                }
            }
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const float pw = gi ? pw1 : pw0;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    v8h b0, b1;
                    if constexpr (I2) {
                        // dword 2 (j % 2) + gi of the quad: both 16-row halves
                        const uint4 c = wq[(r >> 1) & 1][t][0];
                        const uint32_t dw = (r & 1) ? (gi ? c.w : c.z) : (gi ? c.y : c.x);
                        b0 = int2_codes_to_f16<0>(dw);
                        b1 = int2_codes_to_f16<1>(dw);
                    } else if constexpr (FMT == MOE_W_INT8_G32) {
                        const uint4 c = wq[jj][t][gi];
                        b0 = codes_to_f16<FMT>(c.x, c.y);
                        b1 = codes_to_f16<FMT>(c.z, c.w);
                    } else {
                        const uint4 c = wq[jj][t][0];
                        b0 = codes_to_f16<FMT>(gi ? c.z : c.x, 0u);
                        b1 = codes_to_f16<FMT>(gi ? c.w : c.y, 0u);
                    }
                    v4f d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[jj][gi], b0, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    v4f d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[jj][gi], b1, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (DBG) {
                        // rows 4h + i of this 16-row tile, columns nl and 16 + nl of
                        // weight tile t, group 2p + gi
                        if (tile[t] < n_tiles) {
                            int32_t* dst = (GATEUP && t) ? a.dbg1 : a.dbg0;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if (4 * h + i >= rows_here) continue;
                                const size_t o = ((size_t)(prow + i) * N + tile[t] * kTile + nl) * G + 2 * p + gi;
                                dst[o] = (int32_t)d0[i];
                                dst[o + (size_t)16 * G] = (int32_t)d1[i];
                            }
                        }
                    }
                    if constexpr (Q8 && ROW) {
                        const float4 x = sx[gi];
                        acc[t][0][0] = fmaf(d0[0], x.x, acc[t][0][0]);
                        acc[t][0][1] = fmaf(d0[1], x.y, acc[t][0][1]);
                        acc[t][0][2] = fmaf(d0[2], x.z, acc[t][0][2]);
                        acc[t][0][3] = fmaf(d0[3], x.w, acc[t][0][3]);
                        acc[t][1][0] = fmaf(d1[0], x.x, acc[t][1][0]);
                        acc[t][1][1] = fmaf(d1[1], x.y, acc[t][1][1]);
                        acc[t][1][2] = fmaf(d1[2], x.z, acc[t][1][2]);
                        acc[t][1][3] = fmaf(d1[3], x.w, acc[t][1][3]);
                    } else if constexpr (Q8) {
                        const float s0 = sc[t][2 * gi], s1 = sc[t][2 * gi + 1];
                        const float4 x = sx[gi];
                        acc[t][0][0] = fmaf(d0[0], s0 * x.x, acc[t][0][0]);
                        acc[t][0][1] = fmaf(d0[1], s0 * x.y, acc[t][0][1]);
                        acc[t][0][2] = fmaf(d0[2], s0 * x.z, acc[t][0][2]);
                        acc[t][0][3] = fmaf(d0[3], s0 * x.w, acc[t][0][3]);
                        acc[t][1][0] = fmaf(d1[0], s1 * x.x, acc[t][1][0]);
                        acc[t][1][1] = fmaf(d1[1], s1 * x.y, acc[t][1][1]);
                        acc[t][1][2] = fmaf(d1[2], s1 * x.z, acc[t][1][2]);
                        acc[t][1][3] = fmaf(d1[3], s1 * x.w, acc[t][1][3]);
                    } else if constexpr (GATEUP) {
                        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[jj][gi], b0, d0, 0, 0, 0);
                        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[jj][gi], b1, d1, 0, 0, 0);
                        const float f0 = ROW ? pw : sc[t][2 * gi] * pw;
                        const float f1 = ROW ? pw : sc[t][2 * gi + 1] * pw;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[t][0][i] = fmaf(d0[i], f0, acc[t][0][i]);
                            acc[t][1][i] = fmaf(d1[i], f1, acc[t][1][i]);
                        }
                    } else {
                        // f32 down: H's power of two differs per row
                        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[jj][gi], b0, d0, 0, 0, 0);
                        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[jj][gi], b1, d1, 0, 0, 0);
                        const float4 x = sx[gi];
                        const float s0 = ROW ? 1.0f : sc[t][2 * gi], s1 = ROW ? 1.0f : sc[t][2 * gi + 1];
                        acc[t][0][0] = fmaf(d0[0], s0 * x.x, acc[t][0][0]);
                        acc[t][0][1] = fmaf(d0[1], s0 * x.y, acc[t][0][1]);
                        acc[t][0][2] = fmaf(d0[2], s0 * x.z, acc[t][0][2]);
                        acc[t][0][3] = fmaf(d0[3], s0 * x.w, acc[t][0][3]);
                        acc[t][1][0] = fmaf(d1[0], s1 * x.x, acc[t][1][0]);
                        acc[t][1][1] = fmaf(d1[1], s1 * x.y, acc[t][1][1]);
                        acc[t][1][2] = fmaf(d1[2], s1 * x.z, acc[t][1][2]);
                        acc[t][1][3] = fmaf(d1[3], s1 * x.w, acc[t][1][3]);
                    }
                }
            }
        };
        // rounds of four pairs: each step computes its ring slot and refills
        // it two pairs ahead; the scale quad of the next round is issued at
        // the start of this one. The refills stay where they are: issued
        // later, their waits would cover the younger loads too (loads retire
        // in order).
        // the first quad goes out first: at the top of every round the quad
        // it waits for is then older than at least two pairs of loads
        load_quad(0);
        load(0, 0, 0);
        load(1, 1, 1);
        int j0 = 0;
        for (; j0 + 4 <= n_my; j0 += 4) {
            sq_cur[0] = sq_next[0];
            sq_cur[1] = sq_next[1];
            __builtin_amdgcn_sched_barrier(0);
            load_quad(j0 / 4 + 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __builtin_amdgcn_sched_barrier(0);
                step(r & 1, j0 + r, r);
                __builtin_amdgcn_sched_barrier(0);
                load(r & 1, j0 + r + 2, (r + 2) & 3);
            }
        }
        // the last n_my % 4 pairs
        sq_cur[0] = sq_next[0];
        sq_cur[1] = sq_next[1];
        const int rest = n_my - j0;
        if (rest > 0) step(0, j0, 0);
        if (rest > 2) load(0, j0 + 2, 2);
        if (rest > 1) step(1, j0 + 1, 1);
        if (rest > 2) step(0, j0 + 2, 2);

        // sum the KS partial results of each output in wave order
        if constexpr (KS > 1) {
            if (ks > 0) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 2; ++r)
#pragma unroll
                        for (int i = 0; i < 4; ++i) red[ks - 1][t][r][i][lane] = acc[t][r][i];
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int w = 0; w < KS - 1; ++w)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int r = 0; r < 2; ++r)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[t][r][i] += red[w][t][r][i][lane];
            }
        }
        if (ks != 0) continue;
        if constexpr (ROW) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[t][r][i] *= srow[t][r];
        }

        if constexpr (GATEUP && Q8) {
            // H = silu(G) * U, then Q8_0 of each token's 32 columns (one group
            // of the down projection's reduction axis) in the fp32 steps of the
            // quantiser: d = amax / 127, q = rne(h * (1 / d))
            const int GN = N / kGroup;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float h0 = silu(acc[0][0][i]) * acc[1][0][i];   // column nl
                const float h1 = silu(acc[0][1][i]) * acc[1][1][i];   // column 16 + nl
                float am = fmaxf(fabsf(h0), fabsf(h1));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0xB1, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x4E, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x141, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x140, 0xF, 0xF, true)));
                const float dd = __fdiv_rn(am, 127.0f);
                const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
                if (4 * h + i < rows_here) {
                    const size_t row = (size_t)(prow + i);
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int kk = 16 * r + nl;
                        const int pos = 8 * (kk >> 3) + k_slot(FMT, kk & 7);
                        const float q = fminf(fmaxf(rintf(__fmul_rn(r ? h1 : h0, inv)), -127.0f), 127.0f);
                        a.hhi[row * N + (size_t)tile[0] * kGroup + pos] = (_Float16)q;
                        if constexpr (DBG) a.dbg_hq[row * N + (size_t)tile[0] * kGroup + kk] = (int8_t)(int)q;
                    }
                    if (nl == 0) a.hpow[row * GN + tile[0]] = dd;
                }
            }
        } else if constexpr (GATEUP) {
            // H = silu(G) * U for tokens 4h + i and columns nl, 16 + nl of the
            // tile: per token, 32 columns (one group of the down projection's
            // reduction axis) under one power of two of their own
            const int GN = N / kGroup;
            float hv[2][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[0][i] = (4 * h + i < rows_here) ? silu(acc[0][0][i]) * acc[1][0][i] : 0.0f;
                hv[1][i] = (4 * h + i < rows_here) ? silu(acc[0][1][i]) * acc[1][1][i] : 0.0f;
                // the token's 32 columns sit in the 16 lanes of this DPP row
                float am = fmaxf(fabsf(hv[0][i]), fabsf(hv[1][i]));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0xB1, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x4E, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x141, 0xF, 0xF, true)));
                am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x140, 0xF, 0xF, true)));
                const int ex = pow2_exponent(am);
                const float up = ldexpf(1.0f, 15 - ex);
                if (4 * h + i < rows_here) {
                    const size_t row = (size_t)(prow + i);
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int kk = 16 * r + nl;                       // k of this column inside the group
                        const int pos = 8 * (kk >> 3) + k_slot(FMT, kk & 7);
                        const float sv = hv[r][i] * up;
                        const _Float16 hh = (_Float16)sv;
                        const size_t off = row * N + (size_t)tile[0] * kGroup + pos;
                        a.hhi[off] = hh;
                        a.hlo[off] = (_Float16)(sv - (float)hh);
                    }
                    if (nl == 0) a.hpow[row * GN + tile[0]] = ldexpf(1.0f, ex - 15);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (tile[t] >= n_tiles) continue;
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * h + i < rows_here)
                            a.y[(size_t)(prow + i) * N + tile[t] * kTile + 16 * r + nl] = acc[t][r][i];
            }
        }
    }
}

// K-split per block: double it while the grid stays within a wave budget and
// every wave keeps at least two pairs of groups. The budgets were measured:
// the f32 path is fastest at ~6 waves per CU (more waves thrash the caches
// between the activation parts and the code streams), the Q8_0 path, which
// reads half the activation bytes, at ~4 times that.
static int choose_ks(int slots, int blocks_x, int P, bool q8) {
    const long budget = q8 ? 12288 : 3072;   // waves x 2
    int ks = 1;
    while (ks < 8 && (long)slots * blocks_x * 2 * ks <= budget && P >= 4 * ks) ks *= 2;
    return ks;
}

hipError_t launch_gemv(const moe_experts& routed, const moe_experts* shared, bool gateup, bool q8, const _Float16* ahi,
                       const _Float16* alo, const float* apow, const int* row_token, int a_rows, int R,
                       const int* slots, const int* meta, int max_slots, _Float16* hhi, _Float16* hlo, float* hpow,
                       float* y, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, int32_t* dbg0, int32_t* dbg1,
                       int8_t* dbg_hq) {
    if (max_slots == 0) return hipSuccess;
    if (dbg0 && !q8) return hipErrorInvalidValue;
    GemvArgs a{};
    a.ahi = ahi;
    a.alo = alo;
    a.apow = apow;
    a.row_token = row_token;
    a.a_rows = a_rows;
    a.slots = reinterpret_cast<const int4*>(slots);
    a.meta = meta;
    a.E = routed.n_experts;
    const int d = routed.d_model, I = routed.d_ff;
    a.K = gateup ? d : I;
    a.N = gateup ? I : d;
    a.R = R;
    if (a.K / kGroup > kMaxGemvGroups) return hipErrorInvalidValue;
    a.q_stride = fmt_code_bytes(routed.format, a.N, a.K);
    a.s_stride = fmt_scale_floats(routed.format, a.N, a.K);
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
    a.dbg0 = dbg0;
    a.dbg1 = dbg1;
    a.dbg_hq = dbg_hq;
    const bool dbg = dbg0 != nullptr;
    const int tiles = a.N / kTile;
    const int bx = gateup ? tiles : (tiles + 1) / 2;
    const int ks = choose_ks(max_slots, bx, a.K / (2 * kGroup), q8);
    const dim3 grid(bx, max_slots);
#define MOE_GEMV(FMT, RW, GU, KSV)                                                                              \
    do {                                                                                                        \
        if (q8 && dbg) launch_timed(gemv_kernel<FMT, GU, KSV, true, RW, true>, grid, dim3(64 * KSV), st, ev0, ev1, a); \
        else if (q8) launch_timed(gemv_kernel<FMT, GU, KSV, true, RW>, grid, dim3(64 * KSV), st, ev0, ev1, a);  \
        else launch_timed(gemv_kernel<FMT, GU, KSV, false, RW>, grid, dim3(64 * KSV), st, ev0, ev1, a);         \
    } while (0)
#define MOE_GEMV_KS(FMT, RW, GU)                \
    if (ks == 1) MOE_GEMV(FMT, RW, GU, 1);      \
    else if (ks == 2) MOE_GEMV(FMT, RW, GU, 2); \
    else if (ks == 4) MOE_GEMV(FMT, RW, GU, 4); \
    else MOE_GEMV(FMT, RW, GU, 8);
#define MOE_GEMV_GU(FMT, RW) \
    if (gateup) { MOE_GEMV_KS(FMT, RW, true) } else { MOE_GEMV_KS(FMT, RW, false) }
    switch (routed.format) {
        case MOE_W_INT8_G32: MOE_GEMV_GU(MOE_W_INT8_G32, false) break;
        case MOE_W_INT4_G32: MOE_GEMV_GU(MOE_W_INT4_G32, false) break;
        case MOE_W_INT2_G32: MOE_GEMV_GU(MOE_W_INT2_G32, false) break;
        case MOE_W_INT8_ROW: MOE_GEMV_GU(MOE_W_INT8_G32, true) break;
        case MOE_W_INT4_ROW: MOE_GEMV_GU(MOE_W_INT4_G32, true) break;
        default: MOE_GEMV_GU(MOE_W_INT2_G32, true) break;
    }
#undef MOE_GEMV_GU
#undef MOE_GEMV_KS
#undef MOE_GEMV
    return hipGetLastError();
}

}  // namespace moe
