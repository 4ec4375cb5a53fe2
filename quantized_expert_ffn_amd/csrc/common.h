// Internal helpers shared by the libmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 32;            // quantisation group along the reduction axis
constexpr int kMaxExperts = 1024;
constexpr int kMaxGroups = 64;        // noaux_tc n_group limit (a bit mask of groups)

// ---------------------------------------------------------------------------
// Workspace layout. Every section is 256-byte aligned; the same function is
// used to size the workspace and to carve it, so the two never disagree.
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t logits = 0;     // f32  [T, E]
    size_t idx = 0;        // i32  [T, k]
    size_t wts = 0;        // f32  [T, k]
    size_t counts = 0;     // i32  [E]
    size_t offsets = 0;    // i32  [E + 1]
    size_t perm = 0;       // i32  [T*k]
    size_t inv_perm = 0;   // i32  [T*k]
    size_t row_token = 0;  // i32  [T*k + T]   permuted row -> token
    size_t slots = 0;      // i32  [E + 1][4]  (expert, row_begin, n_rows, 0)
    size_t tiles = 0;      // i32  [max_tiles][4] (expert, row_begin, row_end, 0); row_end == row_begin: empty
    size_t meta = 0;       // i32  [4]  n_slots, n_tiles, status, 0
    size_t xq = 0;         // Q8_0: f16 codes [T, d]  F32: f16 hi parts [T, d]
    size_t xd = 0;         // Q8_0: f32 [T, d/32]  F32: f16 lo parts [T, d]
    size_t xp = 0;         //                      F32: f32 powers of two [d/32]
    size_t h = 0;          // Q8_0: f16 codes [R, I]  F32: f16 hi parts [R, I];  R = T*k + T*shared
    size_t hd = 0;         // Q8_0: f32 [R, I/32]  F32: f16 lo parts [R, I]
    size_t hp = 0;         //                      F32: f32 powers of two [R, I/32]
    size_t y = 0;          // f32  [R, d]
    size_t xn = 0;         // f32  [T, d]  RMSNorm(x) for the block entry point, T > 16 only
    size_t sgl = 0;        // f32  [S, T]  shared-expert gate logits per d slice (with a shared expert)
    size_t dhist = 0;      // i32  [chunks, E]  multi-block dispatch histograms (T*k > kDispatchWaveMax)
    size_t dbad = 0;       // i32  [chunks]
    size_t rparts = 0;     // the matrix-core router's operands (router_parts_bytes), T > 16 only
    size_t total = 0;
    int max_tiles = 0;
};

constexpr int kTileRows = 128;        // rows (tokens) per prefill matrix-core tile
// Cache policy of a buffer load (its last argument) for data read once per
// call, such as the decode path's weight codes and scales: non-temporal. On a
// 2 GiB stream of 16-byte buffer loads this policy read at ~7.0 TB/s against
// ~6.1 TB/s for the default one.
constexpr int kStreamed = 2;
constexpr int kDispatchWaveMax = 2048;   // assignments a single-wave dispatch takes
constexpr int kDispatchChunk = 1024;     // assignments per block of the multi-block dispatch
inline int dispatch_chunk_count(int64_t n) { return (int)((n + kDispatchChunk - 1) / kDispatchChunk); }

// Router logits: 0 = the small-T kernels; S >= 1 = d cut into S slices, enough
// for ~1024 tiles of 128 tokens x 64 experts (the kernel's tiles are 128
// experts wide where E > 64, so Qwen prefill runs 512 blocks of eight waves,
// one round of two blocks per CU). Measured there, route stage (prep, logits,
// top-k): targets of 512 / 1024 / 2048 tiles gave 67.6 / 69.0 / 80.7 us; the
// 2% at 512 is within the run-to-run spread.
inline int router_splits(int T, int E, int d) {
    if (T <= 16) return 0;
    const int tiles = ((T + 127) / 128) * ((E + 63) / 64);
    int s = (1024 + tiles - 1) / tiles;
    const int smax = d / 128 > 0 ? d / 128 : 1;
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}
// d-slice length: a multiple of 64 (the last slice takes what is left)
inline int router_kslice(int d, int S) { return ((d + S - 1) / S + 63) / 64 * 64; }

// Router logits leave as S partial sums over slices of d ([S, T, E]; the
// shared-expert gate logit as [S, T]); the top-k and the combine add them in
// slice order. T > 16: the matrix-core kernel's router_splits slices;
// T <= kSmallSplitMinT, or T <= 16 with the RMSNorm fused in: one slice (one
// block per router row reads whole rows; the norm needs them); other T <= 16:
// at most kSmallSlicesMax slices of router_small_units units of kSmallUnit
// values each (split over d, so that no block reads all of X).
constexpr int kSmallUnit = 256;
constexpr int kSmallSlicesMax = 8;
constexpr int kSmallSplitMinT = 4;
inline int router_small_units(int d) {
    const int u = (d + kSmallUnit - 1) / kSmallUnit;
    return (u + kSmallSlicesMax - 1) / kSmallSlicesMax;
}
inline int router_slices(int T, int E, int d, bool norm) {
    if (router_splits(T, E, d) > 0) return router_splits(T, E, d);
    if (norm || T <= kSmallSplitMinT) return 1;
    const int u = (d + kSmallUnit - 1) / kSmallUnit, pu = router_small_units(d);
    return (u + pu - 1) / pu;
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Operands of the matrix-core router (router_splits(T, E, d) > 0): every row
// of X [T, d] and of the gate matrix [E, d] as f16 hi + lo parts of x / p,
// with one power of two p per row (kept beside them), rows padded with zeros
// to dp = d rounded up to 32.
struct RouterParts {
    _Float16* xh = nullptr;   // [T, dp]
    _Float16* xl = nullptr;
    _Float16* wh = nullptr;   // [E, dp]
    _Float16* wl = nullptr;
    float* xp = nullptr;      // [T]
    float* wp = nullptr;      // [E]
    int dp = 0;
};
inline int router_row_pad(int d) { return (d + 31) / 32 * 32; }
inline size_t router_parts_bytes(int T, int E, int d) {
    if (router_splits(T, E, d) == 0) return 0;
    const size_t dp = (size_t)router_row_pad(d);
    return 2 * align256((size_t)T * dp * 2) + 2 * align256((size_t)E * dp * 2) + align256((size_t)T * 4) +
           align256((size_t)E * 4);
}
// the parts laid out from base (256-byte aligned), in router_parts_bytes bytes
inline RouterParts router_parts_at(void* base, int T, int E, int d) {
    RouterParts r;
    r.dp = router_row_pad(d);
    char* b = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) { char* q = b + off; off += align256(bytes); return q; };
    r.xh = reinterpret_cast<_Float16*>(take((size_t)T * r.dp * 2));
    r.xl = reinterpret_cast<_Float16*>(take((size_t)T * r.dp * 2));
    r.wh = reinterpret_cast<_Float16*>(take((size_t)E * r.dp * 2));
    r.wl = reinterpret_cast<_Float16*>(take((size_t)E * r.dp * 2));
    r.xp = reinterpret_cast<float*>(take((size_t)T * 4));
    r.wp = reinterpret_cast<float*>(take((size_t)E * 4));
    return r;
}

inline WsLayout ws_layout(int T, int k, int E, int d, int I, int act_mode, int has_shared) {
    WsLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + (bytes ? bytes : 1)); return o; };
    const size_t n = (size_t)T * k;
    const size_t R = n + (has_shared ? (size_t)T : 0);
    // full and partial tiles, plus up to 7 empty ones that even the full
    // tiles out over the 8 XCDs
    L.max_tiles = (int)((n + kTileRows - 1) / kTileRows + (size_t)(E < (long long)n ? E : n) +
                        (has_shared ? (T + kTileRows - 1) / kTileRows : 0)) + (n > 0 ? 7 : 0);
    const int S = router_splits(T, E, d);
    const int SL = router_slices(T, E, d, false);   // the most slices any path writes
    L.logits = take((size_t)SL * T * E * 4);
    L.idx = take(n * 4);
    L.wts = take(n * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.perm = take(n * 4);
    L.inv_perm = take(n * 4);
    L.row_token = take(R * 4);
    L.slots = take((size_t)(E + 1) * 16);
    L.tiles = take((size_t)(L.max_tiles > 0 ? L.max_tiles : 1) * 16);
    L.meta = take(16);
    if (act_mode == MOE_ACT_Q8_0) {
        L.xq = take((size_t)T * d * 2);
        L.xd = take((size_t)T * (d / kGroup) * 4);
        L.h = take(R * I * 2);
        L.hd = take(R * (I / kGroup) * 4);
    } else {
        L.xq = take((size_t)T * d * 2);
        L.xd = take((size_t)T * d * 2);
        L.xp = take((size_t)(d / kGroup) * 4);
        L.h = take(R * I * 2);
        L.hd = take(R * I * 2);
        L.hp = take(R * (I / kGroup) * 4);
    }
    L.y = take(R * d * 4);
    if (S > 0) L.xn = take((size_t)T * d * 4);
    if (has_shared) L.sgl = take((size_t)SL * T * 4);
    if (S > 0) L.rparts = take(router_parts_bytes(T, E, d));
    if (n > (size_t)kDispatchWaveMax) {
        L.dhist = take((size_t)dispatch_chunk_count((int64_t)n) * E * 4);
        L.dbad = take((size_t)dispatch_chunk_count((int64_t)n) * 4);
    }
    L.total = off;
    return L;
}

// ---------------------------------------------------------------------------
// Weight layout in HBM. A matrix of N rows (outputs) and K columns (reduction
// axis), N % 32 == 0 and K % 64 == 0, is cut into NT = N/32 tiles of 32
// rows; G = K / 32 groups, P = G / 2 group pairs. Inside a tile the data is
// ordered by lane of a 64-lane wave: lane l = nl + 16 h (nl < 16, h < 4)
// holds, for one group, the 8 codes k = 8h .. 8h+7 of rows nl and 16 + nl --
// exactly its part of the B operands of two 16x16x32 matrix-core products
// (rows 0-15, 16-31).
//   int8 codes:  1 KB blocks, block (group g, tile t) at (g*NT + t) KB; lane
//                l's 16 bytes at l*16: [row nl: 8 codes][row 16+nl: 8 codes]
//   int4 codes:  1 KB blocks, block (pair p, tile t) at (p*NT + t) KB; lane
//                l's 16 bytes at l*16, four dwords of 8 nibbles (low nibble =
//                lower k): [row nl, g0][row 16+nl, g0][row nl, g1][row 16+nl, g1]
//   int2 codes:  1 KB blocks, block (quad q of groups 4q .. 4q+3, tile t) at
//                (q*NT + t) KB; lane l's 16 bytes at l*16, one dword per group
//                of the quad, each two 16-bit words of 8 two-bit codes (low
//                bits = lower k): [row nl][row 16+nl]
//   scales fp32: 64-float blocks, block (tile t, pair p) at (t*P + p)*64;
//                lane quad nl at nl*4:
//                [row nl, g0][row 16+nl, g0][row nl, g1][row 16+nl, g1]
// (g0 = 2p, g1 = 2p + 1.) Codes are group- (pair-) major, so the waves
// streaming the tiles of one matrix side by side read neighbouring
// kilobytes; scales are tile-major, so one 16-byte load per lane brings a
// wave the scales of four consecutive pairs. A stack of matrices of the same
// shape is stored matrix after matrix.
// ---------------------------------------------------------------------------
constexpr int kTile = 32;

// Weight formats: the code layout (int8, packed int4 or packed int2, all
// described above) and where the scales live (per group as above, or per row:
// one float per matrix row, in row order).
__host__ __device__ constexpr bool fmt_per_row(int fmt) {
    return fmt == MOE_W_INT8_ROW || fmt == MOE_W_INT4_ROW || fmt == MOE_W_INT2_ROW;
}
// the group-scale format with the same codes (what the kernels' code paths
// are keyed on)
__host__ __device__ constexpr int fmt_codes(int fmt) {
    return fmt == MOE_W_INT8_ROW ? MOE_W_INT8_G32 : fmt == MOE_W_INT4_ROW ? MOE_W_INT4_G32
                                                  : fmt == MOE_W_INT2_ROW ? MOE_W_INT2_G32 : fmt;
}
__host__ __device__ constexpr int fmt_bits(int fmt) {
    return fmt_codes(fmt) == MOE_W_INT8_G32 ? 8 : fmt_codes(fmt) == MOE_W_INT4_G32 ? 4 : 2;
}
inline bool fmt_valid(int fmt) { return fmt >= MOE_W_INT8_G32 && fmt <= MOE_W_INT2_ROW; }
// the reduction length K must be a multiple of this (whole code blocks)
inline int fmt_k_multiple(int fmt) { return fmt_bits(fmt) == 2 ? 4 * kGroup : 2 * kGroup; }
// bytes of codes and floats of scales of one N x K matrix
inline int64_t fmt_code_bytes(int fmt, int64_t N, int64_t K) { return N * K * fmt_bits(fmt) / 8; }
inline int64_t fmt_scale_floats(int fmt, int64_t N, int64_t K) { return fmt_per_row(fmt) ? N : N * (K / kGroup); }

// byte offset, inside one matrix of NT tiles, of the 8 int8 codes (row,
// k = 8*k8 .. +7)
__host__ __device__ __forceinline__ size_t int8_code_offset(size_t row, size_t k8, size_t NT) {
    const size_t g = k8 >> 2, h = k8 & 3, r = row % kTile;
    return (g * NT + row / kTile) * 1024 + ((r & 15) + 16 * h) * 16 + (r >> 4) * 8;
}

// byte offset, inside one matrix of NT tiles, of the dword holding the 8 int4
// codes (row, k = 8*k8 .. +7)
__host__ __device__ __forceinline__ size_t int4_code_offset(size_t row, size_t k8, size_t NT) {
    const size_t g = k8 >> 2, h = k8 & 3, r = row % kTile;
    return ((g >> 1) * NT + row / kTile) * 1024 + ((r & 15) + 16 * h) * 16 + ((g & 1) * 2 + (r >> 4)) * 4;
}

// byte offset, inside one matrix of NT tiles, of the 16-bit word holding the
// 8 int2 codes (row, k = 8*k8 .. +7)
__host__ __device__ __forceinline__ size_t int2_code_offset(size_t row, size_t k8, size_t NT) {
    const size_t g = k8 >> 2, h = k8 & 3, r = row % kTile;
    return ((g >> 2) * NT + row / kTile) * 1024 + ((r & 15) + 16 * h) * 16 + (g & 3) * 4 + (r >> 4) * 2;
}

// float index, inside one matrix, of the scale of (row, group g)
__host__ __device__ __forceinline__ size_t scale_index(size_t row, size_t g, size_t G) {
    const size_t r = row % kTile;
    return ((row / kTile) * (G / 2) + (g >> 1)) * 64 + (r & 15) * 4 + (g & 1) * 2 + (r >> 4);
}

// ---------------------------------------------------------------------------
// Activations of the f32 path on the f16 matrix cores. Per group of 32 along
// the reduction axis, a power of two p = 2^(e-15) with max|x| < 2^e over the
// values that share it (X: the whole batch; H: one row), and x/p split
// exactly into two f16 parts
// (hi = f16(x/p), lo = f16(x/p - hi)). Inside each 8-wide slice the parts are
// stored in the order in which the weight-code conversion produces its
// operand slots (int8: bytes (0,2),(1,3) of a dword; int4: nibbles (0,4),
// (1,5), (2,6), (3,7); int2: k order).
// ---------------------------------------------------------------------------
// k offset (0..7) inside an 8-wide slice for operand slot j
__host__ __device__ constexpr int slot_k(int fmt, int j) {
    return fmt == MOE_W_INT8_G32   ? ((j & 4) | ((j & 1) << 1) | ((j >> 1) & 1))
           : fmt == MOE_W_INT4_G32 ? (((j & 1) << 2) | (j >> 1))
                                   : j;
}

// operand slot holding k offset kin (0..7) of an 8-wide slice
__host__ __device__ constexpr int k_slot(int fmt, int kin) {
    return fmt == MOE_W_INT8_G32   ? ((kin & 4) | ((kin & 2) >> 1) | ((kin & 1) << 1))
           : fmt == MOE_W_INT4_G32 ? (((kin & 3) << 1) | (kin >> 2))
                                   : kin;
}

// exponent e with |x| < 2^e for x = amax (0 -> 0), clamped so 2^(15-e) stays finite
__device__ __forceinline__ int pow2_exponent(float amax) {
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);
    return min(max(ex, -100), 120);
}

// Launch on `st`; with events, they are attached to the dispatch itself, so
// their interval is the kernel's own execution (no separate marker packets).
template <typename K, typename... Args>
inline void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1,
                         Args... args) {
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev0, ev1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// SiLU with the hardware reciprocal (about 1 ulp) in place of a rounded
// division; large negative g gives exp -> inf, reciprocal 0, result -0.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
