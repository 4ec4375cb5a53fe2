// Dispatch for batch-union MoE ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
// implemented": a prefill or verification batch loads every expert it selects
// one time, for all of the positions that chose it).
//
// All of it runs in one block, in LDS, with no atomics and no host round
// trip. Small batches (up to kWaveDispatchMax assignments, the decode case)
// take a single wave and never touch a block barrier:
//   1. it walks the flat assignments f = t*k + j 64 at a time; lanes with the
//      same expert find each other with one ballot per bit of the expert id,
//      which ranks every assignment among equal experts of the pass, and a
//      running count per expert in LDS carries the rank across passes;
//   2. each lane scans a run of experts and the runs are scanned across the
//      wave into counts, offsets, slot and tile positions;
//   3. position = offset + rank, so the permutation is stable by construction.
// Large batches rank over many blocks of kRankChunk assignments each (a
// histogram per chunk), one block scans the chunk histograms per expert and
// then over experts, and many blocks place every assignment; without the
// chunk scratch (moe_dispatch called with no workspace) the same steps run
// in one 1024-thread block, a histogram row per wave.
// Both then write the work lists the expert kernels consume: slots (one per
// expert with rows, then the shared expert), prefill tiles of kTileRows rows,
// and the row -> token map.
//
// For small batches the router's top-k runs in the same block first (one wave
// per token), so the routing reaches the dispatch through LDS.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / kWave;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or_zero(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Wave-wide inclusive scan of one value per lane (all 64 lanes active).
// Inside each row of 16 lanes, shifted copies (row_shr 1, 2, 4, 8; zeros
// shift in) are added; then the last lane of row 0 (row 2) is broadcast to
// row 1 (row 3) and the last lane of row 1 to rows 2 and 3 (row_bcast 15 and
// 31, the other rows adding zero).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    int x = v;
    x += dpp_or_zero<0x111, 0xF>(x);   // row_shr:1
    x += dpp_or_zero<0x112, 0xF>(x);   // row_shr:2
    x += dpp_or_zero<0x114, 0xF>(x);   // row_shr:4
    x += dpp_or_zero<0x118, 0xF>(x);   // row_shr:8
    x += dpp_or_zero<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Wave-wide exclusive scan (all 64 lanes active); *total gets the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int* total) {
    const int x = wave_inclusive_scan(v);
    *total = __builtin_amdgcn_readlane(x, kWave - 1);
    return x - v;
}

// Exclusive scan of one value per thread over the whole block (every thread
// of the kDispThreads present). `tmp` holds at least kDispWaves + 1 ints.
// Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) tmp[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        // the wave totals, scanned by wave 0 (one lane each)
        static_assert(kDispWaves <= kWave, "one lane per wave total");
        const int t = lane < kDispWaves ? tmp[lane] : 0;
        const int ti = wave_inclusive_scan(t);
        if (lane < kDispWaves) tmp[lane] = ti - t;
        if (lane == kDispWaves - 1) tmp[kDispWaves] = ti;
    }
    __syncthreads();
    const int res = tmp[wave] + incl - v;
    *total = tmp[kDispWaves];
    __syncthreads();
    return res;
}

// N exclusive scans at once, one value each per thread over the whole block
// (every thread of the kDispThreads present), for the barriers of one scan.
// tmp: N * (kDispWaves + 1) ints. ex[q] gets the exclusive prefix of v[q],
// total[q] the sum.
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(const int (&v)[N], int* tmp, int (&ex)[N], int (&total)[N]) {
    constexpr int W = kDispWaves + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl[N];
#pragma unroll
    for (int q = 0; q < N; ++q) {
        incl[q] = wave_inclusive_scan(v[q]);
        if (lane == kWave - 1) tmp[q * W + wave] = incl[q];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < N; ++q) {
            const int t = lane < kDispWaves ? tmp[q * W + lane] : 0;
            const int ti = wave_inclusive_scan(t);
            if (lane < kDispWaves) tmp[q * W + lane] = ti - t;
            if (lane == kDispWaves - 1) tmp[q * W + kDispWaves] = ti;
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < N; ++q) {
        ex[q] = tmp[q * W + wave] + incl[q] - v[q];
        total[q] = tmp[q * W + kDispWaves];
    }
    __syncthreads();
}

// Size class of a tile of r rows for the tile list's order: 0 for a full
// tile, then partial tiles by the live 16-row tiles the prefill kernel runs
// them with (8, 4, 2, 1).
__device__ __forceinline__ int tile_class(int r, int tile_rows) {
    if (r >= tile_rows) return 0;
    const int m16 = (r + 15) >> 4;
    return m16 > 4 ? 1 : m16 > 2 ? 2 : m16 > 1 ? 3 : 4;
}

// Work lists from counts/offsets (thread e < E holds counts[e], offsets[e]).
// Slots are in expert order (the shared expert last). Tiles are ordered by
// size, largest first: every full tile, then the partial tiles class by
// class (tile_class); a grid that walks the list in order then ends on its
// cheapest blocks. Each tile computes only its own rows, so the order
// changes no result.
// The prefill kernels run tile position p on XCD p % 8 (blocks are dealt to
// the XCDs in turn), and each XCD walks its positions in order. The full
// tiles (routed experts in expert order, then the shared expert's) are cut
// into 8 contiguous runs of ceil(n_full / 8) tiles, and run x takes
// positions x, x + 8, x + 16, ...: every XCD gets the same number of full
// tiles, and an expert's tiles sit on one XCD (two where a run boundary cuts
// it, more only for an expert larger than a run), one after the other, so
// its weights leave HBM for that XCD's L2 about once. The up to 7 positions
// past the last run's end hold empty tiles (no rows), which the kernels
// skip.
__device__ __forceinline__ void build_work_lists(int E, int cnt, int off, int n_rows_routed, int T, int has_shared,
                                 int tile_rows, int* __restrict__ slots, int* __restrict__ tiles,
                                 int* __restrict__ meta) {
    __shared__ int wl_tmp[6 * (kDispWaves + 1)];
    const int e = threadIdx.x;
    const bool valid = e < E;
    const int act = (valid && cnt > 0) ? 1 : 0;
    const int full = valid ? cnt / tile_rows : 0;
    const int part = valid ? cnt - full * tile_rows : 0;
    const int cls = part > 0 ? tile_class(part, tile_rows) : -1;
    // the slot, the first full tile and the place among the partial tiles of
    // its class, all in one set of scans
    const int v[6] = {act, full, cls == 1, cls == 2, cls == 3, cls == 4};
    int ex[6], tot[6];
    block_exclusive_scan_n<6>(v, wl_tmp, ex, tot);
    int n_active = tot[0];
    if (act) {
        int4* s = reinterpret_cast<int4*>(slots) + ex[0];
        *s = make_int4(e, off, cnt, 0);
    }
    int4* tl = reinterpret_cast<int4*>(tiles);
    const int n_full = tot[1], fbase = ex[1];
    const int s_full = has_shared ? T / tile_rows : 0;
    const int s_part = has_shared ? T - s_full * tile_rows : 0;
    const int s_cls = s_part > 0 ? tile_class(s_part, tile_rows) : -1;
    const int run = (n_full + s_full + 7) / 8;                    // full tiles per XCD
    auto fpos = [run](int f) { return (f % run) * 8 + f / run; };  // f-th full tile -> position
    if (full > 0) {   // then run >= 1
        // fpos(fbase + i) for i = 0, 1, ...: one division, then the quotient
        // and remainder step by one (a popular expert has tens of tiles)
        int q = fbase / run, r = fbase - (fbase / run) * run;
        for (int i = 0; i < full; ++i) {
            const int rb = off + i * tile_rows;
            tl[r * 8 + q] = make_int4(e, rb, rb + tile_rows, 0);
            if (++r == run) {
                r = 0;
                ++q;
            }
        }
    }
    for (int i = threadIdx.x; i < s_full; i += blockDim.x) {
        const int rb = n_rows_routed + i * tile_rows;
        tl[fpos(n_full + i)] = make_int4(E, rb, rb + tile_rows, 0);
    }
    for (int f = n_full + s_full + threadIdx.x; f < 8 * run; f += blockDim.x) tl[fpos(f)] = make_int4(0, 0, 0, 0);
    int pos = 8 * run;
#pragma unroll
    for (int c = 1; c <= 4; ++c) {
        if (cls == c) tl[pos + ex[1 + c]] = make_int4(e, off + full * tile_rows, off + cnt, 0);
        pos += tot[1 + c];
        if (s_cls == c) {
            if (threadIdx.x == 0)
                tl[pos] = make_int4(E, n_rows_routed + s_full * tile_rows, n_rows_routed + T, 0);
            pos += 1;
        }
    }
    if (has_shared) {
        if (threadIdx.x == 0) reinterpret_cast<int4*>(slots)[n_active] = make_int4(E, n_rows_routed, T, 0);
        n_active += 1;
    }
    if (threadIdx.x == 0) {
        meta[0] = n_active;
        meta[1] = pos;
    }
}

// The dispatch proper, by the whole block. idx: the T*k expert ids (global
// or LDS); tmp: T*k ints for the ranks between the passes (LDS, or inv_perm
// itself); hist: kDispWaves*E ints of LDS; scan_tmp: kDispWaves+1 ints of LDS.
__device__ __forceinline__ void dispatch_block(const int* idx, int* tmp, int T, int k, int E, int* __restrict__ counts,
                               int* __restrict__ offsets, int* __restrict__ perm, int* __restrict__ inv_perm,
                               int has_shared, int tile_rows, int* __restrict__ row_token, int* __restrict__ slots,
                               int* __restrict__ tiles, int* __restrict__ meta, int* hist, int* scan_tmp,
                               int* bad_flag) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = T * k;
    for (int i = tid; i < kDispWaves * E; i += kDispThreads) hist[i] = 0;
    if (tid == 0) *bad_flag = 0;
    __syncthreads();

    const int chunk = (((n + kDispWaves - 1) / kDispWaves) + kWave - 1) / kWave * kWave;
    const int begin = wave * chunk;
    const int end = min(n, begin + chunk);
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const uint64_t lt = lanemask_lt();
    int* my_hist = hist + wave * E;

    // pass 1: stable rank inside this wave's chunk; the expert ids of kPB
    // segments are fetched together so their loads overlap
    constexpr int kPB = 4;
    for (int base = begin; base < end; base += kPB * kWave) {
        int ev[kPB];
#pragma unroll
        for (int u = 0; u < kPB; ++u) {
            const int f = base + u * kWave + lane;
            ev[u] = f < end ? idx[f] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPB; ++u) {
            const int f = base + u * kWave + lane;
            const bool valid = f < end;
            const int e = ev[u];
            const bool inr = valid && e >= 0 && e < E;
            if (valid && !inr && e != -1) *bad_flag = 1;   // -1: a slot dropped by top-p
            uint64_t peers = __ballot(inr);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t m = __ballot(inr && bit);
                peers &= bit ? m : ~m;
            }
            const int rank = __popcll(peers & lt);
            const int prior = inr ? my_hist[e] : 0;
            // the last lane of each peer set advances the histogram; every lane has
            // read it above, and a wave executes its LDS operations in order
            if (inr && rank == __popcll(peers) - 1) my_hist[e] = prior + __popcll(peers);
            if (inr) tmp[f] = prior + rank;
        }
    }
    __syncthreads();

    // pass 2: scan over waves (per expert), then over experts
    int cnt = 0;
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < kDispWaves; ++w) {
            const int c = hist[w * E + tid];
            hist[w * E + tid] = run;
            run += c;
        }
        cnt = run;
    }
    int total = 0;
    const int off = block_exclusive_scan(tid < E ? cnt : 0, scan_tmp, &total);
    if (tid < E) {
        counts[tid] = cnt;
        offsets[tid] = off;
        for (int w = 0; w < kDispWaves; ++w) hist[w * E + tid] += off;
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();

    // pass 3: final positions
    for (int base = begin; base < end; base += kPB * kWave) {
        int ev[kPB], rv[kPB];
#pragma unroll
        for (int u = 0; u < kPB; ++u) {
            const int f = base + u * kWave + lane;
            ev[u] = f < end ? idx[f] : -1;
            rv[u] = (f < end && ev[u] >= 0 && ev[u] < E) ? tmp[f] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPB; ++u) {
            const int f = base + u * kWave + lane;
            const int e = ev[u];
            if (f >= end) continue;
            if (e < 0 || e >= E) {
                inv_perm[f] = -1;
                continue;
            }
            const int pos = my_hist[e] + rv[u];
            perm[pos] = f;
            inv_perm[f] = pos;
            if (row_token) row_token[pos] = f / k;
        }
    }
    for (int p = total + tid; p < n; p += kDispThreads) perm[p] = -1;
    if (row_token && has_shared)
        for (int t = tid; t < T; t += kDispThreads) row_token[n + t] = t;

    if (slots) {
        build_work_lists(E, cnt, off, n, T, has_shared, tile_rows, slots, tiles, meta);
        __syncthreads();
        if (tid == 0) meta[2] = *bad_flag;
    }
}


// The same dispatch by one wave, for small batches (the decode case): no
// block barrier anywhere, every LDS access is the wave's own and in order.
// cnt_l, off_l: E ints of LDS each; rank_l: n ints (LDS or global).
constexpr int kWaveDispatchMax = kDispatchWaveMax;   // assignments (32 passes of 64)
__device__ __forceinline__ void dispatch_wave(const int* idx, int* rank_l, int T, int k, int E,
                                              int* __restrict__ counts, int* __restrict__ offsets,
                                              int* __restrict__ perm, int* __restrict__ inv_perm, int has_shared,
                                              int tile_rows, int* __restrict__ row_token, int* __restrict__ slots,
                                              int* __restrict__ tiles, int* __restrict__ meta, int* cnt_l,
                                              int* off_l) {
    const int lane = threadIdx.x & 63;
    const int n = T * k;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const uint64_t lt = lanemask_lt();
    for (int e = lane; e < E; e += kWave) cnt_l[e] = 0;
    bool bad = false;
    // stable rank among equal experts: earlier passes through the running
    // count, earlier lanes of this pass through the ballots
    for (int base = 0; base < n; base += kWave) {
        const int f = base + lane;
        const bool valid = f < n;
        const int e = valid ? idx[f] : 0;
        const bool inr = valid && e >= 0 && e < E;
        bad |= valid && !inr && e != -1;   // -1: a slot dropped by top-p
        uint64_t peers = __ballot(inr);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(inr && bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lt);
        const int prior = inr ? cnt_l[e] : 0;
        if (inr && rank == __popcll(peers) - 1) cnt_l[e] = prior + __popcll(peers);
        if (inr) rank_l[f] = prior + rank;
    }
    // offsets: each lane scans a contiguous run of experts, the runs are
    // scanned across the wave
    const int epl = (E + kWave - 1) / kWave;
    const int e0 = min(lane * epl, E), e1 = min(e0 + epl, E);
    int run = 0, act = 0, ntl = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt_l[e];
        run += c;
        act += c > 0;
        ntl += (c + tile_rows - 1) / tile_rows;
    }
    int total = 0, n_active = 0, n_tiles = 0;
    int off = wave_exclusive_scan(run, &total);
    int slot = wave_exclusive_scan(act, &n_active);
    int tile = wave_exclusive_scan(ntl, &n_tiles);
    for (int e = e0; e < e1; ++e) {
        const int c = cnt_l[e];
        counts[e] = c;
        offsets[e] = off;
        off_l[e] = off;
        if (slots && c > 0) {
            reinterpret_cast<int4*>(slots)[slot++] = make_int4(e, off, c, 0);
            for (int rb = off; rb < off + c; rb += tile_rows)
                reinterpret_cast<int4*>(tiles)[tile++] = make_int4(e, rb, min(off + c, rb + tile_rows), 0);
        }
        off += c;
    }
    if (lane == 0) offsets[E] = total;
    // final positions; assignments not dispatched get inv_perm -1 and the
    // permutation's unused tail is -1
    for (int base = 0; base < n; base += kWave) {
        const int f = base + lane;
        if (f >= n) break;
        const int e = idx[f];
        if (e < 0 || e >= E) {
            inv_perm[f] = -1;
            continue;
        }
        const int pos = off_l[e] + rank_l[f];
        perm[pos] = f;
        inv_perm[f] = pos;
        if (row_token) row_token[pos] = f / k;
    }
    for (int p = total + lane; p < n; p += kWave) perm[p] = -1;
    if (row_token && has_shared)
        for (int t = lane; t < T; t += kWave) row_token[n + t] = t;
    if (slots) {
        if (has_shared) {
            const int shared_tiles = (T + tile_rows - 1) / tile_rows;
            for (int i = lane; i < shared_tiles; i += kWave) {
                const int rb = n + i * tile_rows;
                reinterpret_cast<int4*>(tiles)[n_tiles + i] = make_int4(E, rb, min(n + T, rb + tile_rows), 0);
            }
            if (lane == 0) reinterpret_cast<int4*>(slots)[n_active] = make_int4(E, n, T, 0);
            n_tiles += shared_tiles;
            n_active += 1;
        }
        const bool any_bad = __ballot(bad) != 0;
        if (lane == 0) {
            meta[0] = n_active;
            meta[1] = n_tiles;
            meta[2] = any_bad ? 1 : 0;
        }
    }
}

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(const int* __restrict__ idx, int T, int k, int E,
                                                                 int* __restrict__ counts, int* __restrict__ offsets,
                                                                 int* __restrict__ perm, int* __restrict__ inv_perm,
                                                                 int has_shared, int tile_rows,
                                                                 int* __restrict__ row_token,
                                                                 int* __restrict__ slots, int* __restrict__ tiles,
                                                                 int* __restrict__ meta) {
    extern __shared__ __attribute__((aligned(16))) int lds[];
    __shared__ int bad_flag;
    if (T * k <= kWaveDispatchMax) {
        // ranks between the passes go through inv_perm itself
        if (threadIdx.x < kWave)
            dispatch_wave(idx, inv_perm, T, k, E, counts, offsets, perm, inv_perm, has_shared, tile_rows, row_token,
                          slots, tiles, meta, lds, lds + E);
        return;
    }
    dispatch_block(idx, inv_perm, T, k, E, counts, offsets, perm, inv_perm, has_shared, tile_rows, row_token, slots,
                   tiles, meta, lds, lds + kDispWaves * E, &bad_flag);
}

// ---------------------------------------------------------------------------
// Multi-block dispatch for large batches. Chunk c = assignments
// [c * kRankChunk, (c + 1) * kRankChunk); each of a block's four waves ranks
// a quarter of it, 64 at a time. The three kernels run in stream order.
// ---------------------------------------------------------------------------
constexpr int kRankChunk = kDispatchChunk;
constexpr int kRankPasses = kRankChunk / (4 * kWave);   // passes of 64 per wave

int dispatch_chunks(int64_t n) { return dispatch_chunk_count(n); }

// 1. ranks: tmp[f] = rank of f among the chunk's assignments to its expert;
//    chunk_hist[c][e] = the chunk's count of expert e; chunk_bad[c] = 1 when
//    the chunk holds an id outside [0, E) other than -1.
__global__ __launch_bounds__(256) void dispatch_rank_kernel(const int* __restrict__ idx, int n, int E,
                                                            int* __restrict__ tmp, int* __restrict__ chunk_hist,
                                                            int* __restrict__ chunk_bad) {
    extern __shared__ __attribute__((aligned(16))) int hist[];   // [4][E]
    __shared__ int bad_any;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x;
    for (int i = tid; i < 4 * E; i += 256) hist[i] = 0;
    if (tid == 0) bad_any = 0;
    __syncthreads();
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const uint64_t lt = lanemask_lt();
    int* my_hist = hist + wave * E;
    const int base = c * kRankChunk + wave * (kRankPasses * kWave);
    int ev[kRankPasses], rv[kRankPasses];
#pragma unroll
    for (int u = 0; u < kRankPasses; ++u) {
        const int f = base + u * kWave + lane;
        ev[u] = f < n ? idx[f] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kRankPasses; ++u) {
        const int f = base + u * kWave + lane;
        const int e = ev[u];
        const bool inr = f < n && e >= 0 && e < E;
        bad |= f < n && !inr && e != -1;   // -1: a slot dropped by top-p
        uint64_t peers = __ballot(inr);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(inr && bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lt);
        const int prior = inr ? my_hist[e] : 0;
        // the last lane of each peer set advances the count; every lane has
        // read it above, and a wave executes its LDS operations in order
        if (inr && rank == __popcll(peers) - 1) my_hist[e] = prior + __popcll(peers);
        rv[u] = prior + rank;
        ev[u] = inr ? e : -1;
    }
    if (bad) bad_any = 1;
    __syncthreads();
    // per expert: the waves' counts become wave offsets inside the chunk
    for (int e = tid; e < E; e += 256) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int v = hist[w * E + e];
            hist[w * E + e] = run;
            run += v;
        }
        chunk_hist[(size_t)c * E + e] = run;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRankPasses; ++u) {
        const int f = base + u * kWave + lane;
        if (ev[u] >= 0) tmp[f] = my_hist[ev[u]] + rv[u];
    }
    if (tid == 0) chunk_bad[c] = bad_any;
}

// 2. one block: per expert, chunk offsets (exclusive over chunks, in place)
//    and the count; offsets over experts. Then the perm tail, the shared rows
//    of row_token and the work lists.
__global__ __launch_bounds__(kDispThreads) void dispatch_scan_kernel(int* __restrict__ chunk_hist,
                                                                     const int* __restrict__ chunk_bad, int nch,
                                                                     int T, int k, int E, int* __restrict__ counts,
                                                                     int* __restrict__ offsets,
                                                                     int* __restrict__ perm, int has_shared,
                                                                     int tile_rows, int* __restrict__ row_token,
                                                                     int* __restrict__ slots, int* __restrict__ tiles,
                                                                     int* __restrict__ meta) {
    __shared__ int scan_tmp[kDispWaves + 1];
    const int tid = threadIdx.x;
    const int n = T * k;
    // the chunks' bad-id flags, one per thread (more, rarely, after the
    // scan), so that the load overlaps the counts' loads below
    int bad = (slots && tid < nch) ? chunk_bad[tid] : 0;
    int cnt = 0;
    constexpr int kB = 32;
    if (2 * E <= kDispThreads && nch <= 2 * kB) {
        // two threads per expert, each with half of the chunks: one round of
        // loads; thread e (< E) ends with the total, thread e + 512 offsets
        // its half's prefixes by the first half's sum
        __shared__ int half_sum[2][kDispThreads / 2];
        constexpr int kHalf = kDispThreads / 2;
        const int part = tid / kHalf, e = tid - part * kHalf;
        const int nh = (nch + 1) / 2, cb = part * nh, nmine = min(nch, cb + nh) - cb;
        int v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = (e < E && u < nmine) ? chunk_hist[(size_t)(cb + u) * E + e] : 0;
        int local = 0;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int x = v[u];
            v[u] = local;
            local += x;
        }
        if (e < E) half_sum[part][e] = local;
        __syncthreads();
        const int base = (part == 1 && e < E) ? half_sum[0][e] : 0;
        if (e < E) {
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (u < nmine) chunk_hist[(size_t)(cb + u) * E + e] = base + v[u];
        }
        if (part == 0 && e < E) cnt = local + half_sum[1][e];
    } else if (tid < E) {
        // 32 chunks' loads in flight at a time
        for (int c0 = 0; c0 < nch; c0 += kB) {
            int v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = c0 + u < nch ? chunk_hist[(size_t)(c0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                if (c0 + u < nch) chunk_hist[(size_t)(c0 + u) * E + tid] = cnt;
                cnt += v[u];
            }
        }
    }
    int total = 0;
    const int off = block_exclusive_scan(tid < E ? cnt : 0, scan_tmp, &total);
    if (tid < E) {
        counts[tid] = cnt;
        offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    for (int p = total + tid; p < n; p += kDispThreads) perm[p] = -1;
    if (row_token && has_shared)
        for (int t = tid; t < T; t += kDispThreads) row_token[n + t] = t;
    if (slots) {
        build_work_lists(E, cnt, off, n, T, has_shared, tile_rows, slots, tiles, meta);
        for (int c = tid + kDispThreads; c < nch; c += kDispThreads) bad |= chunk_bad[c];
        const int any_bad = __syncthreads_or(bad);
        if (tid == 0) meta[2] = any_bad;
    }
}

// 3. positions: pos = offsets[e] + rows of e in earlier chunks + rank in the
//    chunk
__global__ __launch_bounds__(256) void dispatch_place_kernel(const int* __restrict__ idx, int n, int k, int E,
                                                             const int* __restrict__ offsets,
                                                             const int* __restrict__ chunk_hist,
                                                             int* __restrict__ perm, int* __restrict__ inv_perm,
                                                             int* __restrict__ row_token) {
    const int c = blockIdx.x;
#pragma unroll
    for (int u = 0; u < kRankChunk / 256; ++u) {
        const int f = c * kRankChunk + u * 256 + threadIdx.x;
        if (f >= n) break;
        const int e = idx[f];
        if (e < 0 || e >= E) {
            inv_perm[f] = -1;
            continue;
        }
        const int pos = offsets[e] + chunk_hist[(size_t)c * E + e] + inv_perm[f];   // inv_perm holds the rank here
        perm[pos] = f;
        inv_perm[f] = pos;
        if (row_token) row_token[pos] = f / k;
    }
}

// Top-k of T <= kDispWaves tokens (wave t takes token t), then the dispatch,
// in one block; the expert ids and ranks stay in LDS.
template <int EPL>
__global__ __launch_bounds__(kDispThreads) void route_dispatch_kernel(const TopkArgs a, int* __restrict__ idx_out,
                                                                       float* __restrict__ w_out,
                                                                       int* __restrict__ counts,
                                                                       int* __restrict__ offsets,
                                                                       int* __restrict__ perm,
                                                                       int* __restrict__ inv_perm, int has_shared,
                                                                       int tile_rows, int* __restrict__ row_token,
                                                                       int* __restrict__ slots,
                                                                       int* __restrict__ tiles,
                                                                       int* __restrict__ meta) {
    extern __shared__ __attribute__((aligned(16))) int lds[];
    __shared__ int bad_flag;
    const int T = a.T, k = a.k, E = a.E, n = T * k;
    const bool noaux = a.mode == MOE_ROUTER_SIGMOID_NOAUX_TC;
    float* keybuf = reinterpret_cast<float*>(lds);           // [kDispWaves][E], noaux_tc only
    int* idx_l = lds + (noaux ? kDispWaves * E : 0);         // [n]
    int* rank_l = idx_l + n;                                 // [n]
    int* hist = rank_l + n;                                  // [kDispWaves][E]
    int* scan_tmp = hist + kDispWaves * E;                   // [kDispWaves + 1]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool active = wave < T;
    int my_e;
    float my_w;
    topk_token<EPL>(a, wave, active, keybuf + (noaux ? wave * E : 0), &my_e, &my_w);
    if (active && lane < k) {
        idx_out[wave * k + lane] = my_e;
        w_out[wave * k + lane] = my_w;
        idx_l[wave * k + lane] = my_e;
    }
    __syncthreads();
    (void)scan_tmp;
    (void)bad_flag;
    if (wave == 0)
        dispatch_wave(idx_l, rank_l, T, k, E, counts, offsets, perm, inv_perm, has_shared, tile_rows, row_token, slots,
                      tiles, meta, hist, hist + E);
}

// Work lists for moe_expert_ffn from a caller's counts / offsets / perm.
__global__ __launch_bounds__(kDispThreads) void plan_kernel(const int* __restrict__ counts,
                                                             const int* __restrict__ offsets,
                                                             const int* __restrict__ perm, int T, int k, int E,
                                                             int has_shared, int tile_rows,
                                                             int* __restrict__ row_token, int* __restrict__ slots,
                                                             int* __restrict__ tiles, int* __restrict__ meta) {
    __shared__ int scan_tmp[kDispWaves + 1];
    const int tid = threadIdx.x;
    const int n = T * k;
    for (int p = tid; p < n; p += kDispThreads) {
        const int f = perm[p];
        row_token[p] = (f >= 0 && f < n) ? f / k : 0;
    }
    if (has_shared)
        for (int t = tid; t < T; t += kDispThreads) row_token[n + t] = t;
    // A caller's counts / offsets are clamped so that every row stays inside
    // the permuted range [0, T*k) and the counts sum to at most T*k: then
    // the tiles number at most ceil(T*k / tile_rows) + min(E, T*k) (plus the
    // shared expert's and up to 7 empty ones), the size of the tile list. Counts and offsets that
    // are not the exclusive prefix sum of each other set the status flag
    // meta[2] (the results are then unspecified, but every access stays in
    // bounds).
    const int off_in = tid < E ? offsets[tid] : 0;
    const int cnt_in = tid < E ? counts[tid] : 0;
    const int off = min(max(off_in, 0), n);
    int cnt = min(max(cnt_in, 0), n - off);
    int total = 0;
    const int before = block_exclusive_scan(cnt, scan_tmp, &total);
    cnt = min(cnt, max(n - before, 0));
    const int bad = __syncthreads_or(tid < E && (off_in != before || cnt != cnt_in));
    build_work_lists(E, cnt, off, n, T, has_shared, tile_rows, slots, tiles, meta);
    if (tid == 0) meta[2] = bad;
}

size_t dispatch_lds_bytes(int E) { return (size_t)(kDispWaves * E + kDispWaves + 1) * sizeof(int); }

size_t route_dispatch_lds_bytes(int T, int k, int E, int mode) {
    const size_t keybuf = mode == MOE_ROUTER_SIGMOID_NOAUX_TC ? (size_t)kDispWaves * E : 0;
    return (keybuf + 2 * (size_t)T * k + dispatch_lds_bytes(E) / sizeof(int)) * sizeof(int);
}

hipError_t launch_route_dispatch(const float* logits, int T, int S, const moe_router_params& p, int* idx, float* w,
                                 int* counts, int* offsets, int* perm, int* inv_perm, int has_shared,
                                 int* row_token, int* slots, int* tiles, int* meta, hipStream_t st) {
    if (T > kDispWaves) return hipErrorInvalidValue;
    const TopkArgs a = topk_args(logits, T, S, p);
    const size_t lds = route_dispatch_lds_bytes(T, p.top_k, p.n_experts, p.mode);
    const int threads = (T > 0 ? T : 1) * kWave;   // one wave per token; wave 0 then dispatches
#define MOE_RD(EPL)                                                                                              \
    hipLaunchKernelGGL(route_dispatch_kernel<EPL>, dim3(1), dim3(threads), lds, st, a, idx, w, counts, offsets,     \
                       perm, inv_perm, has_shared, kTileRows, row_token, slots, tiles, meta)
    switch (topk_epl(p.n_experts)) {
        case 1: MOE_RD(1); break;
        case 2: MOE_RD(2); break;
        case 4: MOE_RD(4); break;
        case 8: MOE_RD(8); break;
        default: MOE_RD(16); break;
    }
#undef MOE_RD
    return hipGetLastError();
}

hipError_t launch_dispatch(const int* idx, int T, int k, int E, int* counts, int* offsets, int* perm,
                           int* inv_perm, int has_shared, int* row_token, int* slots, int* tiles, int* meta,
                           int* chunk_hist, int* chunk_bad, hipStream_t st) {
    const int64_t n = (int64_t)T * k;
    if (n > kWaveDispatchMax && chunk_hist && chunk_bad) {
        const int nch = dispatch_chunks(n);
        hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nch), dim3(256), (size_t)4 * E * sizeof(int), st, idx, (int)n,
                           E, inv_perm, chunk_hist, chunk_bad);
        hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kDispThreads), 0, st, chunk_hist, chunk_bad, nch, T, k,
                           E, counts, offsets, perm, has_shared, kTileRows, row_token, slots, tiles, meta);
        hipLaunchKernelGGL(dispatch_place_kernel, dim3(nch), dim3(256), 0, st, idx, (int)n, k, E, offsets, chunk_hist,
                           perm, inv_perm, row_token);
        return hipGetLastError();
    }
    // small batches: one wave does it all (dispatch_wave)
    const int threads = n <= kWaveDispatchMax ? kWave : kDispThreads;
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(threads), dispatch_lds_bytes(E), st, idx, T, k, E, counts,
                       offsets, perm, inv_perm, has_shared, kTileRows, row_token, slots, tiles, meta);
    return hipGetLastError();
}

hipError_t launch_plan(const int* counts, const int* offsets, const int* perm, int T, int k, int E, int has_shared,
                       int* row_token, int* slots, int* tiles, int* meta, hipStream_t st) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kDispThreads), 0, st, counts, offsets, perm, T, k, E, has_shared,
                       kTileRows, row_token, slots, tiles, meta);
    return hipGetLastError();
}

}  // namespace moe
