// Reference kernels for pricing the layer's kernels against what the chip
// reaches in practice (include/moe_calib.h), next to the vendor peaks: a
// plain streaming read of HBM, and the prefill GEMM's own stage computation
// (q8_stage.h) run on operands that stay in LDS, with no global memory and no
// barriers, which bounds what the GEMM's instruction mix can reach.
#include "common.h"
#include "kernels.h"
#include "moe_calib.h"
#include "q8_stage.h"

namespace moe {

// Every thread reads 16-byte words at a grid-wide stride, kUnroll of them in
// flight, through a buffer resource whose reads past the end return zeros
// (so the tail needs no branch), with the non-temporal cache policy the
// decode kernels use for their weight codes. The XOR of all words goes to
// one word per block, so no load can be dropped.
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
constexpr uint64_t kStreamWindow = (uint64_t)1 << 30;   // bytes per buffer resource (32-bit offsets)
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint8_t* __restrict__ buf, uint64_t bytes,
                                                                      uint32_t* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kStreamThreads * 16;
    const uint64_t step = stride * kStreamUnroll;
    uint32_t acc = 0;
    for (uint64_t base = 0; base < bytes; base += kStreamWindow) {
        // one resource per 1 GiB window; an offset past the window reads zeros
        const uint64_t win = bytes - base < kStreamWindow ? bytes - base : kStreamWindow;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)(buf + base), 0, (int)win, 0x00020000);
        for (uint64_t o = ((uint64_t)blockIdx.x * kStreamThreads + threadIdx.x) * 16; o < win; o += step) {
            v4u_t v[kStreamUnroll];
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u) {
                const uint64_t off = o + u * stride;
                const uint32_t voff = off < win ? (uint32_t)off : 0x80000000u;
                v[u] = __builtin_bit_cast(v4u_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kStreamed));
            }
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
    }
    // one word per block: the lanes' XOR through the wave, then wave 0's
    __shared__ uint32_t red[kStreamThreads / kWave];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) s ^= red[w];
        sink[blockIdx.x] = s;
    }
}

// The prefill GEMM's stage (int4 weight codes, group scales, all eight
// 16-token tiles live) over and over on one stage of operands resident in
// LDS: the instruction mix of its inner loop alone. Two stage buffers are
// allocated and alternated, as in the GEMM, so the occupancy is the same
// (two blocks of eight waves per CU). Operands: token codes 1, weight codes
// 1, activation scales 1, weight scales 2^-20 (the sums stay finite).
constexpr int kMixLive = 8;
constexpr int kMixThreads = 64 * kGemmWaves;
__global__ __launch_bounds__(kMixThreads) void prefill_mix_kernel(int stages, float* __restrict__ sink) {
    constexpr int FMT = MOE_W_INT4_G32;
    constexpr int kW = lds_w_bytes<FMT>();
    constexpr int kStage = lds_gemm_buffer_bytes<FMT>();
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int b = 0; b < 2; ++b) {
        uint32_t* w = reinterpret_cast<uint32_t*>(b ? lds1 : lds0);
        for (int i = tid; i < kLdsTok / 4; i += kMixThreads) w[i] = 0x3C003C00u;             // f16 1.0, 1.0
        for (int i = tid; i < kW / 4; i += kMixThreads) w[kLdsTok / 4 + i] = 0x11111111u;     // int4 codes 1
        float* f = reinterpret_cast<float*>(b ? lds1 : lds0) + (kLdsTok + kW) / 4;
        for (int i = tid; i < kLdsSX / 4; i += kMixThreads) f[i] = 1.0f;
        for (int i = tid; i < kLdsSW / 4; i += kMixThreads) f[kLdsSX / 4 + i] = 0x1p-20f;
    }
    __syncthreads();
    auto opaque = [](int v) __attribute__((always_inline)) {
        asm volatile("" : "+v"(v));
        return v;
    };
    const int nl = lane & 15, rq = lane >> 4;
    const StageOffsets o{opaque(lane * 16), opaque(kLdsTok + lds_w_wave<FMT>(wave) + lane * 16),
                         opaque(kLdsTok + kW + nl * 4), opaque(kLdsTok + kW + kLdsSX + wave * 256 + rq * 64)};
    v4f acc[kMixLive][2];
#pragma unroll
    for (int i = 0; i < kMixLive; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) acc[i][hh] = v4f{0.f, 0.f, 0.f, 0.f};
    auto none = [](int, int, const v4f&) __attribute__((always_inline)) {};
    for (int st = 0; st < stages; st += 2) {
        q8_stage<FMT, false, kMixLive>((const lds_byte*)lds0, o, acc, none);
        q8_stage<FMT, false, kMixLive>((const lds_byte*)lds1, o, acc, none);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < kMixLive; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sum += acc[i][hh][0] + acc[i][hh][1] + acc[i][hh][2] + acc[i][hh][3];
    sink[(size_t)blockIdx.x * kMixThreads + tid] = sum;
}

}  // namespace moe

extern "C" moe_status moe_calib_prefill_mix(int32_t blocks, int32_t stages, float* sink, uint64_t* ops,
                                            hipStream_t stream) {
    if (sink == nullptr || blocks < 1 || stages < 2 || (stages & 1)) return MOE_ERR_INVALID_ARG;
    if (ops) *ops = (uint64_t)blocks * stages * moe::kGemmWaves * (2 * moe::kMixLive * 2) /* products */ * 16384;
    hipLaunchKernelGGL(moe::prefill_mix_kernel, dim3(blocks), dim3(moe::kMixThreads), 0, stream, stages, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status moe_calib_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks,
                                            hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || blocks < 1 || bytes == 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::stream_read_kernel, dim3(blocks), dim3(moe::kStreamThreads), 0, stream,
                       static_cast<const uint8_t*>(buf), bytes, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
