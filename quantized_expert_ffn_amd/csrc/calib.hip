// Reference kernels for pricing the layer's kernels against what the chip
// reaches in practice (include/moe_calib.h), next to the vendor peaks: a
// plain streaming read of HBM. Nothing of the layer's arithmetic is here.
#include "common.h"
#include "kernels.h"
#include "moe_calib.h"

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

}  // namespace moe

extern "C" moe_status moe_calib_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks,
                                            hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || blocks < 1 || bytes == 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::stream_read_kernel, dim3(blocks), dim3(moe::kStreamThreads), 0, stream,
                       static_cast<const uint8_t*>(buf), bytes, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
