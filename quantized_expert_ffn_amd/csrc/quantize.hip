// Quantisers: weights (int8 / packed int4 / packed int2, a scale per group of
// 32 or per row) and Q8_0 activations.
//
// Weights: "mtlm-7m-base" (huggingface.co), section "Files" (int8, group size
// 32) and "Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented" (int8 / packed
// int4 quantisation kernels, per-row scales). Activations: the same section's Q8_0-style int8
// activations. Codes are decided in fp32 with IEEE division and
// round-half-to-even, so a host implementation using the same fp32 steps
// reaches the same bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

// Codes of one group of 32 weights (row, group g of its matrix) with scale
// sc, written to their places in the lane-tiled layout (common.h).
template <int BITS>
__device__ __forceinline__ void encode_group(const float (&v)[kGroup], float sc, size_t row, size_t g, size_t NT,
                                             uint8_t* __restrict__ q) {
    constexpr float qmax = BITS == 8 ? 127.0f : BITS == 4 ? 7.0f : 1.0f;
    int code[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        float r = sc > 0.0f ? rintf(__fdiv_rn(v[i], sc)) : 0.0f;
        r = fminf(fmaxf(r, -qmax), qmax);
        code[i] = (int)r;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const size_t k8 = 4 * g + h;
        if constexpr (BITS == 8) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= (uint32_t)(code[8 * h + j] & 0xff) << (8 * j);
                hi |= (uint32_t)(code[8 * h + 4 + j] & 0xff) << (8 * j);
            }
            *reinterpret_cast<uint2*>(q + int8_code_offset(row, k8, NT)) = make_uint2(lo, hi);
        } else if constexpr (BITS == 4) {
            uint32_t p = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) p |= (uint32_t)(code[8 * h + j] & 0xf) << (4 * j);
            *reinterpret_cast<uint32_t*>(q + int4_code_offset(row, k8, NT)) = p;
        } else {
            uint32_t p = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) p |= (uint32_t)(code[8 * h + j] & 0x3) << (2 * j);
            *reinterpret_cast<uint16_t*>(q + int2_code_offset(row, k8, NT)) = (uint16_t)p;
        }
    }
}

__device__ __forceinline__ void load_group(const float* __restrict__ src, float (&v)[kGroup]) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int i = 0; i < kGroup / 4; ++i) {
        const float4 f = s4[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

// Group scales: one thread per group of 32 consecutive weights of one row;
// the codes and the scale go to their places in the lane-tiled layout of the
// row's matrix (a stack of matrices of matrix_rows rows each).
template <int BITS>
__global__ __launch_bounds__(256) void quantize_weights_kernel(const float* __restrict__ w,
                                                               int64_t n_groups, int G, int matrix_rows,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ s) {
    const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= n_groups) return;
    const size_t grow = (size_t)(gi / G), g = (size_t)(gi % G);
    const size_t mat = grow / matrix_rows, row = grow % matrix_rows, NT = matrix_rows / kTile;
    const size_t mat_elems = (size_t)matrix_rows * G * kGroup;
    q += mat * mat_elems * BITS / 8;
    s += mat * (size_t)matrix_rows * G;
    float v[kGroup];
    load_group(w + gi * kGroup, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float sc = __fdiv_rn(amax, BITS == 8 ? 127.0f : BITS == 4 ? 7.0f : 1.0f);
    s[scale_index(row, g, (size_t)G)] = sc;
    encode_group<BITS>(v, sc, row, g, NT, q);
}

// Row scales: one wave per row. The row's amax first (lane-strided float4
// reads, then a wave max), then each lane encodes groups lane, lane + 64, ...
// of the row with the row's scale.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ w, int64_t rows, int G,
                                                            int matrix_rows, uint8_t* __restrict__ q,
                                                            float* __restrict__ s) {
    const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (grow >= rows) return;
    const int lane = threadIdx.x & 63;
    const size_t cols = (size_t)G * kGroup;
    const float* src = w + (size_t)grow * cols;
    float amax = 0.0f;
    for (size_t c = 4 * (size_t)lane; c < cols; c += 4 * kWave) {
        const float4 f = *reinterpret_cast<const float4*>(src + c);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
    amax = wave_max(amax);
    const float sc = __fdiv_rn(amax, BITS == 8 ? 127.0f : BITS == 4 ? 7.0f : 1.0f);
    const size_t mat = (size_t)grow / matrix_rows, row = (size_t)grow % matrix_rows, NT = matrix_rows / kTile;
    const size_t mat_elems = (size_t)matrix_rows * cols;
    q += mat * mat_elems * BITS / 8;
    if (lane == 0) s[grow] = sc;
    for (int g = lane; g < G; g += kWave) {
        float v[kGroup];
        load_group(src + (size_t)g * kGroup, v);
        encode_group<BITS>(v, sc, row, (size_t)g, NT, q);
    }
}

// One thread per group of 32 activations of one row (fp32 steps).
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x, int64_t n_groups,
                                                            int8_t* __restrict__ q, float* __restrict__ d) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_groups) return;
    float v[kGroup];
    load_group(x + g * kGroup, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float dd = __fdiv_rn(amax, 127.0f);
    const float inv = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
    uint32_t packed[kGroup / 4];
#pragma unroll
    for (int i = 0; i < kGroup / 4; ++i) {
        uint32_t p = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = rintf(__fmul_rn(v[4 * i + j], inv));
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            p |= ((uint32_t)((int)r & 0xff)) << (8 * j);
        }
        packed[i] = p;
    }
    d[g] = dd;
    uint4* dst = reinterpret_cast<uint4*>(q + g * kGroup);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

hipError_t launch_quantize_weights(const float* w, int64_t rows, int cols, int matrix_rows, int format, void* q,
                                   float* s, hipStream_t st) {
    const int G = cols / kGroup;
    const int64_t n_groups = rows * G;
    if (n_groups == 0) return hipSuccess;
    const int bits = fmt_bits(format);
    if (fmt_per_row(format)) {
        const dim3 grid((unsigned)((rows + 3) / 4));
#define MOE_QR(B) hipLaunchKernelGGL(quantize_rows_kernel<B>, grid, dim3(256), 0, st, w, rows, G, matrix_rows, (uint8_t*)q, s)
        if (bits == 8) MOE_QR(8);
        else if (bits == 4) MOE_QR(4);
        else MOE_QR(2);
#undef MOE_QR
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n_groups + 255) / 256));
#define MOE_QW(B) \
    hipLaunchKernelGGL(quantize_weights_kernel<B>, grid, dim3(256), 0, st, w, n_groups, G, matrix_rows, (uint8_t*)q, s)
    if (bits == 8) MOE_QW(8);
    else if (bits == 4) MOE_QW(4);
    else MOE_QW(2);
#undef MOE_QW
    return hipGetLastError();
}

hipError_t launch_quantize_q8_0(const float* x, int64_t rows, int cols, int8_t* q, float* d, hipStream_t st) {
    const int64_t n_groups = rows * (cols / kGroup);
    if (n_groups == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_groups + 255) / 256));
    hipLaunchKernelGGL(quantize_q8_0_kernel, grid, dim3(256), 0, st, x, n_groups, q, d);
    return hipGetLastError();
}

}  // namespace moe
