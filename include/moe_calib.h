/*
 * moe_calib.h - reference kernels of libmoe for roofline pricing.
 *
 * The layer's kernels are priced against the MI355X's published peaks and,
 * beside them, against what a minimal kernel reaches on the same GPU in the
 * same run. These entry points are measurement references only: they compute
 * nothing of the layer. Same conventions as moe.h (caller-owned device
 * memory, asynchronous on `stream`, no allocation).
 */
#ifndef MOE_CALIB_H
#define MOE_CALIB_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of HBM: reads every byte of buf once with 16-byte vector
 * loads (non-temporal cache policy, as the decode kernels' weight streams)
 * from `blocks` workgroups of 256 threads, and writes one 32-bit XOR of the
 * data per workgroup to sink[0 .. blocks-1] (so no read can be dropped).
 *   buf    device, 16-byte aligned; bytes a multiple of 16, > 0 (a buffer
 *          much larger than the 256 MB last-level cache measures HBM)
 *   sink   device uint32 [blocks]
 * Returns MOE_ERR_INVALID_ARG for a null pointer, an unaligned buffer, a
 * size that is zero or not a multiple of 16, or blocks < 1.
 */
moe_status moe_calib_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks,
                                 hipStream_t stream);

/* The prefill grouped GEMM's inner loop alone: each of `blocks` workgroups of
 * eight waves runs the GEMM's stage computation (int4 weight codes with group
 * scales, eight 16-token tiles, two 16-row weight halves per wave; see
 * moe.h, moe_expert_ffn with MOE_ACT_Q8_0) `stages` times over operands that
 * stay in LDS: no global memory, no barriers. Its rate bounds what that
 * instruction mix can reach. Writes one float per thread to sink
 * (device fp32 [blocks * 512]) so no work can be dropped, and, if ops is
 * not NULL, the useful int8 operations the launch performs to *ops (host):
 * 2 * 16 * 16 * 32 per matrix-core product.
 * Returns MOE_ERR_INVALID_ARG for a null sink, blocks < 1, or a stage count
 * that is not even and >= 2.
 */
moe_status moe_calib_prefill_mix(int32_t blocks, int32_t stages, float* sink, uint64_t* ops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H */
