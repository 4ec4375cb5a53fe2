// Weight codes to f16 matrix-core operands, shared by the decode GEMV and the
// prefill grouped GEMM.
//
// Every int8 code (|q| <= 127) and int4 code (|q| <= 7) is an exact f16
// number, and so is the product of two codes; a 16x16x32 f16 matrix-core
// product with fp32 accumulation therefore sums 32 such products exactly as
// long as the partial sums stay below 2^24 (a 32-group of int8 x int8 codes
// stays below 32 * 127 * 127 = 516,128).
//
// Codes to f16 without a conversion instruction: an unsigned byte u ORed
// into 0x6400 is the f16 number 1024 + u, and a packed f16 subtract of 1152
// (int8 after XOR 0x80) leaves the signed code. An int4 nibble u (after XOR
// 0x8) in bits 0-3 of a half gives 1024 + u, less 1032; in bits 4-7 it gives
// 1024 + 16 u, and a packed fused multiply-add by 1/16 less 72 leaves the
// code (every step exact). That pairs bytes (0,2),(1,3) of an int8 dword and
// nibbles (0,4),(1,5),(2,6),(3,7) of an int4 dword, so the eight operand
// slots of a lane hold the k offsets slot_k(fmt, 0..7) of its 8-wide slice
// (common.h); the other operand is stored in the same order.
//
// An int2 code (|q| <= 1) is a 2-bit field u (after XOR 0b10, u = q + 2). The
// 16-bit word of a lane's 8 codes is copied into both halves of a dword; a
// mask then leaves one field in each half at bit 0, 2, 4 or 6, giving
// 1024 + u * 2^b, and a packed fused multiply-add by 2^-b less (1024 / 2^b +
// 2) leaves q. Eight codes take four such pairs, in k order.
#pragma once

#include "common.h"

namespace moe {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// (a & m) | o in one v_bitop3_b32 (truth table 0xEA)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    return __builtin_amdgcn_bitop3_b32(a, m, o, 0xEA);
}

// 8 codes of one lane slice -> 8 f16 in slot order (int8: two dwords w0, w1;
// int4: one dword w0 of 8 nibbles, w1 unused)
template <int FMT>
__device__ __forceinline__ v8h codes_to_f16(uint32_t w0, uint32_t w1) {
    union {
        uint32_t u[4];
        v8h h;
    } r;
    if constexpr (FMT == MOE_W_INT8_G32) {
        // byte pick: (code byte 0 or 1, 0x64) and (code byte 2 or 3, 0x64)
        const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
        r.u[0] = __builtin_amdgcn_perm(a, 0x64646464u, 0x00060004u);
        r.u[1] = __builtin_amdgcn_perm(a, 0x64646464u, 0x00070005u);
        r.u[2] = __builtin_amdgcn_perm(b, 0x64646464u, 0x00060004u);
        r.u[3] = __builtin_amdgcn_perm(b, 0x64646464u, 0x00070005u);
        const v2h off = v2h{(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) r.u[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, r.u[i]) + off);
        return r.h;
    } else {
        // nibbles (0,4) and (2,6) land on bits 0-3 of each half: 1024 + u;
        // nibbles (1,5) and (3,7) on bits 4-7: 1024 + 16 u, scaled by 1/16
        // in the same fused multiply-add (both exact)
        const uint32_t a = w0 ^ 0x88888888u, b = a >> 8;
        r.u[0] = and_or(a, 0x000f000fu, 0x64006400u);
        r.u[1] = and_or(a, 0x00f000f0u, 0x64006400u);
        r.u[2] = and_or(b, 0x000f000fu, 0x64006400u);
        r.u[3] = and_or(b, 0x00f000f0u, 0x64006400u);
        const v2h off = v2h{(_Float16)-1032.0f, (_Float16)-1032.0f};
        const v2h sixteenth = v2h{(_Float16)0.0625f, (_Float16)0.0625f};
        const v2h off16 = v2h{(_Float16)-72.0f, (_Float16)-72.0f};
        r.u[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, r.u[0]) + off);
        r.u[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(v2h, r.u[1]), sixteenth, off16));
        r.u[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, r.u[2]) + off);
        r.u[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(v2h, r.u[3]), sixteenth, off16));
        (void)w1;
        return r.h;
    }
}

// 8 int2 codes (one 16-bit word of dword w: rows nl (HALF 0) or 16 + nl
// (HALF 1)) -> 8 f16 in k order
template <int HALF>
__device__ __forceinline__ v8h int2_codes_to_f16(uint32_t w) {
    union {
        uint32_t u[4];
        v8h h;
    } r;
    const uint32_t a = w ^ 0xAAAAAAAAu;
    // the word in both halves: k0..k7 at bits 0..15 and 16..31
    const uint32_t y = __builtin_amdgcn_perm(a, a, HALF ? 0x03020302u : 0x01000100u);
    // k4..k7 at bits 0..7 of the low half and of the high half
    const uint32_t z = y >> 8;
    r.u[0] = and_or(y, 0x000C0003u, 0x64006400u);   // k0 at bit 0, k1 at bit 2 (of its half)
    r.u[1] = and_or(y, 0x00C00030u, 0x64006400u);   // k2 at bit 4, k3 at bit 6
    r.u[2] = and_or(z, 0x000C0003u, 0x64006400u);   // k4, k5
    r.u[3] = and_or(z, 0x00C00030u, 0x64006400u);   // k6, k7
    const v2h m01 = v2h{(_Float16)1.0f, (_Float16)0.25f}, o01 = v2h{(_Float16)-1026.0f, (_Float16)-258.0f};
    const v2h m23 = v2h{(_Float16)0.0625f, (_Float16)0.015625f}, o23 = v2h{(_Float16)-66.0f, (_Float16)-18.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.u[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(v2h, r.u[i]),
                                                                        (i & 1) ? m23 : m01, (i & 1) ? o23 : o01));
    return r.h;
}

}  // namespace moe
