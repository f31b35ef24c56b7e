// E4M3 (OCP 8-bit floating point, "fn" variant) conversions shared by the kernels that
// read or write an E4M3 KV pool.  Device code only; internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace unipin {

typedef uint32_t e4m3_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t e4m3_u32x4 __attribute__((ext_vector_type(4)));

// E4M3 code (OCP "fn" format: bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN)
// of the bf16 value with bits b: magnitudes from 448 up (infinity included) saturate to
// 448, the rest round to the nearest E4M3 value with ties to the even mantissa; NaN
// stays NaN.  Integer arithmetic on the bf16 fields, so no rounding mode is involved.
__device__ __forceinline__ uint32_t e4m3_from_bf16(uint32_t b) {
    const uint32_t s = (b >> 8) & 0x80u;
    const uint32_t a = b & 0x7fffu;
    if (a > 0x7f80u) return s | 0x7fu;            // NaN
    if (a >= 0x43e0u) return s | 0x7eu;           // |x| >= 448 = 1.75 * 2^8
    const int e = (int)(a >> 7) - 127;            // unbiased exponent
    const uint32_t m = a & 0x7fu;                 // 7 mantissa bits
    if (e >= -6) {
        // normal: biased exponent and the top 3 mantissa bits; a carry out of the
        // mantissa moves into the exponent, which is the correct rounding
        const uint32_t q = ((uint32_t)(e + 7) << 3) | (m >> 4), rem = m & 0xfu;
        return s | (q + ((rem > 8u || (rem == 8u && (q & 1u))) ? 1u : 0u));
    }
    // subnormal: the number of 2^-9 steps, (128 + m) * 2^(e + 2); below 2^-10 it is 0
    const int sh = -e - 2;                        // >= 5
    if (sh > 8) return s;
    const uint32_t full = 128u + m, q = full >> sh, rem = full & ((1u << sh) - 1u), half = 1u << (sh - 1);
    return s | (q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u));
}

// 8 bf16 values (16 bytes) -> their 8 E4M3 codes (8 bytes, element order kept).
__device__ __forceinline__ e4m3_u32x2 e4m3x8_from_bf16x8(const e4m3_u32x4 &x) {
    e4m3_u32x2 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t lo = x[2 * i], hi = x[2 * i + 1];
        r[i] = e4m3_from_bf16(lo & 0xffffu) | (e4m3_from_bf16(lo >> 16) << 8) | (e4m3_from_bf16(hi & 0xffffu) << 16) |
               (e4m3_from_bf16(hi >> 16) << 24);
    }
    return r;
}

// 16 bf16 values (32 bytes) -> their 16 E4M3 codes (16 bytes).
__device__ __forceinline__ e4m3_u32x4 e4m3x16_from_bf16x16(const e4m3_u32x4 &lo, const e4m3_u32x4 &hi) {
    const e4m3_u32x2 a = e4m3x8_from_bf16x8(lo), b = e4m3x8_from_bf16x8(hi);
    return e4m3_u32x4{a[0], a[1], b[0], b[1]};
}

// The four E4M3 codes of a 32-bit word (byte 0 first) as floats; every E4M3 value is
// exact in fp32.  The gfx950 conversion instruction reads the OCP E4M3 format.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float (&f)[4]) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

}  // namespace unipin
