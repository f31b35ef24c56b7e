// E4M3 (OCP 8-bit floating point, "fn" variant) conversions shared by the kernels that
// read or write an E4M3 KV pool.  Device code only; internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace unipin {

typedef uint32_t e4m3_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t e4m3_u32x4 __attribute__((ext_vector_type(4)));

// Two bf16 values (the low and high halves of w) -> their two E4M3 codes (OCP "fn"
// format: bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN) in the low 16 bits,
// low half first.  Magnitudes from 448 up (infinity included) saturate to 448, the rest
// round to the nearest E4M3 value with ties to the even mantissa, NaN stays NaN: the
// values are clamped to +-448 before the hardware conversion (which rounds to nearest
// even), so its own overflow handling never comes into play, and a NaN skips the clamp.
__device__ __forceinline__ uint32_t e4m3x2_from_bf16x2(uint32_t w) {
    float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
    lo = __builtin_isnan(lo) ? lo : fminf(fmaxf(lo, -448.f), 448.f);
    hi = __builtin_isnan(hi) ? hi : fminf(fmaxf(hi, -448.f), 448.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false) & 0xffffu;
}

// 8 bf16 values (16 bytes) -> their 8 E4M3 codes (8 bytes, element order kept).
__device__ __forceinline__ e4m3_u32x2 e4m3x8_from_bf16x8(const e4m3_u32x4 &x) {
    e4m3_u32x2 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) r[i] = e4m3x2_from_bf16x2(x[2 * i]) | (e4m3x2_from_bf16x2(x[2 * i + 1]) << 16);
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

// The four E4M3 codes of a 32-bit word (byte 0 first) as four bf16 values in two 32-bit
// words, element order kept; exact, since every E4M3 value is a bf16 value.  One gfx950
// instruction per pair (the scaled conversion, with scale 1), which reads the OCP E4M3
// format like the fp32 one.
__device__ __forceinline__ e4m3_u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    typedef __bf16 pair_t __attribute__((ext_vector_type(2)));
    const pair_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const pair_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return e4m3_u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

}  // namespace unipin
