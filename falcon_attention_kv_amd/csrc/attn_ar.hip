// One autoregressive step of the retrieval side, for gfx950: each (user, head) has one
// new query token that attends to the N rows already in its pool slot (the history and
// the tokens generated before) and to itself, and whose K/V are stored at row N.
//
// Every K/V byte is used by one query, so the step is bound by HBM bandwidth, and the
// matrix cores have nothing to do (a single query row).  One workgroup per (user, head):
// 8 waves take the slot's rows in 64-key chunks in turn (wave w: chunks w, w+8, ...).
// A wave loads a chunk's K and V rows with 16-byte lane loads, R = row bytes / 16 lanes
// per row and 64 / R rows per wave-wide load, so that every load instruction reads
// whole contiguous rows.  A lane dots its 16 bytes of a key row with the same 16 bytes
// of the query (bf16 pairs: exact products, fp32 sums) and the R lanes of a row add up
// their parts with cross-lane exchanges.  The softmax is the online form in fp32 with
// base-2 exponentials (scale*log2(e) applied to the fp32 score); the value rows are
// weighted in fp32.  At the end the waves' partial states (running max, sum and
// accumulator) are merged through LDS, the new token enters as the last key, and the
// output row is normalised and stored; the new K/V row is copied into the slot.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace unipin {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

template <typename T>
struct Elem;
template <>
struct Elem<bf16> {
    static constexpr int kPer16 = 8;   // elements per 16 bytes
};
template <>
struct Elem<float> {
    static constexpr int kPer16 = 4;
};

// The 16 bytes x as floats (exact for both element types).
template <typename T>
__device__ __forceinline__ void widen(const u32x4 &x, float (&f)[Elem<T>::kPer16]) {
    if constexpr (Elem<T>::kPer16 == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(x[i] << 16);
            f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
    }
}

// Dot product of two 16-byte pieces, fp32 sum of exact products.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4 &a, const u32x4 &b) {
    float s = 0.f;
    if constexpr (Elem<T>::kPer16 == 8) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const bf16x2 pa = {av[i], av[i + 1]}, pb = {bv[i], bv[i + 1]};
            s = __builtin_amdgcn_fdot2_f32_bf16(pa, pb, s, false);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), s);
    }
    return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Sum (or max) over the lanes whose ids differ only in the bits of [lo, 64).
template <int LO>
__device__ __forceinline__ float xsum(float x) {
#pragma unroll
    for (int m = LO; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}
template <int LO>
__device__ __forceinline__ float xmax(float x) {
#pragma unroll
    for (int m = LO; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
// Sum over the lanes whose ids differ only in the bits below HI.
template <int HI>
__device__ __forceinline__ float lowsum(float x) {
#pragma unroll
    for (int m = 1; m < HI; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads) ar_decode_kernel(AttnArgs a) {
    constexpr int ROW = D * (int)sizeof(T);    // bytes per row
    constexpr int R = ROW / 16;                // lanes per row
    constexpr int RPI = 64 / R;                // rows per wave-wide load
    constexpr int PER = Elem<T>::kPer16;       // elements per lane per load
    constexpr int LPC = RPI >= 4 ? 64 / RPI : 16;   // loads per chunk and matrix
    constexpr int CH = LPC * RPI;              // keys per chunk
    static_assert(R >= 1 && R <= 64 && 64 % R == 0, "row must split into 16-byte lanes");
    __shared__ float part[kWaves][D + 2];      // per wave: accumulator, max, sum

    const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int N = a.lens[b];
    const int s = a.slot[b];
    const bool bad_len = N < 0 || N > a.len_limit;
    const bool bad_slot = s < 0 || s >= a.S;
    if (bad_len || bad_slot) {
        if (threadIdx.x == 0 && h == 0) atomicOr(a.status, (bad_len ? kFlagBadLen : 0u) | (bad_slot ? kFlagBadSlot : 0u));
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int sub = lane % R, grp = lane / R;
    const long bh = (long)b * a.H + h;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    const T *pk = static_cast<const T *>(a.pool_k) + slot_off;
    const T *pv = static_cast<const T *>(a.pool_v) + slot_off;
    const __amdgpu_buffer_rsrc_t rk = rsrc(pk, (uint32_t)N * ROW);   // rows >= N read as zero
    const __amdgpu_buffer_rsrc_t rv = rsrc(pv, (uint32_t)N * ROW);
    const u32x4 qx = load16(rsrc(static_cast<const T *>(a.q) + bh * D, ROW), sub * 16);

    float m = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;

    for (int c0 = wave * CH; c0 < N; c0 += kWaves * CH) {
        u32x4 kx[LPC], vx[LPC];
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const uint32_t off = (uint32_t)(c0 + i * RPI + grp) * ROW + sub * 16;
            kx[i] = load16(rk, off);
            vx[i] = load16(rv, off);
        }
        float sc[LPC];
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const float d = lowsum<R>(dot16<T>(qx, kx[i]));
            sc[i] = c0 + i * RPI + grp < N ? d * a.c : -INFINITY;
            cm = fmaxf(cm, sc[i]);
        }
        cm = xmax<R>(cm);   // chunk max over the wave (finite: row c0 < N is valid)
        const float mn = fmaxf(m, cm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] *= alpha;
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - m);
            l += p;   // the R lanes of a row hold the same weight; only rows are summed below
            float vf[PER];
            widen<T>(vx[i], vf);
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(p, vf[e], acc[e]);
        }
    }
    // the wave's state: sum the row groups (lanes with the same sub hold the same dims)
    l = xsum<R>(l);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = xsum<R>(acc[e]);
    if (grp == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) part[wave][sub * PER + e] = acc[e];
        if (sub == 0) {
            part[wave][D] = m;
            part[wave][D + 1] = l;
        }
    }
    __syncthreads();
    if (wave != 0) return;

    // Wave 0: the new token as the last key, merge of the 8 partial states, output.
    const u32x4 knew = load16(rsrc(static_cast<const T *>(a.k) + bh * D, ROW), sub * 16);
    const u32x4 vnew = load16(rsrc(static_cast<const T *>(a.v) + bh * D, ROW), sub * 16);
    const float snew = lowsum<R>(dot16<T>(qx, knew)) * a.c;
    float mt = snew;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, part[w][D]);
    const float pnew = __builtin_amdgcn_exp2f(snew - mt);
    float lt = pnew, out[PER];
    float vf[PER];
    widen<T>(vnew, vf);
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = pnew * vf[e];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(part[w][D] - mt);   // 0 for a wave that saw no row
        lt = __builtin_fmaf(wt, part[w][D + 1], lt);
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] = __builtin_fmaf(wt, part[w][sub * PER + e], out[e]);
    }
    const float inv = 1.f / lt;
    if (grp == 0) {
        u32x4 ox;
        if constexpr (PER == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x2 pr = {(bf16)(out[2 * i] * inv), (bf16)(out[2 * i + 1] * inv)};
                ox[i] = __builtin_bit_cast(uint32_t, pr);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ox[i] = __float_as_uint(out[i] * inv);
        }
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(static_cast<T *>(a.o) + bh * D) + sub * 16) = ox;
        // the new token's K/V row goes to slot row N, bit for bit
        T *dk = static_cast<T *>(a.pool_k) + slot_off + (long)N * D;
        T *dv = static_cast<T *>(a.pool_v) + slot_off + (long)N * D;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(dk) + sub * 16) = knew;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(dv) + sub * 16) = vnew;
    }
}

template <typename T>
hipError_t launch_typed(const AttnArgs &a, int D, hipStream_t stream) {
    const dim3 grid((unsigned)((long)a.B * a.H)), block(kThreads);
    switch (D) {
        case 32: hipLaunchKernelGGL((ar_decode_kernel<T, 32>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((ar_decode_kernel<T, 64>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((ar_decode_kernel<T, 128>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ar_decode(const AttnArgs &a, int D, bool bf16_elems, hipStream_t stream) {
    if ((long)a.B * a.H <= 0) return hipSuccess;
    return bf16_elems ? launch_typed<bf16>(a, D, stream) : launch_typed<float>(a, D, stream);
}

}  // namespace unipin
