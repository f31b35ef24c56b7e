// Row kernels of the transformer block around the masked attention, for gfx950:
// LayerNorm over rows of the hidden state (HBM-bound: each lane moves 16 bytes per
// access and a wave reads and writes whole rows), and a pseudo-random fill that gives
// the GEMM tuner operands of realistic size.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_launch.h"

namespace unipin {
namespace {

typedef __bf16 bf16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const u32x4 &x, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(x[i] << 16);
        f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16 lo = (bf16)f[2 * i], hi = (bf16)f[2 * i + 1];   // round to nearest even
        r[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return r;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// y = (x - mean) / sqrt(var + eps) * w + b over each row of C values (population
// variance, fp32 statistics, bf16 out).  One wave per RPW rows, whose loads all go out
// before any arithmetic; lane l holds 16-byte pieces l, l + 64, ... of a row (P of
// them, C <= 512 P).
constexpr int kLnRowsPerWave = 1;

template <int P>
__global__ void __launch_bounds__(256) layernorm_kernel(const bf16 *__restrict__ x, const bf16 *__restrict__ w,
                                                        const bf16 *__restrict__ b, bf16 *__restrict__ y, long M,
                                                        int C, float eps) {
    constexpr int RPW = kLnRowsPerWave;
    const long row0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    const int lane = threadIdx.x & 63;
    if (row0 >= M) return;
    const int pieces = C / 8;
    u32x4 raw[RPW][P];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = lane + 64 * p;
            raw[r][p] = row0 + r < M && i < pieces ? reinterpret_cast<const u32x4 *>(x + (row0 + r) * C)[i]
                                                   : u32x4{0u, 0u, 0u, 0u};
        }
    float wf[P][8], bf[P][8];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int i = lane + 64 * p;
        const u32x4 wz = i < pieces ? reinterpret_cast<const u32x4 *>(w)[i] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 bz = i < pieces ? reinterpret_cast<const u32x4 *>(b)[i] : u32x4{0u, 0u, 0u, 0u};
        unpack8(wz, wf[p]);
        unpack8(bz, bf[p]);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        if (row0 + r >= M) break;
        float v[P][8];
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            unpack8(raw[r][p], v[p]);   // pieces past C are zero and add nothing
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[p][e];
        }
        const float mean = wave_sum(s) / (float)C;
        float q = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (lane + 64 * p < pieces) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = v[p][e] - mean;
                    q = __builtin_fmaf(d, d, q);
                }
            }
        }
        const float rstd = 1.f / sqrtf(wave_sum(q) / (float)C + eps);
        u32x4 *yr = reinterpret_cast<u32x4 *>(y + (row0 + r) * C);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = lane + 64 * p;
            if (i < pieces) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf((v[p][e] - mean) * rstd, wf[p][e], bf[p][e]);
                yr[i] = pack8(o);
            }
        }
    }
}

// Fills n bf16 values with a hash of (seed, index) mapped to [-amp, amp): operands for
// timing GEMM kernels on data of realistic size and spread.
__global__ void __launch_bounds__(256) fill_random_kernel(bf16 *__restrict__ dst, size_t n, unsigned seed,
                                                          float amp) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    uint32_t h = (uint32_t)i * 0x9e3779b1u ^ seed * 0x85ebca77u;
    h ^= h >> 15;
    h *= 0x2c1b3c6du;
    h ^= h >> 12;
    h *= 0x297a2d39u;
    h ^= h >> 15;
    dst[i] = (bf16)(amp * ((float)(h >> 8) * (1.f / 8388608.f) - 1.f));
}

// The LayerNorm folded into the product after it: for column n of W [C, N],
// wf[k][n] = bf16(gamma[k] W[k][n]), u[n] = sum_k wf[k][n] (of the rounded values, so that
// the mean term cancels what x wf carries of it) and v[n] = sum_k beta[k] W[k][n] + b[n],
// in fp32.  One thread per column; the rows are read and written coalesced.
__global__ void __launch_bounds__(256) fold_layernorm_kernel(const bf16 *__restrict__ gamma,
                                                             const bf16 *__restrict__ beta,
                                                             const bf16 *__restrict__ w, const bf16 *__restrict__ b,
                                                             int C, int N, bf16 *__restrict__ wf,
                                                             float *__restrict__ uv) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float u = 0.f, v = 0.f;
    for (int k = 0; k < C; ++k) {
        const float wk = (float)w[(long)k * N + n];
        const bf16 f = (bf16)((float)gamma[k] * wk);   // round to nearest even
        wf[(long)k * N + n] = f;
        u += (float)f;
        v = __builtin_fmaf((float)beta[k], wk, v);
    }
    uv[n] = u;
    uv[N + n] = v + (float)b[n];
}

// The same sequence as fp32 values (operands for timing, tuning only).
__global__ void __launch_bounds__(256) fill_random_f32_kernel(float *__restrict__ dst, size_t n, unsigned seed,
                                                              float amp) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    uint32_t h = (uint32_t)i * 0x9e3779b1u ^ seed * 0x85ebca77u;
    h ^= h >> 15;
    h *= 0x2c1b3c6du;
    h ^= h >> 12;
    h *= 0x297a2d39u;
    h ^= h >> 15;
    dst[i] = amp * ((float)(h >> 8) * (1.f / 8388608.f) - 1.f);
}

unsigned blocks_for(long threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

hipError_t launch_layernorm(const void *x, const void *w, const void *b, void *y, long M, int C, float eps,
                            hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if (C % 8 != 0 || C > 2048) return hipErrorInvalidValue;
    const long waves = (M + kLnRowsPerWave - 1) / kLnRowsPerWave;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    const bf16 *xs = static_cast<const bf16 *>(x), *ws = static_cast<const bf16 *>(w),
               *bs = static_cast<const bf16 *>(b);
    bf16 *ys = static_cast<bf16 *>(y);
    if (C <= 512)
        hipLaunchKernelGGL(layernorm_kernel<1>, grid, block, 0, stream, xs, ws, bs, ys, M, C, eps);
    else if (C <= 1024)
        hipLaunchKernelGGL(layernorm_kernel<2>, grid, block, 0, stream, xs, ws, bs, ys, M, C, eps);
    else
        hipLaunchKernelGGL(layernorm_kernel<4>, grid, block, 0, stream, xs, ws, bs, ys, M, C, eps);
    return hipGetLastError();
}

hipError_t launch_fold_layernorm(const void *gamma, const void *beta, const void *w, const void *b, int C, int N,
                                 void *wf, void *uv, hipStream_t stream) {
    if (C <= 0 || N <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fold_layernorm_kernel, dim3(blocks_for(N)), dim3(256), 0, stream, static_cast<const bf16 *>(gamma),
                       static_cast<const bf16 *>(beta), static_cast<const bf16 *>(w), static_cast<const bf16 *>(b), C,
                       N, static_cast<bf16 *>(wf), static_cast<float *>(uv));
    return hipGetLastError();
}

hipError_t launch_fill_random(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_random_kernel, dim3(blocks_for((long)n)), dim3(256), 0, stream, static_cast<bf16 *>(dst),
                       n, seed, amp);
    return hipGetLastError();
}

hipError_t launch_fill_random_f32(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_random_f32_kernel, dim3(blocks_for((long)n)), dim3(256), 0, stream,
                       static_cast<float *>(dst), n, seed, amp);
    return hipGetLastError();
}

}  // namespace unipin
