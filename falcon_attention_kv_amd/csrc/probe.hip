// Measurement probes for gfx950, built into their own library (libunipin_probe.so) and
// used only by the benchmark: they bound what the attention kernels can reach on this
// chip, beside the plain device copy that bounds HBM.
//   * unipin_probe_mfma: the achievable bf16 matrix-core rate -- every SIMD runs two waves
//     of independent v_mfma_f32_32x32x16_bf16 (four accumulators each);
//   * unipin_probe_overlap: whether a SIMD overlaps matrix-core work with vector work --
//     the same loop with only MFMAs, only exponentials (v_exp_f32 and a subtraction), both
//     in each wave, or MFMAs in one wave and exponentials in the other wave of the SIMD;
//     and the first and third with the same matrix work as v_mfma_f32_16x16x32_bf16
//     (twice as many instructions of half the work), the finer grain an attention loop
//     could interleave with its exponentials;
//   * unipin_probe_lds: the LDS read rate of the two operand reads the attention tiles
//     use, ds_read_b128 (the K operand) and ds_read_b64_tr_b16 (the transposed V
//     operand), with 16 waves per CU as in the ranking decode.
// Each writes one float per thread (so that nothing is optimised away) into a buffer of
// blocks x threads floats owned by the caller.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kLdsProbeBytes = 65536;   // LDS per block: two blocks fit on a CU

// ROLE 0: every wave runs the MFMAs (if NM) and the exponentials (if NE); ROLE 1: even
// waves the MFMAs, odd waves the exponentials.  NM counts 32x32x16 MFMAs; SMALL issues
// the same work as twice as many 16x16x32 MFMAs.
template <int NM, int NE, int ROLE, bool SMALL = false>
__global__ void __launch_bounds__(512) probe_kernel(float *out, int iters) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const bool do_m = NM > 0 && (ROLE == 0 || (wave & 1) == 0);
    const bool do_e = NE > 0 && (ROLE == 0 || (wave & 1) == 1);
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    f32x4 sm0 = {}, sm1 = {}, sm2 = {}, sm3 = {};
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (tid + i));
        b[i] = (__bf16)(0.002f * (tid - i));
    }
    float x[16];
    for (int i = 0; i < 16; ++i) x[i] = -0.001f * (tid + i);
    for (int it = 0; it < iters; ++it) {
        if (do_m && !SMALL) {
#pragma unroll
            for (int k = 0; k < NM; k += 4) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
                acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
            }
        }
        if (do_m && SMALL) {
#pragma unroll
            for (int k = 0; k < 2 * NM; k += 4) {
                sm0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sm0, 0, 0, 0);
                sm1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sm1, 0, 0, 0);
                sm2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sm2, 0, 0, 0);
                sm3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sm3, 0, 0, 0);
            }
        }
        if (do_e) {
#pragma unroll
            for (int k = 0; k < NE; ++k) x[k & 15] = __builtin_amdgcn_exp2f(x[k & 15]) - 1.0f;
        }
    }
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i] + acc2[i] + acc3[i] + x[i];
    for (int i = 0; i < 4; ++i) s += sm0[i] + sm1[i] + sm2[i] + sm3[i];
    out[blockIdx.x * blockDim.x + tid] = s;
}

// LDS reads: every wave reads 8 KiB per iteration, as 8 ds_read_b128 (TR false: each
// lane 16 consecutive bytes, a wave 1 KiB in a row) or 16 ds_read_b64_tr_b16 (TR true:
// each lane 8 consecutive bytes, a wave 512 B in a row).  The addresses move with the
// iteration (so no read can be hoisted) and are masked into the block's 64 KiB, aligned
// to the access; the values are summed into one word per thread, with little enough
// vector work (one or two three-input adds per read) that the LDS sets the pace.
template <bool TR>
__global__ void __launch_bounds__(512) lds_probe_kernel(float *out, int iters) {
    __shared__ __attribute__((aligned(16))) char lds_raw[kLdsProbeBytes];
    LDS_AS char *lds = (LDS_AS char *)lds_raw;
    const int tid = threadIdx.x;
    for (int i = tid * 16; i < kLdsProbeBytes; i += 512 * 16)
        *reinterpret_cast<LDS_AS u32x4 *>(lds + i) = u32x4{(unsigned)i, (unsigned)i + 1u, (unsigned)i + 2u,
                                                             (unsigned)i + 3u};
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    unsigned acc = 0u;
    for (int it = 0; it < iters; ++it) {
        const unsigned base = (unsigned)(wave * 8192 + it * 4096);
        if (!TR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned a = (base + (unsigned)(j * 1024 + lane * 16)) & (unsigned)(kLdsProbeBytes - 16);
                const u32x4 v = *reinterpret_cast<const LDS_AS u32x4 *>(lds + a);
                acc = acc + v[0] + v[1] + v[2] + v[3];   // two three-input adds per read
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const unsigned a = (base + (unsigned)(j * 512 + lane * 8)) & (unsigned)(kLdsProbeBytes - 8);
                const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                              (LDS_AS i16x4 *)(lds + a)));
                acc = acc + w[0] + w[1];   // one three-input add per read
            }
        }
    }
    out[blockIdx.x * blockDim.x + tid] = (float)acc;
}

template <bool TR>
int timed_lds(float *buf, int blocks, int iters, float *ms) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -1;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -1;
    }
    hipLaunchKernelGGL((lds_probe_kernel<TR>), dim3(blocks), dim3(512), 0, 0, buf, iters);   // warm-up
    hipError_t e = hipEventRecord(e0, 0);
    hipLaunchKernelGGL((lds_probe_kernel<TR>), dim3(blocks), dim3(512), 0, 0, buf, iters);
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int NM, int NE, int ROLE, bool SMALL = false>
int timed(float *buf, int blocks, int threads, int iters, float *ms) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1;
    hipLaunchKernelGGL((probe_kernel<NM, NE, ROLE, SMALL>), dim3(blocks), dim3(threads), 0, 0, buf, iters);   // warm-up
    hipError_t e = hipEventRecord(e0, 0);
    hipLaunchKernelGGL((probe_kernel<NM, NE, ROLE, SMALL>), dim3(blocks), dim3(threads), 0, 0, buf, iters);
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

extern "C" {

// One launch of blocks x 512 threads (two waves per SIMD when blocks = CUs), each wave
// `iters` x 8 MFMAs of 32x32x16 bf16 (32768 FLOP each).  *tflops receives the rate.
// buf: blocks * 512 floats of device memory.  Returns 0 or -1 (HIP error).
int unipin_probe_mfma(float *buf, int blocks, int iters, double *tflops) {
    float ms = 0.f;
    if (timed<8, 0, 0>(buf, blocks, 512, iters, &ms)) return -1;
    *tflops = (double)blocks * 8 * iters * 8 * 32768.0 / (ms * 1e-3) / 1e12;
    return 0;
}

// Nanoseconds per loop iteration of one SIMD (blocks x 512 threads: two waves per SIMD)
// for: [0] MFMAs only (8 per wave), [1] exponentials only (32 per wave), [2] both in each
// wave, [3] 8 MFMAs in one wave and 32 exponentials in the other, [4] and [5] as [0] and
// [2] with 16 MFMAs of 16x16x32 instead of 8 of 32x32x16.  ns: 6 doubles; buf as above.
int unipin_probe_overlap(float *buf, int blocks, int iters, double *ns) {
    float ms = 0.f;
    if (timed<8, 0, 0>(buf, blocks, 512, iters, &ms)) return -1;
    ns[0] = ms * 1e6 / iters;
    if (timed<0, 32, 0>(buf, blocks, 512, iters, &ms)) return -1;
    ns[1] = ms * 1e6 / iters;
    if (timed<8, 32, 0>(buf, blocks, 512, iters, &ms)) return -1;
    ns[2] = ms * 1e6 / iters;
    if (timed<8, 32, 1>(buf, blocks, 512, iters, &ms)) return -1;
    ns[3] = ms * 1e6 / iters;
    if (timed<8, 0, 0, true>(buf, blocks, 512, iters, &ms)) return -1;
    ns[4] = ms * 1e6 / iters;
    if (timed<8, 32, 0, true>(buf, blocks, 512, iters, &ms)) return -1;
    ns[5] = ms * 1e6 / iters;
    return 0;
}

// LDS read rate in bytes per nanosecond and CU, for blocks x 512 threads (two blocks per
// CU when blocks = 2 x cus: 16 waves per CU), each wave `iters` x 8 KiB: [0] as
// ds_read_b128, [1] as ds_read_b64_tr_b16.  buf: blocks * 512 floats of device memory;
// rate: 2 doubles.  Returns 0 or -1 (HIP error or bad sizes).
int unipin_probe_lds(float *buf, int blocks, int iters, int cus, double *rate) {
    if (blocks < 1 || iters < 1 || cus < 1) return -1;
    const double bytes = (double)blocks * 8 * iters * 8192.0;
    float ms = 0.f;
    if (timed_lds<false>(buf, blocks, iters, &ms)) return -1;
    rate[0] = bytes / (ms * 1e6) / cus;
    if (timed_lds<true>(buf, blocks, iters, &ms)) return -1;
    rate[1] = bytes / (ms * 1e6) / cus;
    return 0;
}

}  // extern "C"
