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
//     could interleave with its exponentials.
// Each writes one float per thread (so that nothing is optimised away) into a buffer of
// blocks x threads floats owned by the caller.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
    hipEventDestroy(e0);
    hipEventDestroy(e1);
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

}  // extern "C"
