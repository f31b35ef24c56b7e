// Internal interface between the block's host code (block.cpp) and its kernels
// (block_kernels.hip, gemm_bf16.hip).  Not installed; the public interface is include/unipin.h.
// All tensors are bf16, contiguous, 16-byte aligned device memory.
#pragma once

#include <hip/hip_runtime.h>

namespace unipin {

// y[M, C] = LayerNorm(x[M, C]) * w + b, eps as given; C % 8 == 0, C <= 2048.
hipError_t launch_layernorm(const void *x, const void *w, const void *b, void *y, long M, int C, float eps,
                            hipStream_t stream);
// The LayerNorm (gamma, beta over C) folded into the product that follows it, x W + b
// with W [C, N]: wf = bf16(diag(gamma) W) [C, N] and uv = fp32 [2][N] (u = column sums of
// wf, v = beta W + b), for the kGemmLn* epilogues.
hipError_t launch_fold_layernorm(const void *gamma, const void *beta, const void *w, const void *b, int C, int N,
                                 void *wf, void *uv, hipStream_t stream);
// n bf16 values of a fixed pseudo-random sequence (seed), uniform in [-amp, amp).
hipError_t launch_fill_random(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream);
// n fp32 values of the same sequence.
hipError_t launch_fill_random_f32(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream);

// y[M, N] = epilogue(x[M, K] @ w[K, N] + bias[N]) with this library's MFMA kernel
// (gemm_bf16.hip), fp32 accumulation, one rounding to bf16.  kGemmBiasResidual adds the
// old y (in place).  cfg 0 .. kGemmConfigs-1 picks the workgroup tile: 64, 128 or 256
// rows by 128 columns with 32-deep stages, or 128 x 128 with 64-deep stages.  Needs
// N % 128 == 0, K a multiple of the stage depth and byte sizes below 2^31
// (gemm_bf16_supported).
// kGemmLnBias / kGemmLnBiasGelu fold the LayerNorm of x into the product: x is the
// un-normalised input, w = diag(gamma) W (launch_fold_layernorm) and bias points to fp32
// [2][N]: u = the column sums of that w, then v = beta W + b.  The kernel takes each row's
// mean and 1/sqrt(var + kGemmLnEps) from the X tiles it streams and writes
// rstd (x w - mean u) + v, which is LN(x) W + b (then the GELU).
enum GemmEpilogue : int { kGemmBias = 0, kGemmBiasGelu = 1, kGemmBiasResidual = 2, kGemmLnBias = 3, kGemmLnBiasGelu = 4 };
constexpr float kGemmLnEps = 1e-5f;
constexpr int kGemmConfigs = 4;
bool gemm_bf16_supported(long M, int N, int K, int cfg);
hipError_t launch_gemm_bf16(const void *x, const void *w, const void *bias, void *y, long M, int N, int K, int epi,
                            int cfg, hipStream_t stream);

}  // namespace unipin
