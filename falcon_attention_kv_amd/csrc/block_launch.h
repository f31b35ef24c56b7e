// Internal interface between the block's host code (block.cpp) and its kernels
// (block_kernels.hip, gemm_bf16.hip).  Not installed; the public interface is include/unipin.h.
// All tensors are bf16, contiguous, 16-byte aligned device memory.
#pragma once

#include <hip/hip_runtime.h>

namespace unipin {

// y[M, C] = LayerNorm(x[M, C]) * w + b, eps as given; C % 8 == 0, C <= 2048.
hipError_t launch_layernorm(const void *x, const void *w, const void *b, void *y, long M, int C, float eps,
                            hipStream_t stream);
// n bf16 values of a fixed pseudo-random sequence (seed), uniform in [-amp, amp).
hipError_t launch_fill_random(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream);

// y[M, N] = epilogue(x[M, K] @ w[K, N] + bias[N]) with this library's MFMA kernel
// (gemm_bf16.hip), fp32 accumulation, one rounding to bf16.  kGemmBiasResidual adds the
// old y (in place).  Needs N % 128 == 0, K % 32 == 0 and byte sizes below 2^31
// (gemm_bf16_supported).  cfg 0 .. kGemmConfigs-1 picks the workgroup tile: 64, 128 or 256
// rows (gemm_bf16_rows_per_tile) by 128 columns.
enum GemmEpilogue : int { kGemmBias = 0, kGemmBiasGelu = 1, kGemmBiasResidual = 2 };
constexpr int kGemmConfigs = 3;
bool gemm_bf16_supported(long M, int N, int K);
int gemm_bf16_rows_per_tile(int cfg);
hipError_t launch_gemm_bf16(const void *x, const void *w, const void *bias, void *y, long M, int N, int K, int epi,
                            int cfg, hipStream_t stream);

}  // namespace unipin
