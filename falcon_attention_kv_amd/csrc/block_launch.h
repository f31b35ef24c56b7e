// Internal interface between the block's host code (block.cpp) and its kernels
// (block_kernels.hip).  Not installed; the public interface is include/unipin.h.
// All tensors are bf16, contiguous, 16-byte aligned device memory.
#pragma once

#include <hip/hip_runtime.h>

namespace unipin {

// y[M, C] = LayerNorm(x[M, C]) * w + b, eps as given; C % 8 == 0, C <= 2048.
hipError_t launch_layernorm(const void *x, const void *w, const void *b, void *y, long M, int C, float eps,
                            hipStream_t stream);
// n bf16 values of a fixed pseudo-random sequence (seed), uniform in [-amp, amp).
hipError_t launch_fill_random(void *dst, size_t n, unsigned seed, float amp, hipStream_t stream);

}  // namespace unipin
