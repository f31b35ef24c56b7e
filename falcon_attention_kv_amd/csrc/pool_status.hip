// Sticky per-pool status flags.  Kernels OR flags into their pool's word when a user's
// device-side slot or length is invalid (that user is skipped); unipin_pool_status takes
// and clears the word in one device-side atomic exchange, ordered on the caller's stream,
// so a flag raised by a kernel on another stream is either in this read or kept for the
// next one.  The words are file-scope device arrays, one entry per live pool descriptor,
// so no call ever allocates for them: their addresses are looked up once per device with
// hipGetSymbolAddress and only those addresses reach kernels and copies.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "attn_launch.h"

namespace unipin {

__device__ unsigned int g_pool_flags[kMaxPools];   // flags raised since the last take
__device__ unsigned int g_pool_taken[kMaxPools];   // the value the last take exchanged out

namespace {

constexpr int kMaxDevices = 64;
struct Words {
    unsigned int *flags, *taken;
};
std::atomic<bool> g_ready[kMaxDevices];
Words g_words[kMaxDevices];
std::mutex g_words_mu;

__global__ void take_flags_kernel(unsigned int *flags, unsigned int *taken) {
    *taken = atomicExch(flags, 0u);
}

hipError_t device_words(Words *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_ready[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(g_words_mu);
        if (!g_ready[dev].load(std::memory_order_relaxed)) {
            void *f = nullptr, *t = nullptr;
            e = hipGetSymbolAddress(&f, HIP_SYMBOL(g_pool_flags));
            if (e != hipSuccess) return e;
            e = hipGetSymbolAddress(&t, HIP_SYMBOL(g_pool_taken));
            if (e != hipSuccess) return e;
            g_words[dev] = {static_cast<unsigned int *>(f), static_cast<unsigned int *>(t)};
            g_ready[dev].store(true, std::memory_order_release);
        }
    }
    *out = g_words[dev];
    return hipSuccess;
}

}  // namespace

hipError_t pool_flag_word(int index, unsigned int **out) {
    if (index < 0 || index >= kMaxPools) return hipErrorInvalidValue;
    Words w;
    const hipError_t e = device_words(&w);
    if (e != hipSuccess) return e;
    *out = w.flags + index;
    return hipSuccess;
}

hipError_t clear_pool_flags(int index, hipStream_t stream) {
    if (index < 0 || index >= kMaxPools) return hipErrorInvalidValue;
    Words w;
    hipError_t e = device_words(&w);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(take_flags_kernel, dim3(1), dim3(1), 0, stream, w.flags + index, w.taken + index);
    return hipGetLastError();
}

hipError_t take_pool_flags(int index, hipStream_t stream, unsigned int *host) {
    hipError_t e = clear_pool_flags(index, stream);
    if (e != hipSuccess) return e;
    Words w;
    e = device_words(&w);
    if (e != hipSuccess) return e;
    e = hipMemcpyAsync(host, w.taken + index, sizeof(unsigned int), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(stream);
}

}  // namespace unipin
