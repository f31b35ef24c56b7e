// Sticky per-device status word.  Kernels OR flags into it when a user's device-side
// slot or length is invalid (that user is skipped); unipin_device_status reads and
// clears it.  It is a file-scope device variable, so no call ever allocates for it:
// its address is looked up once per device with hipGetSymbolAddress and only that
// address is handed to kernels and copies.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "attn_launch.h"

namespace unipin {

__device__ unsigned int g_unipin_status = 0;

namespace {
constexpr int kMaxDevices = 64;
std::atomic<unsigned int *> g_word[kMaxDevices];
std::mutex g_word_mu;
}  // namespace

hipError_t device_status_word(unsigned int **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    unsigned int *p = g_word[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_word_mu);
        p = g_word[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_unipin_status));
            if (e != hipSuccess) return e;
            p = static_cast<unsigned int *>(addr);
            g_word[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace unipin
