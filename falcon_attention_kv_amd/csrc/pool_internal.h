// The pool descriptor behind the opaque unipin_pool_t of the C ABI, shared by the host
// sources of the library (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

// Round-robin state of a pool: word 0 counts the hand-outs so far, word 1 + s the
// hand-outs of slot s.  It lives in the descriptor's own host memory, or, once the pool
// is shared with another process, in a shared memory page that the other process maps
// read-only.  Words are accessed with atomic builtins, which work across processes on a
// shared mapping.
struct unipin_pool {
    void *k;
    void *v;
    int L, S, H, n_max, D, dtype;
    int elem;                            // bytes per pool element
    int flag_index;                      // entry in the per-device flag arrays
    std::atomic<bool> clear_flags;       // the entry may hold an earlier owner's flags
    bool readonly;                       // imported from another process: rank decode only
    uint64_t *ring;                      // [1 + S] cursor, then per-slot generations
    uint64_t *ring_own;                  // the private ring (freed with the descriptor)
    // sharing between processes (pool_share.cpp)
    void *shm_addr;                      // mapping of the shared ring page, or null
    size_t shm_bytes;
    char shm_name[64];                   // POSIX name of the page ("" if none)
    bool shm_owner;                      // this process created the page (unlinks it)
    void *ipc_k, *ipc_v;                 // bases of allocations opened from handles
};

namespace unipin {

// Before a pool's kernel: clears a reused flag entry once, on `stream`, and returns the
// device address of the pool's flag word.  UNIPIN_* status.
int pool_kernel_prologue(unipin_pool *pool, hipStream_t stream, unsigned int **flag_word);

// Releases what pool_share.cpp attached to a descriptor (mappings, IPC handles).
void pool_share_release(unipin_pool *pool);

inline uint64_t ring_load(const uint64_t *w) { return __atomic_load_n(w, __ATOMIC_ACQUIRE); }

}  // namespace unipin
