// Sharing one pool between processes on one GPU: the retrieval process exports its
// pool, the ranking process imports it and reads the slots in place ([notes] section 6,
// cross-process KV sharing: the pool's IPC handle goes to a file at start-up and the
// other process maps the same memory; [review] section 2.4).
//
// The share file holds the pool's dims, an IPC handle for each device allocation that
// holds the K or V array with the array's byte offset inside it, and the POSIX name of
// a shared host page.  At export the pool's round-robin state (hand-out cursor and
// per-slot generations) moves into that page; the exporter keeps counting there and
// importers map it read-only, so a ranking call can compare a request's generation with
// the live one without any message between the processes.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include <hip/hip_runtime.h>

#include "unipin.h"
#include "attn_launch.h"
#include "pool_internal.h"

namespace {

constexpr char kMagic[8] = {'U', 'N', 'I', 'P', 'I', 'N', 'P', '1'};
constexpr uint32_t kShareVersion = 1;
constexpr size_t kMaxShareAlloc = (size_t)2 << 30;   // one shared allocation stays under 2 GiB

struct ShareRecord {
    char magic[8];
    uint32_t version;
    uint32_t record_bytes;
    int32_t L, S, H, n_max, D, dtype;
    int32_t same_alloc;          // K and V arrays live in one allocation (one handle)
    int32_t owner_pid;
    uint64_t k_offset, v_offset; // byte offset of each array inside its allocation
    uint64_t k_alloc, v_alloc;   // allocation sizes (bytes)
    hipIpcMemHandle_t k_handle, v_handle;
    char shm_name[64];
    uint64_t ring_bytes;
};

std::atomic<unsigned> g_share_counter{0};

size_t ring_page_bytes(int S) {
    const size_t page = (size_t)sysconf(_SC_PAGESIZE);
    const size_t need = ((size_t)S + 1) * sizeof(uint64_t);
    return (need + page - 1) / page * page;
}

int alloc_of(void *p, void **base, size_t *bytes) {
    hipDeviceptr_t b = nullptr;
    size_t n = 0;
    if (hipMemGetAddressRange(&b, &n, reinterpret_cast<hipDeviceptr_t>(p)) != hipSuccess || !b) return UNIPIN_EINVAL;
    *base = reinterpret_cast<void *>(b);
    *bytes = n;
    return UNIPIN_OK;
}

bool write_file(const char *path, const ShareRecord &r) {
    const std::string tmp = std::string(path) + ".tmp";
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (!f) return false;
    const bool ok = std::fwrite(&r, sizeof(r), 1, f) == 1;
    if (std::fclose(f) != 0 || !ok) {
        std::remove(tmp.c_str());
        return false;
    }
    if (std::rename(tmp.c_str(), path) != 0) {
        std::remove(tmp.c_str());
        return false;
    }
    return true;
}

}  // namespace

namespace unipin {

void pool_share_release(unipin_pool *pool) {
    if (pool->ipc_k) (void)hipIpcCloseMemHandle(pool->ipc_k);
    if (pool->ipc_v && pool->ipc_v != pool->ipc_k) (void)hipIpcCloseMemHandle(pool->ipc_v);
    pool->ipc_k = pool->ipc_v = nullptr;
    if (pool->shm_addr) {
        munmap(pool->shm_addr, pool->shm_bytes);
        if (pool->shm_owner) shm_unlink(pool->shm_name);
    }
    pool->shm_addr = nullptr;
    pool->ring = pool->ring_own;
}

}  // namespace unipin

extern "C" {

int unipin_pool_export(unipin_pool_t *pool, const char *path) {
    if (!pool || !path || !*path) return UNIPIN_EINVAL;
    if (pool->readonly || pool->shm_addr) return UNIPIN_EINVAL;   // imported, or exported already
    ShareRecord r;
    std::memset(&r, 0, sizeof(r));
    std::memcpy(r.magic, kMagic, sizeof(kMagic));
    r.version = kShareVersion;
    r.record_bytes = sizeof(ShareRecord);
    r.L = pool->L;
    r.S = pool->S;
    r.H = pool->H;
    r.n_max = pool->n_max;
    r.D = pool->D;
    r.dtype = pool->dtype;
    r.owner_pid = (int32_t)getpid();
    const size_t array_bytes = (size_t)pool->L * pool->S * pool->H * pool->n_max * pool->D * pool->elem;
    void *kb = nullptr, *vb = nullptr;
    size_t kn = 0, vn = 0;
    int rc = alloc_of(pool->k, &kb, &kn);
    if (rc) return rc;
    rc = alloc_of(pool->v, &vb, &vn);
    if (rc) return rc;
    if (kn >= kMaxShareAlloc || vn >= kMaxShareAlloc) return UNIPIN_EINVAL;
    r.k_offset = (uint64_t)(static_cast<char *>(pool->k) - static_cast<char *>(kb));
    r.v_offset = (uint64_t)(static_cast<char *>(pool->v) - static_cast<char *>(vb));
    if (r.k_offset + array_bytes > kn || r.v_offset + array_bytes > vn) return UNIPIN_EINVAL;
    r.k_alloc = kn;
    r.v_alloc = vn;
    r.same_alloc = kb == vb;
    if (hipIpcGetMemHandle(&r.k_handle, kb) != hipSuccess) return UNIPIN_EHIP;
    if (!r.same_alloc && hipIpcGetMemHandle(&r.v_handle, vb) != hipSuccess) return UNIPIN_EHIP;

    // the shared ring page
    std::snprintf(r.shm_name, sizeof(r.shm_name), "/unipin-%d-%d-%u", (int)getpid(), pool->flag_index,
                  g_share_counter.fetch_add(1));
    r.ring_bytes = ring_page_bytes(pool->S);
    const int fd = shm_open(r.shm_name, O_CREAT | O_EXCL | O_RDWR, 0600);
    if (fd < 0) return UNIPIN_EIO;
    void *addr = MAP_FAILED;
    if (ftruncate(fd, (off_t)r.ring_bytes) == 0)
        addr = mmap(nullptr, r.ring_bytes, PROT_READ | PROT_WRITE, MAP_SHARED, fd, 0);
    close(fd);
    if (addr == MAP_FAILED) {
        shm_unlink(r.shm_name);
        return UNIPIN_EIO;
    }
    uint64_t *ring = static_cast<uint64_t *>(addr);
    for (int i = 0; i <= pool->S; ++i) __atomic_store_n(&ring[i], unipin::ring_load(&pool->ring_own[i]), __ATOMIC_RELAXED);
    __atomic_thread_fence(__ATOMIC_RELEASE);
    pool->shm_addr = addr;
    pool->shm_bytes = r.ring_bytes;
    std::memcpy(pool->shm_name, r.shm_name, sizeof(r.shm_name));
    pool->shm_owner = true;
    pool->ring = ring;
    if (!write_file(path, r)) {
        unipin::pool_share_release(pool);
        return UNIPIN_EIO;
    }
    return UNIPIN_OK;
}

int unipin_pool_import(unipin_pool_t **out, const char *path) {
    if (!out) return UNIPIN_EINVAL;
    *out = nullptr;
    if (!path || !*path) return UNIPIN_EINVAL;
    ShareRecord r;
    FILE *f = std::fopen(path, "rb");
    if (!f) return UNIPIN_EIO;
    const bool got = std::fread(&r, sizeof(r), 1, f) == 1;
    std::fclose(f);
    if (!got || std::memcmp(r.magic, kMagic, sizeof(kMagic)) != 0 || r.version != kShareVersion ||
        r.record_bytes != sizeof(ShareRecord) || r.shm_name[0] != '/' ||
        std::memchr(r.shm_name, 0, sizeof(r.shm_name)) == nullptr || r.S < 1 ||
        r.ring_bytes != ring_page_bytes(r.S))
        return UNIPIN_EIO;

    void *kb = nullptr, *vb = nullptr;
    if (hipIpcOpenMemHandle(&kb, r.k_handle, hipIpcMemLazyEnablePeerAccess) != hipSuccess) return UNIPIN_EHIP;
    if (r.same_alloc) {
        vb = kb;
    } else if (hipIpcOpenMemHandle(&vb, r.v_handle, hipIpcMemLazyEnablePeerAccess) != hipSuccess) {
        (void)hipIpcCloseMemHandle(kb);
        return UNIPIN_EHIP;
    }
    unipin_pool_t *p = nullptr;
    int rc = unipin_pool_create(&p, static_cast<char *>(kb) + r.k_offset, static_cast<char *>(vb) + r.v_offset, r.L,
                                r.S, r.H, r.n_max, r.D, r.dtype);
    if (rc) {
        if (vb != kb) (void)hipIpcCloseMemHandle(vb);
        (void)hipIpcCloseMemHandle(kb);
        return rc == UNIPIN_ENOMEM ? rc : UNIPIN_EIO;
    }
    p->ipc_k = kb;
    p->ipc_v = vb;
    p->readonly = true;
    const int fd = shm_open(r.shm_name, O_RDONLY, 0);
    void *addr = fd < 0 ? MAP_FAILED : mmap(nullptr, r.ring_bytes, PROT_READ, MAP_SHARED, fd, 0);
    if (fd >= 0) close(fd);
    if (addr == MAP_FAILED) {
        unipin_pool_destroy(p);
        return UNIPIN_EIO;
    }
    p->shm_addr = addr;
    p->shm_bytes = r.ring_bytes;
    std::memcpy(p->shm_name, r.shm_name, sizeof(r.shm_name));
    p->shm_owner = false;
    p->ring = static_cast<uint64_t *>(addr);
    *out = p;
    return UNIPIN_OK;
}

}  // extern "C"
