// C ABI of the library (include/unipin.h): pool descriptor, round-robin slot hand-out,
// host-side argument checks, and dispatch to the HIP kernels by element type and head
// dimension.  Nothing here allocates device memory; the only HIP calls are kernel
// launches (prefill, rank decode, autoregressive step) and the status read-back.
#include "unipin.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <new>

#include "attn_launch.h"

struct unipin_pool {
    void *k;
    void *v;
    int L, S, H, n_max, D, dtype;
    int elem;                              // bytes per element
    std::atomic<uint64_t> cursor;          // hand-outs so far
    std::atomic<uint64_t> *gen;            // [S] hand-outs per slot
};

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool supported_d(int D) { return D == 32 || D == 64 || D == 128; }

// Resolves the score scale: non-positive or NaN means 1/sqrt(D); infinity is rejected.
int resolve_scale(float scale, int D, float *c) {
    if (std::isinf(scale)) return UNIPIN_EINVAL;
    const double s = (std::isnan(scale) || scale <= 0.f) ? 1.0 / std::sqrt((double)D) : (double)scale;
    *c = (float)(s * 1.4426950408889634);  // scale * log2(e)
    return UNIPIN_OK;
}

// bf16 kernels serve bf16 and E4M3 pools (bf16 activations); fp32 pools the fp32 ones.
bool bf16_kernels(const unipin_pool *pool) { return pool->dtype != UNIPIN_FP32; }

// bytes of one activation element (q, k, v, o) for this pool
int act_bytes(const unipin_pool *pool) { return pool->dtype == UNIPIN_FP32 ? 4 : 2; }

int fill_pool_args(unipin::AttnArgs &a, const unipin_pool *pool, int layer) {
    const long long per_layer = (long long)pool->S * pool->H * pool->n_max * pool->D;
    a.pool_k = static_cast<char *>(pool->k) + (long long)layer * per_layer * pool->elem;
    a.pool_v = static_cast<char *>(pool->v) + (long long)layer * per_layer * pool->elem;
    a.n_max = pool->n_max;
    a.S = pool->S;
    a.H = pool->H;
    return UNIPIN_OK;
}

int launch(const unipin::AttnArgs &a, const unipin_pool *pool, bool prefill, void *stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (bf16_kernels(pool)) {
        const bool pool8 = pool->dtype == UNIPIN_FP8_E4M3;
        e = prefill ? unipin::launch_prefill_bf16(a, pool->D, pool8, st)
                    : unipin::launch_decode_bf16(a, pool->D, pool8, st);
    }
    else
        e = prefill ? unipin::launch_prefill_fp32(a, pool->D, st) : unipin::launch_decode_fp32(a, pool->D, st);
    return e == hipSuccess ? UNIPIN_OK : UNIPIN_EHIP;
}

int rows_per_block(const unipin_pool *pool, bool prefill) {
    if (!bf16_kernels(pool)) return unipin::kFp32RowsPerBlock;
    return prefill ? unipin::bf16_prefill_rows_per_block(pool->D) : unipin::bf16_decode_rows_per_item(pool->D);
}

}  // namespace

namespace unipin {

int attention_call(bool prefill, const void *q, const void *k, const void *v, RowLayout in, void *o, RowLayout out,
                   ::unipin_pool *pool, const int32_t *slot, const int32_t *lens, int layer, int B, int rows,
                   float scale, void *stream) {
    if (!pool || !q || !k || !v || !lens || !slot || !o) return UNIPIN_EINVAL;
    if (B < 1 || rows < 1 || (prefill && rows > pool->n_max)) return UNIPIN_EINVAL;
    if (layer < 0 || layer >= pool->L) return UNIPIN_ERANGE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lens, 4) ||
        !aligned(slot, 4))
        return UNIPIN_EALIGN;
    const int D = pool->D, H = pool->H;
    const bool dense = in.rstride == D && in.hstride == (long)rows * D && in.bstride == (long)H * rows * D &&
                       out.rstride == D && out.hstride == (long)rows * D && out.bstride == (long)H * rows * D;
    if (!dense) {
        // other layouts: bf16 only, rows at least D elements apart, every row 16-byte aligned
        // and every byte offset within 32 bits
        if (!bf16_kernels(pool)) return UNIPIN_EDTYPE;
        const RowLayout *ls[2] = {&in, &out};
        for (const RowLayout *l : ls) {
            if (l->rstride < D || l->rstride % 8 || l->hstride % 8 || l->bstride % 8 || l->hstride < 0 ||
                l->bstride < 0)
                return UNIPIN_EINVAL;
            if ((long long)rows * l->rstride * act_bytes(pool) >= 0x7fffffffLL) return UNIPIN_EINVAL;
        }
    }
    const int rpb = rows_per_block(pool, prefill);
    const long long blocks = (long long)B * H * ((rows + rpb - 1) / rpb);
    if (blocks > 0x7fffffffLL) return UNIPIN_EINVAL;
    unipin::AttnArgs a{};
    int rc = resolve_scale(scale, D, &a.c);
    if (rc) return rc;
    fill_pool_args(a, pool, layer);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lens = lens;
    a.slot = slot;
    a.B = B;
    a.rows = rows;
    a.len_limit = prefill ? rows : pool->n_max;
    a.tiles = (rows + rpb - 1) / rpb;
    a.xcd_remap = bf16_kernels(pool) && ((long long)B * H) % 8 == 0;
    a.in_bstride = in.bstride;
    a.in_hstride = in.hstride;
    a.in_rstride = in.rstride;
    a.out_bstride = out.bstride;
    a.out_hstride = out.hstride;
    a.out_rstride = out.rstride;
    if (unipin::device_status_word(&a.status) != hipSuccess) return UNIPIN_EHIP;
    return launch(a, pool, prefill, stream);
}

}  // namespace unipin

extern "C" {

int unipin_pool_create(unipin_pool_t **out, void *k_pool, void *v_pool, int L, int S, int H,
                       int n_max, int D, int dtype) {
    if (!out) return UNIPIN_EINVAL;
    *out = nullptr;
    if (!k_pool || !v_pool) return UNIPIN_EINVAL;
    if (L < 1 || S < 1 || H < 1 || n_max < 1 || !supported_d(D)) return UNIPIN_EINVAL;
    if (dtype != UNIPIN_FP32 && dtype != UNIPIN_BF16 && dtype != UNIPIN_FP8_E4M3) return UNIPIN_EDTYPE;
    if (dtype == UNIPIN_FP8_E4M3 && D != 64 && D != 128) return UNIPIN_EINVAL;
    if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return UNIPIN_EALIGN;
    const long long elems = (long long)L * S * H * n_max * D;
    if (elems / L / S / H / n_max != D || elems > (1LL << 46)) return UNIPIN_EINVAL;
    unipin_pool *p = new (std::nothrow) unipin_pool;
    if (!p) return UNIPIN_ENOMEM;
    p->gen = new (std::nothrow) std::atomic<uint64_t>[S];
    if (!p->gen) {
        delete p;
        return UNIPIN_ENOMEM;
    }
    for (int i = 0; i < S; ++i) p->gen[i].store(0, std::memory_order_relaxed);
    p->cursor.store(0, std::memory_order_relaxed);
    p->k = k_pool;
    p->v = v_pool;
    p->L = L;
    p->S = S;
    p->H = H;
    p->n_max = n_max;
    p->D = D;
    p->dtype = dtype;
    p->elem = dtype == UNIPIN_FP32 ? 4 : dtype == UNIPIN_BF16 ? 2 : 1;
    *out = p;
    return UNIPIN_OK;
}

int unipin_pool_destroy(unipin_pool_t *pool) {
    if (!pool) return UNIPIN_OK;
    delete[] pool->gen;
    delete pool;
    return UNIPIN_OK;
}

int unipin_pool_acquire(unipin_pool_t *pool, int32_t *slot, uint64_t *generation) {
    if (!pool || !slot) return UNIPIN_EINVAL;
    const uint64_t i = pool->cursor.fetch_add(1, std::memory_order_relaxed);
    const int32_t s = (int32_t)(i % (uint64_t)pool->S);
    const uint64_t g = pool->gen[s].fetch_add(1, std::memory_order_acq_rel) + 1;
    *slot = s;
    if (generation) *generation = g;
    return UNIPIN_OK;
}

int unipin_pool_generation(const unipin_pool_t *pool, int32_t slot, uint64_t *generation) {
    if (!pool || !generation) return UNIPIN_EINVAL;
    if (slot < 0 || slot >= pool->S) return UNIPIN_ERANGE;
    *generation = pool->gen[slot].load(std::memory_order_acquire);
    return UNIPIN_OK;
}

int unipin_pool_dims(const unipin_pool_t *pool, int *L, int *S, int *H, int *n_max, int *D,
                     int *dtype) {
    if (!pool) return UNIPIN_EINVAL;
    if (L) *L = pool->L;
    if (S) *S = pool->S;
    if (H) *H = pool->H;
    if (n_max) *n_max = pool->n_max;
    if (D) *D = pool->D;
    if (dtype) *dtype = pool->dtype;
    return UNIPIN_OK;
}

int unipin_prefill(const void *q, const void *k, const void *v, const int32_t *lens,
                   unipin_pool_t *pool, const int32_t *slot, int layer, int B, int n,
                   float scale, void *o, void *stream) {
    if (!pool || !q || !k || !v || !lens || !slot || !o) return UNIPIN_EINVAL;
    if (B < 1 || n < 1 || n > pool->n_max) return UNIPIN_EINVAL;
    const unipin::RowLayout dense{(long)pool->H * n * pool->D, (long)n * pool->D, pool->D};
    return unipin::attention_call(true, q, k, v, dense, o, dense, pool, slot, lens, layer, B, n, scale, stream);
}

int unipin_rank_decode(const void *qc, const void *kc, const void *vc,
                       const unipin_pool_t *pool, const int32_t *slot, const int32_t *lens,
                       int layer, int B, int k, float scale, void *oc, void *stream) {
    if (!pool || !qc || !kc || !vc || !lens || !slot || !oc) return UNIPIN_EINVAL;
    if (B < 1 || k < 1) return UNIPIN_EINVAL;
    const unipin::RowLayout dense{(long)pool->H * k * pool->D, (long)k * pool->D, pool->D};
    return unipin::attention_call(false, qc, kc, vc, dense, oc, dense, const_cast<unipin_pool_t *>(pool), slot, lens,
                                  layer, B, k, scale, stream);
}

int unipin_ar_decode(const void *q, const void *k, const void *v, unipin_pool_t *pool,
                     const int32_t *slot, const int32_t *lens, int layer, int B, float scale,
                     void *o, void *workspace, size_t workspace_bytes, void *stream) {
    if (!pool || !q || !k || !v || !lens || !slot || !o) return UNIPIN_EINVAL;
    if (B < 1) return UNIPIN_EINVAL;
    if (layer < 0 || layer >= pool->L) return UNIPIN_ERANGE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lens, 4) || !aligned(slot, 4))
        return UNIPIN_EALIGN;
    if ((long long)B * pool->H > 0x7fffffffLL) return UNIPIN_EINVAL;
    unipin::AttnArgs a{};
    int rc = resolve_scale(scale, pool->D, &a.c);
    if (rc) return rc;
    fill_pool_args(a, pool, layer);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lens = lens;
    a.slot = slot;
    a.B = B;
    a.rows = 1;
    a.len_limit = pool->n_max - 1;
    a.tiles = 1;
    const int kind = pool->dtype;
    int parts = 1;
    if (workspace) {
        if (!aligned(workspace, 16)) return UNIPIN_EALIGN;
        parts = unipin::ar_splits((long)B * pool->H, pool->n_max, pool->D, kind);
        if (workspace_bytes < unipin::ar_workspace_bytes((long)B * pool->H, parts, pool->D)) return UNIPIN_EINVAL;
    }
    if (unipin::device_status_word(&a.status) != hipSuccess) return UNIPIN_EHIP;
    const hipError_t e = unipin::launch_ar_decode(a, pool->D, kind, static_cast<float *>(workspace), parts,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? UNIPIN_OK : UNIPIN_EHIP;
}

size_t unipin_ar_decode_workspace_bytes(const unipin_pool_t *pool, int B) {
    if (!pool || B < 1) return 0;
    const long bh = (long)B * pool->H;
    return unipin::ar_workspace_bytes(bh, unipin::ar_splits(bh, pool->n_max, pool->D, pool->dtype),
                                      pool->D);
}

int unipin_device_status(void *stream, int *flags) {
    if (flags) *flags = 0;
    unsigned int *word = nullptr;
    if (unipin::device_status_word(&word) != hipSuccess) return UNIPIN_EHIP;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned int host = 0;
    if (hipStreamSynchronize(st) != hipSuccess) return UNIPIN_EHIP;
    if (hipMemcpy(&host, word, sizeof(host), hipMemcpyDeviceToHost) != hipSuccess) return UNIPIN_EHIP;
    if (host) {
        if (hipMemset(word, 0, sizeof(host)) != hipSuccess) return UNIPIN_EHIP;
    }
    if (flags) *flags = (int)host;
    return host ? UNIPIN_EDEVICE : UNIPIN_OK;
}

const char *unipin_strerror(int status) {
    switch (status) {
        case UNIPIN_OK: return "ok";
        case UNIPIN_EINVAL: return "invalid argument (null pointer, size or head dim)";
        case UNIPIN_ERANGE: return "layer or slot out of range";
        case UNIPIN_EDTYPE: return "unsupported element type";
        case UNIPIN_EALIGN: return "tensor pointer not 16-byte aligned";
        case UNIPIN_EDEVICE: return "a kernel skipped a user with an invalid slot or length";
        case UNIPIN_EHIP: return "HIP runtime error";
        case UNIPIN_ENOMEM: return "out of host memory";
        default: return "unknown status";
    }
}

int unipin_version(void) { return kVersion; }

}  // extern "C"
