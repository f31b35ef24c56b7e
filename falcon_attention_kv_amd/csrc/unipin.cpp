// C ABI of the library (include/unipin.h): pool descriptor, round-robin slot hand-out,
// host-side argument checks, and dispatch to the HIP kernels by element type and head
// dimension.  Nothing here allocates device memory; the only HIP calls are kernel
// launches (prefill, rank decode, autoregressive step, the flag exchange) and the
// status read-back.
#include "unipin.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>

#include "attn_launch.h"
#include "pool_internal.h"

namespace {

constexpr int kVersion = 10100;  // 1.1.0: folded LayerNorm weights in unipin_block_weights_t

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte offsets inside one (user, head)'s rows and inside one pool slot row block are
// 32-bit in the kernels (buffer record counts, scalar offsets).
constexpr long long kMaxOffset = 0x7fffffffLL;

// Entries of the per-device flag arrays, one per live descriptor; an entry that served
// an earlier descriptor may still hold that descriptor's flags, so its new owner clears
// it before its first kernel.
std::mutex g_index_mu;
bool g_index_used[unipin::kMaxPools];
bool g_index_dirty[unipin::kMaxPools];

int take_flag_index(bool *dirty) {
    std::lock_guard<std::mutex> lock(g_index_mu);
    for (int i = 0; i < unipin::kMaxPools; ++i)
        if (!g_index_used[i]) {
            g_index_used[i] = true;
            *dirty = g_index_dirty[i];
            g_index_dirty[i] = true;
            return i;
        }
    return -1;
}

void release_flag_index(int i) {
    std::lock_guard<std::mutex> lock(g_index_mu);
    if (i >= 0 && i < unipin::kMaxPools) g_index_used[i] = false;
}

bool supported_d(int D) { return D == 32 || D == 64 || D == 128; }

// Resolves the score scale: non-positive or NaN means 1/sqrt(D); infinity is rejected.
int resolve_scale(float scale, int D, unipin::AttnArgs &a) {
    if (std::isinf(scale)) return UNIPIN_EINVAL;
    const double s = (std::isnan(scale) || scale <= 0.f) ? 1.0 / std::sqrt((double)D) : (double)scale;
    a.c = (float)(s * 1.4426950408889634);  // scale * log2(e)
    a.scale64 = s;
    return UNIPIN_OK;
}

// bf16 kernels serve bf16 and E4M3 pools (bf16 activations); fp32 pools the fp32 ones.
bool bf16_kernels(const unipin_pool *pool) { return pool->dtype != UNIPIN_FP32; }

// bytes of one activation element (q, k, v, o) for this pool
int act_bytes(const unipin_pool *pool) { return pool->dtype == UNIPIN_FP32 ? 4 : 2; }

}  // namespace

namespace unipin {

int pool_kernel_prologue(unipin_pool *pool, hipStream_t stream, unsigned int **flag_word) {
    if (pool->clear_flags.load(std::memory_order_acquire) && pool->clear_flags.exchange(false)) {
        if (clear_pool_flags(pool->flag_index, stream) != hipSuccess) {
            pool->clear_flags.store(true);
            return UNIPIN_EHIP;
        }
    }
    return pool_flag_word(pool->flag_index, flag_word) == hipSuccess ? UNIPIN_OK : UNIPIN_EHIP;
}

}  // namespace unipin

namespace {

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

DecodeSplit decode_split_plan(const ::unipin_pool *pool, int B, int k) {
    // Histories shorter than 16 tiles (1024 keys) take the one-pass kernel: their decode
    // is short enough that the merge's launch and the parts' states cost more than the
    // split gains (measured: 0.88-0.90x at 512 keys).  A part takes at least four 64-key
    // tiles, and each part costs a header and an fp32 state of its 256 rows, written and
    // merged again: as many bytes as four bf16 K/V tiles at D = 64.  So the split pays
    // only while the candidate tiles (items) are few next to the history's tiles: at
    // most 2 per tile at D <= 64 and 3 per tile at D = 128 (one workgroup per CU there),
    // the break-even points of a sweep over requests, history and candidate counts
    // (beyond them the split took 0.5-0.9x of the one-pass time, inside them 1.1-2.4x).
    // The decode keeps two workgroups per CU resident at D <= 64 and one at D = 128 (256
    // CUs): the split also needs the candidate tiles to fill at most half of those, and
    // gives each tile's history as many parts as fit in one round of them.  The plan
    // counts on histories up to n_max (the lengths are on the device); parts past a
    // shorter history leave at once.
    constexpr int kMinPartTiles = 4;
    DecodeSplit p{1, 0, 0};
    if (!pool || B < 1 || k < 1 || !bf16_kernels(pool)) return p;
    const int rpb = bf16_decode_rows_per_item(pool->D);
    const long items = (long)B * pool->H * ((k + rpb - 1) / rpb);
    const long resident = pool->D <= 64 ? 512 : 256;
    if (items * 2 > resident) return p;
    const int hist_tiles = (pool->n_max + 63) / 64;
    if (hist_tiles < 16) return p;
    if (items > (pool->D <= 64 ? 2L : 3L) * hist_tiles) return p;
    int parts = (int)std::min<long>(resident / items, hist_tiles / kMinPartTiles);
    if (parts < 2) return p;
    const int part_tiles = (hist_tiles + parts - 1) / parts;
    parts = (hist_tiles + part_tiles - 1) / part_tiles;
    if (parts < 2) return p;
    p.parts = parts;
    p.part_tiles = part_tiles;
    p.bytes = (size_t)items * parts * rpb * (pool->D + 2) * sizeof(float);
    return p;
}

int attention_call(bool prefill, const void *q, const void *k, const void *v, RowLayout in, void *o, RowLayout out,
                   ::unipin_pool *pool, const int32_t *slot, const int32_t *lens, int layer, int B, int rows,
                   float scale, void *stream, float *part_state, int parts, int part_tiles) {
    if (!pool || !q || !k || !v || !lens || !slot || !o) return UNIPIN_EINVAL;
    if (B < 1 || rows < 1 || (prefill && rows > pool->n_max)) return UNIPIN_EINVAL;
    if (layer < 0 || layer >= pool->L) return UNIPIN_ERANGE;
    if (prefill && pool->readonly) return UNIPIN_EPERM;
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
        }
    }
    // one (user, head)'s rows of every operand within 32-bit byte offsets
    const RowLayout *ls[2] = {&in, &out};
    for (const RowLayout *l : ls)
        if ((long long)rows * l->rstride * act_bytes(pool) >= kMaxOffset) return UNIPIN_EINVAL;
    const int rpb = rows_per_block(pool, prefill);
    const long long blocks = (long long)B * H * ((rows + rpb - 1) / rpb);
    if (blocks > 0x7fffffffLL) return UNIPIN_EINVAL;
    unipin::AttnArgs a{};
    int rc = resolve_scale(scale, D, a);
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
    rc = pool_kernel_prologue(pool, static_cast<hipStream_t>(stream), &a.status);
    if (rc) return rc;
    if (!prefill && part_state && parts >= 2 && bf16_kernels(pool)) {
        a.parts = parts;
        a.part_tiles = part_tiles;
        a.part_state = part_state;
        return launch_decode_split_bf16(a, D, pool->dtype == UNIPIN_FP8_E4M3, static_cast<hipStream_t>(stream)) ==
                       hipSuccess
                   ? UNIPIN_OK
                   : UNIPIN_EHIP;
    }
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
    const int elem = dtype == UNIPIN_FP32 ? 4 : dtype == UNIPIN_BF16 ? 2 : 1;
    const long long elems = (long long)L * S * H * n_max * D;
    if (elems / L / S / H / n_max != D || elems > (1LL << 46)) return UNIPIN_EINVAL;
    if ((long long)n_max * D * elem >= kMaxOffset) return UNIPIN_EINVAL;   // one slot row block
    unipin_pool *p = new (std::nothrow) unipin_pool;
    if (!p) return UNIPIN_ENOMEM;
    p->ring_own = new (std::nothrow) uint64_t[(size_t)S + 1];
    if (!p->ring_own) {
        delete p;
        return UNIPIN_ENOMEM;
    }
    bool dirty = false;
    p->flag_index = take_flag_index(&dirty);
    if (p->flag_index < 0) {
        delete[] p->ring_own;
        delete p;
        return UNIPIN_ENOMEM;
    }
    p->clear_flags.store(dirty, std::memory_order_relaxed);
    for (int i = 0; i <= S; ++i) p->ring_own[i] = 0;
    p->ring = p->ring_own;
    p->k = k_pool;
    p->v = v_pool;
    p->L = L;
    p->S = S;
    p->H = H;
    p->n_max = n_max;
    p->D = D;
    p->dtype = dtype;
    p->elem = elem;
    p->readonly = false;
    p->shm_addr = nullptr;
    p->shm_bytes = 0;
    p->shm_name[0] = 0;
    p->shm_owner = false;
    p->ipc_k = p->ipc_v = nullptr;
    *out = p;
    return UNIPIN_OK;
}

int unipin_pool_destroy(unipin_pool_t *pool) {
    if (!pool) return UNIPIN_OK;
    unipin::pool_share_release(pool);
    release_flag_index(pool->flag_index);
    delete[] pool->ring_own;
    delete pool;
    return UNIPIN_OK;
}

int unipin_pool_acquire(unipin_pool_t *pool, int32_t *slot, uint64_t *generation) {
    if (!pool || !slot) return UNIPIN_EINVAL;
    if (pool->readonly) return UNIPIN_EPERM;
    const uint64_t i = __atomic_fetch_add(&pool->ring[0], 1, __ATOMIC_RELAXED);
    const int32_t s = (int32_t)(i % (uint64_t)pool->S);
    const uint64_t g = __atomic_add_fetch(&pool->ring[1 + s], 1, __ATOMIC_ACQ_REL);
    *slot = s;
    if (generation) *generation = g;
    return UNIPIN_OK;
}

uint64_t unipin_pool_generation(const unipin_pool_t *pool, int32_t slot) {
    if (!pool || slot < 0 || slot >= pool->S) return 0;
    return unipin::ring_load(&pool->ring[1 + slot]);
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

size_t unipin_rank_decode_workspace_bytes(const unipin_pool_t *pool, int B, int k) {
    return unipin::decode_split_plan(pool, B, k).bytes;
}

int unipin_rank_decode_split(const void *qc, const void *kc, const void *vc, const unipin_pool_t *pool,
                             const int32_t *slot, const int32_t *lens, int layer, int B, int k, float scale,
                             void *oc, void *workspace, size_t workspace_bytes, void *stream) {
    if (!pool || !qc || !kc || !vc || !lens || !slot || !oc) return UNIPIN_EINVAL;
    if (B < 1 || k < 1) return UNIPIN_EINVAL;
    const unipin::RowLayout dense{(long)pool->H * k * pool->D, (long)k * pool->D, pool->D};
    const unipin::DecodeSplit plan = unipin::decode_split_plan(pool, B, k);
    float *ws = nullptr;
    if (workspace && plan.parts >= 2) {
        if (!aligned(workspace, 16)) return UNIPIN_EALIGN;
        if (workspace_bytes < plan.bytes) return UNIPIN_EINVAL;
        ws = static_cast<float *>(workspace);
    }
    return unipin::attention_call(false, qc, kc, vc, dense, oc, dense, const_cast<unipin_pool_t *>(pool), slot, lens,
                                  layer, B, k, scale, stream, ws, ws ? plan.parts : 1, plan.part_tiles);
}

}  // extern "C"

namespace {

// The autoregressive step's shared body.  ws: the split path's state buffer (null: one
// pass), or, with own_scratch, the library's static array.
int ar_decode_call(const void *q, const void *k, const void *v, unipin_pool_t *pool, const int32_t *slot,
                   const int32_t *lens, int layer, int B, float scale, void *o, void *workspace,
                   size_t workspace_bytes, bool own_scratch, void *stream) {
    if (!pool || !q || !k || !v || !lens || !slot || !o) return UNIPIN_EINVAL;
    if (B < 1) return UNIPIN_EINVAL;
    if (layer < 0 || layer >= pool->L) return UNIPIN_ERANGE;
    if (pool->readonly) return UNIPIN_EPERM;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lens, 4) || !aligned(slot, 4))
        return UNIPIN_EALIGN;
    if ((long long)B * pool->H > 0x7fffffffLL) return UNIPIN_EINVAL;
    unipin::AttnArgs a{};
    int rc = resolve_scale(scale, pool->D, a);
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
    float *ws = nullptr;
    if (own_scratch) {
        parts = unipin::ar_splits((long)B * pool->H, pool->n_max, pool->D, kind);
        if (unipin::ar_workspace_bytes((long)B * pool->H, parts, pool->D) > unipin::ar_scratch_bytes())
            return UNIPIN_ESCRATCH;
        if (parts > 1 && unipin::ar_scratch(&ws) != hipSuccess) return UNIPIN_EHIP;
    } else if (workspace) {
        if (!aligned(workspace, 16)) return UNIPIN_EALIGN;
        parts = unipin::ar_splits((long)B * pool->H, pool->n_max, pool->D, kind);
        if (workspace_bytes < unipin::ar_workspace_bytes((long)B * pool->H, parts, pool->D)) return UNIPIN_EINVAL;
        ws = static_cast<float *>(workspace);
    }
    rc = unipin::pool_kernel_prologue(pool, static_cast<hipStream_t>(stream), &a.status);
    if (rc) return rc;
    const hipError_t e =
        kind == UNIPIN_FP32
            ? unipin::launch_ar_decode_fp32(a, pool->D, static_cast<hipStream_t>(stream))
            : unipin::launch_ar_decode(a, pool->D, kind, ws, parts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? UNIPIN_OK : UNIPIN_EHIP;
}

}  // namespace

extern "C" {

int unipin_ar_decode(const void *q, const void *k, const void *v, unipin_pool_t *pool,
                     const int32_t *slot, const int32_t *lens, int layer, int B, float scale,
                     void *o, void *workspace, size_t workspace_bytes, void *stream) {
    return ar_decode_call(q, k, v, pool, slot, lens, layer, B, scale, o, workspace, workspace_bytes, false, stream);
}

int unipin_ar_decode_noalloc(const void *q, const void *k, const void *v, unipin_pool_t *pool,
                             const int32_t *slot, const int32_t *lens, int layer, int B, float scale,
                             void *o, void *stream) {
    return ar_decode_call(q, k, v, pool, slot, lens, layer, B, scale, o, nullptr, 0, true, stream);
}

size_t unipin_ar_decode_workspace_bytes(const unipin_pool_t *pool, int B) {
    if (!pool || B < 1) return 0;
    const long bh = (long)B * pool->H;
    return unipin::ar_workspace_bytes(bh, unipin::ar_splits(bh, pool->n_max, pool->D, pool->dtype),
                                      pool->D);
}

int unipin_pool_status(unipin_pool_t *pool, void *stream, int *flags) {
    if (flags) *flags = 0;
    if (!pool) return UNIPIN_EINVAL;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // a reused entry's earlier flags are dropped by the exchange below like any others;
    // they belong to no call on this pool only if nothing ran on it yet
    const bool stale = pool->clear_flags.exchange(false);
    unsigned int host = 0;
    if (unipin::take_pool_flags(pool->flag_index, st, &host) != hipSuccess) {
        if (stale) pool->clear_flags.store(true);
        return UNIPIN_EHIP;
    }
    if (stale) host = 0;
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
        case UNIPIN_ENOMEM: return "out of host memory or pool descriptors";
        case UNIPIN_EPERM: return "the pool is imported read-only (rank decode only)";
        case UNIPIN_EIO: return "a pool share file or shared page could not be written, read or mapped";
        case UNIPIN_ESCRATCH: return "the call needs more scratch than the library's static array holds";
        default: return "unknown status";
    }
}

int unipin_version(void) { return kVersion; }

}  // extern "C"
