// One autoregressive step of the retrieval side, for gfx950: each (user, head) has one
// new query token that attends to the N rows already in its pool slot (the history and
// the tokens generated before) and to itself, and whose K/V are stored at row N.
//
// Every K/V byte is used by one query, so the step is bound by HBM bandwidth, and the
// matrix cores have nothing to do (a single query row).  One workgroup per (user, head):
// 8 waves take the slot's rows in 64-key chunks in turn (wave w: chunks w, w+8, ...).
// A wave loads a chunk's K and V rows with 16-byte lane loads, R = row bytes / 16 lanes
// per row and 64 / R rows per wave-wide load, so that every load instruction reads
// whole contiguous rows.  A lane dots its 16 bytes of a key row with the same 16 bytes
// of the query (bf16 pairs: exact products, fp32 sums) and the R lanes of a row add up
// their parts with cross-lane exchanges.  The softmax is the online form in fp32 with
// base-2 exponentials (scale*log2(e) applied to the fp32 score); the value rows are
// weighted in fp32.  At the end the waves' partial states (running max, sum and
// accumulator) are merged through LDS, the new token enters as the last key, and the
// output row is normalised and stored; the new K/V row is copied into the slot.
//
// An E4M3 pool (bf16 activations) halves the row bytes: a lane's 16-byte load then
// holds 16 codes, which it decodes to fp32 and dots with the matching 32 bytes of the
// bf16 query; the new token's K/V row is stored as codes (clamped to +-448, rounded to
// nearest with ties to even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attn_launch.h"
#include "e4m3.h"

namespace unipin {

// The split path's part states for callers that cannot allocate
// (unipin_ar_decode_noalloc): one array per device, held until the process ends, shared
// by every such call on that device.  Its size covers every shape the split rule makes:
// at most 256 (user, head, part) states of D + 4 floats, D <= 128.
constexpr size_t kArScratchBytes = (size_t)256 << 10;
static __device__ __align__(256) float scratch[kArScratchBytes / sizeof(float)];

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

template <typename T>
struct Elem;
template <>
struct Elem<bf16> {
    static constexpr int kPer16 = 8;   // elements per 16 bytes
};
template <>
struct Elem<float> {
    static constexpr int kPer16 = 4;
};

// The 16 bytes x as floats (exact for both element types).
template <typename T>
__device__ __forceinline__ void widen(const u32x4 &x, float (&f)[Elem<T>::kPer16]) {
    if constexpr (Elem<T>::kPer16 == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(x[i] << 16);
            f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
    }
}

// Dot product of two 16-byte pieces, fp32 sum of exact products.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4 &a, const u32x4 &b) {
    float s = 0.f;
    if constexpr (Elem<T>::kPer16 == 8) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const bf16x2 pa = {av[i], av[i + 1]}, pb = {bv[i], bv[i + 1]};
            s = __builtin_amdgcn_fdot2_f32_bf16(pa, pb, s, false);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), s);
    }
    return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Sum (or max) over the lanes whose ids differ only in the bits of [lo, 64).
template <int LO>
__device__ __forceinline__ float xsum(float x) {
#pragma unroll
    for (int m = LO; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}
template <int LO>
__device__ __forceinline__ float xmax(float x) {
#pragma unroll
    for (int m = LO; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
// Sum over the lanes whose ids differ only in the bits below HI.
template <int HI>
__device__ __forceinline__ float lowsum(float x) {
#pragma unroll
    for (int m = 1; m < HI; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// Element kind: activations (q, k, v, o) of type T; the pool holds T as well, or E4M3
// codes (P8).  A lane's 16-byte pool load holds PER elements; the matching activation
// piece is AB = PER * sizeof(T) bytes (16, or 32 for an E4M3 pool).
template <typename T, bool P8>
struct Kind {
    using Act = T;
    static constexpr bool kP8 = P8;
    static constexpr int PB = P8 ? 1 : (int)sizeof(T);   // pool bytes per element
    static constexpr int PER = 16 / PB;
    static constexpr int AB = PER * (int)sizeof(T);
    static_assert(!P8 || sizeof(T) == 2, "an E4M3 pool pairs with bf16 activations");
};

// One lane's piece of an activation row (a query, key or value of the new token).
template <typename K>
struct ActPiece {
    u32x4 x[K::AB / 16];
};

template <typename K, int D>
__device__ __forceinline__ ActPiece<K> load_act(const typename K::Act *row, int sub) {
    const __amdgpu_buffer_rsrc_t r = rsrc(row, (uint32_t)(D * sizeof(typename K::Act)));
    ActPiece<K> a;
#pragma unroll
    for (int j = 0; j < K::AB / 16; ++j) a.x[j] = load16(r, sub * K::AB + 16 * j);
    return a;
}

// The lane's query piece dotted with its 16 bytes of a pool row.
template <typename K>
__device__ __forceinline__ float dot_pool(const ActPiece<K> &q, const u32x4 &kx) {
    if constexpr (!K::kP8) {
        return dot16<typename K::Act>(q.x[0], kx);
    } else {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float kf[4], qf[8];
            e4m3x4_to_f32(kx[w], kf);
            widen<bf16>(q.x[w / 2], qf);
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_fmaf(qf[(w % 2) * 4 + e], kf[e], s);
        }
        return s;
    }
}

// The lane's query piece dotted with the same piece of another activation row.
template <typename K>
__device__ __forceinline__ float dot_act(const ActPiece<K> &q, const ActPiece<K> &k) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < K::AB / 16; ++j) s += dot16<typename K::Act>(q.x[j], k.x[j]);
    return s;
}

template <typename K>
__device__ __forceinline__ void widen_pool(const u32x4 &x, float (&f)[K::PER]) {
    if constexpr (!K::kP8) {
        widen<typename K::Act>(x, f);
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float g[4];
            e4m3x4_to_f32(x[w], g);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * w + e] = g[e];
        }
    }
}

template <typename K>
__device__ __forceinline__ void widen_act(const ActPiece<K> &a, float (&f)[K::PER]) {
    constexpr int E = 16 / (int)sizeof(typename K::Act);   // elements per 16 bytes
#pragma unroll
    for (int j = 0; j < K::AB / 16; ++j) {
        float g[E];
        widen<typename K::Act>(a.x[j], g);
#pragma unroll
        for (int e = 0; e < E; ++e) f[j * E + e] = g[e];
    }
}

// Geometry of one (element kind, head dim): a pool row is R lanes of 16 bytes, a
// wave-wide load covers RPI rows, a chunk (one wave's unit of work) is LPC loads = CH
// rows.
template <typename K, int D>
struct Geo {
    static constexpr int ROW = D * K::PB;
    static constexpr int R = ROW / 16;
    static constexpr int RPI = 64 / R;
    static constexpr int PER = K::PER;
    static constexpr int LPC = RPI >= 4 ? 64 / RPI : 16;
    static constexpr int CH = LPC * RPI;
    static_assert(R >= 1 && R <= 64 && 64 % R == 0, "row must split into 16-byte lanes");
};

// Online-softmax state of one lane: running max m (log2 domain), running sum l over the
// rows this lane's row group saw, and the weighted sum of its 16-byte piece of V.
template <int PER>
struct State {
    float m, l, acc[PER];
    __device__ void clear() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    }
};

// The wave folds chunks c_first, c_first + stride, ... below c_end (chunk c = rows
// [c*CH, c*CH + CH), rows >= N masked) into st.
template <typename K, int D>
__device__ __forceinline__ void scan_chunks(State<Geo<K, D>::PER> &st, __amdgpu_buffer_rsrc_t rk,
                                            __amdgpu_buffer_rsrc_t rv, const ActPiece<K> &qx, float c, int N,
                                            int c_first, int c_end, int stride, int sub, int grp) {
    using G = Geo<K, D>;
    for (int ch = c_first; ch < c_end; ch += stride) {
        const int c0 = ch * G::CH;
        u32x4 kx[G::LPC], vx[G::LPC];
#pragma unroll
        for (int i = 0; i < G::LPC; ++i) {
            const uint32_t off = (uint32_t)(c0 + i * G::RPI + grp) * G::ROW + sub * 16;
            kx[i] = load16(rk, off);
            vx[i] = load16(rv, off);
        }
        float sc[G::LPC];
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < G::LPC; ++i) {
            const float d = lowsum<G::R>(dot_pool<K>(qx, kx[i]));
            sc[i] = c0 + i * G::RPI + grp < N ? d * c : -INFINITY;
            cm = fmaxf(cm, sc[i]);
        }
        cm = xmax<G::R>(cm);   // chunk max over the wave (finite: row c0 < N is valid)
        const float mn = fmaxf(st.m, cm);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
        st.m = mn;
        st.l *= alpha;
#pragma unroll
        for (int e = 0; e < G::PER; ++e) st.acc[e] *= alpha;
#pragma unroll
        for (int i = 0; i < G::LPC; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - st.m);
            st.l += p;   // the R lanes of a row hold the same weight; only rows are summed later
            float vf[G::PER];
            widen_pool<K>(vx[i], vf);
#pragma unroll
            for (int e = 0; e < G::PER; ++e) st.acc[e] = __builtin_fmaf(p, vf[e], st.acc[e]);
        }
    }
}

// Sums the wave's row groups (lanes with the same sub hold the same dims) and leaves the
// wave's state in part[wave]: accumulator [0, D), max at D, sum at D + 1.
template <typename K, int D, int WAVES>
__device__ __forceinline__ void publish(State<Geo<K, D>::PER> &st, float (*part)[D + 2], int wave, int sub,
                                        int grp) {
    using G = Geo<K, D>;
    st.l = xsum<G::R>(st.l);
#pragma unroll
    for (int e = 0; e < G::PER; ++e) st.acc[e] = xsum<G::R>(st.acc[e]);
    if (grp == 0) {
#pragma unroll
        for (int e = 0; e < G::PER; ++e) part[wave][sub * G::PER + e] = st.acc[e];
        if (sub == 0) {
            part[wave][D] = st.m;
            part[wave][D + 1] = st.l;
        }
    }
}

// Flags and skips an invalid user; true when (b) must be skipped.
__device__ __forceinline__ bool invalid_user(const AttnArgs &a, int b, int N, int s, bool flag) {
    const bool bad_len = N < 0 || N > a.len_limit;
    const bool bad_slot = s < 0 || s >= a.S;
    if ((bad_len || bad_slot) && flag)
        atomicOr(a.status, (bad_len ? kFlagBadLen : 0u) | (bad_slot ? kFlagBadSlot : 0u));
    return bad_len || bad_slot;
}

// The last step shared by both paths: the new token enters as one more key with weight
// exp2(snew - mt); out already holds the other keys' weighted values rescaled to mt and
// lt their weight sum.  Stores the output row and the token's K/V row into slot row N
// (as it is, or as E4M3 codes).  Lanes with grp == 0 (one per pool piece) store.
template <typename K, int D>
__device__ __forceinline__ void finish(const AttnArgs &a, long bh, long slot_off, int N, const ActPiece<K> &knew,
                                       const ActPiece<K> &vnew, float pnew, float lt, float (&out)[Geo<K, D>::PER],
                                       int sub, int grp) {
    using G = Geo<K, D>;
    using T = typename K::Act;
    float vf[G::PER];
    widen_act<K>(vnew, vf);
#pragma unroll
    for (int e = 0; e < G::PER; ++e) out[e] = __builtin_fmaf(pnew, vf[e], out[e]);
    const float inv = 1.f / (lt + pnew);
    if (grp == 0) {
        char *orow = reinterpret_cast<char *>(static_cast<T *>(a.o) + bh * D) + sub * K::AB;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int j = 0; j < K::AB / 16; ++j) {
                u32x4 ox;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16x2 pr = {(bf16)(out[8 * j + 2 * i] * inv), (bf16)(out[8 * j + 2 * i + 1] * inv)};
                    ox[i] = __builtin_bit_cast(uint32_t, pr);
                }
                *reinterpret_cast<u32x4 *>(orow + 16 * j) = ox;
            }
        } else {
            u32x4 ox;
#pragma unroll
            for (int i = 0; i < 4; ++i) ox[i] = __float_as_uint(out[i] * inv);
            *reinterpret_cast<u32x4 *>(orow) = ox;
        }
        char *dk = static_cast<char *>(a.pool_k) + (slot_off + (long)N * D) * K::PB + sub * 16;
        char *dv = static_cast<char *>(a.pool_v) + (slot_off + (long)N * D) * K::PB + sub * 16;
        if constexpr (K::kP8) {
            *reinterpret_cast<u32x4 *>(dk) = e4m3x16_from_bf16x16(knew.x[0], knew.x[1]);
            *reinterpret_cast<u32x4 *>(dv) = e4m3x16_from_bf16x16(vnew.x[0], vnew.x[1]);
        } else {
            // bit for bit
            *reinterpret_cast<u32x4 *>(dk) = knew.x[0];
            *reinterpret_cast<u32x4 *>(dv) = vnew.x[0];
        }
    }
}

// One pass per (user, head): kWaves waves take the slot's chunks in turn, then wave 0
// merges their states with the new token.
template <typename K, int D>
__global__ void __launch_bounds__(kThreads) ar_decode_kernel(AttnArgs a) {
    using G = Geo<K, D>;
    using T = typename K::Act;
    __shared__ float part[kWaves][D + 2];

    const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int sub = lane % G::R, grp = lane / G::R;
    const long bh = (long)b * a.H + h;
    // the token's own rows do not depend on the slot: q for every wave, and k, v for wave
    // 0 (which merges at the end), all in the first round trip
    const ActPiece<K> qx = load_act<K, D>(static_cast<const T *>(a.q) + bh * D, sub);
    ActPiece<K> knew{}, vnew{};
    if (wave == 0) {
        knew = load_act<K, D>(static_cast<const T *>(a.k) + bh * D, sub);
        vnew = load_act<K, D>(static_cast<const T *>(a.v) + bh * D, sub);
    }
    const int N = a.lens[b];
    const int s = a.slot[b];
    if (invalid_user(a, b, N, s, threadIdx.x == 0 && h == 0)) return;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;   // in elements
    const char *pk = static_cast<const char *>(a.pool_k) + slot_off * K::PB;
    const char *pv = static_cast<const char *>(a.pool_v) + slot_off * K::PB;
    const __amdgpu_buffer_rsrc_t rk = rsrc(pk, (uint32_t)N * G::ROW);   // rows >= N read as zero
    const __amdgpu_buffer_rsrc_t rv = rsrc(pv, (uint32_t)N * G::ROW);

    State<G::PER> st;
    st.clear();
    scan_chunks<K, D>(st, rk, rv, qx, a.c, N, wave, (N + G::CH - 1) / G::CH, kWaves, sub, grp);
    publish<K, D, kWaves>(st, part, wave, sub, grp);
    __syncthreads();
    if (wave != 0) return;

    const float snew = lowsum<G::R>(dot_act<K>(qx, knew)) * a.c;
    float mt = snew;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, part[w][D]);
    float lt = 0.f, out[G::PER];
#pragma unroll
    for (int e = 0; e < G::PER; ++e) out[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(part[w][D] - mt);   // 0 for a wave that saw no row
        lt = __builtin_fmaf(wt, part[w][D + 1], lt);
#pragma unroll
        for (int e = 0; e < G::PER; ++e) out[e] = __builtin_fmaf(wt, part[w][sub * G::PER + e], out[e]);
    }
    finish<K, D>(a, bh, slot_off, N, knew, vnew, __builtin_amdgcn_exp2f(snew - mt), lt, out, sub, grp);
}

// Split-K across workgroups: a (user, head) with nc chunks cuts them into
// ceil(nc / cps) parts of cps = ceil(nc / P) chunks; part p is one workgroup.
__device__ __forceinline__ int split_chunks(int nc, int P) { return (nc + P - 1) / P; }

// Pass 1 of the split path: workgroup (bh, p) folds its part's chunks and writes the
// part's state (accumulator, max, sum) to ws[(bh * P + p) * (D + 4)].
template <typename K, int D>
__global__ void __launch_bounds__(kThreads) ar_split_kernel(AttnArgs a, float *ws, int P) {
    using G = Geo<K, D>;
    using T = typename K::Act;
    __shared__ float part[kWaves][D + 2];

    const long bh = blockIdx.x / P;
    const int p = blockIdx.x % P;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int sub = lane % G::R, grp = lane / G::R;
    const ActPiece<K> qx = load_act<K, D>(static_cast<const T *>(a.q) + bh * D, sub);   // slot-independent
    const int N = a.lens[b];
    const int s = a.slot[b];
    if (invalid_user(a, b, N, s, threadIdx.x == 0 && h == 0 && p == 0)) return;
    const int nc = (N + G::CH - 1) / G::CH;
    const int cps = split_chunks(nc, P);
    const int c_begin = p * cps, c_end = min(nc, c_begin + cps);
    if (c_begin >= c_end) return;   // this part is empty: the merge pass skips it too
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    const __amdgpu_buffer_rsrc_t rk =
        rsrc(static_cast<const char *>(a.pool_k) + slot_off * K::PB, (uint32_t)N * G::ROW);
    const __amdgpu_buffer_rsrc_t rv =
        rsrc(static_cast<const char *>(a.pool_v) + slot_off * K::PB, (uint32_t)N * G::ROW);

    State<G::PER> st;
    st.clear();
    scan_chunks<K, D>(st, rk, rv, qx, a.c, N, c_begin + wave, c_end, kWaves, sub, grp);
    publish<K, D, kWaves>(st, part, wave, sub, grp);
    __syncthreads();
    if (wave != 0) return;

    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, part[w][D]);   // finite: chunk c_begin has rows
    float lt = 0.f, out[G::PER];
#pragma unroll
    for (int e = 0; e < G::PER; ++e) out[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(part[w][D] - mt);
        lt = __builtin_fmaf(wt, part[w][D + 1], lt);
#pragma unroll
        for (int e = 0; e < G::PER; ++e) out[e] = __builtin_fmaf(wt, part[w][sub * G::PER + e], out[e]);
    }
    float *dst = ws + ((long)bh * P + p) * (D + 4);
    if (grp == 0) {
#pragma unroll
        for (int e = 0; e < G::PER; ++e) dst[sub * G::PER + e] = out[e];
        if (sub == 0) {
            dst[D] = mt;
            dst[D + 1] = lt;
        }
    }
}

// Pass 2 of the split path: one wave per (user, head) merges the non-empty parts with
// the new token, stores the output row and the token's K/V row.  Lane p holds part p's
// max and sum (at most 64 parts); the accumulators are read by the lane groups in
// rounds of 4 RPI parts, whose loads overlap.
template <typename K, int D>
__global__ void __launch_bounds__(64) ar_merge_kernel(AttnArgs a, const float *ws, int P) {
    using G = Geo<K, D>;
    using T = typename K::Act;
    constexpr int SD = D + 4;   // floats per part state
    const long bh = blockIdx.x;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int lane = threadIdx.x;
    const int sub = lane % G::R, grp = lane / G::R;
    // the token's rows do not depend on the slot: their loads go out first
    const ActPiece<K> qx = load_act<K, D>(static_cast<const T *>(a.q) + bh * D, sub);
    const ActPiece<K> knew = load_act<K, D>(static_cast<const T *>(a.k) + bh * D, sub);
    const ActPiece<K> vnew = load_act<K, D>(static_cast<const T *>(a.v) + bh * D, sub);
    // an invalid user (flagged by pass 1) merges nothing and stores nothing; no early
    // exit, so that the loads above are not held back behind the check
    const bool ok = !invalid_user(a, b, a.lens[b], a.slot[b], false);
    const int N = ok ? a.lens[b] : 0;
    const long slot_off = ok ? ((long)a.slot[b] * a.H + h) * (long)a.n_max * D : 0;
    const int nc = (N + G::CH - 1) / G::CH;
    const int parts = nc == 0 ? 0 : (nc + split_chunks(nc, P) - 1) / split_chunks(nc, P);
    const float *src = ws + (long)bh * P * SD;
    const float mp = lane < parts ? src[lane * SD + D] : -INFINITY;
    const float lp = lane < parts ? src[lane * SD + D + 1] : 0.f;
    const float snew = lowsum<G::R>(dot_act<K>(qx, knew)) * a.c;
    const float mt = fmaxf(snew, xmax<1>(mp));
    const float wp = __builtin_amdgcn_exp2f(mp - mt);   // 0 past the last part
    const float lt = xsum<1>(wp * lp);
    // The parts' accumulators are spread over the wave's RPI lane groups (the lanes of a
    // group cover one row's dims), four parts per group per round, so that up to 4 RPI
    // parts cost one round trip; the groups' sums are added at the end.
    float out[G::PER];
#pragma unroll
    for (int e = 0; e < G::PER; ++e) out[e] = 0.f;
    for (int p0 = 0; p0 < parts; p0 += 4 * G::RPI) {
        float x[4][G::PER];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = p0 + j * G::RPI + grp;
            const float *pp = src + (long)min(pi, parts - 1) * SD + sub * G::PER;
#pragma unroll
            for (int e = 0; e < G::PER; ++e) x[j][e] = pp[e];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = p0 + j * G::RPI + grp;
            const float w = __shfl(wp, min(pi, 63));   // part pi's weight sits in lane pi
            const float wv = pi < parts ? w : 0.f;
#pragma unroll
            for (int e = 0; e < G::PER; ++e) out[e] = __builtin_fmaf(wv, x[j][e], out[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < G::PER; ++e) out[e] = xsum<G::R>(out[e]);
    if (ok) finish<K, D>(a, bh, slot_off, N, knew, vnew, __builtin_amdgcn_exp2f(snew - mt), lt, out, sub, grp);
}

template <typename K, int D>
hipError_t launch_dim(const AttnArgs &a, float *ws, int P, hipStream_t stream) {
    const long bh = (long)a.B * a.H;
    if (P <= 1) {
        hipLaunchKernelGGL((ar_decode_kernel<K, D>), dim3((unsigned)bh), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((ar_split_kernel<K, D>), dim3((unsigned)(bh * P)), dim3(kThreads), 0, stream, a, ws, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ar_merge_kernel<K, D>), dim3((unsigned)bh), dim3(64), 0, stream, a, ws, P);
    return hipGetLastError();
}

template <typename K>
hipError_t launch_kind(const AttnArgs &a, int D, float *ws, int P, hipStream_t stream) {
    switch (D) {
        case 32:
            if constexpr (K::kP8) return hipErrorInvalidValue;   // a 32-byte E4M3 row is below one 16-byte lane pair
            else return launch_dim<K, 32>(a, ws, P, stream);
        case 64: return launch_dim<K, 64>(a, ws, P, stream);
        case 128: return launch_dim<K, 128>(a, ws, P, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename K>
int chunk_rows(int D) {
    switch (D) {
        case 32: return Geo<K, 32>::CH;
        case 64: return Geo<K, 64>::CH;
        case 128: return Geo<K, 128>::CH;
        default: return 0;
    }
}

using KindBf16 = Kind<bf16, false>;
using KindBf16P8 = Kind<bf16, true>;

}  // namespace

int ar_splits(long bh, int n_max, int D, int kind) {
    // The one-pass kernel streams a pair's rows from one workgroup, about 3 us plus the
    // rows' bytes at some 72 GB/s (bf16), while the split costs at least its two
    // launches, about 13 us.  So a pair is split only when its slot at capacity holds at
    // least 240 Ki elements per matrix (rows x D; 3840 rows at D = 64, 1920 at D = 128):
    // in a sweep over 8-1024 pairs and 1024-8192 rows the split lost below that (0.70-0.97x
    // at 512-750 KB of bf16 per pair) and won above it (1.1-3.3x), on bf16 and E4M3 pools
    // alike when counted in elements (the E4M3 kernel spends longer per byte decoding).
    // The rows are then cut into parts of at least 4 chunks, up to about 256 workgroups
    // over all pairs (more only add merge work; HBM is busy by then) and 64 parts per
    // pair (one per lane of the merge wave); fewer than 3 parts (128 or more pairs) lost
    // in that sweep (0.83-0.94x) and keep the one-pass kernel.
    // fp32 pools (kind 0) run the fp64 one-pass kernel and never split.
    constexpr long kMinSplitElements = 240L << 10;
    constexpr long kMinParts = 3;
    if (bh <= 0 || n_max < 2 || kind == 0) return 1;
    const long rows = n_max - 1;
    if (rows * D < kMinSplitElements) return 1;
    const int ch = kind == 1 ? chunk_rows<KindBf16>(D) : chunk_rows<KindBf16P8>(D);
    if (ch == 0) return 1;
    const long nc = (rows + ch - 1) / ch;
    long P = (nc + 3) / 4;
    if (P > 256 / bh) P = 256 / bh;
    if (P > 64) P = 64;
    return P < kMinParts ? 1 : (int)P;
}

size_t ar_workspace_bytes(long bh, int P, int D) { return P <= 1 ? 0 : (size_t)bh * P * (D + 4) * sizeof(float); }

size_t ar_scratch_bytes() { return kArScratchBytes; }

hipError_t ar_scratch(float **out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<float *> ptrs[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float *p = ptrs[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = ptrs[dev].load(std::memory_order_relaxed);
        if (!p) {
            // the device address of this device's copy; the host-side name is not one
            e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            ptrs[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_ar_decode(const AttnArgs &a, int D, int kind, float *ws, int P, hipStream_t stream) {
    if ((long)a.B * a.H <= 0) return hipSuccess;
    switch (kind) {
        case 1: return launch_kind<KindBf16>(a, D, ws, P, stream);
        case 2: return launch_kind<KindBf16P8>(a, D, ws, P, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace unipin
