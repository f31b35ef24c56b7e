// bf16 M-FALCON attention kernels for gfx950 (CDNA4): causal prefill with the fused
// pool write, and the ranking decode over a pool slot with the candidate's own key fused.
//
// The method (UniPinRec review, sections 2.2 and 2.4; UniPinRec reading notes,
// sections 3 and 6): history tokens attend causally; each candidate attends to every
// cached history key of its user plus its own key, never to another candidate.
//
// Work decomposition (both kernels):
//   * one workgroup = 4 waves of 64 lanes; each wave owns 64 query rows, held in
//     registers for the whole kernel as the B operand of v_mfma_f32_32x32x16_bf16;
//   * the workgroup streams 64-key tiles of K and V through LDS (double buffered,
//     16-byte coalesced global loads issued one tile ahead);
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA result each lane
//     holds one query and 16 keys: the softmax row statistics are lane-local plus one
//     exchange with the lane 32 away;
//   * the PV product is computed as O^T = V^T P^T: P^T, rounded to bf16, is used in the
//     very registers the score MFMA left it in, and O^T again keeps one query per lane,
//     so rescaling by the running max is lane-local;
//   * fp32 online softmax in the log2 domain (scale*log2(e) folded into one FMA), with a
//     lazy rescale: the running max only moves when a tile's max exceeds it by more
//     than 2^8, which bounds P by 256 and skips almost every rescale;
//   * the row sum is accumulated from the bf16-rounded P (v_dot2 with ones), so the
//     normaliser matches the weights the PV product used.
//
// Layout facts of v_mfma_f32_32x32x16_bf16 this relies on: result element i of lane l
// is row 8*(i/4) + 4*(l/32) + (i%4), column l%32; the A and B operands distribute the
// contraction index over (lane/32, element) in the same way, so any consistent
// assignment of keys to (lane/32, element) is a valid contraction order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace unipin {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 64;                   // query rows per wave
constexpr int kQT = kWaves * kQW;         // query rows per workgroup
constexpr int kTK = 64;                   // keys per LDS tile
static_assert(kQT == kBf16RowsPerBlock, "rows per block must match the host's grid math");
static_assert(kQT % kTK == 0, "a query tile must cover whole key tiles");

// Lazy-rescale threshold in log2 units: P stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct Tile {
    static constexpr int KC = D / 16;           // 16-deep contraction chunks over the head dim
    static constexpr int DB = D / 32;           // 32-row blocks of the head dim in O^T
    static constexpr int KSTR = D + 8;          // K tile row stride in elements (16 B pad)
    static constexpr int K_ELEMS = kTK * KSTR;  // K tile, [key][d], padded rows
    static constexpr int V_ELEMS = D * kTK;     // V^T tile, [d][key position], XOR-swizzled
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int C8 = D / 8;            // 16-byte chunks per row
    static constexpr int K_CHUNKS = kTK * C8 / kThreads;          // K chunks per thread
    static constexpr int V_UNITS = (kTK / 2) * C8;                // key pairs x chunks
    static constexpr int V_PER_THREAD = (V_UNITS + kThreads - 1) / kThreads;
    static_assert(kTK * C8 % kThreads == 0, "K tile must split evenly over the threads");
};

// Position of key offset r (0..63) inside a V^T row: the two middle 4-key groups of
// every 16-key chunk are swapped, so that the 8 keys one lane needs for one PV MFMA
// (keys 16c + 8(e/4) + 4(l/32) + e%4 for e = 0..7, dictated by the score layout) sit at
// 8 consecutive positions.  The map is its own inverse.
__device__ __forceinline__ int vt_pos(int r) {
    return (r & ~12) | ((r >> 1) & 4) | ((r << 1) & 8);
}

// Element index of (d, position p) in the V^T tile.  16-byte blocks of a row are
// XOR-swizzled with a function of d so that both the transposing writes (8 lanes, same
// key pair, 8 different d-groups) and the operand reads (8 lanes, 8 consecutive d, same
// block) spread over all LDS banks.
__device__ __forceinline__ int vt_index(int d, int p) {
    const int sw = (d ^ (d >> 3)) & 7;
    return d * kTK + ((((p >> 3) ^ sw)) << 3) + (p & 7);
}

__device__ __forceinline__ u32x4 load16(const bf16 *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
    return __builtin_bit_cast(bf16x8, x);
}

// Staged copy of one K/V tile held in registers between its global load and its LDS
// store (and, for the prefill's own rows, its pool store).
template <int D>
struct Stage {
    u32x4 k[Tile<D>::K_CHUNKS];
    u32x4 v0[Tile<D>::V_PER_THREAD];
    u32x4 v1[Tile<D>::V_PER_THREAD];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const bf16 *ksrc, const bf16 *vsrc,
                                           int kbase, int N, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::K_CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int r = c / T::C8, c8 = c % T::C8;
        const int key = kbase + r;
        st.k[i] = key < N ? load16(ksrc + (long)key * D + c8 * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < T::V_PER_THREAD; ++i) {
        const int u = tid + i * kThreads;
        const int rp = u / T::C8, c8 = u % T::C8;
        const int key = kbase + 2 * rp;
        const bool in = u < T::V_UNITS;
        st.v0[i] = (in && key < N) ? load16(vsrc + (long)key * D + c8 * 8) : u32x4{0, 0, 0, 0};
        st.v1[i] = (in && key + 1 < N) ? load16(vsrc + (long)(key + 1) * D + c8 * 8)
                                       : u32x4{0, 0, 0, 0};
    }
}

template <int D>
__device__ __forceinline__ void stage_store_lds(const Stage<D> &st, bf16 *buf, int tid) {
    using T = Tile<D>;
    bf16 *ks = buf;
    bf16 *vt = buf + T::K_ELEMS;
#pragma unroll
    for (int i = 0; i < T::K_CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int r = c / T::C8, c8 = c % T::C8;
        *reinterpret_cast<u32x4 *>(ks + r * T::KSTR + c8 * 8) = st.k[i];
    }
#pragma unroll
    for (int i = 0; i < T::V_PER_THREAD; ++i) {
        const int u = tid + i * kThreads;
        if (u >= T::V_UNITS) break;
        const int rp = u / T::C8, c8 = u % T::C8;
        const int p = vt_pos(2 * rp);  // even; the pair's second key sits at p + 1
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = st.v0[i][j], b = st.v1[i][j];
            const uint32_t lo = (a & 0xffffu) | (b << 16);          // d = c8*8 + 2j
            const uint32_t hi = (a >> 16) | (b & 0xffff0000u);      // d = c8*8 + 2j + 1
            const int d = c8 * 8 + 2 * j;
            *reinterpret_cast<uint32_t *>(vt + vt_index(d, p)) = lo;
            *reinterpret_cast<uint32_t *>(vt + vt_index(d + 1, p)) = hi;
        }
    }
}

template <int D>
__device__ __forceinline__ void stage_store_pool(const Stage<D> &st, bf16 *pk, bf16 *pv,
                                                 int kbase, int N, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::K_CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int r = c / T::C8, c8 = c % T::C8;
        const int key = kbase + r;
        if (key < N) *reinterpret_cast<u32x4 *>(pk + (long)key * D + c8 * 8) = st.k[i];
    }
#pragma unroll
    for (int i = 0; i < T::V_PER_THREAD; ++i) {
        const int u = tid + i * kThreads;
        if (u >= T::V_UNITS) break;
        const int rp = u / T::C8, c8 = u % T::C8;
        const int key = kbase + 2 * rp;
        if (key < N) *reinterpret_cast<u32x4 *>(pv + (long)key * D + c8 * 8) = st.v0[i];
        if (key + 1 < N) *reinterpret_cast<u32x4 *>(pv + (long)(key + 1) * D + c8 * 8) = st.v1[i];
    }
}

// Maps the linear block id to (user*H + head, query tile).  With xcd_remap, blocks are
// dispatched round-robin over the 8 XCDs; the map makes the `tiles` consecutive blocks
// an XCD receives belong to one (user, head), so that its K/V is fetched from HBM once
// into that XCD's L2 and re-read from there by the other tiles.
__device__ __forceinline__ void block_coords(const AttnArgs &a, int &group, int &tile) {
    const int bid = blockIdx.x;
    if (a.xcd_remap) {
        const int xcd = bid & 7, local = bid >> 3;
        group = (local / a.tiles) * 8 + xcd;
        tile = local % a.tiles;
    } else {
        group = bid / a.tiles;
        tile = bid % a.tiles;
    }
}

template <int D, bool PREFILL>
__global__ void __launch_bounds__(kThreads, D <= 64 ? 2 : 1) attn_bf16_kernel(AttnArgs a) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::BUF_ELEMS];

    int group, tile;
    block_coords(a, group, tile);
    const int b = group / a.H, h = group % a.H;
    if (b >= a.B) return;
    // Causal prefill: hand out the heaviest (last) query tiles first.
    const int qtile = PREFILL ? (a.tiles - 1 - tile) : tile;

    const int N = a.lens[b];
    const int s = a.slot[b];
    if (N < 0 || N > a.len_limit || s < 0 || s >= a.S) {
        if (threadIdx.x == 0 && tile == 0)
            atomicOr(a.status, (N < 0 || N > a.len_limit ? kFlagBadLen : 0u) |
                                   (s < 0 || s >= a.S ? kFlagBadSlot : 0u));
        return;
    }

    const int q0 = qtile * kQT;
    const int qlimit = PREFILL ? N : a.rows;   // valid query rows are < qlimit
    if (q0 >= qlimit) return;

    const long bh = (long)b * a.H + h;
    const bf16 *qsrc = static_cast<const bf16 *>(a.q) + bh * a.rows * D;
    bf16 *odst = static_cast<bf16 *>(a.o) + bh * a.rows * D;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    bf16 *pk = static_cast<bf16 *>(a.pool_k) + slot_off;
    bf16 *pv = static_cast<bf16 *>(a.pool_v) + slot_off;
    // Key/value source: the history inputs (prefill) or the pool slot (decode).
    const bf16 *ksrc = PREFILL ? static_cast<const bf16 *>(a.k) + bh * a.rows * D : pk;
    const bf16 *vsrc = PREFILL ? static_cast<const bf16 *>(a.v) + bh * a.rows * D : pv;
    const int kend = PREFILL ? min(q0 + kQT, N) : N;
    const int ntiles = (kend + kTK - 1) / kTK;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int wq0 = q0 + wave * kQW;

    // Query rows of this lane: wq0 + qb*32 + col, qb in {0,1}.  Operand layout: chunk c
    // holds head dims c*16 + g*8 .. +7.
    bf16x8 qreg[2][T::KC];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = wq0 + qb * 32 + col;
#pragma unroll
        for (int c = 0; c < T::KC; ++c)
            qreg[qb][c] = as_bf16x8(row < qlimit ? load16(qsrc + (long)row * D + c * 16 + g * 8)
                                                 : u32x4{0, 0, 0, 0});
    }

    // Online-softmax state per query block: running max m (log2 domain), this half's
    // share of the row sum l, and O^T accumulators (lane = query, 16 head dims per block).
    float m[2], l[2];
    f32x16 acc[T::DB][2];
    if constexpr (PREFILL) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            m[qb] = -INFINITY;
            l[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) acc[db][qb] = f32x16{};
        }
    } else {
        // The candidate's own key enters first: it sets the running max, contributes
        // weight exp2(0) = 1 to the row sum (counted once, by the lower half) and its
        // value vc_j to the accumulator.  An empty history therefore yields vc_j exactly.
        const bf16 *kcs = static_cast<const bf16 *>(a.k) + bh * a.rows * D;
        const bf16 *vcs = static_cast<const bf16 *>(a.v) + bh * a.rows * D;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = wq0 + qb * 32 + col;
            const bool ok = row < qlimit;
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < T::KC; ++c) {
                const bf16x8 kk =
                    as_bf16x8(ok ? load16(kcs + (long)row * D + c * 16 + g * 8) : u32x4{0, 0, 0, 0});
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2 qa = {qreg[qb][c][e], qreg[qb][c][e + 1]};
                    const bf16x2 ka = {kk[e], kk[e + 1]};
                    part = __builtin_amdgcn_fdot2_f32_bf16(qa, ka, part, false);
                }
            }
            const float self = part + __shfl_xor(part, 32);
            m[qb] = self * a.c;
            l[qb] = g == 0 ? 1.f : 0.f;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = db * 32 + 8 * j + 4 * g;
                    u32x2 raw = ok ? *reinterpret_cast<const u32x2 *>(vcs + (long)row * D + d0)
                                   : u32x2{0, 0};
                    const bf16x4 vv = __builtin_bit_cast(bf16x4, raw);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[db][qb][4 * j + e] = (float)vv[e];
                }
            }
        }
    }

    Stage<D> st;
    if (ntiles > 0) {
        stage_load<D>(st, ksrc, vsrc, 0, kend, tid);
        if (PREFILL && q0 == 0) stage_store_pool<D>(st, pk, pv, 0, kend, tid);
        stage_store_lds<D>(st, smem, tid);
    }
    __syncthreads();

    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

    for (int t = 0; t < ntiles; ++t) {
        const int kbase = t * kTK;
        const bool has_next = t + 1 < ntiles;
        if (has_next) stage_load<D>(st, ksrc, vsrc, kbase + kTK, kend, tid);

        const bf16 *buf = smem + (t & 1) * T::BUF_ELEMS;
        const bf16 *ks = buf;
        const bf16 *vt = buf + T::K_ELEMS;

        // A wave skips tiles it cannot see (causal) and waves with no valid row.
        const bool active = wq0 < qlimit && (!PREFILL || kbase <= wq0 + kQW - 1);
        if (active) {
            // ---- S^T = K Q^T: 2 key blocks x 2 query blocks of 32x32.
            f32x16 sc[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) sc[kb][qb] = f32x16{};
#pragma unroll
            for (int c = 0; c < T::KC; ++c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 ka = as_bf16x8(
                        *reinterpret_cast<const u32x4 *>(ks + (kb * 32 + col) * T::KSTR + c * 16 + g * 8));
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], sc[kb][qb], 0, 0, 0);
                }
            }

            // ---- mask: keys past the history, and (prefill) keys after the query.
            const bool need_mask = (kbase + kTK > kend) || (PREFILL && kbase + kTK - 1 > wq0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        const int query = wq0 + qb * 32 + col;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                            const bool off = key >= kend || (PREFILL && key > query);
                            sc[kb][qb][i] = off ? -INFINITY : sc[kb][qb][i];
                        }
                    }
            }

            // ---- running max (log2 domain) with lazy rescale.
            float mt[2];
            bool grow = false;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = sc[0][qb][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[0][qb][i]);
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[1][qb][i]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                mt[qb] = mx * a.c;
                grow |= mt[qb] > m[qb] + kRescaleThreshold;
            }
            if (__any(grow)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const float mn = fmaxf(m[qb], mt[qb]);
                    if (mt[qb] > m[qb] + kRescaleThreshold) {
                        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
                        l[qb] *= alpha;
#pragma unroll
                        for (int db = 0; db < T::DB; ++db) acc[db][qb] *= alpha;
                        m[qb] = mn;
                    }
                }
            }

            // ---- P = exp2(s*c - m), rounded to bf16 in the B-operand layout of the PV
            // MFMA; the row sum takes the rounded values.
            bf16x8 pb[2][2][2];  // [kb][chunk of 16 keys][qb]
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float nm = -m[qb];
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        bf16x8 p;
#pragma unroll
                        for (int e = 0; e < 8; e += 2) {
                            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][c2 * 8 + e], a.c, nm));
                            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][c2 * 8 + e + 1], a.c, nm));
                            const bf16x2 pp = {(bf16)p0, (bf16)p1};
                            p[e] = pp[0];
                            p[e + 1] = pp[1];
                            lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
                        }
                        pb[kb][c2][qb] = p;
                    }
                l[qb] += lsum;
            }

            // ---- O^T += V^T P^T.
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        const int d = db * 32 + col;
                        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                            vt + vt_index(d, kb * 32 + c2 * 16 + g * 8)));
#pragma unroll
                        for (int qb = 0; qb < 2; ++qb)
                            acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][c2][qb], acc[db][qb], 0, 0, 0);
                    }
        }

        if (has_next) {
            if (PREFILL && kbase + kTK >= q0) stage_store_pool<D>(st, pk, pv, kbase + kTK, kend, tid);
            stage_store_lds<D>(st, smem + ((t + 1) & 1) * T::BUF_ELEMS, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: combine the two halves' row sums, normalise, store bf16 rows.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = l[qb] + __shfl_xor(l[qb], 32);
        const float inv = 1.f / lt;
        const int row = wq0 + qb * 32 + col;
        if (row < qlimit) {
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = db * 32 + 8 * j + 4 * g;
                    bf16x4 ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[db][qb][4 * j + e] * inv);
                    *reinterpret_cast<u32x2 *>(odst + (long)row * D + d0) = __builtin_bit_cast(u32x2, ov);
                }
        }
    }
}

template <bool PREFILL>
hipError_t launch_bf16(const AttnArgs &a, int D, hipStream_t stream) {
    const long blocks = (long)a.B * a.H * a.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (D) {
        case 32: hipLaunchKernelGGL((attn_bf16_kernel<32, PREFILL>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((attn_bf16_kernel<64, PREFILL>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((attn_bf16_kernel<128, PREFILL>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_bf16<true>(a, D, stream);
}

hipError_t launch_decode_bf16(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_bf16<false>(a, D, stream);
}

}  // namespace unipin
