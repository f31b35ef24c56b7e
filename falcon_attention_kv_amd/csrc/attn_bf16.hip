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
//   * 64-key tiles of K and V are copied HBM -> LDS by the buffer-to-LDS DMA path
//     (buffer_load_dwordx4 ... lds), three tiles in flight: no staging registers, no
//     VALU work, and every row past the history reads as zero (the buffer's record
//     count is the history length), so ragged histories need no branches;
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA result each lane
//     holds one query and 16 keys: softmax row statistics are lane-local plus one
//     exchange with the lane 32 away;
//   * the PV product is computed as O^T = V^T P^T: P^T, rounded to bf16, is used in the
//     very registers the score MFMA left it in; V stays in its natural [key][d] layout
//     in LDS and ds_read_b64_tr_b16 delivers it transposed;
//   * fp32 online softmax in the log2 domain (scale*log2(e) folded into one FMA), with a
//     lazy rescale: the running max only moves when a tile's max exceeds it by more
//     than 2^8, which bounds P by 256 and skips almost every rescale;
//   * the row sum is accumulated from the bf16-rounded P (v_dot2 with ones), so the
//     normaliser matches the weights the PV product used;
//   * masking code runs only on tiles that cross the history end or the causal diagonal.
//
// Hardware facts relied on (checked on gfx950 with small in-bounds probes):
//   * v_mfma_f32_32x32x16_bf16 result element i of lane l is row 8*(i/4) + 4*(l/32)
//     + (i%4), column l%32; A and B spread the contraction index over (lane/32,
//     element) in the same way, so any consistent assignment of keys to (lane/32,
//     element) is a valid contraction order;
//   * ds_read_b64_tr_b16: in each group of 16 lanes, lane c receives element c%4 of the
//     8-byte rows addressed by lanes 4e + c/4 (e = 0..3): a 4 x 16 -> 16 x 4 transpose;
//   * buffer loads to LDS write 16 bytes per lane at consecutive LDS addresses (M0 base
//     + 16 * lane) and write zeros for offsets past the record count.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace unipin {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 64;                   // query rows per wave
constexpr int kQT = kWaves * kQW;         // query rows per workgroup
constexpr int kTK = 64;                   // keys per LDS tile
constexpr int kBufs = 3;                  // LDS tiles in flight
static_assert(kQT == kBf16RowsPerBlock, "rows per block must match the host's grid math");
static_assert(kQT % kTK == 0, "a query tile must cover whole key tiles");

constexpr uint32_t kBufferWord3 = 0x00020000u;   // gfx9 buffer descriptor, raw 32-bit access

// Lazy-rescale threshold in log2 units: P stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct Tile {
    static constexpr int KC = D / 16;                 // 16-deep contraction chunks of the head dim
    static constexpr int DB = D / 32;                 // 32-row blocks of the head dim in O^T
    static constexpr int R = D / 8;                   // 16-byte blocks per key row
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int MAT_BYTES = kTK * ROW_BYTES;  // one K or V tile
    static constexpr int BUF_BYTES = 2 * MAT_BYTES;    // K tile then V tile
    static constexpr int DMA_PER_MAT = MAT_BYTES / 1024;              // 1 KB per wave-wide DMA
    static constexpr int DMA_PER_WAVE = 2 * DMA_PER_MAT / kWaves;     // per wave per tile
    static_assert(2 * DMA_PER_MAT % kWaves == 0, "tile DMA must split evenly over the waves");
};

// 16-byte block swizzles inside a key row (XOR keeps the block inside the row).  K is
// read 8 lanes at a time, one row each, same logical block; V is read with transpose
// loads, 16 lanes covering 4 consecutive rows x 32 bytes.  Both patterns then touch
// every LDS bank exactly once.
template <int D>
__device__ __forceinline__ int k_swz(int key) {
    return Tile<D>::R >= 8 ? (key & 7) : ((key >> 1) & 3);
}
template <int D>
__device__ __forceinline__ int v_swz(int key) {
    return Tile<D>::R >= 8 ? ((key & 3) << 1) : (((key >> 1) & 1) << 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kBufferWord3);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// DMA of one K/V tile (keys kbase .. kbase+63) into LDS buffer `buf`.  Wave w moves
// its share of the 1 KB pieces; lane l of piece j fills LDS block 64*j + l, i.e. key row
// (64*j + l) / R, swizzled block (64*j + l) % R, taken from the matching unswizzled block.
template <int D>
__device__ __forceinline__ void dma_tile(LDS_AS char *buf, __amdgpu_buffer_rsrc_t rk,
                                         __amdgpu_buffer_rsrc_t rv, int kbase, int wave, int lane) {
    using T = Tile<D>;
#pragma unroll
    for (int j = 0; j < T::DMA_PER_WAVE; ++j) {
        const int piece = wave * T::DMA_PER_WAVE + j;          // wave-uniform
        const bool is_v = piece >= T::DMA_PER_MAT;
        const int pj = is_v ? piece - T::DMA_PER_MAT : piece;
        const int p = pj * 64 + lane;
        const int key = p / T::R, blks = p % T::R;
        const int blk = blks ^ (is_v ? v_swz<D>(key) : k_swz<D>(key));
        const uint32_t goff = (uint32_t)((kbase + key) * T::ROW_BYTES + blk * 16);
        LDS_AS char *dst = buf + (is_v ? T::MAT_BYTES : 0) + pj * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? rv : rk, (LDS_AS void *)dst, 16, (int)goff, 0, 0, 0);
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

// Per-wave attention state and the per-tile step.
template <int D>
struct WaveState {
    bf16x8 qreg[2][Tile<D>::KC];   // B operand: query rows wq0 + qb*32 + col, dims c*16 + g*8 ..
    f32x16 acc[Tile<D>::DB][2];    // O^T accumulators: lane = query, 16 head dims per block
    float m[2];                    // running max (log2 domain), shared by both lane halves
    float l[2];                    // this lane half's share of the row sum
};

template <int D, bool PREFILL, bool MASK>
__device__ __forceinline__ void tile_step(WaveState<D> &ws, const LDS_AS char *kt, const LDS_AS char *vt,
                                          int kbase, int kend, int wq0, int col, int g,
                                          int k_off0, const int *k_xor, int v_off, const int *v_blk, float c) {
    using T = Tile<D>;
    // ---- S^T = K Q^T: 2 key blocks x 2 query blocks of 32x32.
    f32x16 sc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sc[kb][qb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < T::KC; ++cc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 ka = *reinterpret_cast<const LDS_AS bf16x8 *>(kt + k_off0 + kb * 32 * T::ROW_BYTES + k_xor[cc]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ws.qreg[qb][cc], sc[kb][qb], 0, 0, 0);
        }
    }

    // ---- mask: keys past the history, and (prefill) keys after the query.  Element i
    // of block (kb, qb) is key kbase + kb*32 + 4g + off(i), off(i) = 8*(i/4) + i%4, so
    // one per-lane bound per block decides all 16: the key is visible iff off(i) <= lim.
    if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int base = kbase + kb * 32 + 4 * g;
                int lim = kend - 1 - base;
                if (PREFILL) lim = min(lim, wq0 + qb * 32 + col - base);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 8 * (i >> 2) + (i & 3);
                    sc[kb][qb][i] = off > lim ? -INFINITY : sc[kb][qb][i];
                }
            }
    }

    // ---- running max (log2 domain) with lazy rescale.  The rescale branch is wave-wide
    // and rare (first visible tile, or a late jump of the max by more than 2^8).
    float mt[2];
    bool grow[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float mx = sc[0][qb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[0][qb][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[1][qb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mt[qb] = mx * c;
        grow[qb] = mt[qb] > ws.m[qb] + kRescaleThreshold;
    }
    if (__any(grow[0] || grow[1])) {
        // keeps the compiler from flattening this rare path into the hot block
        asm volatile("" ::: "memory");
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mn = grow[qb] ? fmaxf(ws.m[qb], mt[qb]) : ws.m[qb];
            const float alpha = grow[qb] ? __builtin_amdgcn_exp2f(ws.m[qb] - mn) : 1.f;
            ws.l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) ws.acc[db][qb] *= alpha;
            ws.m[qb] = mn;
        }
    }

    // ---- per 32-key block: P = exp2(s*c - m), rounded to bf16 in the B-operand layout
    // of the PV MFMA (the row sum takes the rounded values), then O^T += V^T P^T.
    // Lane (d, g) needs, for chunk (kb, c2), V at keys kb*32 + 16*c2 + {4g..4g+3}
    // (elements 0..3) and kb*32 + 16*c2 + 8 + {4g..4g+3} (elements 4..7): two transpose
    // loads of 4 keys x 16 dims each.
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        bf16x8 pb[2][2];  // [chunk of 16 keys][qb]
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float nm = -ws.m[qb];
            float lsum = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                bf16x8 p;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][c2 * 8 + e], c, nm));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][c2 * 8 + e + 1], c, nm));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    p[e] = pp[0];
                    p[e + 1] = pp[1];
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
                }
                pb[c2][qb] = p;
            }
            ws.l[qb] += lsum;
        }
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const LDS_AS char *src = vt + v_off + v_blk[db] + (kb * 32 + 16 * c2) * T::ROW_BYTES;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)src);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(src + 8 * T::ROW_BYTES));
                const i16x4 lh[2] = {lo, hi};
                const bf16x8 va = __builtin_bit_cast(bf16x8, lh);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    ws.acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c2][qb], ws.acc[db][qb], 0, 0, 0);
            }
    }
}

template <int D, bool PREFILL>
__device__ __forceinline__ void attn_body(const AttnArgs &a) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) char smem_raw[kBufs * T::BUF_BYTES];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

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
    // Rows at or past kend read as zeros.
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(ksrc, (uint32_t)kend * T::ROW_BYTES);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vsrc, (uint32_t)kend * T::ROW_BYTES);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int wq0 = q0 + wave * kQW;

    // Start the first two tiles' DMA before anything else.
    if (ntiles > 0) dma_tile<D>(smem, rk, rv, 0, wave, lane);
    if (ntiles > 1) dma_tile<D>(smem + T::BUF_BYTES, rk, rv, kTK, wave, lane);

    WaveState<D> ws;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qsrc, (uint32_t)qlimit * T::ROW_BYTES);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const uint32_t row = (uint32_t)(wq0 + qb * 32 + col);
#pragma unroll
        for (int cc = 0; cc < T::KC; ++cc)
            ws.qreg[qb][cc] = as_bf16x8(bload16(rq, row * T::ROW_BYTES + cc * 32 + g * 16));
    }

    if constexpr (PREFILL) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            ws.m[qb] = -INFINITY;
            ws.l[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) ws.acc[db][qb] = f32x16{};
        }
    } else {
        // The candidate's own key enters first: it sets the running max, contributes
        // weight exp2(0) = 1 to the row sum (counted once, by the lower half) and its
        // value vc_j to the accumulator.  An empty history therefore yields vc_j exactly.
        const __amdgpu_buffer_rsrc_t rkc =
            make_rsrc(static_cast<const bf16 *>(a.k) + bh * a.rows * D, (uint32_t)qlimit * T::ROW_BYTES);
        const __amdgpu_buffer_rsrc_t rvc =
            make_rsrc(static_cast<const bf16 *>(a.v) + bh * a.rows * D, (uint32_t)qlimit * T::ROW_BYTES);
        const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
        (void)ones;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const uint32_t row = (uint32_t)(wq0 + qb * 32 + col);
            float part = 0.f;
#pragma unroll
            for (int cc = 0; cc < T::KC; ++cc) {
                const bf16x8 kk = as_bf16x8(bload16(rkc, row * T::ROW_BYTES + cc * 32 + g * 16));
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2 qa = {ws.qreg[qb][cc][e], ws.qreg[qb][cc][e + 1]};
                    const bf16x2 ka = {kk[e], kk[e + 1]};
                    part = __builtin_amdgcn_fdot2_f32_bf16(qa, ka, part, false);
                }
            }
            const float self = part + __shfl_xor(part, 32);
            ws.m[qb] = self * a.c;
            ws.l[qb] = g == 0 ? 1.f : 0.f;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = db * 32 + 8 * j + 4 * g;
                    const bf16x4 vv = __builtin_bit_cast(bf16x4, bload8(rvc, row * T::ROW_BYTES + d0 * 2));
#pragma unroll
                    for (int e = 0; e < 4; ++e) ws.acc[db][qb][4 * j + e] = (float)vv[e];
                }
            }
        }
    }

    // Per-lane LDS offsets.  K operand: row kb*32 + col, logical block 2*cc + g.
    const int k_off0 = col * T::ROW_BYTES;
    int k_xor[T::KC];
#pragma unroll
    for (int cc = 0; cc < T::KC; ++cc) k_xor[cc] = ((2 * cc + g) ^ k_swz<D>(col)) * 16;
    // V transpose loads: in 16-lane group (g, sub), lane i addresses key 4g + i/4 (plus the
    // chunk's key base) and head dims db*32 + 16*sub + 4*(i%4) .. +3.
    const int ti = lane & 15, sub = (lane >> 4) & 1;
    const int vkey = 4 * g + (ti >> 2);
    const int v_off = vkey * T::ROW_BYTES + (ti & 1) * 8;
    int v_blk[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        v_blk[db] = ((db * 4 + 2 * sub + ((ti & 3) >> 1)) ^ v_swz<D>(vkey)) * 16;

    // Tiles [0, t_plain) need no mask for any wave of the block: they end before the
    // history end and (prefill) at or before the block's first query.  The remaining
    // tiles run the masked step; a wave skips tiles that lie wholly after its queries.
    const int t_plain = PREFILL ? min(kend / kTK, q0 / kTK) : kend / kTK;
    const bool wave_rows_valid = wq0 < qlimit;
    auto pipeline = [&](int t) {
        if (t + 1 < ntiles) wait_vmcnt<T::DMA_PER_WAVE>(); else wait_vmcnt<0>();
        __syncthreads();
        if (t + 2 < ntiles) dma_tile<D>(smem + ((t + 2) % kBufs) * T::BUF_BYTES, rk, rv, (t + 2) * kTK, wave, lane);
    };
    for (int t = 0; t < t_plain; ++t) {
        pipeline(t);
        const LDS_AS char *kt = smem + (t % kBufs) * T::BUF_BYTES;
        if (wave_rows_valid)
            tile_step<D, PREFILL, false>(ws, kt, kt + T::MAT_BYTES, t * kTK, kend, wq0, col, g,
                                         k_off0, k_xor, v_off, v_blk, a.c);
    }
    for (int t = t_plain; t < ntiles; ++t) {
        pipeline(t);
        const int kbase = t * kTK;
        const LDS_AS char *kt = smem + (t % kBufs) * T::BUF_BYTES;
        if (wave_rows_valid && (!PREFILL || kbase <= wq0 + kQW - 1))
            tile_step<D, PREFILL, true>(ws, kt, kt + T::MAT_BYTES, kbase, kend, wq0, col, g,
                                        k_off0, k_xor, v_off, v_blk, a.c);
    }

    // ---- epilogue: combine the two halves' row sums, normalise, store bf16 rows.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = ws.l[qb] + __shfl_xor(ws.l[qb], 32);
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
                    for (int e = 0; e < 4; ++e) ov[e] = (bf16)(ws.acc[db][qb][4 * j + e] * inv);
                    *reinterpret_cast<u32x2 *>(odst + (long)row * D + d0) = __builtin_bit_cast(u32x2, ov);
                }
        }
    }

    // ---- prefill: fused pool write of this block's own history rows, bit for bit.
    if constexpr (PREFILL) {
        const int r1 = min(q0 + kQT, N);
        const int chunks = (r1 - q0) * T::R;
        for (int i = tid; i < chunks; i += kThreads) {
            const long off = (long)q0 * D + (long)i * 8;
            *reinterpret_cast<u32x4 *>(pk + off) = *reinterpret_cast<const u32x4 *>(ksrc + off);
            *reinterpret_cast<u32x4 *>(pv + off) = *reinterpret_cast<const u32x4 *>(vsrc + off);
        }
    }
}

template <int D>
__global__ void __launch_bounds__(kThreads, D <= 64 ? 2 : 1) prefill_bf16_kernel(AttnArgs a) {
    attn_body<D, true>(a);
}

template <int D>
__global__ void __launch_bounds__(kThreads, D <= 64 ? 2 : 1) rank_decode_bf16_kernel(AttnArgs a) {
    attn_body<D, false>(a);
}

template <bool PREFILL>
hipError_t launch_bf16(const AttnArgs &a, int D, hipStream_t stream) {
    const long blocks = (long)a.B * a.H * a.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
#define UNIPIN_LAUNCH(DD)                                                                      \
    if (PREFILL) hipLaunchKernelGGL(prefill_bf16_kernel<DD>, grid, block, 0, stream, a);       \
    else hipLaunchKernelGGL(rank_decode_bf16_kernel<DD>, grid, block, 0, stream, a);
    switch (D) {
        case 32: UNIPIN_LAUNCH(32) break;
        case 64: UNIPIN_LAUNCH(64) break;
        case 128: UNIPIN_LAUNCH(128) break;
        default: return hipErrorInvalidValue;
    }
#undef UNIPIN_LAUNCH
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
