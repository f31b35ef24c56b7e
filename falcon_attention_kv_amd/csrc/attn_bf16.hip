// bf16 M-FALCON attention kernels for gfx950 (CDNA4): causal prefill with the fused
// pool write, and the ranking decode over a pool slot with the candidate's own key fused.
//
// The method (UniPinRec review, sections 2.2 and 2.4; UniPinRec reading notes,
// sections 3 and 6): history tokens attend causally; each candidate attends to every
// cached history key of its user plus its own key, never to another candidate.
//
// Work decomposition:
//   * a workgroup covers 256 query rows: 8 waves of 32 rows at every head dimension; a
//     wave holds its rows in registers as the B operand of v_mfma_f32_32x32x16_bf16.  At
//     D <= 64 two workgroups share a CU (4 waves per SIMD); at D = 128 the LDS ring (four
//     32 KB slots) leaves room for one (2 waves per SIMD, up to 256 registers);
//   * everything a workgroup reads from HBM arrives through the buffer-to-LDS DMA path
//     (buffer_load_dwordx4 ... lds) into a ring of four LDS slots: 64-key tiles of K
//     and V, up to three tiles ahead of use, and the 256-row blocks of queries (and, in
//     the decode, of the candidates' own keys and values).  Each DMA instruction moves
//     1 KB of whole rows (no VGPRs, no VALU work), and every row past the record count
//     reads as zero, so ragged histories need no branches;
//   * outputs go back through LDS too, so that the global stores write whole rows;
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA result each lane
//     holds one query and 16 keys: softmax row statistics are lane-local plus one
//     v_permlane32_swap with the lane 32 away;
//   * the PV product is computed as O^T = V^T P^T: P^T, rounded to bf16, is used in the
//     very registers the score MFMA left it in; V stays in its natural [key][d] layout
//     in LDS and ds_read_b64_tr_b16 delivers it transposed;
//   * fp32 online softmax in the log2 domain (scale*log2(e) folded into one FMA), with a
//     lazy rescale: a tile's weights are taken against the running max as it stands,
//     and the max only moves (and the tile is redone) when a row's weights would leave
//     the range 2^64, so no tile computes its maximum on the common path;
//   * the row sum is accumulated from the bf16-rounded P (v_dot2 with ones), so the
//     normaliser matches the weights the PV product used;
//   * masking runs only on tiles that cross the history end or the causal diagonal.
//
// The prefill launches one workgroup per (user, head, 256-row query tile) that holds
// history rows, the ranking decode one per (user, head, 256-candidate tile); both hand
// out their work longest history first (see the schedules below).
//
// Hardware facts relied on (checked on gfx950 with small in-bounds probes):
//   * v_mfma_f32_32x32x16_bf16 result element i of lane l is row 8*(i/4) + 4*(l/32)
//     + (i%4), column l%32; A and B spread the contraction index over (lane/32,
//     element) in the same way, so any consistent assignment of keys to (lane/32,
//     element) is a valid contraction order;
//   * ds_read_b64_tr_b16: in each group of 16 lanes, lane c receives element c%4 of the
//     8-byte rows addressed by lanes 4e + c/4 (e = 0..3): a 4 x 16 -> 16 x 4 transpose;
//   * buffer loads to LDS write 16 bytes per lane at consecutive LDS addresses (M0 base
//     + 16 * lane) and write zeros for offsets past the record count;
//   * a wave's vector-memory loads complete in issue order, so waiting until at most X
//     loads are outstanding guarantees every load older than the X most recent.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"
#include "e4m3.h"
#include "lds_dma.h"

namespace unipin {
namespace {

constexpr int kTK = 64;                   // keys per LDS tile
// LDS slots of the DMA ring (one 64-key K/V tile or 128 query rows each): 64 KB per
// workgroup at D = 64, so that two workgroups share a CU.
constexpr int kBufs = 4;

// A workgroup covers 256 query rows: 8 waves of one 32-row query block each (QB = 1; the
// tile code is written for QB blocks per wave, and two blocks per wave measured slower
// at every head dimension, since the register file then caps the CU at 4 waves).  At
// D <= 64 two workgroups share a CU (4 waves per SIMD, at most 128 registers per lane);
// at D = 128 the LDS ring holds one workgroup per CU (2 waves per SIMD, up to 256).
constexpr int kBlockRows = 256;
template <int D> constexpr int query_blocks() { return 1; }
template <int D> constexpr int wave_rows() { return 32 * query_blocks<D>(); }
template <int D> constexpr int block_waves() { return kBlockRows / wave_rows<D>(); }
// Minimum waves per SIMD the kernels are compiled for (the second __launch_bounds__
// argument).
template <int D> constexpr int min_waves_per_simd() { return D <= 64 ? 4 : 2; }


template <int D>
struct Tile {
    static constexpr int KC = D / 16;                 // 16-deep contraction chunks of the head dim
    static constexpr int DB = D / 32;                 // 32-row blocks of the head dim in O^T
    static constexpr int R = D / 8;                   // 16-byte blocks per key row
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int MAT_BYTES = kTK * ROW_BYTES;  // one K or V tile
    static constexpr int BUF_BYTES = 2 * MAT_BYTES;    // K tile then V tile
    static constexpr int DMA_PER_MAT = MAT_BYTES / 1024;              // 1 KB per wave-wide DMA
};

// DMA work split of one K/V tile over W waves: the first W/2 waves move K, the others V.
template <int D, int W>
struct KvDma {
    static constexpr int PER_WAVE = 2 * Tile<D>::DMA_PER_MAT / W;
    static_assert(PER_WAVE >= 1 && 2 * Tile<D>::DMA_PER_MAT == PER_WAVE * W, "tile DMA must split evenly");
};

// 16-byte block swizzles inside a key row (XOR keeps the block inside the row).  The
// gfx950 LDS has 64 four-byte banks: a 16-byte-per-lane read is served 16 lanes at a
// time, an 8-byte transpose read 32 lanes at a time.  K is read 16 rows at a time, same
// logical block; V with transpose loads, 4 consecutive rows x 64 bytes per 32 lanes.
// These swizzles put each such group on 64 distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int key) {
    constexpr int R = Tile<D>::R;
    return R >= 16 ? (key & 15) : R == 8 ? ((key >> 1) & 7) : ((key >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int v_swz(int key) {
    constexpr int R = Tile<D>::R;
    return R >= 16 ? ((key & 3) << 2) : R == 8 ? (((key >> 1) & 1) << 2) : 0;
}

// Value exchange with the lane 32 away (v_permlane32_swap: no LDS round trip).  r[0]
// holds the lower half's value in both halves, r[1] the upper half's.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane source offsets of this wave's DMA pieces within a tile.  Piece j of wave w
// moves 1 KB: lane l fills LDS block 64*pj + l of its matrix (pj = the piece's index
// within that matrix), i.e. key row (64*pj + l) / R at swizzled block (64*pj + l) % R,
// taken from the matching unswizzled 16-byte block of that row.
template <int D, int W>
__device__ __forceinline__ void dma_offsets(int (&voff)[(KvDma<D, W>::PER_WAVE)], int wave, int lane,
                                            int row_stride) {
    using T = Tile<D>;
#pragma unroll
    for (int j = 0; j < KvDma<D, W>::PER_WAVE; ++j) {
        const int piece = wave * KvDma<D, W>::PER_WAVE + j;
        const bool is_v = piece >= T::DMA_PER_MAT;
        const int pj = is_v ? piece - T::DMA_PER_MAT : piece;
        const int p = pj * 64 + lane;
        const int key = p / T::R, blks = p % T::R;
        const int blk = blks ^ (is_v ? v_swz<D>(key) : k_swz<D>(key));
        voff[j] = key * row_stride + blk * 16;
    }
}

// DMA of this wave's share of one K/V tile (keys kbase .. kbase+63) into LDS buffer
// `buf`; `rsrc` is the K or V buffer of the wave's half.
template <int D, int W>
__device__ __forceinline__ void dma_tile(LDS_AS char *buf, i32x4 rsrc, int kbase,
                                         const int (&voff)[(KvDma<D, W>::PER_WAVE)], int wave, int row_stride) {
    using T = Tile<D>;
    const bool is_v = wave >= W / 2;
    const int first = wave * KvDma<D, W>::PER_WAVE - (is_v ? T::DMA_PER_MAT : 0);
    const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(buf) + (is_v ? T::MAT_BYTES : 0) + first * 1024;
    const int soff = kbase * row_stride;
#pragma unroll
    for (int j = 0; j < KvDma<D, W>::PER_WAVE; ++j) dma16(dst + j * 1024, rsrc, voff[j], soff);
}

// DMA of ROWS consecutive query (or candidate) rows from row0 into LDS with the K
// swizzle (or, VL, the V swizzle): 16-byte block bi of the block in LDS order is row
// bi / R, logical block (bi % R) ^ swz(row).  Rows past the record count read as zero.
// A 256-row block fills two LDS slots, a 128-row half block one.
template <int D, int W, int ROWS, bool VL = false>
__device__ __forceinline__ void dma_rows(LDS_AS char *dst, i32x4 rsrc, int row0, int wave, int lane,
                                         int row_stride) {
    using T = Tile<D>;
    constexpr int PW = ROWS * T::ROW_BYTES / 1024 / W;   // 1 KB pieces per wave
    static_assert(PW >= 1 && PW * W * 1024 == ROWS * T::ROW_BYTES, "the block must split evenly");
    const uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(dst);
    const int soff = row0 * row_stride;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int piece = wave * PW + j;
        const int bi = piece * 64 + lane;
        const int row = bi / T::R, blk = (bi % T::R) ^ (VL ? v_swz<D>(row) : k_swz<D>(row));
        dma16(base + piece * 1024, rsrc, row * row_stride + blk * 16, soff);
    }
}

// Copies keys [kbase, min(kbase + 64, kend)) of a staged K/V tile into the pool slot
// rows (pk, pv: the slot's K and V rows 0.., of P8 ? 1 : 2 bytes per element), undoing
// the LDS swizzles: whole rows, 16 bytes of the tile per lane (as E4M3 codes, 8 bytes),
// rows at or past kend untouched.
template <int D, int W, bool P8>
__device__ __forceinline__ void tile_to_pool(const LDS_AS char *tile, void *pk, void *pv, int kbase, int kend,
                                             int tid) {
    using T = Tile<D>;
    constexpr int BLOCKS = kTK * T::R;   // 16-byte blocks of one matrix
#pragma unroll
    for (int i0 = 0; i0 < BLOCKS; i0 += W * 64) {
        const int i = i0 + tid;
        const int key = i / T::R, blk = i % T::R;
        if (i < BLOCKS && kbase + key < kend) {
            const u32x4 kx = *reinterpret_cast<const LDS_AS u32x4 *>(tile + key * T::ROW_BYTES +
                                                                     ((blk ^ k_swz<D>(key)) * 16));
            const u32x4 vx = *reinterpret_cast<const LDS_AS u32x4 *>(tile + T::MAT_BYTES + key * T::ROW_BYTES +
                                                                     ((blk ^ v_swz<D>(key)) * 16));
            const long off = (long)(kbase + key) * D + blk * 8;   // in elements
            if constexpr (P8) {
                *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(pk) + off) = e4m3x8_from_bf16x8(kx);
                *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(pv) + off) = e4m3x8_from_bf16x8(vx);
            } else {
                *reinterpret_cast<u32x4 *>(static_cast<bf16 *>(pk) + off) = kx;
                *reinterpret_cast<u32x4 *>(static_cast<bf16 *>(pv) + off) = vx;
            }
        }
    }
}

// Per-wave attention state.
template <int D>
struct WaveState {
    static constexpr int QB = query_blocks<D>();
    bf16x8 qreg[QB][Tile<D>::KC];   // B operand: query rows wq0 + qb*32 + col, dims cc*16 + g*8 ..
    f32x16 acc[Tile<D>::DB][QB];    // O^T accumulators: lane = query, 16 head dims per block
    float m[QB];                    // running max (log2 domain), shared by both lane halves
    float l[QB];                    // this lane half's share of the row sum
};

// Per-lane LDS addressing of the operand reads, fixed for the whole kernel.
template <int D>
struct LaneAddr {
    int k_off0;                 // K operand: row col of the block
    int k_xor[Tile<D>::KC];     // swizzled 16-byte block 2*cc + g of that row
    int v_off;                  // V transpose loads: key 4g + i/4, byte (i%2)*8 of the block
    int v_blk[Tile<D>::DB];     // swizzled block of head dims db*32 + 16*sub + 4*(i%4)
};

template <int D>
__device__ __forceinline__ LaneAddr<D> lane_addr(int lane) {
    using T = Tile<D>;
    const int col = lane & 31, g = lane >> 5;
    LaneAddr<D> la;
    la.k_off0 = col * T::ROW_BYTES;
#pragma unroll
    for (int cc = 0; cc < T::KC; ++cc) la.k_xor[cc] = ((2 * cc + g) ^ k_swz<D>(col)) * 16;
    // V transpose loads: in 16-lane group (g, sub), lane i addresses key 4g + i/4 (plus the
    // chunk's key base) and head dims db*32 + 16*sub + 4*(i%4) .. +3.
    const int ti = lane & 15, sub = (lane >> 4) & 1;
    const int vkey = 4 * g + (ti >> 2);
    la.v_off = vkey * T::ROW_BYTES + (ti & 1) * 8;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        la.v_blk[db] = ((db * 4 + 2 * sub + ((ti & 3) >> 1)) ^ v_swz<D>(vkey)) * 16;
    return la;
}

// ------------------------------------------------------------------ one 64-key tile
// Scores are held transposed, [key block kb][query block qb]: element i of lane (col, g)
// of block (kb, qb) is the score of query wq0 + qb*32 + col against key kbase + kb*32 +
// 4g + off(i), off(i) = 8*(i/4) + i%4.

// S^T = K Q^T for key block kb of one tile (the tile's K rows in LDS at kt): KC MFMAs
// per query block.
template <int D>
__device__ __forceinline__ void block_scores(f32x16 (&sc)[query_blocks<D>()], const WaveState<D> &ws,
                                             const LDS_AS char *kt, const LaneAddr<D> &la, int kb) {
    using T = Tile<D>;
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) sc[qb] = f32x16{};
    bf16x8 ka[T::KC];
#pragma unroll
    for (int cc = 0; cc < T::KC; ++cc)
        ka[cc] = *reinterpret_cast<const LDS_AS bf16x8 *>(kt + la.k_off0 + kb * 32 * T::ROW_BYTES + la.k_xor[cc]);
#pragma unroll
    for (int cc = 0; cc < T::KC; ++cc)
#pragma unroll
        for (int qb = 0; qb < query_blocks<D>(); ++qb)
            sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cc], ws.qreg[qb][cc], sc[qb], 0, 0, 0);
    if (D >= 128) {
        // All of the block's operand reads first, then its MFMAs: left to itself the
        // compiler keeps two operands in flight and each MFMA waits out an LDS latency.
        __builtin_amdgcn_sched_group_barrier(0x100, T::KC, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, T::KC * query_blocks<D>(), 0);
    }
}

// Sets to -inf the scores of key block kb at or past kend and, for the prefill, of keys
// after the query: element i is visible iff off(i) <= lim.
template <int D, bool PREFILL>
__device__ __forceinline__ void block_mask(f32x16 (&sc)[query_blocks<D>()], int kbase, int kend, int wq0, int col,
                                           int g, int kb) {
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        const int base = kbase + kb * 32 + 4 * g;
        int lim = kend - 1 - base;
        if (PREFILL) lim = min(lim, wq0 + qb * 32 + col - base);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int off = 8 * (i >> 2) + (i & 3);
            sc[qb][i] = off > lim ? -INFINITY : sc[qb][i];
        }
    }
}

// P = exp2(s*c - m) for key block kb against the current running max m, rounded to bf16
// in the B-operand layout of the PV MFMA, pb[chunk of 16 keys][qb]; lsum[qb] takes the
// rounded values (so that the normaliser matches the weights the PV product uses).
template <int D>
__device__ __forceinline__ void tile_exp(bf16x8 (&pb)[2][query_blocks<D>()], float (&lsum)[query_blocks<D>()],
                                         const f32x16 (&sc)[2][query_blocks<D>()], int kb, const WaveState<D> &ws,
                                         float c) {
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        const float nm = -ws.m[qb];
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
                lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum[qb], false);
            }
            pb[c2][qb] = p;
        }
    }
}

// Lazy rescale, per 32-key block.  The running max m of a row only has to keep the
// weights in range: a key block is first evaluated against the current m, and only a
// row whose lane sum of weights exceeds kFastSumLimit, or is not finite (m = -inf
// before the row's first block), moves m to max(m, block max), scales its accumulator
// and row sum by exp2(m_old - m_new) and re-evaluates the block.  With the limit at 2^64
// a weight never exceeds 2^64, so for histories up to 2^20 keys the fp32 row sum and
// accumulators stay below 2^84 |v|: far from overflow, and the bf16 weights keep their
// full relative precision.  In practice only a row's first block takes the slow path.
// The decision is per row (both lane halves of a row agree), so a row's arithmetic
// never depends on the other rows of the wave; the branch is wave-wide.  Working per key
// block lets the PV product of one block run on the matrix cores while the vector ALU
// computes the weights of the next.
constexpr float kFastSumLimit = 18446744073709551616.0f;   // 2^64

template <int D>
__device__ __forceinline__ void block_softmax(bf16x8 (&pb)[2][query_blocks<D>()], WaveState<D> &ws,
                                              const f32x16 (&sc)[2][query_blocks<D>()], int kb, float c) {
    using T = Tile<D>;
    constexpr int QB = query_blocks<D>();
    float lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] = 0.f;
    tile_exp<D>(pb, lsum, sc, kb, ws, c);
    bool slow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) slow |= !(lsum[qb] <= kFastSumLimit);
    if (__any(slow)) {
        // keeps the compiler from flattening this rare path into the hot block
        asm volatile("" ::: "memory");
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mine = !(lsum[qb] <= kFastSumLimit) ? 1.f : 0.f;
            const bool grow = half_max(mine) > 0.f;   // either half of the row
            float mx = sc[kb][qb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[kb][qb][i]);
            const float mt = half_max(mx) * c;
            const float mn = grow ? fmaxf(ws.m[qb], mt) : ws.m[qb];
            const float alpha = grow ? __builtin_amdgcn_exp2f(ws.m[qb] - mn) : 1.f;
            ws.l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) ws.acc[db][qb] *= alpha;
            ws.m[qb] = mn;
            lsum[qb] = 0.f;
        }
        tile_exp<D>(pb, lsum, sc, kb, ws, c);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ws.l[qb] += lsum[qb];
}

// O^T += V^T P^T for key block kb of the tile (its V rows in LDS at vt).  Lane (d, g)
// needs, for chunk c2, V at keys kb*32 + 16*c2 + {4g..4g+3} (elements 0..3) and
// kb*32 + 16*c2 + 8 + {4g..4g+3} (elements 4..7): two transpose loads of 4 keys x 16
// dims each.
template <int D>
__device__ __forceinline__ void tile_pv(WaveState<D> &ws, const bf16x8 (&pb)[2][query_blocks<D>()], int kb, const LDS_AS char *vt,
                                        const LaneAddr<D> &la) {
    using T = Tile<D>;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            const LDS_AS char *src = vt + la.v_off + la.v_blk[db] + (kb * 32 + 16 * c2) * T::ROW_BYTES;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)src);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(src + 8 * T::ROW_BYTES));
            const i16x4 lh[2] = {lo, hi};
            const bf16x8 va = __builtin_bit_cast(bf16x8, lh);
#pragma unroll
            for (int qb = 0; qb < query_blocks<D>(); ++qb)
                ws.acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c2][qb], ws.acc[db][qb], 0, 0, 0);
        }
}

// One whole tile for one wave: scores, optional mask, then per 32-key block the weights
// with the lazy rescale and the PV product.
template <int D, bool PREFILL>
__device__ __forceinline__ void tile_step(WaveState<D> &ws, const LDS_AS char *kt, const LDS_AS char *vt,
                                          int kbase, int kend, int wq0, bool masked,
                                          const LaneAddr<D> &la, int col, int g, float c) {
    f32x16 sc[2][query_blocks<D>()];
    block_scores<D>(sc[0], ws, kt, la, 0);
    block_scores<D>(sc[1], ws, kt, la, 1);
    if (masked) {
        block_mask<D, PREFILL>(sc[0], kbase, kend, wq0, col, g, 0);
        block_mask<D, PREFILL>(sc[1], kbase, kend, wq0, col, g, 1);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        bf16x8 pb[2][query_blocks<D>()];
        block_softmax<D>(pb, ws, sc, kb, c);
        tile_pv<D>(ws, pb, kb, vt, la);
    }
}

// Runs the wave over K/V tiles 0 .. ntiles-1.  next_tile(u) makes tile u current (wait
// for its DMA, workgroup barrier, further DMA) and returns its LDS buffer; every wave
// calls it for every tile.  The wave computes tiles 0 .. tlast only (tlast < 0: none).
// Tiles that reach kend (or, for the prefill, cross the causal diagonal) are masked.
template <int D, bool PREFILL, class NextTile>
__device__ __forceinline__ void run_tiles(WaveState<D> &ws, int ntiles, int tlast, int kend, int wq0,
                                          const LaneAddr<D> &la, int col, int g, float c, NextTile &&next_tile) {
    using T = Tile<D>;
    for (int t = 0; t < ntiles; ++t) {
        const LDS_AS char *kt = next_tile(t);
        if (t <= tlast) {
            const bool masked = t * kTK + kTK > kend || (PREFILL && t * kTK + kTK - 1 > wq0);
            tile_step<D, PREFILL>(ws, kt, kt + T::MAT_BYTES, t * kTK, kend, wq0, masked, la, col, g, c);
        }
    }
}

// The wave's rows of a staged row block (dma_rows), read into the B-operand layout
// of the score MFMA: lane (col, g) gets row qb*32 + col, dims 16cc + 8g .. +7.  The
// wave's rows start at a multiple of 32, so k_swz(row) = k_swz(col).
template <int D>
__device__ __forceinline__ void staged_operand(bf16x8 (&r)[query_blocks<D>()][Tile<D>::KC], const LDS_AS char *rows,
                                               const LaneAddr<D> &la) {
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb)
#pragma unroll
        for (int cc = 0; cc < Tile<D>::KC; ++cc)
            r[qb][cc] = *reinterpret_cast<const LDS_AS bf16x8 *>(rows + la.k_off0 + qb * 32 * Tile<D>::ROW_BYTES +
                                                               la.k_xor[cc]);
}

// Element (row qb*32 + col, dims d0 .. d0+3) of a staged row block, d0 = db*32 + 8j + 4g:
// logical block 4db + j, bytes 8g .. 8g+7 of it.
template <int D>
__device__ __forceinline__ int staged_acc_off(int qb, int db, int j, int col, int g) {
    return (qb * 32 + col) * Tile<D>::ROW_BYTES + (((db * 4 + j) ^ k_swz<D>(col)) * 16) + 8 * g;
}

// Normalises the wave's O^T and stores it as bf16 rows of o (rows < qlimit).  The rows go
// through the wave's own region of LDS first, so that the global stores write whole
// rows: 16 bytes per lane, 64 / R rows per instruction.
template <int D>
__device__ __forceinline__ void store_o(const WaveState<D> &ws, LDS_AS char *stage, bf16 *odst, int qlimit, int wq0,
                                        int col, int g, int lane, int row_stride) {
    using T = Tile<D>;
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        const float inv = 1.f / half_sum(ws.l[qb]);
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (bf16)(ws.acc[db][qb][4 * j + e] * inv);
                *reinterpret_cast<LDS_AS bf16x4 *>(stage + staged_acc_off<D>(qb, db, j, col, g)) = ov;
            }
    }
    constexpr int RPI = 64 / T::R;   // rows per store instruction
    const int blk = lane % T::R;
#pragma unroll
    for (int i = 0; i < wave_rows<D>() / RPI; ++i) {
        const int row = i * RPI + lane / T::R;
        const u32x4 v = *reinterpret_cast<const LDS_AS u32x4 *>(stage + row * T::ROW_BYTES +
                                                                ((blk ^ k_swz<D>(row)) * 16));
        if (wq0 + row < qlimit) *reinterpret_cast<u32x4 *>(odst + (long)(wq0 + row) * row_stride + blk * 8) = v;
    }
}

// The candidate's own key, score s_j = scale*log2(e) * qc_j . kc_j, merged after the
// history.  On the bf16 pool the own keys arrive with the values at the end of the
// stream, so the history starts from an empty state (m = -inf) and the merge moves the
// max to max(m, s_j), scaling what the history summed by exp2(m - m'); on the E4M3 pool
// the own score starts the running max (m = s_j) and the merge weight exp2(s_j - m) is
// at most 1.  An empty history yields vc_j exactly on both, and for finite inputs
// nothing of another candidate reaches a candidate's output.  kc and vc come from staged
// row blocks.
template <int D>
__device__ __forceinline__ void self_key_score(const WaveState<D> &ws, float (&sself)[query_blocks<D>()],
                                               const LDS_AS char *kc_rows, const LaneAddr<D> &la, float c) {
    bf16x8 kk[query_blocks<D>()][Tile<D>::KC];
    staged_operand<D>(kk, kc_rows, la);
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        float part = 0.f;
#pragma unroll
        for (int cc = 0; cc < Tile<D>::KC; ++cc)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 qa = {ws.qreg[qb][cc][e], ws.qreg[qb][cc][e + 1]};
                const bf16x2 ka = {kk[qb][cc][e], kk[qb][cc][e + 1]};
                part = __builtin_amdgcn_fdot2_f32_bf16(qa, ka, part, false);
            }
        sself[qb] = half_sum(part) * c;
    }
}

// The state before any key: no max yet, empty sums.
template <int D>
__device__ __forceinline__ void reset_state(WaveState<D> &ws) {
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        ws.m[qb] = -INFINITY;
        ws.l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < Tile<D>::DB; ++db) ws.acc[db][qb] = f32x16{};
    }
}

// The own score, which then starts the running max (the E4M3 path).
template <int D>
__device__ __forceinline__ void self_key_scores(WaveState<D> &ws, float (&sself)[query_blocks<D>()],
                                                const LDS_AS char *kc_rows, const LaneAddr<D> &la, float c) {
    self_key_score<D>(ws, sself, kc_rows, la, c);
    reset_state<D>(ws);
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) ws.m[qb] = sself[qb];
}

// Adds the own key: weight w_j = exp2(s_j - m) on vc_j.  While every row of the wave has
// s_j <= m + 64 (the lazy bound of the history's weights) the max stays; otherwise
// (an own score far above the history's, or an empty history with m = -inf) each row
// moves it to max(m, s_j) and scales its sums by exp2(m - m').  The weight is rounded to
// bf16 like the history's, counted once in the row sum, and vc_j w_j enters O^T through
// the matrix cores: O^T += Vc^T diag(w) over the wave's 32 candidates, with vc staged in
// the V layout and diag(w) built in the register layout of the P^T operand (lane (col,
// g) element e stands for key 16 c2 + 4 g + e, or 8 + 4 g + e - 4 for e >= 4).  An empty
// history gives w = 1 and vc_j exactly; for finite inputs nothing of another candidate
// reaches a row (its terms are vc times an exact zero).
template <int D>
__device__ __forceinline__ void self_key_merge(WaveState<D> &ws, const float (&sself)[query_blocks<D>()],
                                               const LDS_AS char *vc_rows, const LaneAddr<D> &la, int col, int g) {
    using T = Tile<D>;
    constexpr int QB = query_blocks<D>();
    bool far = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) far |= !(sself[qb] <= ws.m[qb] + 64.f);
    if (__any(far)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mn = fmaxf(ws.m[qb], sself[qb]);
            const float alpha = __builtin_amdgcn_exp2f(ws.m[qb] - mn);
            ws.m[qb] = mn;
            ws.l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) ws.acc[db][qb] *= alpha;
        }
    }
    // lane (col, g) holds its row's weight at chunk col / 16, element e* when g matches
    const int r = col & 15;
    const bool mine = g == ((r >> 2) & 1);
    const int estar = (r & 3) + ((r >> 3) << 2);
    bf16x8 pd[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const bf16 w = (bf16)__builtin_amdgcn_exp2f(sself[qb] - ws.m[qb]);
        ws.l[qb] += g == 0 ? (float)w : 0.f;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pd[c2][qb][e] = (mine && (col >> 4) == c2 && e == estar) ? w : (bf16)0.f;
    }
    tile_pv<D>(ws, pd, 0, vc_rows, la);
}

__device__ __forceinline__ bool user_valid(const AttnArgs &a, int N, int s, bool report) {
    const bool bad_len = N < 0 || N > a.len_limit;
    const bool bad_slot = s < 0 || s >= a.S;
    if ((bad_len || bad_slot) && report && threadIdx.x == 0)
        atomicOr(a.status, (bad_len ? kFlagBadLen : 0u) | (bad_slot ? kFlagBadSlot : 0u));
    return !(bad_len || bad_slot);
}

// ------------------------------------------------------------------ longest-first schedules
// Both kernels hand their blocks out longest history first, so that the long (user,
// head) pairs start at once and the short ones fill the CUs at the end, and the prefill
// launches no block for query tiles past a history.  The order is by the key
// ceil(len / 64) (the history's 64-row tiles), descending, ties by user index; a length
// outside [0, limit] ranks as the longest (its blocks only raise the flag).  Every wave
// loads the keys of all B users (up to kOrderUsers, one register per 64 users) and
// finds the user of a rank by a binary search over key values, one ballot per 64 users
// per probe.  Beyond kOrderUsers users the blocks keep the user order.
constexpr int kOrderUsers = 256;

struct UserKeys {
    int key[kOrderUsers / 64];   // this lane's users lane, 64 + lane, ...; -1 past B
    int len[kOrderUsers / 64];   // their lengths and slots (read only when asked for)
    int slot[kOrderUsers / 64];
    int chunks, kmax;
};

// slots may be null (the slots are then not loaded).
__device__ __forceinline__ UserKeys load_keys(const int32_t *__restrict__ lens, const int32_t *__restrict__ slots,
                                              int B, int limit) {
    UserKeys k;
    k.chunks = (B + 63) / 64;
    k.kmax = (limit + kTK - 1) / kTK;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < kOrderUsers / 64; ++c) {
        const int u = c * 64 + lane;
        k.len[c] = u < B ? lens[u] : 0;
        k.slot[c] = (slots && u < B) ? slots[u] : 0;
    }
#pragma unroll
    for (int c = 0; c < kOrderUsers / 64; ++c) {
        const int u = c * 64 + lane, N = k.len[c];
        k.key[c] = u >= B ? -1 : (N < 0 || N > limit) ? k.kmax : (N + kTK - 1) / kTK;
    }
    return k;
}

// User b's length and slot out of the loaded registers (wave-uniform b < B).
__device__ __forceinline__ void user_len_slot(const UserKeys &k, int b, int &N, int &s) {
    const int c = b >> 6, l = b & 63;
    N = s = 0;
#pragma unroll
    for (int i = 0; i < kOrderUsers / 64; ++i)
        if (i == c) {
            N = __builtin_amdgcn_readlane(k.len[i], l);
            s = __builtin_amdgcn_readlane(k.slot[i], l);
        }
}

// Users whose key is at least K (wave-uniform).
__device__ __forceinline__ int users_key_ge(const UserKeys &k, int K) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < kOrderUsers / 64; ++c)
        if (c < k.chunks) n += __builtin_popcountll(__ballot(k.key[c] >= K));
    return n;
}

// The user at rank r (0 <= r < B) of the longest-first order (wave-uniform).
__device__ __forceinline__ int user_at_rank(const UserKeys &k, int r) {
    int lo = 0, hi = k.kmax;   // the rank's key: the largest K with more than r users at >= K
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (users_key_ge(k, mid) > r) lo = mid;
        else hi = mid - 1;
    }
    int j = r - users_key_ge(k, lo + 1);   // its place among the users with key lo
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < kOrderUsers / 64; ++c) {
        if (c >= k.chunks) break;
        const unsigned long long m = __ballot(k.key[c] == lo);
        const int n = __builtin_popcountll(m);
        if (j < n) {
            const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
            const unsigned long long pick = __ballot(((m >> lane) & 1) && below == j);
            return c * 64 + __builtin_ctzll(pick);
        }
        j -= n;
    }
    return r;   // not reached for 0 <= r < B
}

// Whether a user other than b with a valid, non-empty history (1 .. limit rows) names
// slot s (wave-uniform b and s): then both prefills write the slot and race.  One
// ballot per 64 users.
__device__ __forceinline__ bool slot_shared(const int32_t *__restrict__ lens, const int32_t *__restrict__ slots,
                                            int B, int b, int s, int limit) {
    const int lane = threadIdx.x & 63;
    bool dup = false;
    for (int u0 = 0; u0 < B && !dup; u0 += 64) {
        const int u = u0 + lane;
        const int n = u < B ? lens[u] : 0;
        const int su = u < B ? slots[u] : -1;
        dup = __ballot(u != b && n > 0 && n <= limit && su == s) != 0;
    }
    return dup;
}

// ------------------------------------------------------------------ causal prefill

// Maps the linear block id to (user*H + head, query tile).  With xcd_remap, blocks are
// dispatched round-robin over the 8 XCDs and every (user, head) stays on one XCD, so
// that its K/V is fetched from HBM once into that XCD's L2 and re-read from there by its
// other tiles.  TILE_MAJOR hands out tile 0 of every (user, head) first, then tile 1,
// and so on (the prefill's tiles differ in cost and the heaviest come first); otherwise
// the tiles of one (user, head) are consecutive.
template <bool TILE_MAJOR>
__device__ __forceinline__ void block_coords(const AttnArgs &a, int &group, int &tile) {
    const int bid = blockIdx.x;
    const int G = a.B * a.H;
    if (a.xcd_remap) {
        const int xcd = bid & 7, local = bid >> 3, gx = G >> 3;
        if (TILE_MAJOR) {
            group = (local % gx) * 8 + xcd;
            tile = local / gx;
        } else {
            group = (local / a.tiles) * 8 + xcd;
            tile = local % a.tiles;
        }
    } else if (TILE_MAJOR) {
        group = bid % G;
        tile = bid / G;
    } else {
        group = bid / a.tiles;
        tile = bid % a.tiles;
    }
}

// Waits until the DMA step issued `after` (0 .. 3) steps before the most recent one has
// landed, i.e. with after * DPW of this wave's pieces still allowed in flight.
template <int DPW>
__device__ __forceinline__ void wait_pieces_after(int after) {
    if (after >= 3) wait_vmcnt<3 * DPW>();
    else if (after == 2) wait_vmcnt<2 * DPW>();
    else if (after == 1) wait_vmcnt<DPW>();
    else wait_vmcnt<0>();
}

template <int D, bool P8>
__device__ __forceinline__ void prefill_body(const AttnArgs &a, const int32_t *__restrict__ lens,
                                             const int32_t *__restrict__ slots) {
    using T = Tile<D>;
    constexpr int W = block_waves<D>();
    constexpr int QT = W * wave_rows<D>();
    constexpr int DPW = KvDma<D, W>::PER_WAVE;
    static_assert(QT % kTK == 0, "a query tile must cover whole key tiles");
    static_assert(QT * T::ROW_BYTES == 2 * T::BUF_BYTES, "a 256-row block fills two slots");
    __shared__ __attribute__((aligned(1024))) char smem_raw[kBufs * T::BUF_BYTES];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    int b, h, qtile, N, s;
    if (a.B <= kOrderUsers) {
        // Rounds q = tiles-1 .. 0 of query tile q, longest histories first; a round holds
        // all heads of the users with more than q * 256 rows (key above 4 q).  Blocks past
        // the last round have nothing to do.
        static_assert(QT == 4 * kTK, "a query tile is four key tiles");
        const UserKeys keys = load_keys(lens, slots, a.B, a.len_limit);
        int rem = blockIdx.x;
        qtile = -1;
        for (int q = a.tiles - 1; q >= 0; --q) {
            const int items = users_key_ge(keys, 4 * q + 1) * a.H;
            if (rem < items) {
                qtile = q;
                break;
            }
            rem -= items;
        }
        if (qtile < 0) return;
        b = user_at_rank(keys, rem / a.H);
        h = rem % a.H;
        user_len_slot(keys, b, N, s);
    } else {
        int group, tile;
        block_coords<true>(a, group, tile);
        b = group / a.H;
        h = group % a.H;
        if (b >= a.B) return;
        qtile = a.tiles - 1 - tile;   // heaviest (last) query tiles first
        N = lens[b];
        s = slots[b];
    }
    // One block per (user, head) reports an invalid user: in the longest-first schedule
    // the one of tile 0, which every user with history rows (and every invalid length,
    // ranked longest) has; in user order the one of the last tile.  An empty history
    // writes nothing, and its slot is left to the ranking decode's check.
    if (!user_valid(a, N, s, a.B <= kOrderUsers ? qtile == 0 : qtile == a.tiles - 1)) return;
    const int q0 = qtile * QT;
    if (q0 >= N) return;
    // two users writing one slot: one block per user (its first query tile, head 0)
    // raises the flag; both prefills still run
    if (qtile == 0 && h == 0 && slot_shared(lens, slots, a.B, b, s, a.len_limit) && threadIdx.x == 0)
        atomicOr(a.status, kFlagDupSlot);

    const long in_off = (long)b * a.in_bstride + (long)h * a.in_hstride;
    const int in_rs = a.in_rstride * (int)sizeof(bf16);   // bytes between rows of q, k, v
    const bf16 *qsrc = static_cast<const bf16 *>(a.q) + in_off;
    const bf16 *ksrc = static_cast<const bf16 *>(a.k) + in_off;
    const bf16 *vsrc = static_cast<const bf16 *>(a.v) + in_off;
    bf16 *odst = static_cast<bf16 *>(a.o) + (long)b * a.out_bstride + (long)h * a.out_hstride;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    void *pk = static_cast<char *>(a.pool_k) + slot_off * (P8 ? 1 : (long)sizeof(bf16));
    void *pv = static_cast<char *>(a.pool_v) + slot_off * (P8 ? 1 : (long)sizeof(bf16));
    const int kend = min(q0 + QT, N);
    const int ntiles = (kend + kTK - 1) / kTK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int wq0 = q0 + wave * wave_rows<D>();
    // This wave's K/V DMA source: the K or the V rows of the history, rows >= kend read as 0.
    const i32x4 rsrc = rsrc_words(wave < W / 2 ? ksrc : vsrc, (uint32_t)kend * in_rs);
    int voff[DPW];
    dma_offsets<D, W>(voff, wave, lane, in_rs);
    const LaneAddr<D> la = lane_addr<D>(lane);

    // The block's query rows go to the last two slots, the first K/V tiles to the others;
    // tile t lives in slot t % kBufs.
    dma_rows<D, W, kBlockRows>(smem + (kBufs - 2) * T::BUF_BYTES, rsrc_words(qsrc, (uint32_t)N * in_rs), q0, wave,
                               lane, in_rs);
    int issued = 0;
    for (; issued < kBufs - 2 && issued < ntiles; ++issued)
        dma_tile<D, W>(smem + issued * T::BUF_BYTES, rsrc, issued * kTK, voff, wave, in_rs);
    wait_pieces_after<DPW>(issued);
    __syncthreads();

    WaveState<D> ws;
    staged_operand<D>(ws.qreg, smem + (kBufs - 2) * T::BUF_BYTES + wave * wave_rows<D>() * T::ROW_BYTES, la);
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        ws.m[qb] = -INFINITY;
        ws.l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) ws.acc[db][qb] = f32x16{};
    }

    // A wave skips tiles wholly after its last query but keeps taking part in the tile
    // barriers and DMA.  Making tile t current lets the DMA run up to tile t+kBufs-1,
    // into the slot of tile t-1 (or, for t = 0, the slots the query rows came from).
    const int tlast = wq0 < N ? min(ntiles - 1, (wq0 + wave_rows<D>() - 1) / kTK) : -1;
    // Tiles from q0 on hold the block's own history rows: while such a tile is current,
    // the workgroup also writes it into the pool slot.  (The pool stores count in vmcnt
    // like the DMA and only make the next waits longer, never shorter.)
    auto next_tile = [&](int t) -> const LDS_AS char * {
        wait_pieces_after<DPW>(issued - t - 1);
        __syncthreads();
        for (; issued < ntiles && issued <= t + kBufs - 1; ++issued)
            dma_tile<D, W>(smem + (issued % kBufs) * T::BUF_BYTES, rsrc, issued * kTK, voff, wave, in_rs);
        const LDS_AS char *cur = smem + (t % kBufs) * T::BUF_BYTES;
        if (t * kTK >= q0) tile_to_pool<D, W, P8>(cur, pk, pv, t * kTK, kend, tid);
        return cur;
    };
    run_tiles<D, true>(ws, ntiles, tlast, kend, wq0, la, col, g, a.c, next_tile);
    __syncthreads();   // every wave is done with the tile slots
    store_o<D>(ws, smem + wave * wave_rows<D>() * T::ROW_BYTES, odst, N, wq0, col, g, lane, a.out_rstride);
}

// ------------------------------------------------------------------ ranking decode

// E4M3 K/V tiles.  A tile of codes (K: kTK rows of D bytes, then V) is DMA'd as it is,
// 1 KB per wave-wide piece in plain row order, into a staging area; the workgroup then
// decodes it into the bf16 tile layout (rows of 16-byte blocks at the K and V
// swizzles) that the tile step reads.  An E4M3 value is exact in bf16: one conversion
// instruction turns two codes into two bf16 values.
template <int D, int W>
struct F8Tile {
    static constexpr int MAT = kTK * D;                 // bytes of one staged matrix
    static constexpr int BYTES = 2 * MAT;               // K then V
    static constexpr int PER_WAVE = BYTES / 1024 / W;   // DMA pieces per wave
    static_assert(PER_WAVE >= 1 && PER_WAVE * W * 1024 == BYTES, "an E4M3 tile must split evenly over the waves");
    static_assert(2 * BYTES == Tile<D>::BUF_BYTES, "two staged E4M3 tiles fill one LDS slot");
};

// DMA of this wave's share of E4M3 tile keys kbase .. kbase+63 (plain row order) into
// `stage`; waves 0 .. W/2-1 move K, the others V, from `rsrc`.
template <int D, int W>
__device__ __forceinline__ void dma_tile8(LDS_AS char *stage, i32x4 rsrc, int kbase, int wave, int lane) {
    using F = F8Tile<D, W>;
    const bool is_v = wave >= W / 2;
    const int first = (wave % (W / 2)) * F::PER_WAVE;   // piece index inside the matrix
    const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(stage) + (is_v ? F::MAT : 0) + first * 1024;
#pragma unroll
    for (int j = 0; j < F::PER_WAVE; ++j) dma16(dst + j * 1024, rsrc, ((first + j) * 64 + lane) * 16, kbase * D);
}

// Decodes a staged E4M3 tile into the bf16 tile at `tile`: 16-byte output blocks (8
// values), one per thread per pass.
template <int D, int W>
__device__ __forceinline__ void decode_tile8(const LDS_AS char *stage, LDS_AS char *tile, int tid) {
    using T = Tile<D>;
    using F = F8Tile<D, W>;
    constexpr int BLOCKS = 2 * kTK * T::R;
    static_assert(BLOCKS % (W * 64) == 0, "blocks must split evenly over the threads");
#pragma unroll
    for (int i0 = 0; i0 < BLOCKS; i0 += W * 64) {
        const int i = i0 + tid;
        const int mat = i / (kTK * T::R), key = (i / T::R) % kTK, blk = i % T::R;
        const u32x2 raw = *reinterpret_cast<const LDS_AS u32x2 *>(stage + mat * F::MAT + key * D + blk * 8);
        const u32x2 a = e4m3x4_to_bf16x4(raw[0]), b = e4m3x4_to_bf16x4(raw[1]);
        const u32x4 out = {a[0], a[1], b[0], b[1]};
        const int swz = mat ? v_swz<D>(key) : k_swz<D>(key);
        *reinterpret_cast<LDS_AS u32x4 *>(tile + mat * T::MAT_BYTES + key * T::ROW_BYTES + (blk ^ swz) * 16) = out;
    }
}

// One workgroup per item: (user, head, 256-candidate tile).  The candidate rows arrive
// by DMA like the K/V tiles: q and kc first (slots 0-1 and 2-3: the queries and the own
// key's score), then a stream of steps through the ring, step u in slot u % kBufs:
// the K/V tiles 0 .. ntiles-1, then the two 128-row halves of vc, so that the own
// key's values load in the background while the history is processed.
template <int D, bool P8>
__device__ __forceinline__ void decode_body(const AttnArgs &a, const int32_t *__restrict__ lens,
                                            const int32_t *__restrict__ slots) {
    using T = Tile<D>;
    constexpr int W = block_waves<D>();
    constexpr int QT = W * wave_rows<D>();
    constexpr int DPW = KvDma<D, W>::PER_WAVE;
    constexpr int HALF = kBlockRows / 2;
    static_assert(QT * T::ROW_BYTES == 2 * T::BUF_BYTES, "a 256-row block fills two slots");
    static_assert(HALF * T::ROW_BYTES / 1024 / W == DPW, "a vc half block moves like one K/V tile");
    __shared__ __attribute__((aligned(1024))) char smem_raw[kBufs * T::BUF_BYTES];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    int group, ctile;
    block_coords<false>(a, group, ctile);
    if (group >= a.B * a.H) return;
    // the group's rank in the longest-first order of the users, and its head
    const bool ordered = a.B <= kOrderUsers;
    UserKeys keys;
    if (ordered) keys = load_keys(lens, slots, a.B, a.len_limit);
    const int b = ordered ? user_at_rank(keys, group / a.H) : group / a.H;
    const int h = group % a.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int row0 = ctile * QT;
    const int wq0 = row0 + wave * wave_rows<D>();
    const int qlimit = a.rows;
    const bool active = wq0 < qlimit;
    const long in_off = (long)b * a.in_bstride + (long)h * a.in_hstride;
    const int in_rs = a.in_rstride * (int)sizeof(bf16);   // bytes between candidate rows
    const uint32_t rows_bytes = (uint32_t)a.rows * in_rs;
    // The candidates' q (and, for the E4M3 pool, their own keys) do not depend on the
    // user's slot or history length: their DMA goes out before those are read, so the two
    // loads overlap.  A user with an invalid slot or length waits for that DMA before it
    // leaves (no LDS write may outlive the workgroup).  On the bf16 pool q goes to slots
    // 2 and 3, and the first two steps of the stream follow in the same round trip.
    const i32x4 rsrc_kc = rsrc_words(static_cast<const bf16 *>(a.k) + in_off, rows_bytes);
    dma_rows<D, W, kBlockRows>(smem + (P8 ? 0 : 2 * T::BUF_BYTES),
                               rsrc_words(static_cast<const bf16 *>(a.q) + in_off, rows_bytes), row0, wave, lane, in_rs);
    if constexpr (P8) dma_rows<D, W, kBlockRows>(smem + 2 * T::BUF_BYTES, rsrc_kc, row0, wave, lane, in_rs);
    int N, s;
    if (ordered) {
        user_len_slot(keys, b, N, s);
    } else {
        N = lens[b];
        s = slots[b];
    }
    if (!user_valid(a, N, s, ctile == 0)) {
        wait_vmcnt<0>();
        return;
    }
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;   // in elements
    constexpr int PROW = P8 ? D : T::ROW_BYTES;                      // bytes of one pool row
    const i32x4 rsrc = rsrc_words(static_cast<const char *>(wave < W / 2 ? a.pool_k : a.pool_v) + slot_off * (PROW / D),
                                  (uint32_t)N * PROW);
    const i32x4 rsrc_vc = rsrc_words(static_cast<const bf16 *>(a.v) + in_off, rows_bytes);
    int voff[DPW];
    dma_offsets<D, W>(voff, wave, lane, T::ROW_BYTES);   // the pool's K/V rows
    const LaneAddr<D> la = lane_addr<D>(lane);
    const int ntiles = (N + kTK - 1) / kTK;
    const int wrows = wave * wave_rows<D>() * T::ROW_BYTES;   // this wave's rows inside a staged block
    WaveState<D> ws;
    float sself[query_blocks<D>()];

    if constexpr (!P8) {
        // Steps: the ntiles K/V tiles of the history, then per half hv of the candidates
        // (waves hv*W/2 ..) its own keys and its values, 128 rows each.  Step u lives in
        // slot u % kBufs; steps 0 and 1 went out with q (in slots 2 and 3).  The own key
        // is merged last: the running max starts empty and the merge moves it.
        const int nsteps = ntiles + 4;
        auto issue = [&](int u) {
            LDS_AS char *dst = smem + (u % kBufs) * T::BUF_BYTES;
            if (u < ntiles) {
                dma_tile<D, W>(dst, rsrc, u * kTK, voff, wave, T::ROW_BYTES);
            } else {
                const int e = u - ntiles;   // 0: own keys of half 0, 1: values of half 0, 2, 3: half 1
                if (e & 1) dma_rows<D, W, HALF, true>(dst, rsrc_vc, row0 + (e >> 1) * HALF, wave, lane, in_rs);
                else dma_rows<D, W, HALF>(dst, rsrc_kc, row0 + (e >> 1) * HALF, wave, lane, in_rs);
            }
        };
        int issued = 0;
        for (; issued < 2; ++issued) issue(issued);
        wait_pieces_after<DPW>(issued);   // q has landed
        __syncthreads();
        staged_operand<D>(ws.qreg, smem + 2 * T::BUF_BYTES + wrows, la);
        reset_state<D>(ws);
        // Makes step u current: waits for its DMA, workgroup barrier (after which the slot
        // of step u-1, and for u = 0 the q slots, are free), and lets the DMA run up to
        // step u+kBufs-1.
        auto next_step = [&](int u) -> const LDS_AS char * {
            wait_pieces_after<DPW>(issued - u - 1);
            __syncthreads();
            for (; issued < nsteps && issued <= u + kBufs - 1; ++issued) issue(issued);
            return smem + (u % kBufs) * T::BUF_BYTES;
        };
        run_tiles<D, false>(ws, ntiles, active ? ntiles - 1 : -1, N, wq0, la, col, g, a.c, next_step);
        const int hrows = (wave % (W / 2)) * wave_rows<D>() * T::ROW_BYTES;   // this wave's rows in its half
        // one barrier per half: making the values current also covers the own keys, one
        // step older (the DMA issue is the same as with a barrier per step)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
            const LDS_AS char *vc_half = next_step(ntiles + 2 * hv + 1);
            const LDS_AS char *kc_half = smem + ((ntiles + 2 * hv) % kBufs) * T::BUF_BYTES;
            if (active && wave / (W / 2) == hv) {
                self_key_score<D>(ws, sself, kc_half + hrows, la, a.c);
                self_key_merge<D>(ws, sself, vc_half + hrows, la, col, g);
            }
        }
    } else {
        wait_vmcnt<0>();
        __syncthreads();
        staged_operand<D>(ws.qreg, smem + wrows, la);
        self_key_scores<D>(ws, sself, smem + 2 * T::BUF_BYTES + wrows, la, a.c);
        __syncthreads();   // the header slots are free again
        // E4M3 pool.  LDS: slot 0 the current tile decoded to bf16, slot 1 two staged
        // E4M3 tiles (tile t at half t % 2), slots 2 and 3 the two vc halves.  DMA order
        // per wave: tiles 0 and 1, then one tile per step (tile t + 2 after tile t is
        // decoded), then both vc halves once no tile is left to issue.
        using F = F8Tile<D, W>;
        constexpr int FP = F::PER_WAVE;   // this wave's pieces per staged tile
        LDS_AS char *stage = smem + T::BUF_BYTES;
        LDS_AS char *cur = smem;
        auto issue_vc = [&]() {
            dma_rows<D, W, HALF, true>(smem + 2 * T::BUF_BYTES, rsrc_vc, row0, wave, lane, in_rs);
            dma_rows<D, W, HALF, true>(smem + 3 * T::BUF_BYTES, rsrc_vc, row0 + HALF, wave, lane, in_rs);
        };
        if (ntiles > 0) dma_tile8<D, W>(stage, rsrc, 0, wave, lane);
        if (ntiles > 1) dma_tile8<D, W>(stage + F::BYTES, rsrc, kTK, wave, lane);
        if (ntiles == 0) issue_vc();
        auto next_tile8 = [&](int t) -> const LDS_AS char * {
            // pieces of this wave issued after tile t: tile t + 1 while it exists; at the
            // last tile of two or more, the vc halves (issued one step earlier)
            if (t + 1 < ntiles) wait_vmcnt<FP>();
            else if (ntiles >= 2) wait_vmcnt<2 * DPW>();
            else wait_vmcnt<0>();
            __syncthreads();   // tile t has landed; every wave is done with slot 0
            decode_tile8<D, W>(stage + (t % 2) * F::BYTES, cur, tid);
            __syncthreads();   // slot 0 holds tile t; its staging half is free
            if (t + 2 < ntiles) dma_tile8<D, W>(stage + (t % 2) * F::BYTES, rsrc, (t + 2) * kTK, wave, lane);
            else if (t + 2 == ntiles || (ntiles == 1 && t == 0)) issue_vc();
            return cur;
        };
        run_tiles<D, false>(ws, ntiles, active ? ntiles - 1 : -1, N, wq0, la, col, g, a.c, next_tile8);
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
            if (hv == 0) wait_vmcnt<DPW>();
            else wait_vmcnt<0>();
            __syncthreads();
            const LDS_AS char *vc_half = smem + (2 + hv) * T::BUF_BYTES;
            if (active && wave / (W / 2) == hv)
                self_key_merge<D>(ws, sself, vc_half + (wave % (W / 2)) * wave_rows<D>() * T::ROW_BYTES, la, col, g);
        }
    }
    __syncthreads();   // every wave is done with the slots
    store_o<D>(ws, smem + wrows, static_cast<bf16 *>(a.o) + (long)b * a.out_bstride + (long)h * a.out_hstride, qlimit,
               wq0, col, g, lane, a.out_rstride);
}

// ------------------------------------------------------------------ split ranking decode
// For few (user, head) pairs the candidate tiles alone do not fill the GPU: each tile's
// history is then split over `parts` workgroups.  Part p takes the 64-key tiles
// p * part_tiles .. of the slot and runs the decode's tile loop over them (the same tile
// step, with the key end counted from the part's first tile); it leaves each candidate
// row's running max, row sum and unnormalised accumulator (fp32) in the workspace.  The
// merge then adds the own key and normalises: the online softmax over the parts' states
// and one more key.  bf16 or E4M3 pool (P8), contiguous q, k, v and o.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, bool P8>
__device__ __forceinline__ void decode_part_body(const AttnArgs &a, const int32_t *__restrict__ lens,
                                                 const int32_t *__restrict__ slots) {
    using T = Tile<D>;
    constexpr int W = block_waves<D>();
    constexpr int QT = W * wave_rows<D>();
    constexpr int DPW = KvDma<D, W>::PER_WAVE;
    static_assert(QT * T::ROW_BYTES == 2 * T::BUF_BYTES, "a 256-row block fills two slots");
    __shared__ __attribute__((aligned(1024))) char smem_raw[kBufs * T::BUF_BYTES];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    const int item = blockIdx.x / a.parts, part = blockIdx.x % a.parts;
    const int group = item / a.tiles, ctile = item % a.tiles;
    if (group >= a.B * a.H) return;
    const int b = group / a.H, h = group % a.H;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int row0 = ctile * QT;
    const int wq0 = row0 + wave * wave_rows<D>();
    const bool active = wq0 < a.rows;
    const long in_off = (long)b * a.in_bstride + (long)h * a.in_hstride;
    const int in_rs = a.in_rstride * (int)sizeof(bf16);
    const uint32_t rows_bytes = (uint32_t)a.rows * in_rs;
    // q to slots 2 and 3 (its DMA overlaps the reads of the length and slot)
    dma_rows<D, W, kBlockRows>(smem + 2 * T::BUF_BYTES, rsrc_words(static_cast<const bf16 *>(a.q) + in_off, rows_bytes),
                               row0, wave, lane, in_rs);
    const int N = lens[b], s = slots[b];
    if (!user_valid(a, N, s, ctile == 0 && part == 0)) {
        wait_vmcnt<0>();
        return;
    }
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;   // in elements
    constexpr int PROW = P8 ? D : T::ROW_BYTES;                      // bytes of one pool row
    const i32x4 rsrc = rsrc_words(static_cast<const char *>(wave < W / 2 ? a.pool_k : a.pool_v) + slot_off * (PROW / D),
                                  (uint32_t)N * PROW);
    const LaneAddr<D> la = lane_addr<D>(lane);
    const int ntiles = (N + kTK - 1) / kTK;
    const int t0 = part * a.part_tiles;
    const int nt = max(min(ntiles, t0 + a.part_tiles) - t0, 0);   // this part's tiles
    const int wrows = wave * wave_rows<D>() * T::ROW_BYTES;
    WaveState<D> ws;
    if constexpr (!P8) {
        // step u: the part's tile t0 + u, in slot u % kBufs; steps 0 and 1 go out with q
        int voff[DPW];
        dma_offsets<D, W>(voff, wave, lane, T::ROW_BYTES);
        auto issue = [&](int u) {
            dma_tile<D, W>(smem + (u % kBufs) * T::BUF_BYTES, rsrc, (t0 + u) * kTK, voff, wave, T::ROW_BYTES);
        };
        int issued = 0;
        for (; issued < 2 && issued < nt; ++issued) issue(issued);
        wait_pieces_after<DPW>(issued);   // q has landed
        __syncthreads();
        staged_operand<D>(ws.qreg, smem + 2 * T::BUF_BYTES + wrows, la);
        reset_state<D>(ws);
        auto next_step = [&](int u) -> const LDS_AS char * {
            wait_pieces_after<DPW>(issued - u - 1);
            __syncthreads();
            for (; issued < nt && issued <= u + kBufs - 1; ++issued) issue(issued);
            return smem + (u % kBufs) * T::BUF_BYTES;
        };
        run_tiles<D, false>(ws, nt, active ? nt - 1 : -1, N - t0 * kTK, wq0, la, col, g, a.c, next_step);
    } else {
        // E4M3 pool: slot 0 holds the current tile decoded to bf16, slot 1 two staged
        // tiles of codes (the part's tile t0 + u at half u % 2).  Tiles 0 and 1 go out
        // right after q (slots 2 and 3); tile u + 2 once tile u is decoded.
        using F = F8Tile<D, W>;
        constexpr int FP = F::PER_WAVE;   // this wave's pieces per staged tile
        LDS_AS char *stage = smem + T::BUF_BYTES;
        LDS_AS char *cur = smem;
        auto issue8 = [&](int u) { dma_tile8<D, W>(stage + (u % 2) * F::BYTES, rsrc, (t0 + u) * kTK, wave, lane); };
        if (nt > 0) issue8(0);
        if (nt > 1) issue8(1);
        // q has landed once at most the staged tiles' pieces are in flight
        if (nt > 1) wait_vmcnt<2 * FP>();
        else if (nt == 1) wait_vmcnt<FP>();
        else wait_vmcnt<0>();
        __syncthreads();
        staged_operand<D>(ws.qreg, smem + 2 * T::BUF_BYTES + wrows, la);
        reset_state<D>(ws);
        auto next_tile8 = [&](int u) -> const LDS_AS char * {
            if (u + 1 < nt) wait_vmcnt<FP>();   // tile u + 1 may still be in flight
            else wait_vmcnt<0>();
            __syncthreads();   // tile u has landed; every wave is done with slot 0
            decode_tile8<D, W>(stage + (u % 2) * F::BYTES, cur, tid);
            __syncthreads();   // slot 0 holds tile u; its staging half is free
            if (u + 2 < nt) issue8(u + 2);
            return cur;
        };
        run_tiles<D, false>(ws, nt, active ? nt - 1 : -1, N - t0 * kTK, wq0, la, col, g, a.c, next_tile8);
    }
    // the state of the wave's rows: accumulators (lane (col, g) holds head dims
    // db*32 + 8j + 4g .. +3 of row col), then (m, l) from the lanes of half 0
    const long pbase = ((long)item * a.parts + part) * QT;
    float *acc_out = a.part_state;
    float *ml_out = a.part_state + (long)a.B * a.H * a.tiles * a.parts * QT * D;
#pragma unroll
    for (int qb = 0; qb < query_blocks<D>(); ++qb) {
        const long r = pbase + wave * wave_rows<D>() + qb * 32 + col;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {ws.acc[db][qb][4 * j], ws.acc[db][qb][4 * j + 1], ws.acc[db][qb][4 * j + 2],
                                 ws.acc[db][qb][4 * j + 3]};
                *reinterpret_cast<f32x4 *>(acc_out + r * D + db * 32 + 8 * j + 4 * g) = v;
            }
        const float lrow = half_sum(ws.l[qb]);
        if (g == 0) *reinterpret_cast<f32x2 *>(ml_out + 2 * r) = f32x2{ws.m[qb], lrow};
    }
}

// The merge: per candidate row (b, h, j), the parts' states and the own key (score
// scale * qc_j . kc_j, value vc_j) merged in fp32 and normalised.  D / 2 lanes serve a
// row, lane d of them head dims 2d and 2d + 1 (a wave takes 1, 2 or 4 rows at D = 128, 64
// or 32), so that every load and store moves two values.  A user with an invalid length
// or slot is skipped, as by the one-pass decode.
template <int D>
constexpr int merge_rows_per_wave() { return 128 / D; }

template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(AttnArgs a, const int32_t *__restrict__ lens,
                                                           const int32_t *__restrict__ slots) {
    constexpr int QT = block_waves<D>() * wave_rows<D>();
    constexpr int LPR = D / 2;   // lanes per row
    static_assert(64 % LPR == 0, "a wave holds whole rows");
    const int lane = threadIdx.x & 63;
    const int dl = lane % LPR;
    const long row = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * merge_rows_per_wave<D>() + lane / LPR;
    if (row >= (long)a.B * a.H * a.rows) return;   // whole rows leave together
    const int j = (int)(row % a.rows);
    const int group = (int)(row / a.rows), b = group / a.H, h = group % a.H;
    const int N = lens[b], s = slots[b];
    if (N < 0 || N > a.len_limit || s < 0 || s >= a.S) return;
    const long item = (long)group * a.tiles + j / QT;
    const long in_row = (long)b * a.in_bstride + (long)h * a.in_hstride + (long)j * a.in_rstride + 2 * dl;
    const bf16x2 q2 = *reinterpret_cast<const bf16x2 *>(static_cast<const bf16 *>(a.q) + in_row);
    const bf16x2 k2 = *reinterpret_cast<const bf16x2 *>(static_cast<const bf16 *>(a.k) + in_row);
    const bf16x2 v2 = *reinterpret_cast<const bf16x2 *>(static_cast<const bf16 *>(a.v) + in_row);
    float dot = __builtin_amdgcn_fdot2_f32_bf16(q2, k2, 0.f, false);
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);   // within the row's lanes
    const float sself = dot * a.c;   // log2 domain, like the parts' maxima
    const float *accs = a.part_state;
    const float *mls = a.part_state + (long)a.B * a.H * a.tiles * a.parts * QT * D;
    const long r0 = item * a.parts * QT + j % QT;   // the row's state in part 0; part p is p * QT further
    float m = sself;
    for (int p = 0; p < a.parts; ++p) m = fmaxf(m, mls[2 * (r0 + (long)p * QT)]);
    const float ws = __builtin_amdgcn_exp2f(sself - m);
    float l = ws, acc0 = (float)v2[0] * ws, acc1 = (float)v2[1] * ws;
    for (int p = 0; p < a.parts; ++p) {
        const long r = r0 + (long)p * QT;
        const f32x2 ml = *reinterpret_cast<const f32x2 *>(mls + 2 * r);
        const float f = __builtin_amdgcn_exp2f(ml[0] - m);   // 0 for a part with no key (m = -inf)
        const f32x2 st = *reinterpret_cast<const f32x2 *>(accs + r * D + 2 * dl);
        l = __builtin_fmaf(ml[1], f, l);
        acc0 = __builtin_fmaf(st[0], f, acc0);
        acc1 = __builtin_fmaf(st[1], f, acc1);
    }
    const float inv = 1.f / l;
    const bf16x2 out = {(bf16)(acc0 * inv), (bf16)(acc1 * inv)};
    *reinterpret_cast<bf16x2 *>(static_cast<bf16 *>(a.o) + (long)b * a.out_bstride + (long)h * a.out_hstride +
                                (long)j * a.out_rstride + 2 * dl) = out;
}

template <int D, bool P8>
__global__ void __launch_bounds__(block_waves<D>() * 64, min_waves_per_simd<D>()) rank_decode_part_kernel(AttnArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ slots) {
    decode_part_body<D, P8>(a, lens, slots);
}

template <int D, bool P8>
__global__ void __launch_bounds__(block_waves<D>() * 64, min_waves_per_simd<D>()) prefill_bf16_kernel(AttnArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ slots) {
    prefill_body<D, P8>(a, lens, slots);
}

template <int D, bool P8>
__global__ void __launch_bounds__(block_waves<D>() * 64, min_waves_per_simd<D>()) rank_decode_bf16_kernel(AttnArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ slots) {
    decode_body<D, P8>(a, lens, slots);
}

}  // namespace

int bf16_prefill_rows_per_block(int D) {
    (void)D;
    return kBlockRows;
}

int bf16_decode_rows_per_item(int D) {
    (void)D;
    return kBlockRows;
}

hipError_t launch_prefill_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream) {
    const long blocks = (long)a.B * a.H * a.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
#define UNIPIN_PREFILL(DD, P8) \
    hipLaunchKernelGGL((prefill_bf16_kernel<DD, P8>), grid, dim3(block_waves<DD>() * 64), 0, stream, a, a.lens, a.slot)
    switch (D) {
        case 32: if (pool8) return hipErrorInvalidValue; UNIPIN_PREFILL(32, false); break;
        case 64: if (pool8) UNIPIN_PREFILL(64, true); else UNIPIN_PREFILL(64, false); break;
        case 128: if (pool8) UNIPIN_PREFILL(128, true); else UNIPIN_PREFILL(128, false); break;
        default: return hipErrorInvalidValue;
    }
#undef UNIPIN_PREFILL
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream) {
    const long items = (long)a.B * a.H * a.tiles;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)items);
#define UNIPIN_DECODE(DD, P8) \
    hipLaunchKernelGGL((rank_decode_bf16_kernel<DD, P8>), grid, dim3(block_waves<DD>() * 64), 0, stream, a, a.lens, a.slot)
    switch (D) {
        case 32: if (pool8) return hipErrorInvalidValue; UNIPIN_DECODE(32, false); break;
        case 64: if (pool8) UNIPIN_DECODE(64, true); else UNIPIN_DECODE(64, false); break;
        case 128: if (pool8) UNIPIN_DECODE(128, true); else UNIPIN_DECODE(128, false); break;
        default: return hipErrorInvalidValue;
    }
#undef UNIPIN_DECODE
    return hipGetLastError();
}

hipError_t launch_decode_split_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream) {
    const long items = (long)a.B * a.H * a.tiles * a.parts;
    const long rows = (long)a.B * a.H * a.rows;
    if (items <= 0 || rows <= 0) return hipSuccess;
    if (items > 0x7fffffffL || (rows + 3) / 4 > 0x7fffffffL || a.parts < 1 || a.part_tiles < 1 || !a.part_state)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)items);
    // merge: 4 waves per block, merge_rows_per_wave<D>() rows per wave
#define UNIPIN_SPLIT(DD, P8)                                                                                         \
    hipLaunchKernelGGL((rank_decode_part_kernel<DD, P8>), grid, dim3(block_waves<DD>() * 64), 0, stream, a, a.lens,  \
                       a.slot);                                                                                      \
    hipLaunchKernelGGL((decode_merge_kernel<DD>),                                                                    \
                       dim3((unsigned)((rows + 4 * merge_rows_per_wave<DD>() - 1) / (4 * merge_rows_per_wave<DD>()))), \
                       dim3(256), 0, stream, a, a.lens, a.slot)
    switch (D) {
        case 32: if (pool8) return hipErrorInvalidValue; UNIPIN_SPLIT(32, false); break;
        case 64: if (pool8) { UNIPIN_SPLIT(64, true); } else { UNIPIN_SPLIT(64, false); } break;
        case 128: if (pool8) { UNIPIN_SPLIT(128, true); } else { UNIPIN_SPLIT(128, false); } break;
        default: return hipErrorInvalidValue;
    }
#undef UNIPIN_SPLIT
    return hipGetLastError();
}

}  // namespace unipin
