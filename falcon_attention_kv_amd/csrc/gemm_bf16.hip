// Matrix products of the transformer block around the attention, for gfx950 (CDNA4):
// Y[M, N] = epilogue(X[M, K] W[K, N] + b), all row-major bf16, fp32 accumulation, on
// v_mfma_f32_32x32x16_bf16.  W is "x @ W" [fan_in, fan_out] as the block stores it.
//
//   * a workgroup computes a BM x 128 tile of Y (BM = 64, 128 or 256); its waves sit WM
//     along the rows and 2 along the columns, and each holds 32*MB rows x 64 columns of
//     the tile as MFMA accumulators of Y^T = W^T X^T (the attention's O^T = V^T P^T);
//   * the contraction runs in 32-deep steps: the tile rows' 32 columns of X and the tile
//     columns' 32 rows of W arrive by buffer-to-LDS DMA in a ring of NS stages, NS - 1
//     steps ahead of use; rows of X past M read as zero;
//   * X is read from LDS 16 bytes per lane as the B operand; W stays in its [k][n]
//     layout and ds_read_b64_tr_b16 delivers W^T as the A operand;
//   * the epilogue adds the bias and applies the tanh-form GELU or adds the residual (the
//     output's old value) in fp32, rounds once to bf16 and stores whole rows through LDS;
//   * workgroup b runs on XCD b % 8.  The column tiles of one row tile go to consecutive
//     workgroups of one XCD, so that they share its L2 copy of the X rows, for the first
//     8 floor(mtiles / 8) row tiles; the workgroups of the rest are spread over all XCDs,
//     so that no XCD holds a whole extra row tile (with 64 workgroup slots per XCD, one
//     row tile too many can cost a second round).
//
// The contraction index of an MFMA is spread over (lane / 32, element) the same way in
// A and B: a lane of half g holds k = 8g .. 8g + 7 of its 16-deep chunk.  The X read
// gives exactly that (one 16-byte block); the W transpose reads take rows 8g + e and
// 8g + 4 + e to match.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_launch.h"
#include "lds_dma.h"

namespace unipin {
namespace {

constexpr int kKT = 32;                 // contraction depth of one stage
constexpr int kBN = 128;                // columns of Y per workgroup
constexpr int kXRow = kKT * 2;          // bytes of one X row within a stage: 4 blocks of 16
constexpr int kWRow = kBN * 2;          // bytes of one W row within a stage: 16 blocks of 16
constexpr int kWStage = kKT * kWRow;    // 8 KB

// 16-byte block swizzles (XOR inside a row).  The X read serves 16 lanes at a time: 16
// consecutive rows, one logical block; (row >> 2) & 3 puts them on 64 distinct banks.
// The W transpose read serves 32 lanes at a time: 4 consecutive rows x 64 bytes;
// (row & 3) << 2 puts them on 64 distinct banks.
__device__ __forceinline__ int x_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int w_swz(int row) { return (row & 3) << 2; }

template <int WM, int MB, int NS>
struct GemmCfg {
    static constexpr int W = 2 * WM;                  // waves per workgroup
    static constexpr int BM = WM * 32 * MB;           // rows of Y per workgroup
    static constexpr int XBYTES = BM * kXRow;         // the X part of a stage
    static constexpr int SBYTES = XBYTES + kWStage;   // one stage: X, then W
    static constexpr int XP = XBYTES / 1024;          // 1 KB DMA pieces of X per stage
    static constexpr int PW = SBYTES / 1024 / W;      // pieces per wave per stage
    static constexpr int STAGE_OUT = 32 * MB * 128;   // one wave's output rows, bf16
    static_assert(PW * W * 1024 == SBYTES, "a stage must split evenly over the waves");
    static_assert(NS * SBYTES >= W * STAGE_OUT, "the output staging must fit in the ring");
    static_assert(NS >= 2 && NS <= 4, "waits cover up to three steps in flight");
};

// Waits until this wave's pieces of the step issued `after` steps before the newest
// have landed (loads complete in issue order).
template <int PW>
__device__ __forceinline__ void wait_steps_after(int after) {
    if (after >= 3) wait_vmcnt<3 * PW>();
    else if (after == 2) wait_vmcnt<2 * PW>();
    else if (after == 1) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), written as
// x / (1 + e^(-2u)), which has no cancellation for large negative x.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * x, x * x, x);
    return x / (1.f + __builtin_amdgcn_exp2f(-2.8853900817779268f * u));   // e^(-2u) = 2^(-2u log2 e)
}

template <int WM> constexpr int gemm_threads() { return 2 * WM * 64; }   // = GemmCfg::W * 64

template <int WM, int MB, int NS, int WPS, int EPI>
__global__ void __launch_bounds__(gemm_threads<WM>(), WPS)
    gemm_bf16_kernel(const bf16 *__restrict__ x, const bf16 *__restrict__ w, const bf16 *__restrict__ bias, bf16 *y,
                     int M, int N, int K, int mtiles) {
    using G = GemmCfg<WM, MB, NS>;
    __shared__ __attribute__((aligned(1024))) char smem_raw[NS * G::SBYTES];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    const int ntn = N / kBN;
    const int bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
    const int whole = (mtiles >> 3) * ntn;   // per XCD: workgroups of its whole row tiles
    int mt, nt;
    if (j < whole) {
        mt = xcd + 8 * (j / ntn);
        nt = j % ntn;
    } else {
        const int r = (j - whole) * 8 + xcd;   // the remaining row tiles' workgroups, in turn
        mt = (mtiles & ~7) + r / ntn;
        nt = r % ntn;
    }
    if (mt >= mtiles) return;
    const int m0 = mt * G::BM, n0 = nt * kBN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    // DMA: piece p of a stage (1 KB, lane l its 16-byte block 64 p + l in LDS order) is
    // X block p*64 + l (row / 4, swizzled) for p < XP, else W block (p - XP)*64 + l
    // (row / 16, swizzled).  X is addressed from row m0 on, so that rows past M fall
    // past the record count.
    const i32x4 xr = rsrc_words(x + (long)m0 * K, (uint32_t)((long)(M - m0) * K * 2));
    const i32x4 wr = rsrc_words(w + n0, (uint32_t)(((long)K * N - n0) * 2));
    int voff[G::PW];
#pragma unroll
    for (int q = 0; q < G::PW; ++q) {
        const int p = wave * G::PW + q;
        if (p < G::XP) {
            const int bi = p * 64 + lane, row = bi >> 2;
            voff[q] = row * K * 2 + (((bi & 3) ^ x_swz(row)) * 16);
        } else {
            const int bi = (p - G::XP) * 64 + lane, row = bi >> 4;
            voff[q] = row * N * 2 + (((bi & 15) ^ w_swz(row)) * 16);
        }
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    auto issue = [&](int s) {
        const uint32_t stage = lds0 + (uint32_t)((s % NS) * G::SBYTES);
        const int k0 = s * kKT;
#pragma unroll
        for (int q = 0; q < G::PW; ++q) {
            const int p = wave * G::PW + q;
            if (p < G::XP) dma16(stage + p * 1024, xr, voff[q], k0 * 2);
            else dma16(stage + p * 1024, wr, voff[q], k0 * N * 2);
        }
    };

    // operand reads: X rows of this wave; W transpose reads, 16-lane group (g, sub):
    // lane ti takes row 8g + ti/4 (and 4 rows on), bytes (ti & 1) * 8 of the block
    // holding columns db*32 + 16 sub + 4 (ti & 3) .. + 3
    const int xrow0 = wm * 32 * MB + col;
    const int ti = lane & 15, sub = (lane >> 4) & 1;
    const int wrow = 8 * g + (ti >> 2);
    const int w_off = wrow * kWRow + (ti & 1) * 8;
    int w_blk[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) w_blk[nb] = (((wn * 2 + nb) * 4 + 2 * sub + ((ti & 3) >> 1)) ^ w_swz(wrow)) * 16;

    f32x16 acc[2][MB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};

    const int steps = K / kKT;
    int issued = 0;
    for (; issued < NS - 1 && issued < steps; ++issued) issue(issued);
    for (int s = 0; s < steps; ++s) {
        wait_steps_after<G::PW>(issued - s - 1);
        __syncthreads();   // step s has landed everywhere; the slot of step s-1 is free
        if (issued < steps) issue(issued++);
        const LDS_AS char *xs = smem + (s % NS) * G::SBYTES;
        const LDS_AS char *ws = xs + G::XBYTES;
#pragma unroll
        for (int kk = 0; kk < kKT / 16; ++kk) {
            bf16x8 xb[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = xrow0 + mb * 32;
                xb[mb] = *reinterpret_cast<const LDS_AS bf16x8 *>(xs + row * kXRow + (((2 * kk + g) ^ x_swz(row)) * 16));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const LDS_AS char *src = ws + w_off + w_blk[nb] + kk * 16 * kWRow;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)src);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(src + 4 * kWRow));
                const i16x4 lh[2] = {lo, hi};
                const bf16x8 va = __builtin_bit_cast(bf16x8, lh);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, xb[mb], acc[nb][mb], 0, 0, 0);
            }
        }
    }

    // Epilogue.  Element i of acc[nb][mb] in lane (col, g) is Y[m][n] with m = m0 + wm*32*MB
    // + mb*32 + col, n = n0 + (wn*2 + nb)*32 + 8(i/4) + 4g + i%4.  Each wave stages its
    // 32*MB x 64 outputs as bf16 rows of 128 bytes (16-byte blocks swizzled by row & 7),
    // then stores them as whole 16-byte pieces of rows.
    __syncthreads();   // every wave is done with the ring
    LDS_AS char *stg = smem + wave * G::STAGE_OUT;
    // The epilogue's global loads go out together, one round trip per column block: the
    // bias of the wave's columns, and for the residual the old outputs (a row past M
    // reads row M-1 instead, and its result is never stored).
    bf16x4 bv[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            bv[nb][jj] = *reinterpret_cast<const bf16x4 *>(bias + n0 + (wn * 2 + nb) * 32 + 8 * jj + 4 * g);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        bf16x4 rv[4][MB];
        if (EPI == kGemmBiasResidual) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int m = min(m0 + wm * 32 * MB + mb * 32 + col, M - 1);
                    rv[jj][mb] = *reinterpret_cast<const bf16x4 *>(y + (long)m * N + n0 + (wn * 2 + nb) * 32 + 8 * jj +
                                                                   4 * g);
                }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int r = mb * 32 + col;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[nb][mb][4 * jj + e] + (float)bv[nb][jj][e];
                    if (EPI == kGemmBiasGelu) v[e] = gelu_tanh(v[e]);
                    if (EPI == kGemmBiasResidual) v[e] += (float)rv[jj][mb][e];
                }
                const bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};   // round to nearest even
                *reinterpret_cast<LDS_AS bf16x4 *>(stg + r * 128 + (((nb * 4 + jj) ^ (r & 7)) * 16) + g * 8) = o;
            }
        }
    }
    asm volatile("" ::: "memory");   // a wave's LDS operations run in order: the reads see the writes
#pragma unroll
    for (int i = lane; i < 32 * MB * 8; i += 64) {
        const int r = i >> 3, b = i & 7;
        const u32x4 val = *reinterpret_cast<const LDS_AS u32x4 *>(stg + r * 128 + ((b ^ (r & 7)) * 16));
        const int m = m0 + wm * 32 * MB + r;
        if (m < M) *reinterpret_cast<u32x4 *>(y + (long)m * N + n0 + wn * 64 + b * 8) = val;
    }
}

template <int WM, int MB, int NS, int WPS>
hipError_t launch_cfg(const void *x, const void *w, const void *bias, void *y, int M, int N, int K, int epi,
                      hipStream_t stream) {
    using G = GemmCfg<WM, MB, NS>;
    const int mtiles = (M + G::BM - 1) / G::BM;
    const long ntn = N / kBN;
    const long blocks = 8L * ((mtiles / 8) * ntn + ((mtiles % 8) * ntn + 7) / 8);
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(G::W * 64);
    const bf16 *xs = static_cast<const bf16 *>(x), *ws = static_cast<const bf16 *>(w),
               *bs = static_cast<const bf16 *>(bias);
    bf16 *ys = static_cast<bf16 *>(y);
    switch (epi) {
        case kGemmBias:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, MB, NS, WPS, kGemmBias>), grid, block, 0, stream, xs, ws, bs, ys,
                               M, N, K, mtiles);
            break;
        case kGemmBiasGelu:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, MB, NS, WPS, kGemmBiasGelu>), grid, block, 0, stream, xs, ws, bs,
                               ys, M, N, K, mtiles);
            break;
        case kGemmBiasResidual:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, MB, NS, WPS, kGemmBiasResidual>), grid, block, 0, stream, xs, ws,
                               bs, ys, M, N, K, mtiles);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool gemm_bf16_supported(long M, int N, int K) {
    constexpr long kLim = 1L << 31;   // byte offsets of the buffer descriptors
    return M >= 1 && N >= kBN && N % kBN == 0 && K >= kKT && K % kKT == 0 && M * (long)K * 2 < kLim &&
           (long)K * N * 2 < kLim && M * (long)N * 2 < kLim;
}

int gemm_bf16_rows_per_tile(int cfg) {
    switch (cfg) {
        case 0: return GemmCfg<2, 1, 4>::BM;
        case 1: return GemmCfg<2, 2, 4>::BM;
        case 2: return GemmCfg<4, 2, 3>::BM;
        default: return 0;
    }
}

hipError_t launch_gemm_bf16(const void *x, const void *w, const void *bias, void *y, long M, int N, int K, int epi,
                            int cfg, hipStream_t stream) {
    if (!gemm_bf16_supported(M, N, K)) return hipErrorInvalidValue;
    switch (cfg) {
        // LDS per workgroup 48, 64 and 72 KB: 3, 2 and 2 workgroups per CU (3, 2 and 4 waves per SIMD)
        case 0: return launch_cfg<2, 1, 4, 3>(x, w, bias, y, (int)M, N, K, epi, stream);
        case 1: return launch_cfg<2, 2, 4, 2>(x, w, bias, y, (int)M, N, K, epi, stream);
        case 2: return launch_cfg<4, 2, 3, 4>(x, w, bias, y, (int)M, N, K, epi, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace unipin
