// Matrix products of the transformer block around the attention, for gfx950 (CDNA4):
// Y[M, N] = epilogue(X[M, K] W[K, N] + b), all row-major bf16, fp32 accumulation, on
// v_mfma_f32_32x32x16_bf16.  W is "x @ W" [fan_in, fan_out] as the block stores it.
//
//   * a workgroup computes a BM x BN tile of Y; its waves sit WM along the rows and WN
//     along the columns, and each holds 32*MB rows x 32*NB columns of the tile as MFMA
//     accumulators of Y^T = W^T X^T (the attention's O^T = V^T P^T);
//   * the contraction runs in KT-deep stages (32 or 64): the tile rows' KT columns of X
//     and the tile columns' KT rows of W arrive by buffer-to-LDS DMA in a ring of NS
//     stages, NS - 1 stages ahead of use; rows of X past M read as zero.  Each wave
//     moves a fixed share of every stage (XPW 1 KB pieces of X, WPW of W);
//   * X is read from LDS 16 bytes per lane as the B operand; W stays in its [k][n]
//     layout and ds_read_b64_tr_b16 delivers W^T as the A operand.  The operands of the
//     next 16-deep slice are read while the current slice's MFMAs run, across the stage
//     boundary too: the wait for the next stage and the workgroup barrier come before
//     the last slice of a stage is multiplied;
//   * the epilogue adds the bias and applies the tanh-form GELU or adds the residual (the
//     output's old value) in fp32, rounds once to bf16 and stores whole rows through LDS;
//     with a LayerNorm folded into the weights it first applies each row's mean and
//     1/std, which the workgroup sums from the X tiles as they pass through LDS (exactly,
//     from global memory, for a row whose mean is far above its spread);
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int WM, int WN, int MB, int NB, int KT, int NS>
struct GemmCfg {
    static constexpr int W = WM * WN;              // waves per workgroup
    static constexpr int BM = WM * 32 * MB;        // rows of Y per workgroup
    static constexpr int BN = WN * 32 * NB;        // columns of Y per workgroup
    static constexpr int KK = KT / 16;             // 16-deep slices per stage
    static constexpr int XROW = KT * 2;            // bytes of one X row within a stage
    static constexpr int XBLK = KT / 8;            // its 16-byte blocks
    static constexpr int WROW = BN * 2;            // bytes of one W row within a stage
    static constexpr int WBLK = BN / 8;
    static constexpr int XBYTES = BM * XROW;       // a stage: X, then W
    static constexpr int WBYTES = KT * WROW;
    static constexpr int SBYTES = XBYTES + WBYTES;
    static constexpr int XPW = XBYTES / 1024 / W;  // 1 KB DMA pieces per wave per stage
    static constexpr int WPW = WBYTES / 1024 / W;
    static constexpr int PW = XPW + WPW;
    static constexpr int OROW = NB * 64;           // bytes of one staged output row of a wave
    static constexpr int OBLK = NB * 4;
    static constexpr int STAGE_OUT = 32 * MB * OROW;
    static constexpr int TPR = W * 64 / BM;        // LayerNorm epilogues: threads per row of X
    static constexpr int BPT = XBLK / TPR;         // and the 16-byte blocks each takes per stage
    static_assert(KT == 32 || KT == 64, "stage depth");
    static_assert(TPR >= 1 && TPR <= 4 && 64 % TPR == 0 && BPT * TPR == XBLK, "row statistics split");
    static_assert(KK % 2 == 0, "every stage starts in operand buffer 0");
    static_assert(XPW * W * 1024 == XBYTES && WPW * W * 1024 == WBYTES && XPW >= 1 && WPW >= 1,
                  "a stage must split evenly over the waves");
    static_assert(NS * SBYTES >= W * STAGE_OUT, "the output staging must fit in the ring");
    static_assert(NS >= 2 && (NS - 2) * PW < 64, "vmcnt range");
    static_assert(BN >= 128, "W rows of at least 16 blocks (the W swizzle)");
};

// 16-byte block swizzles (XOR inside a row).  The X read serves 16 lanes at a time: 16
// consecutive rows, one logical block; the XOR puts them on 64 distinct banks (rows of
// 4 blocks: (row >> 2) & 3; rows of 8 blocks: (row >> 1) & 7).  The W transpose read
// serves 32 lanes at a time: 4 consecutive rows x 64 bytes; (row & 3) << 2 puts them on
// 64 distinct banks.
template <int XBLK>
__device__ __forceinline__ int x_swz(int row) {
    return XBLK == 4 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}
__device__ __forceinline__ int w_swz(int row) { return (row & 3) << 2; }

// Waits until at most `after` of this wave's stages are still in flight (loads complete
// in issue order); `after` never exceeds MAXA.
template <int PW, int MAXA>
__device__ __forceinline__ void wait_stages_after(int after) {
    if constexpr (MAXA == 0) {
        wait_vmcnt<0>();
    } else {
        if (after >= MAXA) wait_vmcnt<MAXA * PW>();
        else wait_stages_after<PW, MAXA - 1>(after);
    }
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), written as
// x / (1 + 2^z) with z = -2 log2(e) u = x (a + b x^2), which has no cancellation for
// large negative x.  The reciprocal is v_rcp_f32 (1 ulp), far below the bf16 rounding
// of the result, instead of a full-precision division.
__device__ __forceinline__ float gelu_tanh(float x) {
    constexpr float a = -2.f * 1.4426950408889634f * 0.7978845608028654f;
    constexpr float b = a * 0.044715f;
    const float z = x * __builtin_fmaf(b, x * x, a);
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
}

template <int WM, int WN, int MB, int NB, int KT, int NS, int WPS, int EPI>
__global__ void __launch_bounds__(WM *WN * 64, WPS)
    gemm_bf16_kernel(const bf16 *__restrict__ x, const bf16 *__restrict__ w, const void *__restrict__ bias_, bf16 *y,
                     int M, int N, int K, int mtiles) {
    using G = GemmCfg<WM, WN, MB, NB, KT, NS>;
    constexpr bool LN = EPI == kGemmLnBias || EPI == kGemmLnBiasGelu;
    // the ring, then (LayerNorm epilogues) the mean and 1/std of the tile's rows
    __shared__ __attribute__((aligned(1024))) char smem_raw[NS * G::SBYTES + (LN ? G::BM * 8 : 0)];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    const int ntn = N / G::BN;
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
    const int m0 = mt * G::BM, n0 = nt * G::BN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, g = lane >> 5;
    const int wm = wave / WN, wn = wave % WN;

    // DMA: X piece p of a stage (1 KB, lane l its 16-byte block 64 p + l in LDS order) is
    // X block 64 p + l (row / XBLK, swizzled); W piece p likewise (row / WBLK).  Wave v
    // moves X pieces v*XPW .. and W pieces v*WPW ...  X is addressed from row m0 on, so
    // that rows past M fall past the record count.
    const i32x4 xr = rsrc_words(x + (long)m0 * K, (uint32_t)((long)(M - m0) * K * 2));
    const i32x4 wr = rsrc_words(w + n0, (uint32_t)(((long)K * N - n0) * 2));
    int voff[G::PW];
#pragma unroll
    for (int q = 0; q < G::XPW; ++q) {
        const int bi = (wave * G::XPW + q) * 64 + lane, row = bi / G::XBLK;
        voff[q] = row * K * 2 + (((bi % G::XBLK) ^ x_swz<G::XBLK>(row)) * 16);
    }
#pragma unroll
    for (int q = 0; q < G::WPW; ++q) {
        const int bi = (wave * G::WPW + q) * 64 + lane, row = bi / G::WBLK;
        voff[G::XPW + q] = row * N * 2 + (((bi % G::WBLK) ^ w_swz(row)) * 16);
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    auto issue = [&](int s) {
        const uint32_t stage = lds0 + (uint32_t)((s % NS) * G::SBYTES);
        const int k0 = s * KT;
#pragma unroll
        for (int q = 0; q < G::XPW; ++q) dma16(stage + (wave * G::XPW + q) * 1024, xr, voff[q], k0 * 2);
#pragma unroll
        for (int q = 0; q < G::WPW; ++q)
            dma16(stage + G::XBYTES + (wave * G::WPW + q) * 1024, wr, voff[G::XPW + q], k0 * N * 2);
    };

    // operand reads: X rows of this wave; W transpose reads, 16-lane group (g, sub):
    // lane ti takes row 8g + ti/4 (and 4 rows on), bytes (ti & 1) * 8 of the block
    // holding columns db*32 + 16 sub + 4 (ti & 3) .. + 3
    const int xrow0 = wm * 32 * MB + col;
    const int ti = lane & 15, sub = (lane >> 4) & 1;
    const int wrow = 8 * g + (ti >> 2);
    const int w_off = wrow * G::WROW + (ti & 1) * 8;
    int w_blk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        w_blk[nb] = (((wn * NB + nb) * 4 + 2 * sub + ((ti & 3) >> 1)) ^ w_swz(wrow)) * 16;

    f32x16 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};

    // operands of two 16-deep slices: the one multiplied and the next one being read
    bf16x8 xb[2][MB], va[2][NB];
    auto read = [&](int s, int kk, int buf) {
        const LDS_AS char *xs = smem + (s % NS) * G::SBYTES;
        const LDS_AS char *ws = xs + G::XBYTES;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = xrow0 + mb * 32;
            xb[buf][mb] = *reinterpret_cast<const LDS_AS bf16x8 *>(xs + row * G::XROW +
                                                                  (((2 * kk + g) ^ x_swz<G::XBLK>(row)) * 16));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const LDS_AS char *src = ws + w_off + w_blk[nb] + kk * 16 * G::WROW;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)src);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(src + 4 * G::WROW));
            const i16x4 lh[2] = {lo, hi};
            va[buf][nb] = __builtin_bit_cast(bf16x8, lh);
        }
    };
    auto mfma = [&](int buf) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[buf][nb], xb[buf][mb], acc[nb][mb], 0, 0, 0);
    };

    // LayerNorm epilogues: the row statistics of X come from the stages as they pass
    // through LDS.  Thread t sums blocks (t % TPR)*BPT .. of row t / TPR of every stage:
    // the values and their squares, two v_dot2 per pair of values.  Such one-pass sums
    // lose the variance to cancellation only when a row's mean is far above its spread;
    // a row with mean^2 > 64 var is recomputed exactly (two passes over the row in global
    // memory) before the epilogue.
    const int srow = tid / G::TPR, spart = tid % G::TPR;
    float s1 = 0.f, s2 = 0.f;
    auto stats = [&](int s) {
        const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
        const LDS_AS char *xs = smem + (s % NS) * G::SBYTES + srow * G::XROW;
#pragma unroll
        for (int j = 0; j < G::BPT; ++j) {
            const u32x4 v = *reinterpret_cast<const LDS_AS u32x4 *>(
                xs + (((spart * G::BPT + j) ^ x_swz<G::XBLK>(srow)) * 16));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t word = v[e];   // a plain value first: a bit cast of the vector element reads element 0
                const bf16x2 p = __builtin_bit_cast(bf16x2, word);
                s1 = __builtin_amdgcn_fdot2_f32_bf16(p, ones, s1, false);
                s2 = __builtin_amdgcn_fdot2_f32_bf16(p, p, s2, false);
            }
        }
    };

    // Stage s + NS - 1 is issued into the slot of stage s - 1 once the barrier before
    // stage s has shown that every wave is done reading it.
    const int steps = K / KT;
    int issued = 0;
    for (; issued < NS - 1 && issued < steps; ++issued) issue(issued);
    wait_stages_after<G::PW, NS - 2>(issued - 1);
    __syncthreads();   // stage 0 has landed everywhere
    if (issued < steps) issue(issued++);
    read(0, 0, 0);
    if constexpr (LN) stats(0);
    for (int s = 0; s < steps; ++s) {
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < G::KK) {
                read(s, kk + 1, cur ^ 1);
            } else if (s + 1 < steps) {
                wait_stages_after<G::PW, NS - 2>(issued - s - 2);
                __syncthreads();   // stage s + 1 has landed everywhere; stage s is read
                if (issued < steps) issue(issued++);
                read(s + 1, 0, cur ^ 1);
                if constexpr (LN) stats(s + 1);
            }
            mfma(cur);
        }
    }

    // Epilogue.  Element i of acc[nb][mb] in lane (col, g) is Y[m][n] with m = m0 + wm*32*MB
    // + mb*32 + col, n = n0 + (wn*NB + nb)*32 + 8(i/4) + 4g + i%4.  Each wave stages its
    // 32*MB x 32*NB outputs as bf16 rows of OROW bytes (16-byte blocks swizzled by row),
    // then stores them as whole 16-byte pieces of rows.
    LDS_AS float *rstats = (LDS_AS float *)(smem + NS * G::SBYTES);
    if constexpr (LN) {
#pragma unroll
        for (int o = 1; o < G::TPR; o <<= 1) {
            s1 += __shfl_xor(s1, o);
            s2 += __shfl_xor(s2, o);
        }
        float mean = s1 / (float)K, var = s2 / (float)K - mean * mean;
        // the TPR threads of a row hold the same sums and take this branch together
        if (!(mean * mean <= 64.f * var) && m0 + srow < M) {
            const bf16 *row = x + (long)(m0 + srow) * K;
            float t = 0.f;
            for (int k = spart * 8; k < K; k += 8 * G::TPR) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(row + k);
#pragma unroll
                for (int e = 0; e < 4; ++e) t += __uint_as_float(v[e] << 16) + __uint_as_float(v[e] & 0xffff0000u);
            }
#pragma unroll
            for (int o = 1; o < G::TPR; o <<= 1) t += __shfl_xor(t, o);
            mean = t / (float)K;
            float q = 0.f;
            for (int k = spart * 8; k < K; k += 8 * G::TPR) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(row + k);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(v[e] << 16) - mean, hi = __uint_as_float(v[e] & 0xffff0000u) - mean;
                    q = __builtin_fmaf(lo, lo, __builtin_fmaf(hi, hi, q));
                }
            }
#pragma unroll
            for (int o = 1; o < G::TPR; o <<= 1) q += __shfl_xor(q, o);
            var = q / (float)K;
        }
        if (spart == 0) {
            rstats[2 * srow] = mean;
            rstats[2 * srow + 1] = 1.f / sqrtf(fmaxf(var, 0.f) + kGemmLnEps);
        }
    }
    __syncthreads();   // every wave is done with the ring (and the row statistics are written)
    LDS_AS char *stg = smem + wave * G::STAGE_OUT;
    const bf16 *bias = static_cast<const bf16 *>(bias_);
    const float *uv = static_cast<const float *>(bias_);   // LayerNorm epilogues: u[N], then v[N]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        // the bias of the column block, and for the residual the old outputs (a row past
        // M reads row M-1 instead, and its result is never stored), loaded together
        float bu[4][4], bv[4][4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int n = n0 + (wn * NB + nb) * 32 + 8 * jj + 4 * g;
            if constexpr (LN) {
                const f32x4 u4 = *reinterpret_cast<const f32x4 *>(uv + n), v4 = *reinterpret_cast<const f32x4 *>(uv + N + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bu[jj][e] = u4[e];
                    bv[jj][e] = v4[e];
                }
            } else {
                const bf16x4 b4 = *reinterpret_cast<const bf16x4 *>(bias + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[jj][e] = (float)b4[e];
            }
        }
        bf16x4 rv[4][MB];
        if (EPI == kGemmBiasResidual) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int m = min(m0 + wm * 32 * MB + mb * 32 + col, M - 1);
                    rv[jj][mb] = *reinterpret_cast<const bf16x4 *>(y + (long)m * N + n0 + (wn * NB + nb) * 32 +
                                                                   8 * jj + 4 * g);
                }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int r = mb * 32 + col;
                float mu = 0.f, rs = 1.f;
                if constexpr (LN) {
                    mu = rstats[2 * (wm * 32 * MB + r)];
                    rs = rstats[2 * (wm * 32 * MB + r) + 1];
                }
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // LN(x) W + b = rstd (x W' - mean u) + v, W' = diag(gamma) W, u its column sums
                    if constexpr (LN) v[e] = __builtin_fmaf(rs, __builtin_fmaf(-mu, bu[jj][e], acc[nb][mb][4 * jj + e]), bv[jj][e]);
                    else v[e] = acc[nb][mb][4 * jj + e] + bv[jj][e];
                    if (EPI == kGemmBiasGelu || EPI == kGemmLnBiasGelu) v[e] = gelu_tanh(v[e]);
                    if (EPI == kGemmBiasResidual) v[e] += (float)rv[jj][mb][e];
                }
                const bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};   // round to nearest even
                *reinterpret_cast<LDS_AS bf16x4 *>(stg + r * G::OROW + (((nb * 4 + jj) ^ (r & (G::OBLK - 1))) * 16) +
                                                   g * 8) = o;
            }
        }
    }
    asm volatile("" ::: "memory");   // a wave's LDS operations run in order: the reads see the writes
#pragma unroll
    for (int i = lane; i < 32 * MB * G::OBLK; i += 64) {
        const int r = i / G::OBLK, b = i % G::OBLK;
        const u32x4 val = *reinterpret_cast<const LDS_AS u32x4 *>(stg + r * G::OROW + ((b ^ (r & (G::OBLK - 1))) * 16));
        const int m = m0 + wm * 32 * MB + r;
        if (m < M) *reinterpret_cast<u32x4 *>(y + (long)m * N + n0 + wn * 32 * NB + b * 8) = val;
    }
}

template <int WM, int WN, int MB, int NB, int KT, int NS, int WPS>
hipError_t launch_cfg(const void *x, const void *w, const void *bias, void *y, int M, int N, int K, int epi,
                      hipStream_t stream) {
    using G = GemmCfg<WM, WN, MB, NB, KT, NS>;
    if (N % G::BN || K % KT) return hipErrorInvalidValue;
    const int mtiles = (M + G::BM - 1) / G::BM;
    const long ntn = N / G::BN;
    const long blocks = 8L * ((mtiles / 8) * ntn + ((mtiles % 8) * ntn + 7) / 8);
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(G::W * 64);
    const bf16 *xs = static_cast<const bf16 *>(x), *ws = static_cast<const bf16 *>(w);
    const void *bs = bias;
    bf16 *ys = static_cast<bf16 *>(y);
    switch (epi) {
        case kGemmBias:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, MB, NB, KT, NS, WPS, kGemmBias>), grid, block, 0, stream, xs,
                               ws, bs, ys, M, N, K, mtiles);
            break;
        case kGemmBiasGelu:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, MB, NB, KT, NS, WPS, kGemmBiasGelu>), grid, block, 0, stream,
                               xs, ws, bs, ys, M, N, K, mtiles);
            break;
        case kGemmBiasResidual:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, MB, NB, KT, NS, WPS, kGemmBiasResidual>), grid, block, 0,
                               stream, xs, ws, bs, ys, M, N, K, mtiles);
            break;
        case kGemmLnBias:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, MB, NB, KT, NS, WPS, kGemmLnBias>), grid, block, 0, stream,
                               xs, ws, bs, ys, M, N, K, mtiles);
            break;
        case kGemmLnBiasGelu:
            hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, MB, NB, KT, NS, WPS, kGemmLnBiasGelu>), grid, block, 0,
                               stream, xs, ws, bs, ys, M, N, K, mtiles);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The stage depth of each tile configuration (the contraction must be a multiple of it).
constexpr int kStageDepth[kGemmConfigs] = {32, 32, 32, 64};

}  // namespace

bool gemm_bf16_supported(long M, int N, int K, int cfg) {
    constexpr long kLim = 1L << 31;   // byte offsets of the buffer descriptors
    if (cfg < 0 || cfg >= kGemmConfigs) return false;
    return M >= 1 && N >= 128 && N % 128 == 0 && K >= kStageDepth[cfg] && K % kStageDepth[cfg] == 0 &&
           M * (long)K * 2 < kLim && (long)K * N * 2 < kLim && M * (long)N * 2 < kLim;
}

hipError_t launch_gemm_bf16(const void *x, const void *w, const void *bias, void *y, long M, int N, int K, int epi,
                            int cfg, hipStream_t stream) {
    if (!gemm_bf16_supported(M, N, K, cfg)) return hipErrorInvalidValue;
    switch (cfg) {
        // workgroup tiles 64, 128 and 256 x 128 with 32-deep stages (4, 4 and 8 waves of
        // 32 x 64, 64 x 64 and 64 x 64), and 128 x 128 with 64-deep stages (8 waves of
        // 64 x 32); LDS per workgroup 48, 64, 72 and 128 KB (3, 2, 2 and 1 workgroups
        // per CU: 3, 2, 4 and 2 waves per SIMD)
        case 0: return launch_cfg<2, 2, 1, 2, 32, 4, 3>(x, w, bias, y, (int)M, N, K, epi, stream);
        case 1: return launch_cfg<2, 2, 2, 2, 32, 4, 2>(x, w, bias, y, (int)M, N, K, epi, stream);
        case 2: return launch_cfg<4, 2, 2, 2, 32, 3, 4>(x, w, bias, y, (int)M, N, K, epi, stream);
        case 3: return launch_cfg<2, 4, 2, 1, 64, 4, 2>(x, w, bias, y, (int)M, N, K, epi, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace unipin
