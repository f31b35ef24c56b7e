// fp32 M-FALCON attention kernels for gfx950: the same two operations as the bf16
// kernels (causal prefill with the fused pool write; ranking decode over a pool slot
// with the candidate's own key fused), computed in fp32 on the vector ALUs.  This path
// keeps full fp32 precision (no reduced-precision matrix modes) and serves fp32 pools.
//
// One workgroup = one wave of 64 lanes = 64 query rows of one (user, head); each lane
// owns one query row, keeps q and the output accumulator in registers and walks the
// keys in 32-key tiles staged in LDS (every lane reads the same key row: LDS broadcast).
// Softmax is the online form in the log2 domain, rescaled per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace unipin {
namespace {

constexpr int kLanes = 64;
constexpr int kTK = 32;
static_assert(kLanes == kFp32RowsPerBlock, "rows per block must match the host's grid math");

template <int D, bool PREFILL>
__global__ void __launch_bounds__(kLanes) attn_fp32_kernel(AttnArgs a) {
    __shared__ float ks[kTK][D];
    __shared__ float vs[kTK][D];

    const int bid = blockIdx.x;
    const int group = bid / a.tiles, tile = bid % a.tiles;
    const int b = group / a.H, h = group % a.H;
    if (b >= a.B) return;
    const int N = a.lens[b];
    const int s = a.slot[b];
    if (N < 0 || N > a.len_limit || s < 0 || s >= a.S) {
        if (threadIdx.x == 0 && tile == 0)
            atomicOr(a.status, (N < 0 || N > a.len_limit ? kFlagBadLen : 0u) |
                                   (s < 0 || s >= a.S ? kFlagBadSlot : 0u));
        return;
    }
    const int q0 = tile * kLanes;
    const int qlimit = PREFILL ? N : a.rows;
    if (q0 >= qlimit) return;

    const long bh = (long)b * a.H + h;
    const float *qsrc = static_cast<const float *>(a.q) + bh * a.rows * D;
    float *odst = static_cast<float *>(a.o) + bh * a.rows * D;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    float *pk = static_cast<float *>(a.pool_k) + slot_off;
    float *pv = static_cast<float *>(a.pool_v) + slot_off;
    const float *ksrc = PREFILL ? static_cast<const float *>(a.k) + bh * a.rows * D : pk;
    const float *vsrc = PREFILL ? static_cast<const float *>(a.v) + bh * a.rows * D : pv;

    const int lane = threadIdx.x;
    const int row = q0 + lane;
    const bool valid = row < qlimit;

    // Fused pool write: this block's own history rows go to the slot, bit for bit.
    if (PREFILL && valid) {
        for (int d = 0; d < D; ++d) {
            pk[(long)row * D + d] = ksrc[(long)row * D + d];
            pv[(long)row * D + d] = vsrc[(long)row * D + d];
        }
    }

    float q[D], acc[D];
    for (int d = 0; d < D; ++d) q[d] = valid ? qsrc[(long)row * D + d] : 0.f;
    float m, l;
    if constexpr (PREFILL) {
        m = -INFINITY;
        l = 0.f;
        for (int d = 0; d < D; ++d) acc[d] = 0.f;
    } else {
        // The candidate's own key enters first (weight exp2(0) = 1, value vc_j).
        const float *kc = static_cast<const float *>(a.k) + bh * a.rows * D + (long)row * D;
        const float *vc = static_cast<const float *>(a.v) + bh * a.rows * D + (long)row * D;
        float self = 0.f;
        for (int d = 0; d < D; ++d) self = __builtin_fmaf(q[d], valid ? kc[d] : 0.f, self);
        m = self * a.c;
        l = 1.f;
        for (int d = 0; d < D; ++d) acc[d] = valid ? vc[d] : 0.f;
    }

    const int kend = PREFILL ? min(q0 + kLanes, N) : N;
    for (int kbase = 0; kbase < kend; kbase += kTK) {
        __syncthreads();
        for (int idx = lane; idx < kTK * D; idx += kLanes) {
            const int r = idx / D, d = idx % D;
            const int key = kbase + r;
            ks[r][d] = key < kend ? ksrc[(long)key * D + d] : 0.f;
            vs[r][d] = key < kend ? vsrc[(long)key * D + d] : 0.f;
        }
        __syncthreads();

        float sc[kTK];
        float mx = -INFINITY;
        for (int r = 0; r < kTK; ++r) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q[d], ks[r][d], dot);
            const int key = kbase + r;
            const bool off = key >= kend || (PREFILL && key > row);
            sc[r] = off ? -INFINITY : dot * a.c;
            mx = fmaxf(mx, sc[r]);
        }
        const float mn = fmaxf(m, mx);
        if (mn == -INFINITY) continue;  // nothing visible yet (rows past the history only)
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        m = mn;
        for (int r = 0; r < kTK; ++r) {
            const float p = __builtin_amdgcn_exp2f(sc[r] - m);
            l += p;
            for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vs[r][d], acc[d]);
        }
    }

    if (valid) {
        const float inv = 1.f / l;
        for (int d = 0; d < D; ++d) odst[(long)row * D + d] = acc[d] * inv;
    }
}

template <bool PREFILL>
hipError_t launch_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    const long blocks = (long)a.B * a.H * a.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kLanes);
    switch (D) {
        case 32: hipLaunchKernelGGL((attn_fp32_kernel<32, PREFILL>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((attn_fp32_kernel<64, PREFILL>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((attn_fp32_kernel<128, PREFILL>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_fp32<true>(a, D, stream);
}

hipError_t launch_decode_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_fp32<false>(a, D, stream);
}

}  // namespace unipin
