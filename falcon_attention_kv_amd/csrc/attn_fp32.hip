// fp32 M-FALCON attention kernels for gfx950: the causal prefill with the fused pool
// write, the ranking decode over a pool slot with the candidate's own key fused, and
// the autoregressive step (UniPinRec review, sections 2.2 and 2.4; UniPinRec reading
// notes, sections 3 and 6).  This is the precision path of the library: the inputs and
// outputs are fp32, and everything in between -- the dot products, the score scale,
// the exponentials, the softmax state and the weighted sums of the values -- is fp64 on
// the vector ALUs, rounded to fp32 once at the output.  fp32 arithmetic would leave an
// output that the weights nearly cancel (|o| around 1e-3) with a relative error near
// 1e-4; in fp64 the error stays at the final rounding.
//
// A row group of G = D/16 consecutive lanes owns one query row, each lane 16 of its head
// dims (q as fp32, the accumulator as fp64); a workgroup holds 64 row groups.  The
// score of a key is the sum of the group's 16-dim partial dots (cross-lane exchanges).
//   * prefill and decode: group r takes query row q0 + r and walks the keys in 32-key
//     tiles staged in LDS as fp32; per tile it computes the scores, moves the running
//     max once and adds the weighted values;
//   * autoregressive step: one query row per (user, head); group r takes the slot rows
//     t with t % 64 == r with its own softmax state, and the 64 states are merged in LDS
//     at the end, with the new token's own key last.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace unipin {
namespace {

constexpr int kRows = 64;     // row groups per workgroup
constexpr int kTK = 32;       // keys per LDS tile
constexpr int kDS = 16;       // head dims per lane
static_assert(kRows == kFp32RowsPerBlock, "rows per block must match the host's grid math");

enum Mode { kPrefill, kDecode, kStep };

template <int D>
constexpr int group_lanes() { return D / kDS; }
template <int D>
constexpr int block_threads() { return kRows * group_lanes<D>(); }

// Sum of a group's partial values: G consecutive lanes, G a power of two dividing 64.
template <int G>
__device__ __forceinline__ double group_sum(double x) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ void load16(float (&r)[kDS], const float *src) {
#pragma unroll
    for (int i = 0; i < kDS; i += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(src + i);
        r[i] = v.x;
        r[i + 1] = v.y;
        r[i + 2] = v.z;
        r[i + 3] = v.w;
    }
}

__device__ __forceinline__ void store16(float *dst, const float (&r)[kDS]) {
#pragma unroll
    for (int i = 0; i < kDS; i += 4) *reinterpret_cast<float4 *>(dst + i) = float4{r[i], r[i + 1], r[i + 2], r[i + 3]};
}

__device__ __forceinline__ double dot16(const float (&q)[kDS], const float *k) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kDS; ++i) s = __builtin_fma((double)q[i], (double)k[i], s);   // exact products
    return s;
}

// Online softmax state of one query row (this lane's 16 dims of the accumulator).
struct State {
    double m, l;
    double acc[kDS];
};

// Adds one key with score s (already scaled) and value row vrow to the state.
__device__ __forceinline__ void add_key(State &st, double s, const float *vrow) {
    const double mn = fmax(st.m, s);
    const double alpha = exp(st.m - mn);   // 0 when st.m = -inf
    const double p = exp(s - mn);
    st.l = st.l * alpha + p;
#pragma unroll
    for (int i = 0; i < kDS; ++i) st.acc[i] = __builtin_fma(p, (double)vrow[i], st.acc[i] * alpha);
    st.m = mn;
}

// Merges state o into st (the log-sum-exp combination of two disjoint key sets).
__device__ __forceinline__ void merge_state(State &st, double om, double ol, const double *oacc) {
    const double mn = fmax(st.m, om);
    if (mn == -INFINITY) return;   // both sets empty
    const double wa = exp(st.m - mn), wb = exp(om - mn);
    st.l = st.l * wa + ol * wb;
#pragma unroll
    for (int i = 0; i < kDS; ++i) st.acc[i] = __builtin_fma(oacc[i], wb, st.acc[i] * wa);
    st.m = mn;
}

// LDS of one workgroup: the K and V tiles (prefill, decode) or, for the step, the
// states of half the row groups during the merge.
template <int D>
constexpr int lds_bytes() {
    constexpr int tiles = 2 * kTK * D * 4;
    constexpr int merge = kRows / 2 * (D + 2) * 8;
    return tiles > merge ? tiles : merge;
}

template <int D, Mode M>
__global__ void __launch_bounds__(block_threads<D>()) attn_f64_kernel(AttnArgs a) {
    constexpr int G = group_lanes<D>();
    __shared__ __attribute__((aligned(16))) char smem[lds_bytes<D>()];

    const int bid = blockIdx.x;
    const int group = bid / a.tiles, tile = bid % a.tiles;
    const int b = group / a.H, h = group % a.H;
    if (b >= a.B) return;
    const int N = a.lens[b];
    const int s = a.slot[b];
    if (N < 0 || N > a.len_limit || s < 0 || s >= a.S) {
        if (threadIdx.x == 0 && tile == 0)
            atomicOr(a.status, (N < 0 || N > a.len_limit ? kFlagBadLen : 0u) | (s < 0 || s >= a.S ? kFlagBadSlot : 0u));
        return;
    }
    // two users writing one slot (prefill): one block per user raises the flag, both run
    if (M == kPrefill && tile == 0 && h == 0 && N > 0 && (threadIdx.x >> 6) == 0) {
        bool dup = false;
        for (int u0 = 0; u0 < a.B && !dup; u0 += 64) {
            const int u = u0 + (int)threadIdx.x;
            const int n = u < a.B ? a.lens[u] : 0;
            const int su = u < a.B ? a.slot[u] : -1;
            dup = __ballot(u != b && n > 0 && n <= a.len_limit && su == s) != 0;
        }
        if (dup && threadIdx.x == 0) atomicOr(a.status, kFlagDupSlot);
    }
    const int tid = threadIdx.x;
    const int r = tid / G, gi = tid % G;
    const int d0 = gi * kDS;
    const long bh = (long)b * a.H + h;
    const float *qsrc = static_cast<const float *>(a.q) + bh * a.rows * D;
    const float *kin = static_cast<const float *>(a.k) + bh * a.rows * D;
    const float *vin = static_cast<const float *>(a.v) + bh * a.rows * D;
    float *odst = static_cast<float *>(a.o) + bh * a.rows * D;
    const long slot_off = ((long)s * a.H + h) * (long)a.n_max * D;
    float *pk = static_cast<float *>(a.pool_k) + slot_off;
    float *pv = static_cast<float *>(a.pool_v) + slot_off;
    const double sc = a.scale64;

    if constexpr (M == kStep) {
        // One query row (row 0 of q, k, v); group r takes slot rows r, r + 64, ...
        float q[kDS];
        load16(q, qsrc + d0);
        State st;
        st.m = -INFINITY;
        st.l = 0.0;
#pragma unroll
        for (int i = 0; i < kDS; ++i) st.acc[i] = 0.0;
        for (int t = r; t < N; t += kRows) {
            const double dot = group_sum<G>(dot16(q, pk + (long)t * D + d0));
            add_key(st, sc * dot, pv + (long)t * D + d0);
        }
        // Tree merge over LDS: in each round the upper half of the remaining groups
        // leaves its states, the lower half folds them in.
        double *acc_buf = reinterpret_cast<double *>(smem);                  // [32][D]
        double *ml_buf = acc_buf + kRows / 2 * D;                           // [32][2]
        for (int half = kRows / 2; half >= 1; half >>= 1) {
            __syncthreads();
            if (r >= half && r < 2 * half) {
#pragma unroll
                for (int i = 0; i < kDS; ++i) acc_buf[(r - half) * D + d0 + i] = st.acc[i];
                if (gi == 0) {
                    ml_buf[2 * (r - half)] = st.m;
                    ml_buf[2 * (r - half) + 1] = st.l;
                }
            }
            __syncthreads();
            if (r < half) merge_state(st, ml_buf[2 * r], ml_buf[2 * r + 1], acc_buf + r * D + d0);
        }
        if (r == 0) {
            // the new token's own key enters last; its K/V row goes to slot row N
            float kn[kDS], vn[kDS];
            load16(kn, kin + d0);
            load16(vn, vin + d0);
            add_key(st, sc * group_sum<G>(dot16(q, kn)), vn);
            float out[kDS];
#pragma unroll
            for (int i = 0; i < kDS; ++i) out[i] = (float)(st.acc[i] / st.l);
            store16(odst + d0, out);
            store16(pk + (long)N * D + d0, kn);
            store16(pv + (long)N * D + d0, vn);
        }
        return;
    } else {
        constexpr bool PREFILL = M == kPrefill;
        const int q0 = tile * kRows;
        const int qlimit = PREFILL ? N : a.rows;
        if (q0 >= qlimit) return;
        const int row = q0 + r;
        const bool valid = row < qlimit;
        const float *ksrc = PREFILL ? kin : pk;
        const float *vsrc = PREFILL ? vin : pv;
        float (*ks)[D] = reinterpret_cast<float (*)[D]>(smem);
        float (*vs)[D] = ks + kTK;

        // Fused pool write: this block's own history rows go to the slot, bit for bit.
        if (PREFILL && valid) {
            float x[kDS];
            load16(x, kin + (long)row * D + d0);
            store16(pk + (long)row * D + d0, x);
            load16(x, vin + (long)row * D + d0);
            store16(pv + (long)row * D + d0, x);
        }

        float q[kDS];
        if (valid) load16(q, qsrc + (long)row * D + d0);
        else
#pragma unroll
            for (int i = 0; i < kDS; ++i) q[i] = 0.f;
        State st;
        if constexpr (PREFILL) {
            st.m = -INFINITY;
            st.l = 0.0;
#pragma unroll
            for (int i = 0; i < kDS; ++i) st.acc[i] = 0.0;
        } else {
            // the candidate's own key enters first: weight exp(0) = 1, value vc_j
            float kc[kDS], vc[kDS];
            if (valid) {
                load16(kc, kin + (long)row * D + d0);
                load16(vc, vin + (long)row * D + d0);
            } else {
#pragma unroll
                for (int i = 0; i < kDS; ++i) kc[i] = vc[i] = 0.f;
            }
            st.m = sc * group_sum<G>(dot16(q, kc));
            st.l = 1.0;
#pragma unroll
            for (int i = 0; i < kDS; ++i) st.acc[i] = (double)vc[i];
        }

        const int kend = PREFILL ? min(q0 + kRows, N) : N;
        for (int kbase = 0; kbase < kend; kbase += kTK) {
            __syncthreads();
            for (int idx = tid; idx < kTK * D / 4; idx += block_threads<D>()) {
                const int kr = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
                const int key = kbase + kr;
                const float4 kx = key < kend ? *reinterpret_cast<const float4 *>(ksrc + (long)key * D + c4)
                                             : float4{0.f, 0.f, 0.f, 0.f};
                const float4 vx = key < kend ? *reinterpret_cast<const float4 *>(vsrc + (long)key * D + c4)
                                             : float4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<float4 *>(&ks[kr][c4]) = kx;
                *reinterpret_cast<float4 *>(&vs[kr][c4]) = vx;
            }
            __syncthreads();
            double scr[kTK];
            double mx = -INFINITY;
#pragma unroll
            for (int kr = 0; kr < kTK; ++kr) {
                const double dot = group_sum<G>(dot16(q, &ks[kr][d0]));
                const int key = kbase + kr;
                const bool off = key >= kend || (PREFILL && key > row);
                scr[kr] = off ? -INFINITY : sc * dot;
                mx = fmax(mx, scr[kr]);
            }
            const double mn = fmax(st.m, mx);
            if (mn == -INFINITY) continue;   // nothing visible yet (rows past the history only)
            const double alpha = exp(st.m - mn);
            st.l *= alpha;
#pragma unroll
            for (int i = 0; i < kDS; ++i) st.acc[i] *= alpha;
            st.m = mn;
#pragma unroll
            for (int kr = 0; kr < kTK; ++kr) {
                const double p = exp(scr[kr] - mn);   // 0 for masked keys
                st.l += p;
#pragma unroll
                for (int i = 0; i < kDS; ++i) st.acc[i] = __builtin_fma(p, (double)vs[kr][d0 + i], st.acc[i]);
            }
        }
        if (valid) {
            float out[kDS];
#pragma unroll
            for (int i = 0; i < kDS; ++i) out[i] = (float)(st.acc[i] / st.l);
            store16(odst + (long)row * D + d0, out);
        }
    }
}

template <Mode M>
hipError_t launch_f64(const AttnArgs &a, int D, hipStream_t stream) {
    const long blocks = (long)a.B * a.H * a.tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (D) {
        case 32: hipLaunchKernelGGL((attn_f64_kernel<32, M>), grid, dim3(block_threads<32>()), 0, stream, a); break;
        case 64: hipLaunchKernelGGL((attn_f64_kernel<64, M>), grid, dim3(block_threads<64>()), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((attn_f64_kernel<128, M>), grid, dim3(block_threads<128>()), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_f64<kPrefill>(a, D, stream);
}

hipError_t launch_decode_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    return launch_f64<kDecode>(a, D, stream);
}

hipError_t launch_ar_decode_fp32(const AttnArgs &a, int D, hipStream_t stream) {
    AttnArgs one = a;
    one.tiles = 1;
    return launch_f64<kStep>(one, D, stream);
}

}  // namespace unipin
