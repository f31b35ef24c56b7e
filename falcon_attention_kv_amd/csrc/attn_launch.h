// Internal interface between the C ABI (unipin.cpp) and the HIP kernels.
// Not installed; the public interface is include/unipin.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct unipin_pool;   // the pool descriptor of the C ABI (unipin.cpp)

namespace unipin {

// Arguments of one attention launch.  Both kernels of the library take this struct by
// value.  "rows" are the query rows of the call: the history rows for the prefill, the
// candidate rows for the ranking decode.
struct AttnArgs {
    const void *q, *k, *v;        // prefill: q, k, v [B,H,n,D]; decode: qc, kc, vc [B,H,k,D]
    void *o;                      // [B,H,rows,D]
    const int32_t *lens;          // [B] device
    const int32_t *slot;          // [B] device
    void *pool_k, *pool_v;        // K/V pool arrays, already offset to `layer`: [S,H,n_max,D]
    int B, H, rows;               // rows = n (prefill) or k (decode)
    int n_max, S;
    int len_limit;                // largest valid lens[b]: n (prefill) or n_max (decode)
    int tiles;                    // query tiles per (user, head)
    int xcd_remap;                // 1: map blocks so all tiles of a (user, head) share an XCD
    float c;                      // scale * log2(e)
    double scale64;               // the score scale itself, in fp64 (fp32 kernels)
    unsigned int *status;         // the pool's sticky flag word on this device
    // Row addressing of q, k, v (in) and o (out), in elements: row t of (user b, head h)
    // starts at b * bstride + h * hstride + t * rstride.  The contiguous [B, H, rows, D]
    // layout is bstride = H * rows * D, hstride = rows * D, rstride = D; the bf16 kernels
    // take any layout whose rows and bases are 16-byte aligned (the fp32 kernels and the
    // autoregressive step only the contiguous one).
    long in_bstride, in_hstride, out_bstride, out_hstride;
    int in_rstride, out_rstride;
    // The ranking decode split over the history (launch_decode_split_bf16): each of the
    // `parts` workgroups of a candidate tile takes `part_tiles` 64-key tiles and leaves its
    // state in part_state (fp32: the accumulators [item][part][256][D], then (m, l) pairs
    // [item][part][256]).
    int parts, part_tiles;
    float *part_state;
};

// Row layout of one attention operand, in elements (see AttnArgs).
struct RowLayout {
    long bstride, hstride;
    int rstride;
};

// The prefill (prefill = true) or the ranking decode over the pool, with q, k, v read
// and o written in the given layouts: the public entry points' shared body, after
// their argument checks.  bf16 pools only for a non-contiguous layout.  Returns a
// UNIPIN_* status.
// For the ranking decode, part_state (parts >= 2) selects the split over the history
// (launch_decode_split_bf16; bf16 and E4M3 pools).
int attention_call(bool prefill, const void *q, const void *k, const void *v, RowLayout in, void *o, RowLayout out,
                   ::unipin_pool *pool, const int32_t *slot, const int32_t *lens, int layer, int B, int rows,
                   float scale, void *stream, float *part_state = nullptr, int parts = 1, int part_tiles = 0);

// The split of the ranking decode over the history for B users of k candidates: parts
// (1: the one-pass kernel), 64-key tiles per part and the workspace bytes it needs.
struct DecodeSplit {
    int parts, part_tiles;
    size_t bytes;
};
DecodeSplit decode_split_plan(const ::unipin_pool *pool, int B, int k);

// Flags raised on the device (mirrors UNIPIN_FLAG_* of the public header).
constexpr unsigned int kFlagBadSlot = 1u;
constexpr unsigned int kFlagBadLen = 2u;
constexpr unsigned int kFlagDupSlot = 4u;

// Query rows one workgroup (prefill) or one work item (decode) covers.
constexpr int kFp32RowsPerBlock = 64;
int bf16_prefill_rows_per_block(int D);
int bf16_decode_rows_per_item(int D);

// bf16 activations; pool8: the pool holds E4M3 codes (written by the prefill's fused
// pool write, decoded by the ranking decode as its tiles arrive), else bf16.
hipError_t launch_prefill_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream);
hipError_t launch_decode_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream);
// The split ranking decode with bf16 activations (contiguous layout) on a bf16 pool or,
// with pool8, an E4M3 pool: the parts, then the merge of the parts with each candidate's
// own key into o.
hipError_t launch_decode_split_bf16(const AttnArgs &a, int D, bool pool8, hipStream_t stream);
// fp32 pools: fp32 in and out, fp64 arithmetic inside.
hipError_t launch_prefill_fp32(const AttnArgs &a, int D, hipStream_t stream);
hipError_t launch_decode_fp32(const AttnArgs &a, int D, hipStream_t stream);
hipError_t launch_ar_decode_fp32(const AttnArgs &a, int D, hipStream_t stream);
// One autoregressive step (one new token per user and head) on a bf16 pool (kind 1) or
// with bf16 activations over an E4M3 pool (kind 2) (the unipin_dtype_t codes; fp32
// pools take launch_ar_decode_fp32 and never split).  P = 1: one pass per (user, head).  P > 1: the slot rows are
// split into up to P parts, one workgroup each, whose states go to ws
// (ar_workspace_bytes(B*H, P, D) bytes, fp32) and are merged by a second pass.
int ar_splits(long bh, int n_max, int D, int kind);
size_t ar_workspace_bytes(long bh, int P, int D);
hipError_t launch_ar_decode(const AttnArgs &a, int D, int kind, float *ws, int P, hipStream_t stream);
// The library's own split-path state array on the current device (for callers that cannot
// allocate): its device address, looked up once per device, and its size in bytes.
hipError_t ar_scratch(float **out);
size_t ar_scratch_bytes();

// Per-pool sticky flag words: one entry per live pool descriptor, in file-scope device
// arrays on every device (addresses looked up once per device with hipGetSymbolAddress).
constexpr int kMaxPools = 4096;
// Device address, on the current device, of pool entry `index`'s flag word.
hipError_t pool_flag_word(int index, unsigned int **out);
// Enqueues on `stream` a one-thread kernel that exchanges entry `index`'s flags for 0.
hipError_t clear_pool_flags(int index, hipStream_t stream);
// The same exchange, then a copy of the old value to *host and a wait for `stream`.
hipError_t take_pool_flags(int index, hipStream_t stream, unsigned int *host);

}  // namespace unipin
