// C ABI of the transformer block around the masked attention (include/unipin.h): one
// GPT2-style pre-LayerNorm block, run either as the history forward (causal attention,
// K/V stored in the pool) or as the ranking stage's candidate-only forward (attention
// to the pool's history plus the candidate's own key).
//
// The four projections are bf16 GEMMs with fp32 accumulation and fused epilogues (bias,
// tanh-form GELU, residual add into the hidden state).  They run on hipBLASLt (its
// epilogues, beta = 1 on the hidden state for the residual) or on this library's MFMA
// kernel (gemm_bf16.hip, four workgroup tile configurations), whichever the tuner timed
// fastest for the shape; untuned, on hipBLASLt's first heuristic choice.  LayerNorm is this
// library's kernel (block_kernels.hip); with the weights unipin_block_fold_layernorm
// prepares, the QKV and MLP-up projections may instead run this library's kernel on the
// hidden state itself, the LayerNorm's row statistics taken inside the GEMM and applied in
// its epilogue (the tuner chooses per shape).  The attention is the library's own prefill and rank-decode
// kernels, which read q, k and v straight from the fused projection's rows
// [B, rows, 3, H, D] and write the heads' outputs straight into the merged rows
// [B, rows, H, D] that the output projection reads.  Host code here allocates nothing on
// the device: every intermediate lives in the caller's workspace.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt-ext.hpp>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "attn_launch.h"
#include "block_launch.h"
#include "unipin.h"

namespace {

constexpr float kLnEps = 1e-5f;
constexpr size_t kGemmWorkspace = 32u << 20;   // hipBLASLt's share of the workspace
constexpr size_t kMaxTuneCandidates = 1500;    // GEMM kernels timed per shape by the tuner
constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// out[M, N] (row-major) = in[M, K] (row-major) @ W[K, N] (row-major), seen by the
// column-major library as D[N x M] = W[N x K] * in[K x M]: the bias runs along D's rows.
struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    int own = -1;   // >= 0: this library's kernel with that tile configuration; -1: hipBLASLt
    // >= 0: given folded LayerNorm weights, the QKV or MLP-up projection runs on the hidden
    // state itself in this library's kernel with that configuration (no LayerNorm kernel)
    int ln_own = -1;
};

using PlanKey = std::tuple<long, int, int, int, bool>;   // M, N, K, epilogue, residual

}  // namespace

struct unipin_block_ctx {
    hipblasLtHandle_t handle = nullptr;
    int device = -1;
    int kernel = UNIPIN_GEMM_AUTO;       // unipin_block_ctx_set_gemm
    std::mutex mu;                       // plans and their descriptors are shared by calls
    std::map<PlanKey, GemmPlan> plans;
};

namespace {

void destroy_plan(GemmPlan &p) {
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
}

// This library's GEMM epilogue for a hipBLASLt one.
int own_epilogue(hipblasLtEpilogue_t ep, bool residual) {
    if (ep == HIPBLASLT_EPILOGUE_GELU_BIAS) return unipin::kGemmBiasGelu;
    return residual ? unipin::kGemmBiasResidual : unipin::kGemmBias;
}

// The plan for one GEMM shape and epilogue, made on first use (descriptors, the
// library's first heuristic choice and the kernel selection).  Called with ctx->mu held.
GemmPlan *plan_for(unipin_block_ctx *ctx, long M, int N, int K, hipblasLtEpilogue_t ep, bool residual) {
    const PlanKey key{M, N, K, (int)ep, residual};
    auto it = ctx->plans.find(key);
    if (it != ctx->plans.end()) return &it->second;
    GemmPlan p;
    if (ctx->kernel >= 0 && unipin::gemm_bf16_supported(M, N, K, ctx->kernel)) p.own = p.ln_own = ctx->kernel;
    const hipblasOperation_t op = HIPBLAS_OP_N;
    const hipDataType bias_type = HIP_R_16BF;
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t ws = kGemmWorkspace;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof(op)) == 0 &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof(op)) == 0 &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &ep, sizeof(ep)) == 0 &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                              sizeof(bias_type)) == 0 &&
              hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, N, K, N) == 0 &&
              hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) == 0 &&
              hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, M, N) == 0 &&
              hipblasLtMatmulPreferenceCreate(&pref) == 0 &&
              hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                    sizeof(ws)) == 0 &&
              hipblasLtMatmulAlgoGetHeuristic(ctx->handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &found) ==
                  0 &&
              found > 0;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) {
        destroy_plan(p);
        return nullptr;
    }
    p.algo = res[0].algo;
    return &ctx->plans.emplace(key, p).first->second;
}

// One run of a planned GEMM: out = in @ W + bias (then GELU, with ep = GELU_BIAS);
// residual: out += the old out.  Called with ctx->mu held.
int run_plan(unipin_block_ctx *ctx, GemmPlan *p, const void *in, const void *W, const void *bias, void *out, long M,
             int N, int K, hipblasLtEpilogue_t ep, bool residual, void *ws, hipStream_t stream) {
    if (p->own >= 0)
        return unipin::launch_gemm_bf16(in, W, bias, out, M, N, K, own_epilogue(ep, residual), p->own, stream) ==
                       hipSuccess
                   ? UNIPIN_OK
                   : UNIPIN_EHIP;
    if (hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) != 0)
        return UNIPIN_EHIP;
    const float alpha = 1.f, beta = residual ? 1.f : 0.f;
    const hipblasStatus_t s = hipblasLtMatmul(ctx->handle, p->desc, &alpha, W, p->la, in, p->lb, &beta, out, p->lc,
                                              out, p->lc, &p->algo, ws, kGemmWorkspace, stream);
    return s == HIPBLAS_STATUS_SUCCESS ? UNIPIN_OK : UNIPIN_EHIP;
}

int gemm(unipin_block_ctx *ctx, const void *in, const void *W, const void *bias, void *out, long M, int N, int K,
         hipblasLtEpilogue_t ep, bool residual, void *ws, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(ctx->mu);
    GemmPlan *p = plan_for(ctx, M, N, K, ep, residual);
    if (!p) return UNIPIN_EHIP;
    return run_plan(ctx, p, in, W, bias, out, M, N, K, ep, residual, ws, stream);
}

// The configuration of this library's kernel that runs the projection with its
// LayerNorm folded in, or -1 (LayerNorm kernel, then the planned GEMM).
int ln_choice(unipin_block_ctx *ctx, long M, int N, int K, hipblasLtEpilogue_t ep) {
    std::lock_guard<std::mutex> lock(ctx->mu);
    GemmPlan *p = plan_for(ctx, M, N, K, ep, false);
    return p ? p->ln_own : -1;
}

// Workspace layout for M = B * rows hidden rows of width C (bytes, 256-aligned):
//   [gemm]  hipBLASLt workspace
//   [big]   M x 4C: the fused QKV output (M x 3C), later the MLP's hidden layer
//   [ln]    M x C:  LayerNorm output, then the attention output, then LayerNorm again
//   [tune]  4C x C + 4C: weights and bias for timing the GEMM kernels (tuning only)
//   [uv]    2 x 4C fp32: the folded LayerNorm's column terms for timing (tuning only)
struct Layout {
    size_t gemm, big, ln, tune, uv, total;
};

Layout layout(long M, int C) {
    Layout l;
    const size_t e = 2;
    l.gemm = 0;
    l.big = up(kGemmWorkspace);
    l.ln = l.big + up((size_t)M * 4 * C * e);
    l.tune = l.ln + up((size_t)M * C * e);
    l.uv = l.tune + up(((size_t)4 * C * C + 4 * C) * e);
    l.total = l.uv + up((size_t)8 * C * sizeof(float));
    return l;
}

// The block's four GEMMs for M hidden rows of width C: QKV, output projection (plus
// residual), MLP up (bias and GELU), MLP down (plus residual).
struct GemmShape {
    int N, K;
    hipblasLtEpilogue_t ep;
    bool residual;
};

void block_gemms(int C, GemmShape (&g)[4]) {
    g[0] = {3 * C, C, HIPBLASLT_EPILOGUE_BIAS, false};
    g[1] = {C, C, HIPBLASLT_EPILOGUE_BIAS, true};
    g[2] = {4 * C, C, HIPBLASLT_EPILOGUE_GELU_BIAS, false};
    g[3] = {C, 4 * C, HIPBLASLT_EPILOGUE_BIAS, true};
}

// The optional folded LayerNorm weights: 0 none, 1 both parts of a projection given
// (aligned), -1 half given or misaligned.
int folded(const void *wf, const void *uv) {
    if (!wf && !uv) return 0;
    return wf && uv && aligned16(wf) && aligned16(uv) ? 1 : -1;
}

bool weights_present(const unipin_block_weights_t *w) {
    const void *p[] = {w->ln1_w, w->ln1_b, w->w_qkv, w->b_qkv, w->w_o, w->b_o,
                       w->ln2_w, w->ln2_b, w->w_fc, w->b_fc, w->w_proj, w->b_proj};
    for (const void *q : p)
        if (!q || !aligned16(q)) return false;
    return true;
}

}  // namespace

extern "C" {

int unipin_block_ctx_create(unipin_block_ctx_t **out) {
    if (!out) return UNIPIN_EINVAL;
    *out = nullptr;
    auto *ctx = new (std::nothrow) unipin_block_ctx;
    if (!ctx) return UNIPIN_ENOMEM;
    if (hipGetDevice(&ctx->device) != hipSuccess || hipblasLtCreate(&ctx->handle) != HIPBLAS_STATUS_SUCCESS) {
        delete ctx;
        return UNIPIN_EHIP;
    }
    *out = ctx;
    return UNIPIN_OK;
}

int unipin_block_ctx_destroy(unipin_block_ctx_t *ctx) {
    if (!ctx) return UNIPIN_EINVAL;
    for (auto &kv : ctx->plans) destroy_plan(kv.second);
    hipblasLtDestroy(ctx->handle);
    delete ctx;
    return UNIPIN_OK;
}

int unipin_block_ctx_set_gemm(unipin_block_ctx_t *ctx, int kernel) {
    if (!ctx || kernel < UNIPIN_GEMM_AUTO || kernel >= unipin::kGemmConfigs) return UNIPIN_EINVAL;
    std::lock_guard<std::mutex> lock(ctx->mu);
    for (auto &kv : ctx->plans) destroy_plan(kv.second);
    ctx->plans.clear();
    ctx->kernel = kernel;
    return UNIPIN_OK;
}

size_t unipin_block_workspace_bytes(const unipin_pool_t *pool, int B, int rows) {
    int L, S, H, n_max, D, dt;
    if (!pool || B < 1 || rows < 1 || unipin_pool_dims(pool, &L, &S, &H, &n_max, &D, &dt) != UNIPIN_OK) return 0;
    return layout((long)B * rows, H * D).total;
}

int unipin_block_ctx_tune(unipin_block_ctx_t *ctx, const unipin_pool_t *pool, int B, int rows, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (!ctx || !pool || !workspace || B < 1 || rows < 1) return UNIPIN_EINVAL;
    int L, S, H, n_max, D, dt;
    if (unipin_pool_dims(pool, &L, &S, &H, &n_max, &D, &dt) != UNIPIN_OK) return UNIPIN_EINVAL;
    if (dt == UNIPIN_FP32) return UNIPIN_EDTYPE;   // bf16 activations (bf16 or E4M3 pool)
    const int C = H * D;
    const long M = (long)B * rows;
    const Layout lo = layout(M, C);
    if (!aligned16(workspace)) return UNIPIN_EALIGN;
    if (workspace_bytes < lo.total) return UNIPIN_EINVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != ctx->device) return UNIPIN_EINVAL;
    char *ws = static_cast<char *>(workspace);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // operands: activations in [ln] and [big], weights and bias in [tune]; values of the
    // size the block sees (a GEMM's speed can depend on the data through power)
    if (unipin::launch_fill_random(ws + lo.big, (size_t)M * 4 * C, 1u, 1.f, st) != hipSuccess ||
        unipin::launch_fill_random(ws + lo.tune, (size_t)4 * C * C + 4 * C, 2u, 0.05f, st) != hipSuccess ||
        unipin::launch_fill_random(ws + lo.ln, (size_t)M * C, 3u, 1.f, st) != hipSuccess)
        return UNIPIN_EHIP;
    // and the folded LayerNorm's column terms, values of the size the block sees
    if (unipin::launch_fill_random_f32(ws + lo.uv, (size_t)8 * C, 4u, 1.f, st) != hipSuccess) return UNIPIN_EHIP;
    GemmShape g[4];
    block_gemms(C, g);
    // QKV: ln -> big; output projection: ln -> big (M x C of it); MLP up: ln -> big;
    // MLP down: big -> ln
    void *in_of[4] = {ws + lo.ln, ws + lo.ln, ws + lo.ln, ws + lo.big};
    void *out_of[4] = {ws + lo.big, ws + lo.big, ws + lo.big, ws + lo.ln};
    const void *W = ws + lo.tune, *bias = ws + lo.tune + (size_t)4 * C * C * 2;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return UNIPIN_EHIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return UNIPIN_EHIP;
    }
    int rc = UNIPIN_OK;
    std::lock_guard<std::mutex> lock(ctx->mu);
    for (int i = 0; i < 4 && rc == UNIPIN_OK; ++i) {
        GemmPlan *p = plan_for(ctx, M, g[i].N, g[i].K, g[i].ep, g[i].residual);
        if (!p) {
            rc = UNIPIN_EHIP;
            break;
        }
        // candidates: this library's kernel in each tile configuration, hipBLASLt's
        // heuristic choices, then every kernel hipBLASLt has for a bf16 GEMM that accepts
        // this problem (shape, layouts, epilogue) within the workspace; restricted to one
        // kernel or to hipBLASLt by unipin_block_ctx_set_gemm
        struct Cand {
            int own;
            hipblasLtMatmulAlgo_t algo;
        };
        std::vector<Cand> cands;
        bool own_ok = false;
        if (ctx->kernel >= 0 && unipin::gemm_bf16_supported(M, g[i].N, g[i].K, ctx->kernel)) {
            cands.push_back({ctx->kernel, {}});
            own_ok = true;
        }
        if (ctx->kernel == UNIPIN_GEMM_AUTO)
            for (int c = 0; c < unipin::kGemmConfigs; ++c)
                if (unipin::gemm_bf16_supported(M, g[i].N, g[i].K, c)) {
                    cands.push_back({c, {}});
                    own_ok = true;
                }
        const bool lib = ctx->kernel == UNIPIN_GEMM_LIBRARY || (ctx->kernel == UNIPIN_GEMM_AUTO) || !own_ok;
        hipblasLtMatmulPreference_t pref = nullptr;
        const uint64_t wsz = kGemmWorkspace;
        constexpr int kHeuristic = 32;
        hipblasLtMatmulHeuristicResult_t heur[kHeuristic];
        int found = 0;
        if (hipblasLtMatmulPreferenceCreate(&pref) != 0 ||
            hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz,
                                                  sizeof(wsz)) != 0 ||
            hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) != 0 ||
            hipblasLtMatmulAlgoGetHeuristic(ctx->handle, p->desc, p->la, p->lb, p->lc, p->lc, pref, kHeuristic, heur,
                                            &found) != 0) {
            if (pref) hipblasLtMatmulPreferenceDestroy(pref);
            rc = UNIPIN_EHIP;
            break;
        }
        hipblasLtMatmulPreferenceDestroy(pref);
        for (int a = 0; lib && a < found; ++a)
            if (heur[a].state == HIPBLAS_STATUS_SUCCESS && heur[a].workspaceSize <= kGemmWorkspace)
                cands.push_back({-1, heur[a].algo});
        if (lib) {
            const float al = 1.f, be = g[i].residual ? 1.f : 0.f;
            std::vector<hipblasLtMatmulHeuristicResult_t> all;
            if (hipblaslt_ext::getAllAlgos(ctx->handle, hipblaslt_ext::GemmType::HIPBLASLT_GEMM, HIPBLAS_OP_N,
                                           HIPBLAS_OP_N, HIP_R_16BF, HIP_R_16BF, HIP_R_16BF, HIP_R_16BF,
                                           HIPBLAS_COMPUTE_32F, all) == HIPBLAS_STATUS_SUCCESS) {
                for (auto &r : all) {
                    if (cands.size() >= kMaxTuneCandidates) break;
                    size_t need = 0;
                    if (hipblaslt_ext::matmulIsAlgoSupported(ctx->handle, p->desc, &al, p->la, p->lb, &be, p->lc,
                                                             p->lc, r.algo, need) == HIPBLAS_STATUS_SUCCESS &&
                        need <= kGemmWorkspace)
                        cands.push_back({-1, r.algo});
                }
            }
        }
        // One timing of a candidate: two untimed runs, then `reps` runs between events.
        // 1: the candidate cannot run this problem; -1: an event call failed.
        auto time_plan = [&](GemmPlan &t, int reps, float *ms) -> int {
            auto run = [&]() {
                return run_plan(ctx, &t, in_of[i], W, bias, out_of[i], M, g[i].N, g[i].K, g[i].ep, g[i].residual,
                                ws + lo.gemm, st);
            };
            if (run() != UNIPIN_OK || run() != UNIPIN_OK) return 1;
            if (hipEventRecord(e0, st) != hipSuccess) return -1;
            bool ok = true;
            for (int r = 0; r < reps && ok; ++r) ok = run() == UNIPIN_OK;
            if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(ms, e0, e1) != hipSuccess)
                return -1;
            // the residual GEMMs add into their output each run; start the next timing
            // from the same values as the first so that no candidate sees overflowing data
            if (g[i].residual &&
                unipin::launch_fill_random(out_of[i], (size_t)M * g[i].N, 5u, 1.f, st) != hipSuccess)
                return -1;
            return ok ? 0 : 1;
        };
        // The sweep keeps the fastest of this library's kernels and the fastest of
        // hipBLASLt's.  With over a thousand library candidates, the minimum of single
        // noisy timings favours the library; the two finalists are therefore timed again
        // against each other, in alternating rounds, and the faster in total is kept.
        GemmPlan own_pick = *p, lib_pick = *p;
        float own_ms = 1e30f, lib_ms = 1e30f;
        for (auto &c : cands) {
            GemmPlan trial = *p;
            trial.own = c.own;
            trial.algo = c.algo;
            float ms = 0.f;
            const int r = time_plan(trial, 5, &ms);
            if (r < 0) {
                rc = UNIPIN_EHIP;
                break;
            }
            if (r > 0) continue;
            float &best = c.own >= 0 ? own_ms : lib_ms;
            if (ms < best) {
                best = ms;
                (c.own >= 0 ? own_pick : lib_pick) = trial;
            }
        }
        if (rc != UNIPIN_OK) break;
        if (own_ms < 1e30f && lib_ms < 1e30f) {
            float own_total = 0.f, lib_total = 0.f;
            for (int round = 0; round < 4 && rc == UNIPIN_OK; ++round) {
                float a = 0.f, b = 0.f;
                const int ra = time_plan(own_pick, 10, &a), rb = ra < 0 ? -1 : time_plan(lib_pick, 10, &b);
                if (ra < 0 || rb < 0) rc = UNIPIN_EHIP;
                own_total += ra == 0 ? a : 1e30f;
                lib_total += rb == 0 ? b : 1e30f;
            }
            if (rc != UNIPIN_OK) break;
            own_ms = own_total;
            lib_ms = lib_total;
        }
        if (own_ms < 1e30f || lib_ms < 1e30f) {
            const GemmPlan &pick = own_ms <= lib_ms ? own_pick : lib_pick;
            p->own = pick.own;
            p->algo = pick.algo;
        }
        // The QKV and MLP-up projections can instead run with their LayerNorm folded into
        // the weights (unipin_block_fold_layernorm): this library's kernel on the hidden
        // state, the row statistics taken inside the GEMM.  The fastest configuration is
        // timed against the LayerNorm kernel followed by the GEMM just chosen, in
        // alternating rounds; a pinned kernel is used as it is.
        if (g[i].residual) continue;
        p->ln_own = -1;
        if (ctx->kernel >= 0) {
            if (unipin::gemm_bf16_supported(M, g[i].N, g[i].K, ctx->kernel)) p->ln_own = ctx->kernel;
            continue;
        }
        if (ctx->kernel != UNIPIN_GEMM_AUTO) continue;
        const int lepi = g[i].ep == HIPBLASLT_EPILOGUE_GELU_BIAS ? unipin::kGemmLnBiasGelu : unipin::kGemmLnBias;
        const void *gamma = bias, *beta = static_cast<const char *>(bias) + (size_t)C * 2;
        auto timed = [&](auto &&run, int reps, float *ms) -> int {
            if (!run() || !run()) return 1;
            if (hipEventRecord(e0, st) != hipSuccess) return -1;
            bool ok = true;
            for (int r = 0; r < reps && ok; ++r) ok = run();
            if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(ms, e0, e1) != hipSuccess)
                return -1;
            return ok ? 0 : 1;
        };
        int best_cfg = -1;
        float best_ms = 1e30f;
        for (int c = 0; c < unipin::kGemmConfigs && rc == UNIPIN_OK; ++c) {
            if (!unipin::gemm_bf16_supported(M, g[i].N, g[i].K, c)) continue;
            float ms = 0.f;
            const int r = timed([&]() {
                return unipin::launch_gemm_bf16(in_of[i], W, ws + lo.uv, out_of[i], M, g[i].N, g[i].K, lepi, c, st) ==
                       hipSuccess;
            }, 5, &ms);
            if (r < 0) rc = UNIPIN_EHIP;
            if (r == 0 && ms < best_ms) {
                best_ms = ms;
                best_cfg = c;
            }
        }
        if (rc != UNIPIN_OK) break;
        if (best_cfg < 0) continue;
        float fused_total = 0.f, plain_total = 0.f;
        for (int round = 0; round < 4 && rc == UNIPIN_OK; ++round) {
            float a = 0.f, b = 0.f;
            const int ra = timed([&]() {
                return unipin::launch_gemm_bf16(in_of[i], W, ws + lo.uv, out_of[i], M, g[i].N, g[i].K, lepi,
                                                best_cfg, st) == hipSuccess;
            }, 10, &a);
            // the plain path: LayerNorm (in place, which keeps the operands bounded), then the GEMM
            const int rb = ra < 0 ? -1 : timed([&]() {
                return unipin::launch_layernorm(in_of[i], gamma, beta, in_of[i], M, C, kLnEps, st) == hipSuccess &&
                       run_plan(ctx, p, in_of[i], W, bias, out_of[i], M, g[i].N, g[i].K, g[i].ep, false,
                                ws + lo.gemm, st) == UNIPIN_OK;
            }, 10, &b);
            if (ra < 0 || rb < 0) rc = UNIPIN_EHIP;
            fused_total += ra == 0 ? a : 1e30f;
            plain_total += rb == 0 ? b : 1e30f;
        }
        if (rc != UNIPIN_OK) break;
        if (fused_total < plain_total) p->ln_own = best_cfg;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}

int unipin_block_fold_layernorm(const unipin_block_weights_t *w, int C, void *w_qkv_ln, void *uv_qkv,
                                void *w_fc_ln, void *uv_fc, void *stream) {
    if (!w || !w_qkv_ln || !uv_qkv || !w_fc_ln || !uv_fc) return UNIPIN_EINVAL;
    if (C < 8 || C % 8 != 0 || C > 2048) return UNIPIN_EINVAL;
    if (!weights_present(w)) return w->ln1_w && w->ln1_b && w->w_qkv && w->b_qkv && w->w_o && w->b_o &&
                                           w->ln2_w && w->ln2_b && w->w_fc && w->b_fc && w->w_proj && w->b_proj
                                       ? UNIPIN_EALIGN
                                       : UNIPIN_EINVAL;
    if (!aligned16(w_qkv_ln) || !aligned16(uv_qkv) || !aligned16(w_fc_ln) || !aligned16(uv_fc)) return UNIPIN_EALIGN;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (unipin::launch_fold_layernorm(w->ln1_w, w->ln1_b, w->w_qkv, w->b_qkv, C, 3 * C, w_qkv_ln, uv_qkv, st) !=
            hipSuccess ||
        unipin::launch_fold_layernorm(w->ln2_w, w->ln2_b, w->w_fc, w->b_fc, C, 4 * C, w_fc_ln, uv_fc, st) !=
            hipSuccess)
        return UNIPIN_EHIP;
    return UNIPIN_OK;
}

int unipin_block_forward(unipin_block_ctx_t *ctx, const unipin_block_weights_t *w, int mode, void *x,
                         unipin_pool_t *pool, const int32_t *slot, const int32_t *lens, int layer, int B, int rows,
                         float scale, void *workspace, size_t workspace_bytes, void *stream) {
    if (!ctx || !w || !x || !pool || !slot || !lens || !workspace) return UNIPIN_EINVAL;
    if (mode != UNIPIN_BLOCK_HISTORY && mode != UNIPIN_BLOCK_CANDIDATES) return UNIPIN_EINVAL;
    if (B < 1 || rows < 1) return UNIPIN_EINVAL;
    int L, S, H, n_max, D, dt;
    if (unipin_pool_dims(pool, &L, &S, &H, &n_max, &D, &dt) != UNIPIN_OK) return UNIPIN_EINVAL;
    if (dt == UNIPIN_FP32) return UNIPIN_EDTYPE;   // bf16 activations (bf16 or E4M3 pool)
    if (layer < 0 || layer >= L) return UNIPIN_ERANGE;
    if (mode == UNIPIN_BLOCK_HISTORY && rows > n_max) return UNIPIN_EINVAL;
    const int C = H * D;
    if (C > 2048) return UNIPIN_EINVAL;
    if (!weights_present(w)) return w->ln1_w && w->ln1_b && w->w_qkv && w->b_qkv && w->w_o && w->b_o &&
                                           w->ln2_w && w->ln2_b && w->w_fc && w->b_fc && w->w_proj && w->b_proj
                                       ? UNIPIN_EALIGN
                                       : UNIPIN_EINVAL;
    if (!aligned16(x) || !aligned16(workspace) || !aligned16(slot) || !aligned16(lens)) return UNIPIN_EALIGN;
    const int fold1 = folded(w->w_qkv_ln, w->uv_qkv), fold2 = folded(w->w_fc_ln, w->uv_fc);
    if (fold1 < 0 || fold2 < 0) return (w->w_qkv_ln == nullptr) != (w->uv_qkv == nullptr) ||
                                               (w->w_fc_ln == nullptr) != (w->uv_fc == nullptr)
                                           ? UNIPIN_EINVAL
                                           : UNIPIN_EALIGN;
    const long M = (long)B * rows;
    const Layout lo = layout(M, C);
    if (workspace_bytes < lo.total) return UNIPIN_EINVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != ctx->device) return UNIPIN_EINVAL;

    char *ws = static_cast<char *>(workspace);
    void *gws = ws + lo.gemm, *ln = ws + lo.ln;
    char *big = ws + lo.big;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    int rc;

    // attention half: x += (attention of LN1(x)) @ W_o + b_o.  The QKV rows are
    // [B, rows, 3, H, D]: q, k, v of head h start at columns h*D, C + h*D, 2C + h*D of a
    // row; the heads' outputs land at columns h*D of the merged rows [B, rows, C].
    // With the LayerNorm folded into the weights, the planned kernel may take x itself.
    const int f1 = fold1 ? ln_choice(ctx, M, 3 * C, C, HIPBLASLT_EPILOGUE_BIAS) : -1;
    if (f1 >= 0) {
        if (unipin::launch_gemm_bf16(x, w->w_qkv_ln, w->uv_qkv, big, M, 3 * C, C, unipin::kGemmLnBias, f1, st) !=
            hipSuccess)
            return UNIPIN_EHIP;
    } else {
        if (unipin::launch_layernorm(x, w->ln1_w, w->ln1_b, ln, M, C, kLnEps, st) != hipSuccess) return UNIPIN_EHIP;
        if ((rc = gemm(ctx, ln, w->w_qkv, w->b_qkv, big, M, 3 * C, C, HIPBLASLT_EPILOGUE_BIAS, false, gws, st)))
            return rc;
    }
    const unipin::RowLayout qkv_rows{(long)rows * 3 * C, D, 3 * C}, merged_rows{(long)rows * C, D, C};
    rc = unipin::attention_call(mode == UNIPIN_BLOCK_HISTORY, big, big + (size_t)C * 2, big + (size_t)2 * C * 2,
                                qkv_rows, ln, merged_rows, pool, slot, lens, layer, B, rows, scale, stream);
    if (rc) return rc;
    if ((rc = gemm(ctx, ln, w->w_o, w->b_o, x, M, C, C, HIPBLASLT_EPILOGUE_BIAS, true, gws, st))) return rc;
    // MLP half: x += GELU(LN2(x) @ W_fc + b_fc) @ W_proj + b_proj
    const int f2 = fold2 ? ln_choice(ctx, M, 4 * C, C, HIPBLASLT_EPILOGUE_GELU_BIAS) : -1;
    if (f2 >= 0) {
        if (unipin::launch_gemm_bf16(x, w->w_fc_ln, w->uv_fc, big, M, 4 * C, C, unipin::kGemmLnBiasGelu, f2, st) !=
            hipSuccess)
            return UNIPIN_EHIP;
    } else {
        if (unipin::launch_layernorm(x, w->ln2_w, w->ln2_b, ln, M, C, kLnEps, st) != hipSuccess) return UNIPIN_EHIP;
        if ((rc = gemm(ctx, ln, w->w_fc, w->b_fc, big, M, 4 * C, C, HIPBLASLT_EPILOGUE_GELU_BIAS, false, gws, st)))
            return rc;
    }
    return gemm(ctx, big, w->w_proj, w->b_proj, x, M, C, 4 * C, HIPBLASLT_EPILOGUE_BIAS, true, gws, st);
}

}  // extern "C"
