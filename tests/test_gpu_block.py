"""GPU parity of the transformer block (unipin_block_forward) against the oracle.

The block runs at the precision of a bf16 model: every intermediate (LayerNorm output,
projections, attention output, MLP hidden layer, the hidden state itself) is stored in
bf16, with fp32 accumulation inside each step.  Each store rounds with relative error
at most u = 2^-8 (bf16 keeps 8 significant bits).  An output passes through a handful
of such roundings of quantities of its own size (the two residual adds store the hidden
state itself), so the bounds are relative to the reference's magnitude:
    one block:   max |g - r| <= 4 u max |r|,   mean |g - r| <= 1 u mean |r|
    pool rows:   max |g - r| <= 2 u max |r|,   mean |g - r| <= 1 u mean |r|
                 (one rounding of the projection, after one of the LayerNorm output)
    12 layers:   max <= 12 u, mean <= 4 u: the per-layer errors add along the residual
                 stream, about as a random walk (sqrt(12) x 1 u), with margin.
"""
import sys

import numpy as np
import pytest
import torch

import falcon_attention_kv_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -8


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def check_rel(got, ref, what, max_units=4, mean_units=1):
    g = oracle.as_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - r)
    mx, mn = d.max() / np.abs(r).max(), d.mean() / np.abs(r).mean()
    sys.__stderr__.write(f"  {what}: max {mx / U:.2f} u, mean {mn / U:.3f} u (of |r|)\n")
    assert mx <= max_units * U, f"{what}: max error {mx / U:.2f} u of max|ref| > {max_units} u"
    assert mn <= mean_units * U, f"{what}: mean error {mn / U:.3f} u of mean|ref| > {mean_units} u"


def make(B, n, K, H, D, L=2, S=None, seed=0):
    C = H * D
    S = S or B
    w = W.block_weights(C, torch.bfloat16, seed=seed, device=DEV)
    xh = W.block_inputs(B, n, C, torch.bfloat16, seed=seed + 1, device=DEV)
    xc = W.block_inputs(B, K, C, torch.bfloat16, seed=seed + 2, device=DEV)
    pool = fa.Pool.allocate(L, S, H, n, D, torch.bfloat16, DEV)
    return w, xh, xc, pool


SHAPES = [(3, 70, 33, 4, 32), (2, 130, 65, 8, 64), (2, 64, 20, 2, 128)]


# the block's GEMMs: hipBLASLt, or the library's kernel with each workgroup tile
GEMM_KERNELS = [fa.GEMM_LIBRARY, 0, 1, 2, 3]


@pytest.mark.parametrize("fold", [False, True], ids=["plain", "folded"])
@pytest.mark.parametrize("gemm", GEMM_KERNELS, ids=lambda k: "hipblaslt" if k == fa.GEMM_LIBRARY else f"tile{k}")
@pytest.mark.parametrize("B,n,K,H,D", SHAPES, ids=lambda x: str(x))
def test_block_history_then_candidates(B, n, K, H, D, gemm, fold):
    """History forward (fills the pool), then the candidate-only forward, against the
    oracle's two forwards and its joint pass; the pool rows against the oracle's.  Every
    shape is run with each GEMM kernel (rows B*n and B*K leave ragged row tiles), with
    the plain weights and with the LayerNorms folded into them (with this library's
    kernel pinned, the QKV and MLP-up projections then take the hidden state itself)."""
    announce(f"block history+candidates B={B} n={n} K={K} H={H} D={D} gemm={gemm} fold={fold}")
    w, xh, xc, pool = make(B, n, K, H, D, seed=50)
    wrun = fa.fold_layernorm(w) if fold else w
    lens = [n, n // 2, 0][:B]
    slots = [B - 1 - b for b in range(B)]
    layer = 1
    ctx = fa.BlockContext()
    ctx.set_gemm(gemm)
    xh0, xc0 = xh.clone(), xc.clone()
    fa.block_forward(ctx, wrun, fa.BLOCK_HISTORY, xh, pool, slots, lens, layer)
    fa.block_forward(ctx, wrun, fa.BLOCK_CANDIDATES, xc, pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    wc = {k: v.cpu() for k, v in w.items()}
    nanpool = np.full((2, B, H, n, D), np.nan)
    rh, rk, rv = oracle.block_history(xh0.cpu(), lens, wc, H, nanpool, nanpool.copy(), slots, layer)
    for b, N in enumerate(lens):
        if N:
            check_rel(xh[b, :N], rh[b, :N], f"history user {b}")
            s = slots[b]
            check_rel(pool.k[layer, s, :, :N], rk[layer, s, :, :N], f"pool K user {b}", 2, 1)
            check_rel(pool.v[layer, s, :, :N], rv[layer, s, :, :N], f"pool V user {b}", 2, 1)
    # the candidates against the joint pass over the exact inputs
    _, jc = oracle.block_joint(xh0.cpu(), xc0.cpu(), lens, wc, H)
    check_rel(xc, jc, "candidates vs the joint pass")
    # and against the candidate-only oracle on the pool the GPU wrote
    rc = oracle.block_candidates(xc0.cpu(), wc, H, pool.k.cpu(), pool.v.cpu(), slots, lens, layer)
    check_rel(xc, rc, "candidates over the GPU's pool")
    pool.close()
    ctx.close()


def test_block_candidates_independent_of_each_other():
    """A candidate's output is bitwise the same whatever other candidates share the call."""
    B, n, K, H, D = 2, 100, 40, 8, 64
    announce("block candidate independence")
    w, xh, xc, pool = make(B, n, K, H, D, seed=60)
    lens, slots = [n, 37], [1, 0]
    ctx = fa.BlockContext()
    fa.block_forward(ctx, w, fa.BLOCK_HISTORY, xh, pool, slots, lens, 0)
    full = xc.clone()
    fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, full, pool, slots, lens, 0)
    pick = [5, 17, 39, 0]
    part = xc[:, pick].contiguous()
    fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, part, pool, slots, lens, 0)
    torch.cuda.synchronize()
    # GEMM tiling may differ with the row count; compare to the oracle bound and, for
    # the attention-only part, exactly through a second call of the same size
    again = xc[:, pick].contiguous()
    fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, again, pool, slots, lens, 0)
    torch.cuda.synchronize()
    assert torch.equal(part, again), "repeated calls must be bitwise identical"
    check_rel(part, oracle.as_f64(full[:, pick]), "subset vs full call", 4, 1)
    pool.close()
    ctx.close()


@pytest.mark.parametrize("fold", [False, True], ids=["plain", "folded"])
@pytest.mark.parametrize("gemm", ["tuned", 0, 1, 2, 3], ids=lambda k: k if k == "tuned" else f"tile{k}")
def test_block_table2_shape_sampled(gemm, fold):
    """The pages' Table 2 shape (B=8, history 992, 656 candidates) at width 512
    (8 heads x 64), with the GEMM kernels the tuner picks and with each tile
    configuration of the library's GEMM pinned, with plain and with folded LayerNorm
    weights: history then candidate forward, sampled users against the oracle.  User
    7's candidate rows hold the last, partial 256-row tile of the candidate-side GEMMs
    (5248 rows)."""
    B, n, K, H, D = 8, 992, 656, 8, 64
    announce(f"block Table 2 shape gemm={gemm} fold={fold}")
    w0, xh, xc, pool = make(B, n, K, H, D, L=1, seed=70)
    w = fa.fold_layernorm(w0) if fold else w0
    lens = [n] * B
    slots = list(range(B))
    ctx = fa.BlockContext()
    if gemm == "tuned":
        ctx.tune(pool, B, n)   # the kernels the benchmark times
        ctx.tune(pool, B, K)
    else:
        ctx.set_gemm(gemm)
    xh0, xc0 = xh.clone(), xc.clone()
    fa.block_forward(ctx, w, fa.BLOCK_HISTORY, xh, pool, slots, lens, 0)
    fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, xc, pool, slots, lens, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    wc = {k: v.cpu() for k, v in w0.items()}
    for b in (0, 7):
        _, jc = oracle.block_joint(xh0[b:b + 1].cpu(), xc0[b:b + 1].cpu(), [n], wc, H)
        check_rel(xc[b:b + 1], jc, f"Table 2 shape, candidates of user {b}")
    pool.close()
    ctx.close()


@pytest.mark.parametrize("gemm", [0, 1, 2, 3], ids=lambda k: f"tile{k}")
def test_block_folded_rows_far_off_centre(gemm):
    """Rows whose mean is far above their spread (20 standard deviations; every other row
    of one user, so such rows share tiles with ordinary ones): the folded LayerNorm takes
    their statistics exactly, so the folded and the plain path agree within the block's
    rounding, and both match the oracle."""
    B, n, K, H, D = 2, 130, 65, 8, 64
    announce(f"block folded, rows far off centre, gemm={gemm}")
    w, xh, xc, pool = make(B, n, K, H, D, seed=95)
    for x in (xh, xc):
        x[0] += 20.0
        x[1, ::2] += 20.0
    lens, slots = [n, n], [0, 1]
    outs = {}
    for fold in (False, True):
        ctx = fa.BlockContext()
        ctx.set_gemm(gemm)
        wr = fa.fold_layernorm(w) if fold else w
        a, c = xh.clone(), xc.clone()
        fa.block_forward(ctx, wr, fa.BLOCK_HISTORY, a, pool, slots, lens, 0)
        fa.block_forward(ctx, wr, fa.BLOCK_CANDIDATES, c, pool, slots, lens, 0)
        torch.cuda.synchronize()
        assert pool.status() == 0
        outs[fold] = (a, c)
        ctx.close()
    check_rel(outs[True][0], oracle.as_f64(outs[False][0]), "history, folded vs plain")
    check_rel(outs[True][1], oracle.as_f64(outs[False][1]), "candidates, folded vs plain")
    wc = {k: v.cpu() for k, v in w.items()}
    _, jc = oracle.block_joint(xh.cpu(), xc.cpu(), lens, wc, H)
    check_rel(outs[True][1], jc, "candidates (folded) vs the joint pass")
    pool.close()


def test_fold_layernorm_values():
    """The folded weights: W' bit for bit the bf16 rounding of gamma W, u the column sums
    of W', v = beta W + b (fp32, summation order aside)."""
    C = 512
    w = W.block_weights(C, torch.bfloat16, seed=90, device=DEV)
    f = fa.fold_layernorm(w)
    torch.cuda.synchronize()
    for g, b, wm, bias, wl, uv in (("ln1_w", "ln1_b", "w_qkv", "b_qkv", "w_qkv_ln", "uv_qkv"),
                                   ("ln2_w", "ln2_b", "w_fc", "b_fc", "w_fc_ln", "uv_fc")):
        ref = (w[g].float()[:, None] * w[wm].float()).to(torch.bfloat16)
        assert torch.equal(f[wl], ref), wl
        u = f[wl].double().sum(0)
        v = w[b].double() @ w[wm].double() + w[bias].double()
        got = f[uv].double()
        assert torch.allclose(got[0], u, rtol=1e-5, atol=1e-5 * u.abs().max().item()), uv
        assert torch.allclose(got[1], v, rtol=1e-5, atol=1e-5 * v.abs().max().item()), uv


def test_block_bad_arguments():
    B, n, K, H, D = 1, 16, 4, 2, 32
    w, xh, xc, pool = make(B, n, K, H, D, seed=80)
    ctx = fa.BlockContext()
    with pytest.raises(fa.UnipinError):
        fa.block_forward(ctx, w, 7, xc, pool, [0], [n], 0)            # bad mode
    with pytest.raises(fa.UnipinError):
        fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, xc, pool, [0], [n], 2)   # layer out of range
    small = torch.empty(100, dtype=torch.uint8, device=DEV)
    with pytest.raises(fa.UnipinError):
        fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, xc, pool, [0], [n], 0, workspace=small)
    bad = dict(w)
    bad["w_o"] = w["w_qkv"]   # [C, 3C] where [C, C] belongs
    with pytest.raises(fa.UnipinError):
        fa.block_forward(ctx, bad, fa.BLOCK_CANDIDATES, xc, pool, [0], [n], 0)
    half = fa.fold_layernorm(w)
    del half["uv_qkv"]        # one of a folded pair without the other
    with pytest.raises(fa.UnipinError) as e:
        fa.block_forward(ctx, half, fa.BLOCK_CANDIDATES, xc, pool, [0], [n], 0)
    assert e.value.status == fa.EINVAL
    pool.close()
    ctx.close()


def test_block_twelve_layer_stack():
    """Twelve layers with their own weights: the history side fills each layer's pool
    rows, the candidate side reads them; the candidates' final hidden state against the
    oracle's joint pass chained over the same twelve layers.  Errors add up over the
    layers' residual stream: bound 12 u of max|ref| and 4 u of mean|ref|."""
    B, n, K, H, D, L = 2, 160, 48, 8, 64, 12
    announce("block twelve-layer stack")
    C = H * D
    ws = [W.block_weights(C, torch.bfloat16, seed=90 + l, device=DEV) for l in range(L)]
    xh = W.block_inputs(B, n, C, torch.bfloat16, seed=88, device=DEV)
    xc = W.block_inputs(B, K, C, torch.bfloat16, seed=89, device=DEV)
    pool = fa.Pool.allocate(L, B, H, n, D, torch.bfloat16, DEV)
    lens, slots = [n, 101], [1, 0]
    ctx = fa.BlockContext()
    rh, rc = oracle.as_f64(xh), oracle.as_f64(xc)
    for l in range(L):
        fa.block_forward(ctx, ws[l], fa.BLOCK_HISTORY, xh, pool, slots, lens, l)
        fa.block_forward(ctx, ws[l], fa.BLOCK_CANDIDATES, xc, pool, slots, lens, l)
        rh, rc = oracle.block_joint(rh, rc, lens, {k: v.cpu() for k, v in ws[l].items()}, H)
    torch.cuda.synchronize()
    assert pool.status() == 0
    check_rel(xc, rc, "candidates after 12 layers", 12, 4)
    for b, N in enumerate(lens):
        check_rel(xh[b, :N], rh[b, :N], f"history of user {b} after 12 layers", 12, 4)
    pool.close()
    ctx.close()
