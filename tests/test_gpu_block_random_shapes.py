"""Seeded random shapes through the transformer block (unipin_block_forward) on the GPU,
against the float64 oracle: the history forward into scattered slots, then the
candidate-only forward over the pool it wrote.

Each case draws the head dimension (32, 64 or 128) and head count (width H*D from 32 to
1024), 1-4 users, history and candidate row counts, ragged history lengths (empty and
full ones included), a pool capacity at or above the history rows, the layer of a one-
or two-layer pool, the slots, the pool format (bf16 or, at D = 64 and 128, E4M3), the
GEMM kernels (hipBLASLt, the untuned default, or the library's kernel in one of its
tile configurations) and, with the library's kernel, whether the LayerNorms are folded
into the weights.  Bounds as in test_gpu_block.py, relative to bf16's unit roundoff
u = 2^-8 and to the reference's magnitude: one block max 4 u / mean 1 u; pool rows
(bf16 pools) max 2 u / mean 1 u.  On an E4M3 pool the candidates are checked against
the oracle's candidate forward over the codes the GPU stored.
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
N_CASES = 12
F8 = torch.float8_e4m3fn


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
    assert mx <= max_units * U, f"{what}: max error {mx / U:.2f} u of max|ref| > {max_units} u"
    assert mn <= mean_units * U, f"{what}: mean error {mn / U:.3f} u of mean|ref| > {mean_units} u"


def draw(seed: int) -> dict:
    rng = np.random.default_rng(8000 + seed)
    D = int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 1024 // D + 1))
    B = int(rng.integers(1, 5))
    n, K = int(rng.integers(1, 300)), int(rng.integers(1, 200))
    lens = rng.integers(0, n + 1, size=B)
    if B > 1:
        lens[rng.integers(0, B)] = n
    if B > 2:
        lens[rng.integers(0, B)] = 0
    L = int(rng.integers(1, 3))
    S = B + int(rng.integers(0, 3))
    gemm = int(rng.choice([fa.GEMM_LIBRARY, fa.GEMM_AUTO, 0, 1, 2, 3]))
    return dict(D=D, H=H, B=B, n=n, K=K, lens=[int(x) for x in lens], n_max=n + int(rng.integers(0, 40)), L=L,
                layer=int(rng.integers(0, L)), S=S, slots=[int(x) for x in rng.permutation(S)[:B]],
                e4m3=D >= 64 and bool(rng.random() < 0.3), gemm=gemm, fold=gemm >= 0 and bool(rng.random() < 0.5))


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_block_shape(seed):
    c = draw(seed)
    announce(f"random block shape {seed}: {c}")
    D, H, B, n, K, lens, layer, slots = (c[x] for x in ("D", "H", "B", "n", "K", "lens", "layer", "slots"))
    C = H * D
    w = W.block_weights(C, torch.bfloat16, seed=8100 + seed, device=DEV)
    xh = W.block_inputs(B, n, C, torch.bfloat16, seed=8200 + seed, device=DEV)
    xc = W.block_inputs(B, K, C, torch.bfloat16, seed=8300 + seed, device=DEV)
    shape = (c["L"], c["S"], H, c["n_max"], D)
    if c["e4m3"]:
        pool = fa.Pool(torch.zeros(shape, dtype=F8, device=DEV), torch.zeros(shape, dtype=F8, device=DEV))
    else:
        pool = fa.Pool.allocate(*shape, torch.bfloat16, DEV)
        pool.k.fill_(float("nan"))
        pool.v.fill_(float("nan"))
    ctx = fa.BlockContext()
    ctx.set_gemm(c["gemm"])
    wrun = fa.fold_layernorm(w) if c["fold"] else w
    xh0, xc0 = xh.cpu(), xc.cpu()
    fa.block_forward(ctx, wrun, fa.BLOCK_HISTORY, xh, pool, slots, lens, layer)
    fa.block_forward(ctx, wrun, fa.BLOCK_CANDIDATES, xc, pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    wc = {k: v.cpu() for k, v in w.items()}
    nanpool = np.full(shape, np.nan)
    rh, rk, rv = oracle.block_history(xh0, lens, wc, H, nanpool, nanpool.copy(), slots, layer)
    for b, N in enumerate(lens):
        if not N:
            continue
        check_rel(xh[b, :N], rh[b, :N], f"history user {b} N={N}")
        if not c["e4m3"]:
            s = slots[b]
            check_rel(pool.k[layer, s, :, :N], rk[layer, s, :, :N], f"pool K user {b}", 2, 1)
            check_rel(pool.v[layer, s, :, :N], rv[layer, s, :, :N], f"pool V user {b}", 2, 1)
    if c["e4m3"]:
        pk, pv = oracle.e4m3_decode(codes(pool.k)), oracle.e4m3_decode(codes(pool.v))
    else:
        pk, pv = pool.k.cpu(), pool.v.cpu()
    rc = oracle.block_candidates(xc0, wc, H, pk, pv, slots, lens, layer)
    check_rel(xc, rc, "candidates over the GPU's pool")
    if not c["e4m3"]:
        _, jc = oracle.block_joint(xh0, xc0, lens, wc, H)
        check_rel(xc, jc, "candidates against the joint pass")
    ctx.close()
    pool.close()
