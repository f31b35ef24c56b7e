"""GPU parity of the E4M3 KV pool (UNIPIN_FP8_E4M3) against the oracle.

Codes are integers: every code the GPU stores must equal the oracle's, bit for bit.
The encoding is checked on every finite bf16 value, and the decoding on every code,
through the library's own pool writes and reads.  Attention outputs over E4M3 rows are
bf16 results and take the usual bf16 bounds (max abs 2e-2, mean abs 2e-3).
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
F8 = torch.float8_e4m3fn


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


def check_close(got, ref, what):
    g = oracle.as_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - r)
    assert d.max() <= 2e-2, f"{what}: max abs error {d.max():.3e} > 2e-2"
    assert d.mean() <= 2e-3, f"{what}: mean abs error {d.mean():.3e} > 2e-3"


def e4m3_pool(L, S, H, n_max, D, seed):
    """An E4M3 pool holding the codes of N(0, 1) draws (stand-ins for earlier rows)."""
    k, v = W.random_pool(L, S, H, n_max, D, torch.float32, seed=seed, device=DEV)
    return fa.Pool(k.to(F8), v.to(F8))


def test_prefill_stores_the_code_of_every_finite_bf16_value():
    """Every finite bf16 bit pattern as a key (q = 0, so every score is exactly 0): the
    pool must hold the oracle's code of each, saturation and subnormals included."""
    announce("e4m3 encoding of every finite bf16 value")
    D, n = 64, 1024
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16)
    finite = torch.isfinite(vals.float())
    k = torch.where(finite, vals, torch.zeros_like(vals)).reshape(1, 1, n, D).to(DEV)
    q = torch.zeros_like(k)
    v = torch.zeros_like(k)
    pool = fa.Pool(torch.zeros((1, 1, 1, n, D), dtype=F8, device=DEV), torch.zeros((1, 1, 1, n, D), dtype=F8, device=DEV))
    fa.prefill(q, k, v, [n], pool, [0], 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    got = codes(pool.k).reshape(-1)
    ref = oracle.e4m3_encode(k.cpu()).reshape(-1)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at bf16 bits {int(bits.reshape(-1)[bad[0]]) & 0xffff:#06x}"
    assert not codes(pool.v).any()
    pool.close()


def test_ar_step_reads_every_code_exactly():
    """User c's slot holds one row of code c in every dimension; with q = 0 and a zero
    new token the step returns decode(c) / 2 exactly (equal weights on the row and the
    token), for every non-NaN code."""
    announce("e4m3 decoding of every code")
    D = 64
    cs = [c for c in range(256) if c not in (0x7F, 0xFF)]
    B = len(cs)
    kp = torch.zeros((1, B, 1, 4, D), dtype=torch.uint8)
    for b, c in enumerate(cs):
        kp[0, b, 0, 0] = c
    pool = fa.Pool(kp.to(DEV).view(F8), kp.to(DEV).view(F8).clone())
    z = torch.zeros((B, 1, 1, D), dtype=torch.bfloat16, device=DEV)
    o = fa.ar_decode(z, z, z, pool, list(range(B)), [1] * B, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    exp = oracle.e4m3_decode(np.array(cs, dtype=np.uint8)) / 2
    got = o[:, 0, 0].double().cpu().numpy()
    assert np.array_equal(got, np.repeat(exp[:, None], D, axis=1)), "decoded values differ"
    assert not codes(pool.k)[0, :, 0, 1].any(), "the zero token is stored as code 0 at row 1"
    pool.close()


def test_ar_step_stores_nan_and_extreme_tokens_as_the_oracle_does():
    """The new token's K/V row goes to the pool as codes: NaN stays NaN (sign kept),
    infinities and huge values saturate, subnormal-range values round as specified."""
    announce("e4m3 codes of NaN and extreme token values")
    D = 64
    special = torch.tensor([float("nan"), -float("nan"), float("inf"), -float("inf"), 1e30, -500.0, 464.0, 2.0 ** -10,
                            3 * 2.0 ** -10, -2.0 ** -12, 0.0, -0.0, 447.9, 1.0625, 1.1875, -1.8125], dtype=torch.float32)
    k = special.repeat(D // special.numel()).to(torch.bfloat16).reshape(1, 1, 1, D).to(DEV)
    pool = fa.Pool(torch.zeros((1, 1, 1, 4, D), dtype=F8, device=DEV), torch.zeros((1, 1, 1, 4, D), dtype=F8, device=DEV))
    z = torch.zeros_like(k)
    fa.ar_decode(z, k, k, pool, [0], [2], 0)
    torch.cuda.synchronize()
    got = codes(pool.k)[0, 0, 0, 2]
    ref = oracle.e4m3_encode(k.cpu().reshape(-1))
    assert np.array_equal(got, ref), (got.tolist()[:16], ref.tolist()[:16])
    assert np.array_equal(codes(pool.v)[0, 0, 0, 2], ref)
    pool.status()   # NaN attention output is expected; clear nothing else
    pool.close()


@pytest.mark.parametrize("D,n_max", [(64, 601), (128, 601), (64, 4600), (128, 4600)], ids=str)
def test_ar_step_on_e4m3_pool(D, n_max):
    """Mixed fill levels, one pass (n_max 601) and the split path (n_max 4600)."""
    announce(f"e4m3 retrieval step D={D} n_max={n_max}")
    L, S, H, layer = 2, 9, 2, 1
    lens = [0, 1, 63, 64, 65, 200, 511, min(2047, n_max - 1), n_max - 1]
    slots = [4, 0, 8, 2, 7, 1, 3, 6, 5]
    B = len(lens)
    pool = e4m3_pool(L, S, H, n_max, D, seed=51)
    if n_max > 4000:
        assert fa.ar_decode_workspace_bytes(pool, B) > 0, "this shape must take the split path"
    tok = W.step_tokens(B, H, D, 1, torch.bfloat16, seed=52, device=DEV)
    q, k, v = tok["q"][0], tok["k"][0], tok["v"][0]
    before_k, before_v = codes(pool.k), codes(pool.v)
    o = fa.ar_decode(q, k, v, pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    ref, rk, rv = oracle.ar_decode_e4m3(q.cpu(), k.cpu(), v.cpu(), before_k, before_v, slots, lens, layer)
    check_close(o, ref, f"e4m3 step D={D}")
    assert np.array_equal(codes(pool.k), rk) and np.array_equal(codes(pool.v), rv), "pool codes"
    pool.close()


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_on_e4m3_pool(D):
    """The history attention runs on the bf16 inputs; the pool receives their codes."""
    announce(f"e4m3 prefill D={D}")
    B, H, n = 3, 2, 300
    lens = [300, 129, 0]
    slots = [1, 2, 0]
    inp = W.small_case(B, H, D, n, 8, lens, seed=53, device=DEV)
    pool = e4m3_pool(1, 3, H, n, D, seed=54)
    before_k, before_v = codes(pool.k), codes(pool.v)
    o = fa.prefill(inp["q"], inp["k"], inp["v"], lens, pool, slots, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    ref = oracle.prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), lens)
    for b, N in enumerate(lens):
        if N:
            check_close(o[b, :, :N], ref[b, :, :N], f"prefill user {b}")
    rk, rv = oracle.pool_write_e4m3(before_k, before_v, inp["k"].cpu(), inp["v"].cpu(), lens, slots, 0)
    assert np.array_equal(codes(pool.k), rk) and np.array_equal(codes(pool.v), rv), "pool codes"
    pool.close()


def test_rank_decode_reads_every_code_exactly():
    """User c's slot holds one row of code c; its one candidate has q = k = v = 0, so the
    output is decode(c) / 2 exactly, for every non-NaN code."""
    announce("e4m3 ranking decode of every code")
    D = 64
    cs = [c for c in range(256) if c not in (0x7F, 0xFF)]
    B = len(cs)
    kp = torch.zeros((1, B, 1, 4, D), dtype=torch.uint8)
    for b, c in enumerate(cs):
        kp[0, b, 0, 0] = c
    pool = fa.Pool(kp.to(DEV).view(F8), kp.to(DEV).view(F8).clone())
    z = torch.zeros((B, 1, 1, D), dtype=torch.bfloat16, device=DEV)
    oc = fa.rank_decode(z, z, z, pool, list(range(B)), [1] * B, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    exp = oracle.e4m3_decode(np.array(cs, dtype=np.uint8)) / 2
    assert np.array_equal(oc[:, 0, 0].double().cpu().numpy(), np.repeat(exp[:, None], D, axis=1))
    pool.close()


@pytest.mark.parametrize("D,k", [(64, 1), (64, 300), (64, 600), (128, 100), (128, 513)], ids=str)
def test_rank_decode_on_e4m3_pool(D, k):
    """Histories of 0 to n_max rows (0, 1 and 2 tiles, partial tiles) and 1 to 3
    candidate tiles, against the oracle on the decoded pool."""
    announce(f"e4m3 ranking decode D={D} k={k}")
    L, S, H, n_max, layer = 2, 9, 2, 700, 1
    lens = [0, 1, 63, 64, 65, 128, 200, 511, n_max][: 9]
    slots = [4, 0, 8, 2, 7, 1, 3, 6, 5]
    B = len(lens)
    pool = e4m3_pool(L, S, H, n_max, D, seed=55)
    inp = W.small_case(B, H, D, 8, k, [1] * B, seed=56, device=DEV)
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    pk, pv = oracle.e4m3_decode(codes(pool.k)), oracle.e4m3_decode(codes(pool.v))
    ref = oracle.rank_decode(inp["qc"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), pk, pv, slots, lens, layer)
    check_close(oc, ref, f"e4m3 ranking decode D={D} k={k}")
    pool.close()


def test_serving_shape_on_e4m3_pool_sampled():
    """The 12-layer serving shape (64 requests x 8 heads, history 512, 1000 candidates)
    prefilled into an E4M3 pool and decoded, sampled (layer, user) against the oracle."""
    w = W.WORKLOADS[3]
    announce("e4m3 serving shape")
    lens = W.history_lengths(w).tolist()
    pool = fa.Pool(torch.zeros((w.L, w.S, w.H, w.n, w.D), dtype=F8, device=DEV),
                   torch.zeros((w.L, w.S, w.H, w.n, w.D), dtype=F8, device=DEV))
    slots = pool.acquire_many(w.B)
    checks = [(0, 3), (11, 60)]
    outs = {}
    for l in range(w.L):
        x = W.layer_inputs(w, l, DEV)
        fa.prefill(x["q"], x["k"], x["v"], lens, pool, slots, l)
        oc = fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens, l)
        for (cl, b) in checks:
            if cl == l:
                outs[(l, b)] = (oc[b:b + 1].cpu(), {kk: vv[b:b + 1].cpu() for kk, vv in x.items()})
    torch.cuda.synchronize()
    assert pool.status() == 0
    for (l, b), (got, x) in outs.items():
        s = slots[b]
        pk = oracle.e4m3_decode(codes(pool.k[l:l + 1, s:s + 1]))
        pv = oracle.e4m3_decode(codes(pool.v[l:l + 1, s:s + 1]))
        assert np.array_equal(codes(pool.k[l, s, :, :lens[b]]), oracle.e4m3_encode(x["k"][0, :, :lens[b]]))
        ref = oracle.rank_decode(x["qc"], x["kc"], x["vc"], pk, pv, [0], [lens[b]], 0)
        check_close(got, ref, f"e4m3 serving shape layer {l} user {b}")
    pool.close()


def test_block_on_e4m3_pool():
    """The transformer block with an E4M3 pool: the history forward stores codes, the
    candidate forward reads them; against the oracle's candidate forward on the decoded
    pool the GPU wrote (bf16 bounds relative to the output's size)."""
    announce("block on an e4m3 pool")
    B, n, K, H, D = 2, 130, 65, 8, 64
    C = H * D
    w = W.block_weights(C, torch.bfloat16, seed=57, device=DEV)
    xh = W.block_inputs(B, n, C, torch.bfloat16, seed=58, device=DEV)
    xc = W.block_inputs(B, K, C, torch.bfloat16, seed=59, device=DEV)
    pool = fa.Pool(torch.zeros((1, B, H, n, D), dtype=F8, device=DEV), torch.zeros((1, B, H, n, D), dtype=F8, device=DEV))
    lens, slots = [n, 71], [1, 0]
    ctx = fa.BlockContext()
    xc0 = xc.cpu()
    fa.block_forward(ctx, w, fa.BLOCK_HISTORY, xh, pool, slots, lens, 0)
    fa.block_forward(ctx, w, fa.BLOCK_CANDIDATES, xc, pool, slots, lens, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    pk, pv = oracle.e4m3_decode(codes(pool.k)), oracle.e4m3_decode(codes(pool.v))
    ref = oracle.block_candidates(xc0, {kk: vv.cpu() for kk, vv in w.items()}, H, pk, pv, slots, lens, 0)
    g = oracle.as_f64(xc)
    u = 2.0 ** -8
    assert np.abs(g - ref).max() <= 4 * u * np.abs(ref).max()
    assert np.abs(g - ref).mean() <= 1 * u * np.abs(ref).mean()
    ctx.close()
    pool.close()
