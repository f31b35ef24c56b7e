"""Seeded random shapes through the whole attention path on the GPU, against the float64
oracle: a prefill into scattered slots of a poisoned pool (outputs and pool rows), the
ranking decode through the split entry point (which splits wherever its plan does; the
one-pass kernel is checked too when it does), and one autoregressive step on the same
slots, on bf16, E4M3 and fp32 pools.

Each case draws the pool format, the head dimension (32, 64 or 128; E4M3 pools hold
64 or 128), 1-6 users of 1-4 heads, the pool's row capacity, ragged history lengths
(empty and full ones included), 1-519 candidates, the layer of a one- or two-layer pool,
the slots and, for half of the cases, an explicit score scale (a value fp32 holds
exactly, since the C ABI passes it as a float).  Every fourth case uses a pool of
1000-1399 rows with few users, heads and candidates, the shapes the split plan takes.
Tolerances as in test_gpu_parity.py: fp32 max relative error <= 1e-5 (normwise and
element-wise with a 1e-3 floor); bf16 max abs error <= 2e-2 and mean <= 2e-3; pool rows
and codes bit for bit.
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
N_CASES = 24
F8 = torch.float8_e4m3fn


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def check_close(got: torch.Tensor, ref: np.ndarray, fp32: bool, what: str) -> None:
    g = got.detach().to("cpu").to(torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    diff = np.abs(g - r)
    if fp32:
        rel = diff.max() / max(np.abs(r).max(), 1e-30)
        assert rel <= 1e-5, f"{what}: normwise relative error {rel:.3e} > 1e-5"
        elem = (diff / np.maximum(np.abs(r), 1e-3)).max()
        assert elem <= 1e-5, f"{what}: element-wise relative error {elem:.3e} > 1e-5 (floor 1e-3)"
        return
    assert diff.max() <= 2e-2, f"{what}: max abs error {diff.max():.3e} > 2e-2"
    assert diff.mean() <= 2e-3, f"{what}: mean abs error {diff.mean():.3e} > 2e-3"


def draw(seed: int) -> dict:
    rng = np.random.default_rng(7000 + seed)
    fmt = ("bf16", "e4m3", "fp32")[seed % 3]
    D = int(rng.choice([64, 128])) if fmt == "e4m3" else int(rng.choice([32, 64, 128]))
    long = seed % 4 == 3
    if long:
        n_max, B, H, k = int(rng.integers(1000, 1400)), int(rng.integers(1, 3)), int(rng.integers(1, 3)), \
            int(rng.integers(1, 300))
    else:
        n_max, B, H, k = int(rng.integers(1, 520)), int(rng.integers(1, 7)), int(rng.integers(1, 5)), \
            int(rng.integers(1, 520))
    lens = rng.integers(0, n_max + 1, size=B)
    if B > 1:
        lens[rng.integers(0, B)] = n_max          # a full slot
    if B > 2:
        lens[rng.integers(0, B)] = 0              # an empty history
    L = int(rng.integers(1, 3))
    S = B + int(rng.integers(0, 3))
    return dict(fmt=fmt, D=D, n_max=n_max, B=B, H=H, k=k, lens=[int(x) for x in lens], L=L,
                layer=int(rng.integers(0, L)), S=S, slots=[int(x) for x in rng.permutation(S)[:B]],
                # the C ABI takes the scale as a float: draw one that fp32 holds exactly, so
                # that the oracle computes with the value the kernels receive
                scale=None if rng.random() < 0.5 else float(np.float32(rng.uniform(0.05, 0.3))))


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_through_the_path(seed):
    c = draw(seed)
    announce(f"random shape {seed}: {c}")
    fmt, D, n, B, H, k, lens, layer, slots, scale = (c[x] for x in ("fmt", "D", "n_max", "B", "H", "k", "lens",
                                                                     "layer", "slots", "scale"))
    fp32 = fmt == "fp32"
    act = torch.float32 if fp32 else torch.bfloat16
    inp = W.small_case(B, H, D, n, k, lens, dtype=act, seed=7100 + seed, device=DEV)
    if fmt == "e4m3":
        kp, vp = W.random_pool(c["L"], c["S"], H, n, D, torch.float32, seed=7200 + seed, device=DEV)
        pool = fa.Pool(kp.to(F8), vp.to(F8))
        del kp, vp
    else:
        pool = fa.Pool.allocate(c["L"], c["S"], H, n, D, act, DEV)
        pool.k.fill_(float("nan"))
        pool.v.fill_(float("nan"))
    before_k, before_v = ((codes(pool.k), codes(pool.v)) if fmt == "e4m3" else (pool.k.cpu(), pool.v.cpu()))

    # prefill: outputs of the history rows and the pool rows
    o = fa.prefill(inp["q"], inp["k"], inp["v"], lens, pool, slots, layer, scale=scale)
    torch.cuda.synchronize()
    assert pool.status() == 0
    ref_o = oracle.prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), lens, scale)
    for b, N in enumerate(lens):
        if N:
            check_close(o[b, :, :N], ref_o[b, :, :N], fp32, f"prefill user {b} N={N}")
    if fmt == "e4m3":
        rk, rv = oracle.pool_write_e4m3(before_k, before_v, inp["k"].cpu(), inp["v"].cpu(), lens, slots, layer)
        assert np.array_equal(codes(pool.k), rk) and np.array_equal(codes(pool.v), rv), "pool codes"
        pk, pv = oracle.e4m3_decode(rk), oracle.e4m3_decode(rv)
    else:
        rk, rv = oracle.pool_write(before_k, before_v, inp["k"].cpu(), inp["v"].cpu(), lens, slots, layer)
        gk, gv = oracle.as_f64(pool.k.cpu()), oracle.as_f64(pool.v.cpu())
        # NaN rows stay NaN on both sides; every written row equal
        assert np.array_equal(gk, rk, equal_nan=True) and np.array_equal(gv, rv, equal_nan=True), "pool rows"
        pk, pv = rk, rv

    # ranking decode through the split entry point, and the one-pass kernel where it splits
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer, scale=scale, split=True)
    split = fa.rank_decode_workspace_bytes(pool, B, k) > 0
    one = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer, scale=scale) if split else None
    torch.cuda.synchronize()
    assert pool.status() == 0
    ref_c = oracle.rank_decode(inp["qc"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), pk, pv, slots, lens, layer, scale)
    check_close(oc, ref_c, fp32, f"rank decode ({'split' if split else 'one pass'})")
    if one is not None:
        check_close(one, ref_c, fp32, "rank decode (one pass)")

    # one autoregressive step: user b's token goes to row min(N, n_max - 1)
    lens_ar = [min(N, n - 1) for N in lens]
    tok = W.step_tokens(B, H, D, 1, dtype=act, seed=7300 + seed, device=DEV)
    o1 = fa.ar_decode(tok["q"][0], tok["k"][0], tok["v"][0], pool, slots, lens_ar, layer, scale=scale)
    torch.cuda.synchronize()
    assert pool.status() == 0
    if fmt == "e4m3":
        r1, ak, av = oracle.ar_decode_e4m3(tok["q"][0].cpu(), tok["k"][0].cpu(), tok["v"][0].cpu(), rk, rv, slots,
                                           lens_ar, layer, scale)
        assert np.array_equal(codes(pool.k), ak) and np.array_equal(codes(pool.v), av), "pool codes after the step"
    else:
        r1, ak, av = oracle.ar_decode(tok["q"][0].cpu(), tok["k"][0].cpu(), tok["v"][0].cpu(), rk, rv, slots,
                                      lens_ar, layer, scale)
        gk, gv = oracle.as_f64(pool.k.cpu()), oracle.as_f64(pool.v.cpu())
        assert np.array_equal(gk, ak, equal_nan=True) and np.array_equal(gv, av, equal_nan=True), \
            "pool rows after the step"
    check_close(o1, r1, fp32, "autoregressive step")
    pool.close()
