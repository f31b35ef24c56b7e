"""GPU parity of the ranking decode split over the history (unipin_rank_decode_split),
on bf16 and E4M3 pools, against the float64 oracle, with the bf16 tolerances of
test_gpu_parity.py (max |gpu - oracle| <= 2e-2, mean <= 2e-3).

The split runs when few (user, head) pairs leave the GPU mostly idle: each candidate
tile's history goes to several workgroups, whose softmax states a second kernel merges
with the candidate's own key.  Every case here is small enough that the library plans
such a split (rank_decode_workspace_bytes > 0), and each is also run through the
one-pass kernel as a cross-check.
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


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def check_bf16(got: torch.Tensor, ref, what: str) -> float:
    g = got.detach().to("cpu").to(torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - r)
    assert d.max() <= 2e-2, f"{what}: max abs error {d.max():.3e} > 2e-2"
    assert d.mean() <= 2e-3, f"{what}: mean abs error {d.mean():.3e} > 2e-3"
    return float(d.max())


# (B, H, D, n_max, k, lens, layer)
CASES = [
    (1, 8, 64, 1024, 1000, [1024], 0),         # one request, full history: four parts of four tiles
    (2, 4, 128, 1024, 300, [1000, 37], 0),     # ragged: most of the short user's parts are empty
    (1, 2, 32, 1024, 40, [0], 0),              # empty history: the own value exactly
    (3, 2, 64, 1100, 257, [1100, 1, 64], 0),   # a partial candidate tile, a one-key history
    # D = 32 on the second layer of the pool: eight parts of four tiles over 2048 rows, a
    # 1500-key history ends inside part 5 (its last tile holds 28 keys), parts 6 and 7 are empty
    (1, 4, 32, 2048, 500, [1500], 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}D{c[2]}n{c[3]}k{c[4]}L{c[6]}")
def test_split_decode_against_the_oracle(case):
    B, H, D, n, k, lens, layer = case
    announce(f"split decode {case}")
    inp = W.small_case(B, H, D, n, k, lens, seed=3000 + n + k, device=DEV)
    pool = fa.Pool.allocate(layer + 1, B + 1, H, n, D, torch.bfloat16, DEV)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    slots = list(range(B, 0, -1))
    fa.prefill(inp["q"], inp["k"], inp["v"], lens, pool, slots, layer)
    need = fa.rank_decode_workspace_bytes(pool, B, k)
    assert need > 0, "the case must take the split path"
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer, split=True)
    one = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    for b, N in enumerate(lens):
        s = slots[b]
        pk = oracle.as_f64(pool.k[layer, s, :, :N].cpu()).reshape(1, 1, H, N, D)
        pv = oracle.as_f64(pool.v[layer, s, :, :N].cpu()).reshape(1, 1, H, N, D)
        sub = {key: inp[key][b:b + 1].cpu() for key in ("qc", "kc", "vc")}
        ref = oracle.rank_decode(sub["qc"], sub["kc"], sub["vc"], pk, pv, [0], [N], 0, None)
        check_bf16(oc[b:b + 1], ref, f"split decode user {b} N={N}")
        check_bf16(one[b:b + 1], ref, f"one-pass decode user {b} N={N}")
        if N == 0:
            assert torch.equal(oc[b], inp["vc"][b]), "an empty history must return vc exactly"


F8 = torch.float8_e4m3fn

# (B, H, D, n_max, k, lens, layer) on a pool of E4M3 codes of N(0, 1) draws
E4M3_CASES = [
    (1, 8, 64, 1024, 1000, [1024], 0),          # one request, full history: four parts of four tiles
    (2, 4, 128, 1100, 300, [1100, 37], 1),      # ragged, second layer: the short user's parts mostly empty
    (3, 2, 64, 2048, 257, [1500, 0, 65], 0),    # a history ending inside a part, an empty one, a partial tile
]


@pytest.mark.parametrize("case", E4M3_CASES, ids=lambda c: f"B{c[0]}H{c[1]}D{c[2]}n{c[3]}k{c[4]}L{c[6]}")
def test_split_decode_on_e4m3_pool(case):
    """The split path on an E4M3 pool: each part decodes its staged tiles of codes to bf16
    in LDS; against the oracle on the decoded pool, and through the one-pass kernel."""
    B, H, D, n, k, lens, layer = case
    announce(f"split decode, E4M3 pool {case}")
    kp, vp = W.random_pool(layer + 1, B + 1, H, n, D, torch.float32, seed=3400 + n + k, device=DEV)
    pool = fa.Pool(kp.to(F8), vp.to(F8))
    del kp, vp
    slots = list(range(B, 0, -1))
    inp = W.small_case(B, H, D, 8, k, [1] * B, seed=3500 + n + k, device=DEV)   # qc, kc, vc
    assert fa.rank_decode_workspace_bytes(pool, B, k) > 0, "the case must take the split path"
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer, split=True)
    one = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    pk = oracle.e4m3_decode(pool.k.detach().cpu().view(torch.uint8).numpy())
    pv = oracle.e4m3_decode(pool.v.detach().cpu().view(torch.uint8).numpy())
    ref = oracle.rank_decode(inp["qc"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), pk, pv, slots, lens, layer)
    check_bf16(oc, ref, f"E4M3 split decode {case}")
    check_bf16(one, ref, f"E4M3 one-pass decode {case}")
    for b, N in enumerate(lens):
        if N == 0:
            assert torch.equal(oc[b], inp["vc"][b]), "an empty history must return vc exactly"
    pool.close()


def test_split_decode_repeated_calls_are_bitwise_identical():
    B, H, D, n, k = 1, 8, 64, 1024, 600
    inp = W.small_case(B, H, D, n, k, [980], seed=3100, device=DEV)
    pool = fa.Pool.allocate(1, 1, H, n, D, torch.bfloat16, DEV)
    fa.prefill(inp["q"], inp["k"], inp["v"], [980], pool, [0], 0)
    ws = torch.empty(fa.rank_decode_workspace_bytes(pool, B, k), dtype=torch.uint8, device=DEV)
    a = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0], [980], 0, split=True, workspace=ws)
    ws.fill_(0xff)   # the workspace is scratch: its contents before a call do not matter
    b = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0], [980], 0, split=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_split_decode_invalid_user_is_skipped_and_flagged():
    B, H, D, n, k = 3, 2, 64, 1024, 64
    announce("split decode status flags")
    inp = W.small_case(B, H, D, n, k, [1024, 64, 10], seed=3200, device=DEV)
    pool = fa.Pool.allocate(1, 3, H, n, D, torch.bfloat16, DEV)
    fa.prefill(inp["q"], inp["k"], inp["v"], [1024, 64, 10], pool, [0, 1, 2], 0)
    assert pool.status() == 0
    assert fa.rank_decode_workspace_bytes(pool, B, k) > 0
    oc = torch.full_like(inp["qc"], 7.0)
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0, -1, 2], [1024, 64, 10], 0, oc=oc, split=True)
    assert pool.status() == fa.FLAG_BAD_SLOT
    assert (oc[1] == 7.0).all(), "a skipped user's output must stay untouched"
    assert torch.isfinite(oc[0]).all() and torch.isfinite(oc[2]).all()
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0, 1, 2], [1024, 1025, 10], 0, oc=oc, split=True)
    assert pool.status() == fa.FLAG_BAD_LEN
    assert pool.status() == 0


def test_split_decode_without_a_plan_is_the_one_pass_kernel():
    """Where the plan keeps the one-pass kernel (a 512-row pool; 64 candidate tiles on a
    1024-row one), the split entry point runs it: outputs bitwise equal, a workspace
    passed in is ignored."""
    for (B, H, D, n, k, lens) in ((1, 8, 64, 512, 300, [512]), (2, 8, 64, 1024, 1000, [1024, 700])):
        announce(f"split entry without a split: B={B} H={H} D={D} n={n} k={k}")
        inp = W.small_case(B, H, D, n, k, lens, seed=3600 + n + k, device=DEV)
        pool = fa.Pool.allocate(1, B, H, n, D, torch.bfloat16, DEV)
        slots = list(range(B))
        fa.prefill(inp["q"], inp["k"], inp["v"], lens, pool, slots, 0)
        assert fa.rank_decode_workspace_bytes(pool, B, k) == 0
        ws = torch.full((64,), 0xff, dtype=torch.uint8, device=DEV)
        a = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, 0, split=True, workspace=ws)
        b = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, lens, 0)
        torch.cuda.synchronize()
        assert pool.status() == 0
        assert torch.equal(a, b)


def test_split_decode_workspace_checks():
    B, H, D, n, k = 1, 4, 64, 1024, 100
    inp = W.small_case(B, H, D, n, k, [300], seed=3300, device=DEV)
    pool = fa.Pool.allocate(1, 1, H, n, D, torch.bfloat16, DEV)
    need = fa.rank_decode_workspace_bytes(pool, B, k)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(fa.UnipinError) as e:
        fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0], [300], 0, split=True, workspace=small)
    assert e.value.status == fa.EINVAL
    odd = torch.empty(need + 16, dtype=torch.uint8, device=DEV)[4:]
    with pytest.raises(fa.UnipinError) as e:
        fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0], [300], 0, split=True, workspace=odd)
    assert e.value.status == fa.EALIGN
    # fp32 pools always take the one-pass kernel
    p32 = fa.Pool.allocate(1, 1, H, n, D, torch.float32, DEV)
    assert fa.rank_decode_workspace_bytes(p32, B, k) == 0
