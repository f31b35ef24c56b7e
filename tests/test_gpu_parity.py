"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (applied to history rows t < lens[b] and to every candidate row):
  * fp32: max relative error <= 1e-5, checked two ways: normwise,
    max|gpu - oracle| / max|oracle| per output tensor, and element by element,
    max |gpu - oracle| / max(|oracle|, 1e-3) (the floor keeps outputs near zero, whose
    relative error is undefined, from deciding the figure);
  * bf16 inputs with fp32 accumulation: max|gpu - oracle| <= 2e-2 and
    mean|gpu - oracle| <= 2e-3.
The oracle runs on the exact bits the GPU received (upcast to float64).  Integer and
byte results (pool contents, rows that must stay untouched, permutation and
composition invariance of a candidate's output) are compared bit for bit.
"""
import math
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


def check_close(got: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str):
    g = got.detach().to("cpu").to(torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    diff = np.abs(g - r)
    if dtype == torch.float32:
        rel = diff.max() / max(np.abs(r).max(), 1e-30)
        assert rel <= 1e-5, f"{what}: normwise relative error {rel:.3e} > 1e-5"
        elem = (diff / np.maximum(np.abs(r), 1e-3)).max()
        assert elem <= 1e-5, f"{what}: element-wise relative error {elem:.3e} > 1e-5 (floor 1e-3)"
        return max(rel, elem)
    mx, mean = diff.max(), diff.mean()
    assert mx <= 2e-2, f"{what}: max abs error {mx:.3e} > 2e-2"
    assert mean <= 2e-3, f"{what}: mean abs error {mean:.3e} > 2e-3"
    return mx


def hist_rows(x: torch.Tensor, lens) -> list:
    return [x[b, :, : int(n)] for b, n in enumerate(lens)]


def run_layer(pool, inp, lens, slots, layer, scale=None):
    lens_d = torch.as_tensor(lens, dtype=torch.int32).to(DEV)
    slots_d = torch.as_tensor(slots, dtype=torch.int32).to(DEV)
    o = fa.prefill(inp["q"], inp["k"], inp["v"], lens_d, pool, slots_d, layer, scale=scale)
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots_d, lens_d, layer, scale=scale)
    torch.cuda.synchronize()
    return o, oc


def full_check(inp, lens, o, oc, pool, slots, layer, dtype, users=None, scale=None, tag=""):
    """Oracle on selected users (all heads, all rows); pool rows compared bit for bit."""
    users = range(len(lens)) if users is None else users
    for b in users:
        N = int(lens[b])
        sub = {k: v[b : b + 1].cpu() for k, v in inp.items() if k in ("q", "k", "v", "qc", "kc", "vc")}
        ref_o = oracle.prefill(sub["q"], sub["k"], sub["v"], [N], scale)
        if N:
            check_close(o[b : b + 1, :, :N], ref_o[:, :, :N], dtype, f"{tag} prefill user {b} N={N}")
        s = int(slots[b])
        pk = pool.k[layer, s, :, :N].cpu()
        pv = pool.v[layer, s, :, :N].cpu()
        assert torch.equal(pk, inp["k"][b, :, :N].cpu()), f"{tag} pool K user {b}"
        assert torch.equal(pv, inp["v"][b, :, :N].cpu()), f"{tag} pool V user {b}"
        # decode against the oracle reading the (bitwise-checked) pool rows
        ref_c = oracle.rank_decode(sub["qc"], sub["kc"], sub["vc"],
                                   oracle.as_f64(pk).reshape(1, 1, *pk.shape),
                                   oracle.as_f64(pv).reshape(1, 1, *pv.shape), [0], [N], 0, scale)
        check_close(oc[b : b + 1], ref_c, dtype, f"{tag} decode user {b} N={N}")


# ------------------------------------------------------------------ workload configs

@pytest.mark.parametrize("idx", [0, 1])
def test_workload_full(idx):
    w = W.WORKLOADS[idx]
    announce(f"workload {idx} full: {w.name}")
    lens = W.history_lengths(w).tolist()
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, w.dtype, DEV)
    slots = pool.acquire_many(w.B)
    inp = W.layer_inputs(w, 0, DEV)
    o, oc = run_layer(pool, inp, lens, slots, 0)
    full_check(inp, lens, o, oc, pool, slots, 0, w.dtype, tag=f"w{idx}")
    assert pool.status() == 0


def test_workload_ragged_sampled_users():
    w = W.WORKLOADS[2]
    announce(f"workload 2 sampled users: {w.name}")
    lens = W.history_lengths(w).tolist()
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, w.dtype, DEV)
    slots = pool.acquire_many(w.B)
    inp = W.layer_inputs(w, 0, DEV)
    o, oc = run_layer(pool, inp, lens, slots, 0)
    order = np.argsort(lens)
    # the shortest and longest histories, the users around the length quartiles, and
    # every fourth user (all heads, all rows of each)
    users = sorted(set([int(order[i]) for i in (0, 1, 16, 32, 48, 62, 63)] + list(range(0, 64, 4))))
    assert len(users) >= 16
    full_check(inp, lens, o, oc, pool, slots, 0, w.dtype, users=users, tag="w2")
    assert pool.status() == 0


def test_serving_shape_twelve_layers_sampled():
    """The 12-layer serving shape: 12 prefills into rotating slots, then 12 decodes; two
    request batches so the 64 slots are handed out twice."""
    w = W.WORKLOADS[3]
    announce(f"workload 3 (12 layers), sampled heads: {w.name}")
    lens = W.history_lengths(w).tolist()
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, w.dtype, DEV)
    rng = np.random.default_rng(3)
    for batch in range(2):
        slots = pool.acquire_many(w.B)
        assert slots == list(range(64))
        assert pool.generation(0) == batch + 1
        lens_d = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
        slots_d = torch.as_tensor(slots, dtype=torch.int32, device=DEV)
        layers = [W.layer_inputs(w, l + 100 * batch, DEV) for l in range(w.L)]
        outs = [fa.prefill(x["q"], x["k"], x["v"], lens_d, pool, slots_d, l) for l, x in enumerate(layers)]
        outc = [fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots_d, lens_d, l) for l, x in enumerate(layers)]
        torch.cuda.synchronize()
        for l in (0, 6, 11):
            x = layers[l]
            assert torch.equal(pool.k[l].cpu(), x["k"].cpu()), f"pool K layer {l}"
            assert torch.equal(pool.v[l].cpu(), x["v"].cpu()), f"pool V layer {l}"
            for _ in range(3):
                b, h = int(rng.integers(64)), int(rng.integers(8))
                ref_o = oracle.prefill(x["q"][b:b+1, h:h+1].cpu(), x["k"][b:b+1, h:h+1].cpu(),
                                       x["v"][b:b+1, h:h+1].cpu(), [512])
                check_close(outs[l][b:b+1, h:h+1], ref_o, w.dtype, f"prefill layer {l} b{b} h{h}")
                ref_c = oracle.rank_decode_rows(x["qc"][b, h].cpu(), x["kc"][b, h].cpu(), x["vc"][b, h].cpu(),
                                                pool.k[l, slots[b], h].cpu(), pool.v[l, slots[b], h].cpu(),
                                                range(1000))
                check_close(outc[l][b, h], ref_c, w.dtype, f"decode layer {l} b{b} h{h}")
    assert pool.status() == 0


def test_long_history_sampled():
    """Long histories (D = 128): every head of the shortest, the longest and two more
    users.  Per (user, head): the first and last row of every 256-row query tile and of
    every 256-candidate tile, the rows around each 64-key tile edge of the first tile,
    and random rows; pool rows bit for bit."""
    w = W.WORKLOADS[4]
    announce(f"workload 4 sampled rows: {w.name}")
    lens = W.history_lengths(w).tolist()
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, w.dtype, DEV)
    slots = pool.acquire_many(w.B)
    inp = W.layer_inputs(w, 0, DEV)
    o, oc = run_layer(pool, inp, lens, slots, 0)
    rng = np.random.default_rng(4)
    order = np.argsort(lens)
    users = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2]), 5]))
    assert len(users) >= 4
    tile = 256
    for b in users:
        N = lens[b]
        assert torch.equal(pool.k[0, slots[b], :, :N].cpu(), inp["k"][b, :, :N].cpu())
        assert torch.equal(pool.v[0, slots[b], :, :N].cpu(), inp["v"][b, :, :N].cpu())
        edges = [r for t in range(0, N, tile) for r in (t, min(t + tile, N) - 1)]
        crow_edges = [r for t in range(0, w.k, tile) for r in (t, min(t + tile, w.k) - 1)]
        for h in range(w.H):
            rows = sorted(set(edges + [1, 63, 64, 65, 127, 128] + rng.integers(0, N, 12).tolist()))
            rows = [r for r in rows if r < N]
            ref = oracle.prefill_rows(inp["q"][b, h].cpu(), inp["k"][b, h].cpu(), inp["v"][b, h].cpu(), N, rows)
            check_close(o[b, h, rows], ref, w.dtype, f"prefill b{b} h{h} N={N}")
            crow = sorted(set(crow_edges + rng.integers(0, w.k, 16).tolist()))
            ref = oracle.rank_decode_rows(inp["qc"][b, h].cpu(), inp["kc"][b, h].cpu(), inp["vc"][b, h].cpu(),
                                          inp["k"][b, h, :N].cpu(), inp["v"][b, h, :N].cpu(), crow)
            check_close(oc[b, h, crow], ref, w.dtype, f"decode b{b} h{h} N={N}")
    assert pool.status() == 0


# ------------------------------------------------------------------ edge cases

EDGE = [
    # (dtype, B, H, D, n, k, lens)
    (torch.bfloat16, 3, 2, 64, 300, 70, [0, 1, 300]),       # empty and one-token history, ragged tails
    (torch.bfloat16, 4, 2, 64, 130, 1, [63, 64, 65, 129]),    # k = 1, lengths around a tile edge
    (torch.bfloat16, 2, 4, 32, 257, 257, [257, 100]),          # D = 32, no XCD remap (B*H = 8 -> remap)
    (torch.bfloat16, 1, 3, 128, 520, 300, [511]),              # D = 128, B*H not a multiple of 8
    (torch.bfloat16, 8, 1, 64, 512, 256, [512, 256, 255, 257, 1, 2, 500, 384]),
    # 70 users, lengths in ties of one 64-row key and zeros: the longest-first schedules
    (torch.bfloat16, 70, 1, 64, 200, 40, [(i * 37) % 201 if i % 9 else 0 for i in range(70)]),
    # 300 users: past the ordered schedules' user limit (user order)
    (torch.bfloat16, 300, 1, 64, 70, 9, [(i * 7) % 71 for i in range(300)]),
    # every history 257 .. 512 rows: two query tiles per (user, head), ragged tails
    (torch.bfloat16, 16, 8, 64, 512, 40, [257, 512, 320, 511, 300, 448, 258, 400, 384, 500, 290, 333, 449, 510, 260, 385]),
    (torch.bfloat16, 2, 8, 128, 400, 30, [257, 400]),
    (torch.float32, 2, 2, 64, 100, 33, [100, 37]),
    (torch.float32, 1, 2, 128, 70, 5, [0]),
    (torch.float32, 3, 1, 32, 65, 64, [65, 64, 1]),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}D{c[3]}n{c[4]}k{c[5]}")
def test_edge_shapes(case):
    dtype, B, H, D, n, k, lens = case
    announce(f"edge {case}")
    inp = W.small_case(B, H, D, n, k, lens, dtype=dtype, seed=1000 + n + k, device=DEV)
    pool = fa.Pool.allocate(2, B + 1, H, n, D, dtype, DEV)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    slots = list(range(B, 0, -1))  # not the identity, to catch slot mix-ups
    o, oc = run_layer(pool, inp, lens, slots, 1)
    full_check(inp, lens, o, oc, pool, slots, 1, dtype, tag="edge")
    # rows past each history, other slots and the other layer are untouched (NaN sentinel)
    for b, N in enumerate(lens):
        assert torch.isnan(pool.k[1, slots[b], :, N:]).all() and torch.isnan(pool.v[1, slots[b], :, N:]).all()
    assert torch.isnan(pool.k[0]).all() and torch.isnan(pool.k[1, 0]).all()
    if 0 in lens:
        b = lens.index(0)
        assert torch.equal(oc[b], inp["vc"][b]), "empty history must return vc exactly"
    assert pool.status() == 0


def test_nan_poison_rows_past_history_are_never_read():
    """Inputs and pool rows at or past lens[b] are NaN; outputs must equal the clean run bit for bit."""
    B, H, D, n, k = 4, 2, 64, 333, 90
    lens = [333, 200, 64, 7]
    announce("nan poison")
    clean = W.small_case(B, H, D, n, k, lens, seed=77, device=DEV)
    pois = dict(clean)
    lens_t = torch.as_tensor(lens)
    for name in ("q", "k", "v"):
        pois[name] = W.poison_tail(clean[name], lens_t)
    outs = []
    for inp in (clean, pois):
        pool = fa.Pool.allocate(1, B, H, n, D, torch.bfloat16, DEV)
        pool.k.fill_(float("nan"))
        pool.v.fill_(float("nan"))
        o, oc = run_layer(pool, inp, lens, list(range(B)), 0)
        outs.append((o, oc))
    for b, N in enumerate(lens):
        assert torch.equal(outs[0][0][b, :, :N], outs[1][0][b, :, :N])
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[1][1]).all()


# ------------------------------------------------------------------ invariants

def test_joint_invariant():
    """prefill + rank_decode on the GPU == one pass over [history || candidates] (oracle)."""
    B, H, D, n, k = 3, 2, 64, 200, 50
    lens = [200, 77, 0]
    announce("joint invariant")
    inp = W.small_case(B, H, D, n, k, lens, seed=5, device=DEV)
    pool = fa.Pool.allocate(3, 4, H, n, D, torch.bfloat16, DEV)
    o, oc = run_layer(pool, inp, lens, [3, 1, 0], 2)
    cpu = {key: v.cpu() for key, v in inp.items()}
    jo, jc = oracle.joint(cpu["q"], cpu["k"], cpu["v"], cpu["qc"], cpu["kc"], cpu["vc"], lens)
    for b, N in enumerate(lens):
        if N:
            check_close(o[b, :, :N], jo[b, :, :N], torch.bfloat16, f"joint hist {b}")
    check_close(oc, jc, torch.bfloat16, "joint candidates")


def test_candidate_independence_bitwise():
    """A candidate's output does not depend on the other candidates of the call."""
    B, H, D, n, k = 2, 4, 64, 300, 400
    lens = [300, 123]
    announce("candidate independence")
    inp = W.small_case(B, H, D, n, k, lens, seed=9, device=DEV)
    pool = fa.Pool.allocate(1, 2, H, n, D, torch.bfloat16, DEV)
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    slots_d = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    fa.prefill(inp["q"], inp["k"], inp["v"], lens_d, pool, slots_d, 0)
    dec = lambda qc, kc, vc: fa.rank_decode(qc.contiguous(), kc.contiguous(), vc.contiguous(),
                                            pool, slots_d, lens_d, 0)
    base = dec(inp["qc"], inp["kc"], inp["vc"])
    perm = torch.randperm(k, generator=torch.Generator().manual_seed(1)).to(DEV)
    out = dec(inp["qc"][:, :, perm], inp["kc"][:, :, perm], inp["vc"][:, :, perm])
    assert torch.equal(out, base[:, :, perm])
    keep = torch.arange(0, k, 7, device=DEV)
    out = dec(inp["qc"][:, :, keep], inp["kc"][:, :, keep], inp["vc"][:, :, keep])
    assert torch.equal(out, base[:, :, keep])
    extra = W.small_case(B, H, D, n, 300, lens, seed=10, device=DEV)
    cat = lambda a, e: torch.cat([a, e], dim=2)
    out = dec(cat(inp["qc"], extra["qc"]), cat(inp["kc"], extra["kc"]), cat(inp["vc"], extra["vc"]))
    assert torch.equal(out[:, :, :k], base)


def test_repeated_launches_are_bitwise_identical():
    """Many launches of the same decode and prefill, interleaved with launches of other
    history lengths, give bit-identical outputs.  The kernels stage K/V and the candidate
    rows in LDS by DMA under a counted wait; a missed wait or a hazard on the DMA's LDS
    address shows up here as an occasional differing block of rows."""
    w = W.Workload(90, "repeat", torch.bfloat16, L=1, S=64, B=64, H=8, D=64, n=1024, k=1000,
                   len_lo=0, len_hi=1024)
    announce("repeated launches B64 H8 D64 n1024 k1000")
    x = W.layer_inputs(w, 0, DEV)
    pool = fa.Pool.allocate(1, w.S, w.H, w.n, w.D, w.dtype, DEV)
    slots = torch.arange(w.B, dtype=torch.int32, device=DEV)
    lens = {N: torch.full((w.B,), N, dtype=torch.int32, device=DEV) for N in (0, 512, 1024)}
    fa.prefill(x["q"], x["k"], x["v"], lens[1024], pool, slots, 0)
    other = torch.empty_like(x["qc"])
    o = torch.empty_like(x["q"])
    ref = ref_o = None
    for it in range(120):
        for N in (0, 1024):
            fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens[N], 0, oc=other)
        oc = fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens[512], 0)
        fa.prefill(x["q"], x["k"], x["v"], lens[1024], pool, slots, 0, o=o)
        if ref is None:
            ref, ref_o = oc.clone(), o.clone()
        else:
            assert torch.equal(oc, ref), f"rank_decode differs at launch {it}"
            assert torch.equal(o, ref_o), f"prefill differs at launch {it}"
    torch.cuda.synchronize()
    assert pool.status() == 0


def test_same_data_other_slot_or_layer_is_bitwise_identical():
    B, H, D, n, k = 2, 2, 64, 256, 128
    lens = [256, 190]
    announce("slot/layer placement")
    inp = W.small_case(B, H, D, n, k, lens, seed=11, device=DEV)
    pool = fa.Pool.allocate(3, 5, H, n, D, torch.bfloat16, DEV)
    a = run_layer(pool, inp, lens, [0, 1], 0)
    b = run_layer(pool, inp, lens, [4, 2], 2)
    assert torch.equal(a[1], b[1])
    for i, N in enumerate(lens):
        assert torch.equal(a[0][i, :, :N], b[0][i, :, :N])


@pytest.mark.parametrize("kind", ["peaky", "dominant_key", "scale_arg"])
def test_adversarial_numerics(kind):
    B, H, D, n, k = 2, 2, 64, 384, 128
    lens = [384, 250]
    announce(f"adversarial {kind}")
    inp = W.small_case(B, H, D, n, k, lens, seed=12, device=DEV)
    scale = None
    if kind == "peaky":
        for name in ("q", "qc"):
            inp[name] = (inp[name].float() * 8).to(torch.bfloat16)
    elif kind == "dominant_key":
        # one late history key aligned with every query: the running max jumps late
        kk = inp["k"].clone()
        kk[:, :, 200] = (inp["qc"][:, :, 0].float() * 4).to(torch.bfloat16)
        inp["k"] = kk
        inp["q"] = inp["q"].clone()
        inp["q"][:, :, :] = inp["qc"][:, :, :1]
        inp["qc"] = inp["qc"][:, :, :1].expand(-1, -1, k, -1).contiguous()
    else:
        scale = 0.37
    pool = fa.Pool.allocate(1, 2, H, n, D, torch.bfloat16, DEV)
    o, oc = run_layer(pool, inp, lens, [1, 0], 0, scale=scale)
    full_check(inp, lens, o, oc, pool, [1, 0], 0, torch.bfloat16, scale=scale, tag=kind)


def test_device_side_invalid_user_is_skipped_and_flagged():
    B, H, D, n, k = 3, 2, 64, 128, 64
    announce("device status flags")
    inp = W.small_case(B, H, D, n, k, [128, 64, 10], seed=13, device=DEV)
    pool = fa.Pool.allocate(1, 2, H, n, D, torch.bfloat16, DEV)
    assert pool.status() == 0
    o = torch.full_like(inp["q"], 7.0)
    fa.prefill(inp["q"], inp["k"], inp["v"], [128, 64, 10], pool, [0, 5, 1], 0, o=o)  # slot 5 >= S
    assert pool.status() == fa.FLAG_BAD_SLOT
    assert (o[1] == 7.0).all(), "a skipped user's output must stay untouched"
    fa.prefill(inp["q"], inp["k"], inp["v"], [128, 129, 10], pool, [0, 1, 1], 0, o=o)  # len > n
    assert pool.status() == fa.FLAG_BAD_LEN
    oc = torch.full_like(inp["qc"], 7.0)
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, [0, -1, 1], [128, 64, 10], 0, oc=oc)
    assert pool.status() == fa.FLAG_BAD_SLOT
    assert (oc[1] == 7.0).all()
    assert torch.isfinite(oc[0]).all() and torch.isfinite(oc[2]).all()
    assert pool.status() == 0


@pytest.mark.parametrize("D", [64, 128])
def test_short_user_with_an_invalid_slot_is_flagged(D):
    """A user shorter than the call's padded extent has only its first query tiles in
    the longest-first schedule; an invalid slot of such a user is still flagged (and its
    rows skipped)."""
    B, H, n, k = 3, 8, 600, 16
    announce(f"short user with an invalid slot, D={D}")
    inp = W.small_case(B, H, D, n, k, [600, 50, 300], seed=17, device=DEV)
    pool = fa.Pool.allocate(1, 3, H, n, D, torch.bfloat16, DEV)
    o = torch.full_like(inp["q"], 7.0)
    fa.prefill(inp["q"], inp["k"], inp["v"], [600, 50, 300], pool, [0, 9, 2], 0, o=o)   # slot 9 >= S
    torch.cuda.synchronize()
    assert pool.status() == fa.FLAG_BAD_SLOT
    assert (o[1] == 7.0).all(), "a skipped user's output must stay untouched"
    for b, N in ((0, 600), (2, 300)):
        sub = {kk: v[b:b + 1].cpu() for kk, v in inp.items() if kk in ("q", "k", "v")}
        ref = oracle.prefill(sub["q"], sub["k"], sub["v"], [N])
        check_close(o[b:b + 1, :, :N], ref[:, :, :N], torch.bfloat16, f"user {b} beside the invalid one")


def test_invalid_length_ranks_longest_and_only_flags():
    """One invalid length among two-tile histories: the longest-first schedule ranks the
    invalid user first; its blocks only raise the flag, the other user is exact."""
    B, H, D, n, k = 2, 8, 64, 300, 16
    announce("invalid length in the longest-first prefill schedule")
    inp = W.small_case(B, H, D, n, k, [300, 280], seed=15, device=DEV)
    pool = fa.Pool.allocate(1, 2, H, n, D, torch.bfloat16, DEV)
    o = torch.full_like(inp["q"], 7.0)
    fa.prefill(inp["q"], inp["k"], inp["v"], [300, 301], pool, [1, 0], 0, o=o)   # 301 > n
    torch.cuda.synchronize()
    assert pool.status() == fa.FLAG_BAD_LEN
    assert (o[1] == 7.0).all(), "a skipped user's output must stay untouched"
    sub = {kk: v[0:1].cpu() for kk, v in inp.items() if kk in ("q", "k", "v")}
    ref = oracle.prefill(sub["q"], sub["k"], sub["v"], [300])
    check_close(o[0:1], ref, torch.bfloat16, "valid user beside an invalid one")
    assert torch.equal(pool.k[0, 1].cpu(), inp["k"][0].cpu()) and torch.equal(pool.v[0, 1].cpu(), inp["v"][0].cpu())


def test_two_users_naming_one_slot_are_flagged():
    """A prefill in which two users with histories name the same slot raises
    FLAG_DUP_SLOT (both still run); an empty or invalid history sharing the slot does not
    count.  Also past the ordered schedules' user limit, and on an fp32 pool."""
    announce("duplicate slots in one prefill")
    for dtype, B, lens, slots, want in (
            (torch.bfloat16, 3, [10, 20, 30], [0, 1, 0], fa.FLAG_DUP_SLOT),
            (torch.bfloat16, 3, [10, 20, 0], [0, 1, 0], 0),
            (torch.bfloat16, 3, [10, 65, 30], [0, 0, 1], fa.FLAG_BAD_LEN),        # 65 > n: skipped
            (torch.bfloat16, 3, [64, 64, 64], [2, 1, 0], 0),
            (torch.float32, 3, [10, 20, 30], [1, 1, 0], fa.FLAG_DUP_SLOT),
            (torch.float32, 3, [10, 0, 30], [1, 1, 0], 0),
            (torch.bfloat16, 300, [(i % 64) + 1 for i in range(300)], [i % 300 for i in range(299)] + [7],
             fa.FLAG_DUP_SLOT)):
        H, D, n, k = 1, 64, 64, 8
        inp = W.small_case(B, H, D, n, k, lens, dtype=dtype, seed=16, device=DEV)
        pool = fa.Pool.allocate(1, max(slots) + 1, H, n, D, dtype, DEV)
        fa.prefill(inp["q"], inp["k"], inp["v"], lens, pool, slots, 0)
        torch.cuda.synchronize()
        assert pool.status() == want, (dtype, B, lens[:4], slots[:4])
        pool.close()


def test_flags_belong_to_the_pool_whose_call_raised_them():
    """Two pools on one device: an invalid user in a call on one pool raises that pool's
    flag only."""
    B, H, D, n, k = 2, 2, 64, 64, 32
    announce("per-pool status flags")
    inp = W.small_case(B, H, D, n, k, [64, 20], seed=14, device=DEV)
    pa = fa.Pool.allocate(1, 2, H, n, D, torch.bfloat16, DEV)
    pb = fa.Pool.allocate(1, 3, H, n, D, torch.bfloat16, DEV)
    assert pa.status() == 0 and pb.status() == 0
    fa.prefill(inp["q"], inp["k"], inp["v"], [64, 20], pa, [0, 2], 0)      # slot 2 >= S of pool a
    fa.prefill(inp["q"], inp["k"], inp["v"], [64, 20], pb, [0, 2], 0)      # valid on pool b
    assert pb.status() == 0
    assert pa.status() == fa.FLAG_BAD_SLOT
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pb, [0, 2], [64, n + 1], 0)   # len > n_max on b
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pa, [0, 1], [64, 20], 0)
    assert pa.status() == 0
    assert pb.status() == fa.FLAG_BAD_LEN
    # a flag raised by a kernel on another stream is kept until a status call takes it
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pa, [0, -1], [64, 20], 0)
    side.synchronize()
    assert pb.status() == 0
    assert pa.status() == fa.FLAG_BAD_SLOT
    assert pa.status() == 0
    # a new descriptor that reuses a released entry does not inherit its flags
    fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pa, [0, 7], [64, 20], 0)
    torch.cuda.synchronize()
    pa.close()
    pc = fa.Pool(pb.k, pb.v)
    assert pc.status() == 0
    pc.close()
    pb.close()
