"""GPU parity of the autoregressive retrieval step (unipin_ar_decode) against the oracle.

Same tolerances as the other GPU parity tests: fp32 1e-5 relative, normwise and element
by element (floored at 1e-3); bf16 max abs 2e-2
and mean abs 2e-3.  Pool contents are compared bit for bit: the step must store the
new token's K/V at row lens[b] of its slot and leave every other entry as it was.
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
        return
    assert diff.max() <= 2e-2, f"{what}: max abs error {diff.max():.3e} > 2e-2"
    assert diff.mean() <= 2e-3, f"{what}: mean abs error {diff.mean():.3e} > 2e-3"


CASES = [
    (torch.bfloat16, 64), (torch.bfloat16, 32), (torch.bfloat16, 128),
    (torch.float32, 32), (torch.float32, 64), (torch.float32, 128),
]


@pytest.mark.parametrize("dtype,D", CASES, ids=lambda x: str(x))
def test_ar_decode_one_step(dtype, D):
    """Mixed fill levels (empty slot, partial and whole chunks, the last free row)."""
    L, S, H, n_max, layer = 2, 9, 3, 601, 1
    lens = [0, 1, 63, 64, 65, 200, 511, 513, n_max - 1]
    slots = [4, 0, 8, 2, 7, 1, 3, 6, 5]
    B = len(lens)
    announce(f"ar_decode one step {dtype} D={D}")
    pk, pv = W.random_pool(L, S, H, n_max, D, dtype, seed=31, device=DEV)
    tok = W.step_tokens(B, H, D, 1, dtype, seed=32, device=DEV)
    q, k, v = tok["q"][0], tok["k"][0], tok["v"][0]
    before_k, before_v = pk.cpu(), pv.cpu()
    pool = fa.Pool(pk, pv)
    o = fa.ar_decode(q, k, v, pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    ref_o, ref_k, ref_v = oracle.ar_decode(q.cpu(), k.cpu(), v.cpu(), before_k, before_v, slots, lens, layer)
    check_close(o, ref_o, dtype, f"ar_decode {dtype} D={D}")
    exp_k, exp_v = before_k.clone(), before_v.clone()
    for b, (N, s) in enumerate(zip(lens, slots)):
        exp_k[layer, s, :, N] = k[b, :, 0].cpu()
        exp_v[layer, s, :, N] = v[b, :, 0].cpu()
    assert torch.equal(pk.cpu(), exp_k) and torch.equal(pv.cpu(), exp_v), "pool must change at row lens[b] only"
    assert np.array_equal(oracle.as_f64(pk), ref_k)
    pool.close()


@pytest.mark.parametrize("scale", [None, 0.37])
def test_ar_decode_steps_replay_the_prefill(scale):
    """Prefill N history tokens, then decode T more one step at a time (lens advanced by
    the caller): step j must give row N+j of a causal prefill over all N+T tokens, the
    slot must end up holding all N+T rows, and the ranking decode still sees the history
    it is told to see."""
    B, H, D, N, T, k = 4, 2, 64, 130, 5, 48
    n_max = N + T
    announce(f"ar_decode replay scale={scale}")
    inp = W.small_case(B, H, D, n_max, k, [n_max] * B, seed=33, device=DEV)
    pool = fa.Pool.allocate(1, B, H, n_max, D, torch.bfloat16, DEV)
    slots = [2, 0, 3, 1]
    hist = [N, N - 7, 1, 0]
    fa.prefill(inp["q"], inp["k"], inp["v"], hist, pool, slots, 0, scale=scale)
    lens = torch.as_tensor(hist, dtype=torch.int32, device=DEV)
    outs = []
    for j in range(T):
        rows = lens.long()
        gather = lambda x: torch.stack([x[b, :, int(rows[b]):int(rows[b]) + 1] for b in range(B)])
        outs.append(fa.ar_decode(gather(inp["q"]), gather(inp["k"]), gather(inp["v"]), pool, slots, lens, 0,
                                 scale=scale))
        lens = lens + 1
    torch.cuda.synchronize()
    assert pool.status() == 0
    full = oracle.prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), [n_max] * B, scale)
    for j in range(T):
        ref = np.stack([full[b, :, hist[b] + j] for b in range(B)])[:, :, None]
        check_close(outs[j], ref, torch.bfloat16, f"step {j}")
    for b, s in enumerate(slots):
        m = hist[b] + T
        assert torch.equal(pool.k[0, s, :, :m].cpu(), inp["k"][b, :, :m].cpu())
        assert torch.equal(pool.v[0, s, :, :m].cpu(), inp["v"][b, :, :m].cpu())
    # the ranking decode with the history length alone ignores the generated rows
    oc = fa.rank_decode(inp["qc"], inp["kc"], inp["vc"], pool, slots, hist, 0, scale=scale)
    torch.cuda.synchronize()
    for b in (0, 2):
        s = slots[b]
        ref = oracle.rank_decode(inp["qc"][b:b + 1].cpu(), inp["kc"][b:b + 1].cpu(), inp["vc"][b:b + 1].cpu(),
                                 oracle.as_f64(pool.k[0:1, s:s + 1].cpu()), oracle.as_f64(pool.v[0:1, s:s + 1].cpu()),
                                 [0], [hist[b]], 0, scale)
        check_close(oc[b:b + 1], ref, torch.bfloat16, f"rank decode after steps, user {b}")
    pool.close()


def test_ar_decode_invalid_users_flagged_and_skipped():
    L, S, H, n_max, D = 1, 3, 2, 40, 64
    announce("ar_decode invalid users")
    pk, pv = W.random_pool(L, S, H, n_max, D, torch.bfloat16, seed=34, device=DEV)
    tok = W.step_tokens(3, H, D, 1, torch.bfloat16, seed=35, device=DEV)
    before_k, before_v = pk.clone(), pv.clone()
    pool = fa.Pool(pk, pv)
    o = torch.full_like(tok["q"][0], 7.0)
    fa.ar_decode(tok["q"][0], tok["k"][0], tok["v"][0], pool, [0, 5, 1], [n_max, 3, -1], 0, o=o)
    torch.cuda.synchronize()
    flags = pool.status()
    assert flags == fa.FLAG_BAD_SLOT | fa.FLAG_BAD_LEN
    assert torch.all(o == 7.0), "skipped users' outputs must stay untouched"
    assert torch.equal(pk, before_k) and torch.equal(pv, before_v), "skipped users must not write the pool"
    assert pool.status() == 0
    pool.close()


def test_ar_decode_serving_shape_sampled():
    """The retrieval step at the serving shape (64 requests x 8 heads, history 512, D=64,
    12-layer pool), in the launch configuration the benchmark times; sampled users
    against the oracle, every pool row written checked bit for bit."""
    w = W.WORKLOADS[3]
    T = 4
    n_max = w.n + T
    announce("ar_decode serving shape")
    pk, pv = W.random_pool(w.L, w.S, w.H, n_max, w.D, w.dtype, seed=36, device=DEV)
    pool = fa.Pool(pk, pv)
    tok = W.step_tokens(w.B, w.H, w.D, 1, w.dtype, seed=37, device=DEV)
    slots = list(range(w.B))
    lens = [w.n + 2] * w.B
    layer = 11
    users = [0, 17, 63]
    before = {b: (pk[layer, b, :, :lens[b]].cpu(), pv[layer, b, :, :lens[b]].cpu()) for b in users}
    o = fa.ar_decode(tok["q"][0], tok["k"][0], tok["v"][0], pool, slots, lens, layer)
    torch.cuda.synchronize()
    assert pool.status() == 0
    for b in users:
        # the user's slot as a one-layer, one-slot pool with one free row for the new token
        hk, hv = (np.concatenate([oracle.as_f64(x), np.zeros((w.H, 1, w.D))], axis=1)[None, None]
                  for x in before[b])
        ref, _, _ = oracle.ar_decode(tok["q"][0][b:b + 1].cpu(), tok["k"][0][b:b + 1].cpu(),
                                     tok["v"][0][b:b + 1].cpu(), hk, hv, [0], [lens[b]], 0)
        check_close(o[b:b + 1], ref, w.dtype, f"serving shape user {b}")
    rows_k = torch.stack([pk[layer, b, :, lens[b]] for b in range(w.B)])
    rows_v = torch.stack([pv[layer, b, :, lens[b]] for b in range(w.B)])
    assert torch.equal(rows_k, tok["k"][0][:, :, 0]) and torch.equal(rows_v, tok["v"][0][:, :, 0])
    pool.close()


SPLIT_CASES = [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.bfloat16, 32), (torch.float32, 64),
               (torch.float32, 128)]   # fp32 pools never split (fp64 one-pass kernel): the same cases, one pass


@pytest.mark.parametrize("dtype,D", SPLIT_CASES, ids=lambda x: str(x))
def test_ar_decode_split_path(dtype, D):
    """Few (user, head) pairs on a long slot: the rows are split across workgroups and the
    parts merged by a second pass (bf16; fp32 pools run their one-pass fp64 kernel).
    Lengths cover an empty slot, fewer chunks than parts, part boundaries and the last
    free row; the one-pass kernel must agree with the oracle on the same inputs too."""
    L, S, H, layer = 1, 12, 2, 0
    n_max = 4600 if D >= 64 else 8200   # at least 240 Ki elements per matrix: the slot splits
    lens = [0, 1, 64, 65, 200, 511, 513, 1024, 2047, 3000, 4100, n_max - 1]
    slots = [3, 0, 11, 2, 7, 1, 4, 6, 5, 10, 9, 8]
    B = len(lens)
    announce(f"ar_decode split path {dtype} D={D}")
    pk, pv = W.random_pool(L, S, H, n_max, D, dtype, seed=38, device=DEV)
    tok = W.step_tokens(B, H, D, 1, dtype, seed=39, device=DEV)
    q, k, v = tok["q"][0], tok["k"][0], tok["v"][0]
    before_k, before_v = pk.cpu(), pv.cpu()
    ref_o, ref_k, ref_v = oracle.ar_decode(q.cpu(), k.cpu(), v.cpu(), before_k, before_v, slots, lens, layer)
    for split in (True, False):
        pk.copy_(before_k.to(DEV))
        pv.copy_(before_v.to(DEV))
        pool = fa.Pool(pk, pv)
        if split:
            need = fa.ar_decode_workspace_bytes(pool, B)
            if dtype == torch.float32:
                assert need == 0, "fp32 pools run one pass"
            else:
                assert need > 0, "this shape must take the split path"
        o = fa.ar_decode(q, k, v, pool, slots, lens, layer, split=split)
        torch.cuda.synchronize()
        assert pool.status() == 0
        check_close(o, ref_o, dtype, f"ar_decode split={split} {dtype} D={D}")
        assert np.array_equal(oracle.as_f64(pk), ref_k) and np.array_equal(oracle.as_f64(pv), ref_v)
        pool.close()


def test_ar_decode_split_invalid_users_and_reused_workspace():
    """Invalid users are flagged and skipped by both passes; a workspace filled with NaN
    from an earlier call does not leak into the next one."""
    L, S, H, n_max, D = 1, 4, 2, 4600, 64   # 4599 x 64 elements per matrix: the slot splits
    announce("ar_decode split invalid users")
    pk, pv = W.random_pool(L, S, H, n_max, D, torch.bfloat16, seed=40, device=DEV)
    pool = fa.Pool(pk, pv)
    tok = W.step_tokens(4, H, D, 1, torch.bfloat16, seed=41, device=DEV)
    need = fa.ar_decode_workspace_bytes(pool, 4)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    before_k, before_v = pk.cpu(), pv.cpu()
    o = torch.full_like(tok["q"][0], 7.0)
    slots, lens = [0, 9, 1, 2], [2000, 5, n_max, n_max - 1]
    fa.ar_decode(tok["q"][0], tok["k"][0], tok["v"][0], pool, slots, lens, 0, o=o, workspace=ws)
    torch.cuda.synchronize()
    assert pool.status() == fa.FLAG_BAD_SLOT | fa.FLAG_BAD_LEN
    assert torch.all(o[1:3] == 7.0), "skipped users' outputs must stay untouched"
    ref, _, _ = oracle.ar_decode(tok["q"][0].cpu(), tok["k"][0].cpu(), tok["v"][0].cpu(), before_k, before_v,
                                 [0, 0, 0, 2], [2000, 0, 0, n_max - 1], 0)
    check_close(o[[0, 3]], ref[[0, 3]], torch.bfloat16, "valid users next to invalid ones")
    exp_k = before_k.clone()
    exp_k[0, 0, :, 2000] = tok["k"][0][0, :, 0].cpu()
    exp_k[0, 2, :, n_max - 1] = tok["k"][0][3, :, 0].cpu()
    assert torch.equal(pk.cpu(), exp_k), "only the valid users' rows may change"
    pool.close()


def test_ar_decode_long_history_sampled():
    """The step at the long-history shape (16 users x 16 heads, D=128, histories drawn
    from 1024..4096): 256 (user, head) pairs, one pass; sampled users against the oracle."""
    w = W.WORKLOADS[4]
    _long_history_case(w.B, w.H, w.D, W.history_lengths(w).tolist(), w.n + 1, seed=42, split_expected=False)


def test_ar_decode_few_users_long_history_split():
    """Two requests of 16 heads with 4000 and 2500 rows (D=128): too few pairs to fill the
    GPU, so each pair's rows are split across workgroups."""
    _long_history_case(2, 16, 128, [4000, 2500], 4001, seed=44, split_expected=True)


def _long_history_case(B, H, D, lens, n_max, seed, split_expected):
    announce(f"ar_decode long history B={B} H={H} D={D} split={split_expected}")
    pk, pv = W.random_pool(1, B, H, n_max, D, torch.bfloat16, seed=seed, device=DEV)
    pool = fa.Pool(pk, pv)
    assert (fa.ar_decode_workspace_bytes(pool, B) > 0) == split_expected
    tok = W.step_tokens(B, H, D, 1, torch.bfloat16, seed=seed + 1, device=DEV)
    slots = list(range(B))
    users = sorted({int(np.argmin(lens)), int(np.argmax(lens)), B // 3})
    before = {b: (pk[0, b, :, :lens[b]].cpu(), pv[0, b, :, :lens[b]].cpu()) for b in users}
    o = fa.ar_decode(tok["q"][0], tok["k"][0], tok["v"][0], pool, slots, lens, 0)
    torch.cuda.synchronize()
    assert pool.status() == 0
    for b in users:
        hk, hv = (np.concatenate([oracle.as_f64(x), np.zeros((H, 1, D))], axis=1)[None, None]
                  for x in before[b])
        ref, _, _ = oracle.ar_decode(tok["q"][0][b:b + 1].cpu(), tok["k"][0][b:b + 1].cpu(),
                                     tok["v"][0][b:b + 1].cpu(), hk, hv, [0], [lens[b]], 0)
        check_close(o[b:b + 1], ref, torch.bfloat16, f"long history user {b} (N={lens[b]})")
    rows_k = torch.stack([pk[0, b, :, lens[b]] for b in range(B)])
    rows_v = torch.stack([pv[0, b, :, lens[b]] for b in range(B)])
    assert torch.equal(rows_k, tok["k"][0][:, :, 0]) and torch.equal(rows_v, tok["v"][0][:, :, 0])
    pool.close()
