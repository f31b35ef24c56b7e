"""Pins of the float64 oracle against facts it does not compute itself.

Each check below ties the oracle to something other than its own code:
  * a mask and a worked example written by hand from the pages (tests/golden/);
  * the allowed-pair count N(N+1)/2 + K(N+1), the O(n^2 + nk) cost the pages state
    (review of "UniPinRec: Unifying Generative Retrieval and Ranking at Pinterest
    Scale", section 2.2; reading notes, section 3 "attention mask");
  * an independent scalar brute force (loops, math.fsum) on every tiny shape;
  * closed forms (zero queries give prefix means; constant values give the constant;
    an empty history gives the candidate's own value);
  * a library routine for the textbook special cases (torch float64 causal SDPA);
  * the joint-pass invariant (prefill + pool + rank decode == one pass over
    [history || candidates]) and batch-composition independence (reading notes,
    section 3: candidate scores do not depend on the other candidates);
  * for the autoregressive retrieval step: replaying a sequence one token at a time
    must give the causal prefill's rows and leave the whole sequence in the slot.
The last test plants plausible mistakes in the oracle (on the CPU) and checks that
at least one pin catches each of them.
"""
import itertools
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as OA

GOLDEN = Path(__file__).parent / "golden"
TOL = 1e-12


# ------------------------------------------------------------------ fixtures / helpers

def _num(tok: str) -> float:
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    return float(Fraction(tok))


def load_worked_example():
    rows = {}
    for line in (GOLDEN / "worked_example_N3_K2_D2.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        key, rest = line.split(None, 1)
        if key == "scale":
            rows[key] = float(rest)
        else:
            rows[key] = np.array([[_num(t) for t in grp.split()] for grp in rest.split("|")])
    return rows


def load_mask_golden():
    lines = [l for l in (GOLDEN / "mfalcon_mask_N4_K3.txt").read_text().splitlines()
             if l.strip() and not l.startswith("#")]
    return np.array([[int(t) for t in l.split()] for l in lines], dtype=bool)


def rand_case(rng, N, K, D, B=1, H=1, n=None):
    n = N if n is None else n
    f = lambda *s: rng.standard_normal(s)
    return dict(q=f(B, H, n, D), k=f(B, H, n, D), v=f(B, H, n, D),
                qc=f(B, H, K, D), kc=f(B, H, K, D), vc=f(B, H, K, D))


def _maxerr(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.size == 0 and b.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


# ------------------------------------------------------------------ checks (bool)

def check_mask_golden():
    return np.array_equal(OA.mfalcon_mask(4, 3), load_mask_golden())


def check_pair_count():
    for N in range(0, 9):
        for K in range(0, 7):
            if int(OA.mfalcon_mask(N, K).sum()) != N * (N + 1) // 2 + K * (N + 1):
                return False
    return True


def check_worked_example():
    w = load_worked_example()
    x = {key: w[key][None, None] for key in ("q", "k", "v", "qc", "kc", "vc")}
    oh, oc = OA.joint(x["q"], x["k"], x["v"], x["qc"], x["kc"], x["vc"], [3], scale=w["scale"])
    op = OA.prefill(x["q"], x["k"], x["v"], [3], scale=w["scale"])
    pk, pv = OA.pool_write(np.zeros((1, 1, 1, 3, 2)), np.zeros((1, 1, 1, 3, 2)),
                           x["k"], x["v"], [3], [0], 0)
    od = OA.rank_decode(x["qc"], x["kc"], x["vc"], pk, pv, [0], [3], 0, scale=w["scale"])
    return (_maxerr(oh[0, 0], w["o_hist"]) < TOL and _maxerr(oc[0, 0], w["o_cand"]) < TOL
            and _maxerr(op[0, 0], w["o_hist"]) < TOL and _maxerr(od[0, 0], w["o_cand"]) < TOL)


def check_bruteforce(seed=0):
    rng = np.random.default_rng(seed)
    for N, K, D in itertools.product(range(0, 7), range(1, 6), (1, 2, 4, 8)):
        c = rand_case(rng, N, K, D)
        scale = 1.0 / math.sqrt(D)
        oh, oc = OA.joint(c["q"], c["k"], c["v"], c["qc"], c["kc"], c["vc"], [N], scale)
        bh, bc = OA.bruteforce_joint(*(c[t][0, 0].tolist() for t in ("q", "k", "v", "qc", "kc", "vc")),
                                     N=N, scale=scale)
        if N and _maxerr(oh[0, 0, :N], bh) > TOL:
            return False
        if _maxerr(oc[0, 0], bc) > TOL:
            return False
        # the split path (prefill, pool, rank decode) must agree with brute force as well
        op = OA.prefill(c["q"], c["k"], c["v"], [N], scale)
        pk, pv = OA.pool_write(np.zeros((1, 1, 1, N, D)), np.zeros((1, 1, 1, N, D)),
                               c["k"], c["v"], [N], [0], 0)
        od = OA.rank_decode(c["qc"], c["kc"], c["vc"], pk, pv, [0], [N], 0, scale)
        if N and _maxerr(op[0, 0, :N], bh) > TOL:
            return False
        if _maxerr(od[0, 0], bc) > TOL:
            return False
    return True


def check_closed_forms(seed=1):
    rng = np.random.default_rng(seed)
    for N, K, D in ((0, 3, 4), (1, 1, 2), (5, 4, 8), (17, 6, 16)):
        c = rand_case(rng, N, K, D)
        # zero queries: uniform weights over the visible keys
        z = {**c, "q": np.zeros_like(c["q"]), "qc": np.zeros_like(c["qc"])}
        oh, oc = OA.joint(z["q"], z["k"], z["v"], z["qc"], z["kc"], z["vc"], [N])
        v, vc = c["v"][0, 0], c["vc"][0, 0]
        prefix = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None] if N else np.zeros((0, D))
        if N and _maxerr(oh[0, 0, :N], prefix) > TOL:
            return False
        cand = (v.sum(axis=0)[None, :] + vc) / (N + 1)
        if _maxerr(oc[0, 0], cand) > TOL:
            return False
        # constant values: every output is that constant
        const = rng.standard_normal(D)
        cv = {**c, "v": np.broadcast_to(const, c["v"].shape).copy(),
              "vc": np.broadcast_to(const, c["vc"].shape).copy()}
        oh, oc = OA.joint(cv["q"], cv["k"], cv["v"], cv["qc"], cv["kc"], cv["vc"], [N])
        if (N and _maxerr(oh[0, 0, :N], np.broadcast_to(const, (N, D))) > TOL) or \
                _maxerr(oc[0, 0], np.broadcast_to(const, (K, D))) > TOL:
            return False
    # empty history: a candidate sees only itself
    c = rand_case(rng, 0, 5, 8, n=4)
    pk, pv = np.zeros((1, 1, 1, 4, 8)), np.zeros((1, 1, 1, 4, 8))
    od = OA.rank_decode(c["qc"], c["kc"], c["vc"], pk, pv, [0], [0], 0)
    return np.array_equal(od[0, 0], c["vc"][0, 0])


def check_sdpa(seed=2):
    """Textbook special cases, via torch's float64 CPU scaled_dot_product_attention."""
    F = torch.nn.functional
    rng = np.random.default_rng(seed)
    for N, D in ((1, 4), (7, 8), (33, 16), (64, 32)):
        c = rand_case(rng, N, 1, D, B=2, H=3)
        lens = [N, N]
        op = OA.prefill(c["q"], c["k"], c["v"], lens)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
        ref = F.scaled_dot_product_attention(t(c["q"]), t(c["k"]), t(c["v"]), is_causal=True,
                                             scale=1.0 / math.sqrt(D)).numpy()
        if _maxerr(op, ref) > TOL:
            return False
        # K = 1: a candidate is the last row of causal attention over N + 1 tokens
        cat = lambda a, b: np.concatenate([a, b], axis=2)
        ref = F.scaled_dot_product_attention(t(cat(c["q"], c["qc"])), t(cat(c["k"], c["kc"])),
                                             t(cat(c["v"], c["vc"])), is_causal=True,
                                             scale=1.0 / math.sqrt(D)).numpy()[:, :, N:]
        pk, pv = OA.pool_write(np.zeros((1, 2, 3, N, D)), np.zeros((1, 2, 3, N, D)),
                               c["k"], c["v"], lens, [1, 0], 0)
        od = OA.rank_decode(c["qc"], c["kc"], c["vc"], pk, pv, [1, 0], lens, 0)
        if _maxerr(od, ref) > TOL:
            return False
    return True


def check_joint_invariant(seed=3):
    rng = np.random.default_rng(seed)
    B, H, n, K, D, L, S = 4, 2, 12, 5, 8, 3, 6
    c = rand_case(rng, n, K, D, B=B, H=H)
    lens = [0, 12, 5, 9]
    slot = [4, 0, 5, 2]
    layer = 2
    pk0, pv0 = rng.standard_normal((L, S, H, n, D)), rng.standard_normal((L, S, H, n, D))
    oh, oc = OA.joint(c["q"], c["k"], c["v"], c["qc"], c["kc"], c["vc"], lens)
    op = OA.prefill(c["q"], c["k"], c["v"], lens)
    pk, pv = OA.pool_write(pk0, pv0, c["k"], c["v"], lens, slot, layer)
    od = OA.rank_decode(c["qc"], c["kc"], c["vc"], pk, pv, slot, lens, layer)
    for b in range(B):
        if _maxerr(op[b, :, :lens[b]], oh[b, :, :lens[b]]) > TOL:
            return False
    return _maxerr(od, oc) <= TOL


def check_independence(seed=4):
    rng = np.random.default_rng(seed)
    N, K, D = 9, 7, 8
    c = rand_case(rng, N, K, D, B=1, H=2)
    pk, pv = OA.pool_write(np.zeros((1, 1, 2, N, D)), np.zeros((1, 1, 2, N, D)),
                           c["k"], c["v"], [N], [0], 0)
    dec = lambda qc, kc, vc: OA.rank_decode(qc, kc, vc, pk, pv, [0], [N], 0)
    base = dec(c["qc"], c["kc"], c["vc"])
    perm = rng.permutation(K)
    out = dec(c["qc"][:, :, perm], c["kc"][:, :, perm], c["vc"][:, :, perm])
    if _maxerr(out, base[:, :, perm]) > TOL:
        return False
    keep = [0, 3, 6]
    out = dec(c["qc"][:, :, keep], c["kc"][:, :, keep], c["vc"][:, :, keep])
    if _maxerr(out, base[:, :, keep]) > TOL:
        return False
    extra = rand_case(rng, 0, 4, D, B=1, H=2)
    add = lambda a, e: np.concatenate([a, e], axis=2)
    out = dec(add(c["qc"], extra["qc"]), add(c["kc"], extra["kc"]), add(c["vc"], extra["vc"]))
    return _maxerr(out[:, :, :K], base) <= TOL


def check_pool_write(seed=5):
    rng = np.random.default_rng(seed)
    L, S, H, n, D = 2, 4, 3, 6, 4
    pk0, pv0 = rng.standard_normal((L, S, H, n, D)), rng.standard_normal((L, S, H, n, D))
    k, v = rng.standard_normal((2, H, n, D)), rng.standard_normal((2, H, n, D))
    lens, slot, layer = [3, 6], [2, 0], 1
    pk, pv = OA.pool_write(pk0, pv0, k, v, lens, slot, layer)
    ek, ev = pk0.copy(), pv0.copy()
    for b in range(2):
        for h in range(H):
            for t in range(lens[b]):
                ek[layer, slot[b], h, t] = k[b, h, t]
                ev[layer, slot[b], h, t] = v[b, h, t]
    return np.array_equal(pk, ek) and np.array_equal(pv, ev)


def check_ar_decode_replays_prefill(seed=7):
    """Autoregressive steps reproduce the causal prefill of the same token sequence.

    A history of N tokens is prefilled into a slot, then T more tokens are decoded one
    per step: step j must give prefill row N+j of the whole sequence (each row of a
    causal pass sees exactly the tokens before it and itself), and the slot must end up
    holding all N+T rows.  Starting from an empty slot (N = 0) the first step must
    return the token's own value.
    """
    rng = np.random.default_rng(seed)
    L, S, H, D, layer = 2, 3, 2, 8, 1
    for N, T, s in ((0, 5, 2), (6, 4, 0), (1, 1, 1)):
        n = N + T
        c = rand_case(rng, n, 0, D, B=1, H=H)
        full = OA.prefill(c["q"], c["k"], c["v"], [n])
        pk0, pv0 = rng.standard_normal((L, S, H, n + 2, D)), rng.standard_normal((L, S, H, n + 2, D))
        pk, pv = OA.pool_write(pk0, pv0, c["k"], c["v"], [N], [s], layer)
        for j in range(T):
            t = N + j
            o, pk, pv = OA.ar_decode(c["q"][:, :, t:t + 1], c["k"][:, :, t:t + 1], c["v"][:, :, t:t + 1],
                                     pk, pv, [s], [t], layer)
            if _maxerr(o[0, :, 0], full[0, :, t]) > TOL:
                return False
            if t == 0 and not np.array_equal(o[0, :, 0], c["v"][0, :, 0]):
                return False
        ek, ev = OA.pool_write(pk0, pv0, c["k"], c["v"], [n], [s], layer)
        if not (np.array_equal(pk, ek) and np.array_equal(pv, ev)):
            return False
    return True


def check_ar_decode_bruteforce(seed=8):
    """One step against the scalar brute force, for a batch with mixed slot fill levels."""
    rng = np.random.default_rng(seed)
    L, S, H, nmax, D, layer = 1, 4, 2, 7, 3, 0
    pk0, pv0 = rng.standard_normal((L, S, H, nmax, D)), rng.standard_normal((L, S, H, nmax, D))
    lens, slot = [0, 3, 6], [3, 1, 0]
    q, k, v = (rng.standard_normal((3, H, 1, D)) for _ in range(3))
    scale = 0.7
    o, pk, pv = OA.ar_decode(q, k, v, pk0, pv0, slot, lens, layer, scale=scale)
    for b, (N, s) in enumerate(zip(lens, slot)):
        for h in range(H):
            keys = [list(pk0[layer, s, h, t]) for t in range(N)] + [list(k[b, h, 0])]
            vals = [list(pv0[layer, s, h, t]) for t in range(N)] + [list(v[b, h, 0])]
            ref = OA._softmax_average(list(q[b, h, 0]), keys, vals, scale)
            if _maxerr(o[b, h, 0], ref) > TOL:
                return False
    return True


ALL_CHECKS = [check_mask_golden, check_pair_count, check_worked_example, check_bruteforce,
              check_closed_forms, check_sdpa, check_joint_invariant, check_independence,
              check_pool_write, check_ar_decode_replays_prefill, check_ar_decode_bruteforce]


# ------------------------------------------------------------------ the pins

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    assert check()


def test_slot_ring_round_robin():
    r = oracle.SlotRing(3)
    got = [r.acquire() for _ in range(7)]
    assert got == [(0, 1), (1, 1), (2, 1), (0, 2), (1, 2), (2, 2), (0, 3)]


def test_rows_helpers_match_full_oracle():
    rng = np.random.default_rng(6)
    N, K, D = 10, 6, 8
    c = rand_case(rng, N, K, D)
    pk, pv = OA.pool_write(np.zeros((1, 1, 1, N, D)), np.zeros((1, 1, 1, N, D)),
                           c["k"], c["v"], [N], [0], 0)
    full = OA.rank_decode(c["qc"], c["kc"], c["vc"], pk, pv, [0], [N], 0)
    rows = OA.rank_decode_rows(c["qc"][0, 0], c["kc"][0, 0], c["vc"][0, 0],
                               c["k"][0, 0, :N], c["v"][0, 0, :N], [5, 0, 2])
    assert _maxerr(rows, full[0, 0, [5, 0, 2]]) < TOL
    fullp = OA.prefill(c["q"], c["k"], c["v"], [N])
    rows = OA.prefill_rows(c["q"][0, 0], c["k"][0, 0], c["v"][0, 0], N, [9, 0, 4])
    assert _maxerr(rows, fullp[0, 0, [9, 0, 4]]) < TOL


# ------------------------------------------------------------------ planted mistakes

def _mask_no_self(N, K, include_self=True):
    return OA.__dict__["_orig_mask"](N, K, include_self=False)


def _mask_candidates_see_each_other(N, K, include_self=True):
    M = OA.__dict__["_orig_mask"](N, K)
    M[N:, N:] = True
    return M


def _mask_noncausal_history(N, K, include_self=True):
    M = OA.__dict__["_orig_mask"](N, K)
    M[:N, :N] = True
    return M


def _mask_plain_causal(N, K, include_self=True):
    T = N + K
    return np.tril(np.ones((T, T), dtype=bool))


def _mask_history_off_by_one(N, K, include_self=True):
    M = OA.__dict__["_orig_mask"](N, K)
    for i in range(N):
        M[i, i] = False if i > 0 else True
    return M


def _attn_no_scale(xq, xk, xv, mask, scale):
    return OA.__dict__["_orig_attn"](xq, xk, xv, mask, 1.0)


def _attn_wrong_axis(xq, xk, xv, mask, scale):
    s = np.where(mask, scale * (xq @ xk.T), -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=0, keepdims=True).clip(min=1e-300)
    return p @ xv


def _attn_values_from_keys(xq, xk, xv, mask, scale):
    return OA.__dict__["_orig_attn"](xq, xk, xk, mask, scale)


def _pool_write_short(pool_k, pool_v, k, v, lens, slot, layer):
    return OA.__dict__["_orig_pool_write"](pool_k, pool_v, k, v,
                                           [max(0, int(x) - 1) for x in lens], slot, layer)


def _pool_write_wrong_slot(pool_k, pool_v, k, v, lens, slot, layer):
    S = np.asarray(pool_k).shape[1]
    return OA.__dict__["_orig_pool_write"](pool_k, pool_v, k, v, lens,
                                           [(int(s) + 1) % S for s in slot], layer)


def _ar_without_itself(q, k, v, pool_k, pool_v, slot, lens, layer, scale=None):
    o, pk, pv = OA.__dict__["_orig_ar"](q, k, v, pool_k, pool_v, slot, lens, layer, scale=scale)
    pk0, pv0 = OA.as_f64(pool_k), OA.as_f64(pool_v)
    lens = [int(x) for x in np.asarray(lens).reshape(-1)]
    D = np.asarray(q).shape[-1]
    sc = OA.default_scale(D) if scale is None else scale
    for b, (N, s) in enumerate(zip(lens, [int(x) for x in np.asarray(slot).reshape(-1)])):
        if N == 0:
            continue
        for h in range(np.asarray(q).shape[1]):
            o[b, h] = OA.masked_attention(OA.as_f64(q)[b, h], pk0[layer, s, h, :N], pv0[layer, s, h, :N],
                                          np.ones((1, N), dtype=bool), sc)
    return o, pk, pv


def _ar_writes_previous_row(q, k, v, pool_k, pool_v, slot, lens, layer, scale=None):
    shifted = [max(0, int(x) - 1) for x in np.asarray(lens).reshape(-1)]
    o, _, _ = OA.__dict__["_orig_ar"](q, k, v, pool_k, pool_v, slot, lens, layer, scale=scale)
    _, pk, pv = OA.__dict__["_orig_ar"](q, k, v, pool_k, pool_v, slot, shifted, layer, scale=scale)
    return o, pk, pv


MUTANTS = {
    "autoregressive step does not see itself": ("ar_decode", _ar_without_itself),
    "autoregressive step stores at the previous row": ("ar_decode", _ar_writes_previous_row),
    "candidate does not see itself": ("mfalcon_mask", _mask_no_self),
    "candidates see each other": ("mfalcon_mask", _mask_candidates_see_each_other),
    "history not causal": ("mfalcon_mask", _mask_noncausal_history),
    "plain causal over the joint sequence": ("mfalcon_mask", _mask_plain_causal),
    "history misses its own position": ("mfalcon_mask", _mask_history_off_by_one),
    "scale dropped": ("masked_attention", _attn_no_scale),
    "softmax over the wrong axis": ("masked_attention", _attn_wrong_axis),
    "values taken from keys": ("masked_attention", _attn_values_from_keys),
    "pool write drops the last row": ("pool_write", _pool_write_short),
    "pool write to the wrong slot": ("pool_write", _pool_write_wrong_slot),
}


# a planted mistake may leave a row with no visible key: its NaN is what the pins catch
@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(OA.__dict__, "_orig_mask", OA.mfalcon_mask)
    monkeypatch.setitem(OA.__dict__, "_orig_attn", OA.masked_attention)
    monkeypatch.setitem(OA.__dict__, "_orig_pool_write", OA.pool_write)
    monkeypatch.setitem(OA.__dict__, "_orig_ar", OA.ar_decode)
    monkeypatch.setattr(OA, attr, fn)
    failed = []
    for check in ALL_CHECKS:
        try:
            ok = check()
        except Exception:
            ok = False
        if not ok:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
