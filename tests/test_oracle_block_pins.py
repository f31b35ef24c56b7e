"""Pins of the transformer-block oracle (oracle/block.py) to things other than itself.

* GELU: the value at 1 of the tanh form (torch's own tanh-approximate GELU agrees), the
  identity gelu(x) - gelu(-x) = x, the tails, and closeness to the exact x*Phi(x);
* LayerNorm: the closed form of a normalised row, and torch's layer_norm;
* the whole joint block against an independent float64 assembly of torch.nn.functional
  routines (layer_norm, linear, tanh GELU, scaled_dot_product_attention with the mask
  built here from triangular and identity blocks);
* zero weights make the block the identity;
* the KV-reuse split: the history forward (which fills the pool) followed by the
  candidate-only forward equals the joint pass ([review] section 2.4);
* a candidate's output does not depend on the other candidates ([notes] section 3);
* planted mistakes in the oracle are caught.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.block as OB
import workloads as W


def _w64(C, seed):
    return {k: v.to(torch.float64) for k, v in W.block_weights(C, torch.float32, seed=seed).items()}


def torch_block_joint(xh, xc, lens, w, H, scale):
    """float64 torch.nn.functional assembly of the GPT2 block with the M-FALCON mask."""
    B, n, C = xh.shape
    K = xc.shape[1]
    D = C // H
    yh = torch.full((B, n, C), float("nan"), dtype=torch.float64)
    yc = torch.empty((B, K, C), dtype=torch.float64)
    for b in range(B):
        N = int(lens[b])
        x = torch.cat([xh[b, :N], xc[b]])
        T = N + K
        a = F.layer_norm(x, (C,), w["ln1_w"], w["ln1_b"], eps=1e-5)
        qkv = F.linear(a, w["w_qkv"].T, w["b_qkv"])
        q, k, v = (t.reshape(T, H, D).transpose(0, 1) for t in qkv.split(C, dim=-1))
        mask = torch.zeros(T, T, dtype=torch.bool)
        mask[:N, :N] = torch.tril(torch.ones(N, N, dtype=torch.bool))
        mask[N:, :N] = True
        mask[N:, N:] = torch.eye(K, dtype=torch.bool)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        h = x + F.linear(o.transpose(0, 1).reshape(T, C), w["w_o"].T, w["b_o"])
        m = F.gelu(F.linear(F.layer_norm(h, (C,), w["ln2_w"], w["ln2_b"], eps=1e-5), w["w_fc"].T, w["b_fc"]),
                   approximate="tanh")
        y = h + F.linear(m, w["w_proj"].T, w["b_proj"])
        yh[b, :N] = y[:N]
        yc[b] = y[N:]
    return yh.numpy(), yc.numpy()


# ---------------------------------------------------------------- the checks

def check_gelu_values():
    g = OB.gelu(np.array([1.0, 0.0, 10.0, -10.0]))
    assert abs(g[0] - 0.8411919906082768) < 1e-15          # tanh form at 1 (the erf form gives 0.84134)
    assert g[1] == 0.0
    assert abs(g[2] - 10.0) < 1e-12 and abs(g[3]) < 1e-12
    x = np.linspace(-6, 6, 241)
    assert np.allclose(OB.gelu(x) - OB.gelu(-x), x, atol=1e-13, rtol=0)
    exact = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in x])
    assert np.max(np.abs(OB.gelu(x) - exact)) < 1e-3
    t = torch.tensor(x)
    assert np.allclose(OB.gelu(x), F.gelu(t, approximate="tanh").numpy(), atol=1e-14, rtol=0)


def check_layer_norm():
    rng = np.random.default_rng(3)
    x = rng.normal(2.0, 3.0, size=(5, 64))
    y = OB.layer_norm(x, np.ones(64), np.zeros(64))
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), var / (var + OB.LN_EPS), atol=1e-12)
    w, b = rng.normal(size=64), rng.normal(size=64)
    ref = F.layer_norm(torch.tensor(x), (64,), torch.tensor(w), torch.tensor(b), eps=1e-5).numpy()
    assert np.allclose(OB.layer_norm(x, w, b), ref, atol=1e-12, rtol=0)


def check_block_vs_torch():
    C, H, B, n, K = 32, 4, 3, 9, 5
    w = _w64(C, 11)
    xh = W.block_inputs(B, n, C, torch.float64, seed=12)
    xc = W.block_inputs(B, K, C, torch.float64, seed=13)
    lens = [9, 4, 0]
    for scale in (None, 0.3):
        s = 1 / math.sqrt(C // H) if scale is None else scale
        yh, yc = OB.block_joint(xh, xc, lens, w, H, scale)
        th, tc = torch_block_joint(xh, xc, lens, w, H, s)
        assert np.allclose(yc, tc, atol=1e-11, rtol=0)
        for b, N in enumerate(lens):
            assert np.allclose(yh[b, :N], th[b, :N], atol=1e-11, rtol=0)
            assert np.isnan(yh[b, N:]).all()


def check_zero_weights_is_identity():
    C, H = 16, 2
    w = {k: torch.zeros_like(v) for k, v in _w64(C, 1).items()}
    xh = W.block_inputs(2, 6, C, torch.float64, seed=2)
    xc = W.block_inputs(2, 3, C, torch.float64, seed=3)
    yh, yc = OB.block_joint(xh, xc, [6, 2], w, H)
    assert np.array_equal(yc, xc.numpy())
    assert np.array_equal(yh[0], xh[0].numpy()) and np.array_equal(yh[1, :2], xh[1, :2].numpy())


def check_kv_reuse_equals_joint():
    C, H, B, n, K, L, S = 32, 4, 3, 10, 6, 2, 4
    w = _w64(C, 21)
    xh = W.block_inputs(B, n, C, torch.float64, seed=22)
    xc = W.block_inputs(B, K, C, torch.float64, seed=23)
    lens, slot, layer = [10, 7, 0], [3, 0, 2], 1
    D = C // H
    pk0 = np.full((L, S, H, n, D), np.nan)
    yh, pk, pv = OB.block_history(xh, lens, w, H, pk0, pk0.copy(), slot, layer)
    yc = OB.block_candidates(xc, w, H, pk, pv, slot, lens, layer)
    jh, jc = OB.block_joint(xh, xc, lens, w, H)
    assert np.allclose(yc, jc, atol=1e-12, rtol=0)
    assert np.allclose(np.nan_to_num(yh), np.nan_to_num(jh), atol=1e-12, rtol=0)
    # the pool holds the history's projected keys and values, nothing else
    for b, (N, s) in enumerate(zip(lens, slot)):
        a = OB.layer_norm(xh[b, :N].numpy(), w["ln1_w"].numpy(), w["ln1_b"].numpy())
        kv = a @ w["w_qkv"].numpy() + w["b_qkv"].numpy()
        assert np.allclose(pk[layer, s, :, :N], kv[:, C:2 * C].reshape(N, H, D).transpose(1, 0, 2), atol=1e-13)
        assert np.allclose(pv[layer, s, :, :N], kv[:, 2 * C:].reshape(N, H, D).transpose(1, 0, 2), atol=1e-13)
        assert np.isnan(pk[layer, s, :, N:]).all()
    assert np.isnan(pk[0]).all() and np.isnan(pk[layer, 1]).all()


def check_candidate_independence():
    C, H = 32, 4
    w = _w64(C, 31)
    xh = W.block_inputs(1, 8, C, torch.float64, seed=32)
    xc = W.block_inputs(1, 5, C, torch.float64, seed=33)
    _, full = OB.block_joint(xh, xc, [8], w, H)
    _, two = OB.block_joint(xh, xc[:, [3, 1]], [8], w, H)
    assert np.allclose(two[0], full[0, [3, 1]], atol=1e-13, rtol=0)


ALL_CHECKS = [check_gelu_values, check_layer_norm, check_block_vs_torch, check_zero_weights_is_identity,
              check_kv_reuse_equals_joint, check_candidate_independence]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_block_pin(check):
    check()


# ---------------------------------------------------------------- planted mistakes

def _gelu_erf(x):
    x = OB.as_f64(x)
    return 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))


def _finish_no_attention_residual(x, o, w):
    h = OB._merge(o) @ w["w_o"] + w["b_o"]
    m = OB.gelu(OB.layer_norm(h, w["ln2_w"], w["ln2_b"]) @ w["w_fc"] + w["b_fc"])
    return h + m @ w["w_proj"] + w["b_proj"]


def _finish_post_ln(x, o, w):
    h = OB.layer_norm(x + OB._merge(o) @ w["w_o"] + w["b_o"], w["ln2_w"], w["ln2_b"])
    return h + OB.gelu(h @ w["w_fc"] + w["b_fc"]) @ w["w_proj"] + w["b_proj"]


def _heads_interleaved(y, H):
    T, C = y.shape
    return y.reshape(T, C // H, H).transpose(2, 0, 1)


def _qkv_no_layer_norm(x, w, H):
    C = x.shape[-1]
    y = x @ w["w_qkv"] + w["b_qkv"]
    return OB._heads(y[:, :C], H), OB._heads(y[:, C:2 * C], H), OB._heads(y[:, 2 * C:], H)


def _qkv_k_v_swapped(x, w, H):
    q, k, v = _orig_qkv(x, w, H)
    return q, v, k


_orig_qkv = OB._qkv

MUTANTS = {
    "GELU in the erf form": ("gelu", _gelu_erf),
    "attention residual dropped": ("_finish", _finish_no_attention_residual),
    "post-LayerNorm block": ("_finish", _finish_post_ln),
    "heads taken from interleaved columns": ("_heads", _heads_interleaved),
    "no LayerNorm before the projection": ("_qkv", _qkv_no_layer_norm),
    "keys and values swapped": ("_qkv", _qkv_k_v_swapped),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_block_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OB, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches: {name}"
