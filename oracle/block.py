"""Float64 CPU oracle for one transformer block of the unified model around the masked
attention: the candidate-only forward of the ranking stage and the history forward that
fills the KV pool.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this module; the GPU library never calls it and shares no code
with it.

Pages cited (by title and section):
  [review] "UniPinRec: Unifying Generative Retrieval and Ranking at Pinterest Scale",
           paper review at liuzhao09.github.io/papers/pinterest-unipinrec.html
  [notes]  UniPinRec reading notes, slinene.github.io ai-papers-daily, gen-rec collection

What the pages fix and what is read into them:
  * the history and the candidates pass through one GPT2-style decoder with the
    M-FALCON mask ([review] section 2.2 and Figure 2); ranking runs the candidates
    only, reading the history's per-layer K/V from the pool ([review] section 2.4;
    [notes] section 6).  Table 2 of [notes] times this candidate-only forward over
    12 layers;
  * the model's width is not disclosed ([notes], closing remarks).  The block here
    is the GPT2 block read plainly: pre-LayerNorm (eps 1e-5), fused QKV projection,
    multi-head attention with the M-FALCON mask, output projection and residual,
    pre-LayerNorm MLP of width 4C with the tanh form of GELU, and residual.  C = H*D;
  * inputs, heads and projections outside the block (embedders, input projector,
    action decoder, final LayerNorm) are not part of it.

Weights are a dict of float64 arrays with row-major "x @ W" matrices:
  ln1_w, ln1_b [C]; w_qkv [C, 3C], b_qkv [3C] (columns: q, then k, then v, each
  head-major: column j of a part belongs to head j // D); w_o [C, C], b_o [C];
  ln2_w, ln2_b [C]; w_fc [C, 4C], b_fc [4C]; w_proj [4C, C], b_proj [C].
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

from .attention import as_f64, default_scale, masked_attention, mfalcon_mask

LN_EPS = 1e-5
WEIGHT_KEYS = ("ln1_w", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_w", "ln2_b", "w_fc", "b_fc",
               "w_proj", "b_proj")


def layer_norm(x, w, b, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * w + b, population variance."""
    x = as_f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * as_f64(w) + as_f64(b)


def gelu(x) -> np.ndarray:
    """GELU in the tanh form of the GPT2 code: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = as_f64(x)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def _weights(w: Dict) -> Dict[str, np.ndarray]:
    return {key: as_f64(w[key]) for key in WEIGHT_KEYS}


def _heads(y: np.ndarray, H: int) -> np.ndarray:
    """[T, C] -> [H, T, D]: head h takes columns h*D .. h*D + D - 1."""
    T, C = y.shape
    return y.reshape(T, H, C // H).transpose(1, 0, 2)


def _merge(o: np.ndarray) -> np.ndarray:
    """[H, T, D] -> [T, H*D]."""
    H, T, D = o.shape
    return o.transpose(1, 0, 2).reshape(T, H * D)


def _qkv(x: np.ndarray, w: Dict[str, np.ndarray], H: int):
    """Pre-LayerNorm and fused projection of the rows x [T, C]: q, k, v [H, T, D]."""
    C = x.shape[-1]
    y = layer_norm(x, w["ln1_w"], w["ln1_b"]) @ w["w_qkv"] + w["b_qkv"]
    return _heads(y[:, :C], H), _heads(y[:, C:2 * C], H), _heads(y[:, 2 * C:], H)


def _finish(x: np.ndarray, o: np.ndarray, w: Dict[str, np.ndarray]) -> np.ndarray:
    """Output projection and residual, then the pre-LayerNorm MLP and residual."""
    h = x + _merge(o) @ w["w_o"] + w["b_o"]
    m = gelu(layer_norm(h, w["ln2_w"], w["ln2_b"]) @ w["w_fc"] + w["b_fc"])
    return h + m @ w["w_proj"] + w["b_proj"]


def block_joint(x_hist, x_cand, lens, weights, H: int, scale: float | None = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """The block over each user's joint sequence [history (lens[b] rows) || candidates]
    with the M-FALCON mask, in one pass.  x_hist [B, n, C], x_cand [B, K, C].
    Returns (y_hist [B, n, C] with NaN at rows >= lens[b], y_cand [B, K, C])."""
    xh, xc, w = as_f64(x_hist), as_f64(x_cand), _weights(weights)
    B, n, C = xh.shape
    K = xc.shape[1]
    D = C // H
    scale = default_scale(D) if scale is None else scale
    yh = np.full((B, n, C), np.nan)
    yc = np.empty((B, K, C))
    for b in range(B):
        N = int(lens[b])
        x = np.concatenate([xh[b, :N], xc[b]], axis=0)
        q, k, v = _qkv(x, w, H)
        M = mfalcon_mask(N, K)
        o = np.stack([masked_attention(q[h], k[h], v[h], M, scale) for h in range(H)])
        y = _finish(x, o, w)
        yh[b, :N] = y[:N]
        yc[b] = y[N:]
    return yh, yc


def block_history(x_hist, lens, weights, H: int, pool_k, pool_v, slot, layer: int,
                  scale: float | None = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The history forward of one layer: causal self-attention over each user's lens[b]
    rows, and the history's projected K/V stored in rows 0..lens[b]-1 of slot[b] at
    `layer` ([review] section 2.4: the retrieval side leaves each layer's K/V in the
    request's slot).  Returns (y_hist [B, n, C] with NaN at rows >= lens[b], pool_k',
    pool_v')."""
    xh, w = as_f64(x_hist), _weights(weights)
    pk, pv = as_f64(pool_k).copy(), as_f64(pool_v).copy()
    B, n, C = xh.shape
    D = C // H
    scale = default_scale(D) if scale is None else scale
    yh = np.full((B, n, C), np.nan)
    for b in range(B):
        N, s = int(lens[b]), int(slot[b])
        if N == 0:
            continue
        q, k, v = _qkv(xh[b, :N], w, H)
        pk[layer, s, :, :N] = k
        pv[layer, s, :, :N] = v
        M = mfalcon_mask(N, 0)
        o = np.stack([masked_attention(q[h], k[h], v[h], M, scale) for h in range(H)])
        yh[b, :N] = _finish(xh[b, :N], o, w)
    return yh, pk, pv


def block_candidates(x_cand, weights, H: int, pool_k, pool_v, slot, lens, layer: int,
                     scale: float | None = None) -> np.ndarray:
    """The ranking stage's candidate-only forward of one layer: the candidates' own
    q, k, v; each candidate attends to the lens[b] history rows cached in slot[b] at
    `layer` and to itself, never to another candidate ([review] sections 2.2, 2.4;
    [notes] sections 3, 6).  x_cand [B, K, C] -> y_cand [B, K, C]."""
    xc, w = as_f64(x_cand), _weights(weights)
    pk, pv = as_f64(pool_k), as_f64(pool_v)
    B, K, C = xc.shape
    D = C // H
    scale = default_scale(D) if scale is None else scale
    yc = np.empty((B, K, C))
    for b in range(B):
        N, s = int(lens[b]), int(slot[b])
        qc, kc, vc = _qkv(xc[b], w, H)
        M = mfalcon_mask(N, K)[N:]
        o = np.stack([masked_attention(qc[h], np.concatenate([pk[layer, s, h, :N], kc[h]]),
                                       np.concatenate([pv[layer, s, h, :N], vc[h]]), M, scale)
                      for h in range(H)])
        yc[b] = _finish(xc[b], o, w)
    return yc
