"""Float64 CPU oracle for M-FALCON masked attention over a slotted KV pool.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this module.  The GPU library never calls it, and it shares no
code with the GPU library: it is the plain definition of what that library computes,
written out with an explicit dense mask so that a reader can check it by eye.

Pages cited (by title and section):
  [review] "UniPinRec: Unifying Generative Retrieval and Ranking at Pinterest Scale",
           paper review at liuzhao09.github.io/papers/pinterest-unipinrec.html
  [notes]  UniPinRec reading notes ("unified retrieval/ranking, masked action, KV share"),
           slinene.github.io ai-papers-daily, gen-rec collection

What is computed, for one layer, user b and head h, with N = lens[b] history tokens
and K candidate tokens:
  * the joint sequence is [N history tokens || K candidate tokens], passed through
    the transformer in one pass ([review] section 2.2; [notes] "overall approach");
  * history rows attend causally: row i sees keys 0..i ([notes] section 3, attention
    mask: "the past part is standard causal attention");
  * each candidate row sees all N history positions, and candidates cannot see each
    other ([review] section 2.2; [notes] section 3);
  * a candidate also sees its own position.  The pages say "only the past history"
    in one place and are silent in another; the no-leakage condition of equation (2)
    in [review] section 2.1 ([notes] section 2, "no leakage") makes a token's hidden
    state depend on its own features, i.e. causal attention including the diagonal.
    This reading is the constant INCLUDE_SELF below;
  * scores are scale * q.k with plain softmax attention (a GPT2-style backbone,
    [review] Figure 2); no positional term enters the attention itself;
  * the KV pool is two arrays K and V of shape [L, S, H, n_max, D] (layer, slot,
    KV head, history position, head dim), preallocated once; a request's history
    K/V of layer l is stored in its slot s at rows 0..N-1 ([review] section 2.4;
    [notes] section 6, cross-process KV sharing).  Slots are handed out round-robin
    and reused ([review] section 2.4; [notes] section 6);
  * ranking reads the slot's history K/V and runs only the candidate tokens,
    cost O(nk) ([review] section 2.4; [notes] section 6).  The pages copy the slot
    into a separate decode cache first; reading it in place gives the same values.

All inputs are upcast exactly to float64 before any arithmetic; rows of history
tensors at positions >= lens[b] are never read, and the history outputs there are
returned as NaN ("undefined").
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

# Reading of the pages: a candidate attends to its own position (see module docstring).
INCLUDE_SELF = True


def as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a (CPU or device) torch tensor to float64."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(D: int) -> float:
    """1/sqrt(D): the scale the workloads state; used when a caller passes none."""
    return 1.0 / math.sqrt(D)


def mfalcon_mask(N: int, K: int, include_self: bool = INCLUDE_SELF) -> np.ndarray:
    """Dense boolean mask over the joint sequence [N history || K candidates].

    M[i, j] is True when query position i may attend to key position j
    ([review] section 2.2; [notes] section 3, attention mask).
    """
    T = N + K
    M = np.zeros((T, T), dtype=bool)
    for i in range(N):
        M[i, : i + 1] = True          # history: causal, its own position included
    for j in range(K):
        M[N + j, :N] = True           # a candidate sees every history position
        if include_self:
            M[N + j, N + j] = True    # ... and itself, never another candidate
    return M


def masked_attention(xq: np.ndarray, xk: np.ndarray, xv: np.ndarray,
                     mask: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * xq xk^T restricted to mask) xv, row by row, in float64.

    xq is [R, D], xk and xv are [C, D], mask is [R, C].  Every row must allow at
    least one key (true for the M-FALCON mask with INCLUDE_SELF).
    """
    s = scale * (xq @ xk.T)
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ xv


def joint(q, k, v, qc, kc, vc, lens, scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """One pass over [history || candidates] under the M-FALCON mask.

    q, k, v are [B, H, n, D]; qc, kc, vc are [B, H, K, D]; lens is [B].
    Returns (o_hist [B,H,n,D] with NaN at rows >= lens[b], o_cand [B,H,K,D]).
    """
    q, k, v, qc, kc, vc = (as_f64(t) for t in (q, k, v, qc, kc, vc))
    lens = [int(x) for x in np.asarray(as_f64(lens)).reshape(-1)]
    B, H, n, D = q.shape
    K = qc.shape[2]
    scale = default_scale(D) if scale is None else scale
    o_hist = np.full((B, H, n, D), np.nan)
    o_cand = np.empty((B, H, K, D))
    for b in range(B):
        N = lens[b]
        M = mfalcon_mask(N, K)
        for h in range(H):
            xq = np.concatenate([q[b, h, :N], qc[b, h]], axis=0)
            xk = np.concatenate([k[b, h, :N], kc[b, h]], axis=0)
            xv = np.concatenate([v[b, h, :N], vc[b, h]], axis=0)
            o = masked_attention(xq, xk, xv, M, scale)
            o_hist[b, h, :N] = o[:N]
            o_cand[b, h] = o[N:]
    return o_hist, o_cand


def prefill(q, k, v, lens, scale: float | None = None) -> np.ndarray:
    """Causal attention over each user's history: the N x N block of the joint mask.

    History rows cannot see candidates, so this block alone gives their outputs.
    Returns o [B, H, n, D] with NaN at rows >= lens[b].
    """
    q, k, v = (as_f64(t) for t in (q, k, v))
    lens = [int(x) for x in np.asarray(as_f64(lens)).reshape(-1)]
    B, H, n, D = q.shape
    scale = default_scale(D) if scale is None else scale
    o = np.full((B, H, n, D), np.nan)
    for b in range(B):
        N = lens[b]
        if N == 0:
            continue
        M = mfalcon_mask(N, 0)
        for h in range(H):
            o[b, h, :N] = masked_attention(q[b, h, :N], k[b, h, :N], v[b, h, :N], M, scale)
    return o


def pool_write(pool_k, pool_v, k, v, lens, slot, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """The pool after a prefill: rows 0..N-1 of slot[b] at `layer` hold k/v[b] exactly.

    pool_k, pool_v are [L, S, H, n_max, D]; every other entry is left as it was.
    """
    pk, pv = as_f64(pool_k).copy(), as_f64(pool_v).copy()
    k, v = as_f64(k), as_f64(v)
    lens = [int(x) for x in np.asarray(as_f64(lens)).reshape(-1)]
    slot = [int(x) for x in np.asarray(as_f64(slot)).reshape(-1)]
    for b, (N, s) in enumerate(zip(lens, slot)):
        pk[layer, s, :, :N] = k[b, :, :N]
        pv[layer, s, :, :N] = v[b, :, :N]
    return pk, pv


def rank_decode(qc, kc, vc, pool_k, pool_v, slot, lens, layer: int,
                scale: float | None = None) -> np.ndarray:
    """Candidate rows of the joint mask, with history K/V read from the pool slot.

    Row j of the K x (N + K) block sees the N history keys of slot[b] and its own
    key; it is the ranking decode of [review] section 2.4 / [notes] section 6.
    Returns oc [B, H, K, D].
    """
    qc, kc, vc = (as_f64(t) for t in (qc, kc, vc))
    pk, pv = as_f64(pool_k), as_f64(pool_v)
    lens = [int(x) for x in np.asarray(as_f64(lens)).reshape(-1)]
    slot = [int(x) for x in np.asarray(as_f64(slot)).reshape(-1)]
    B, H, K, D = qc.shape
    scale = default_scale(D) if scale is None else scale
    oc = np.empty((B, H, K, D))
    for b in range(B):
        N, s = lens[b], slot[b]
        M = mfalcon_mask(N, K)[N:, :]
        for h in range(H):
            xk = np.concatenate([pk[layer, s, h, :N], kc[b, h]], axis=0)
            xv = np.concatenate([pv[layer, s, h, :N], vc[b, h]], axis=0)
            oc[b, h] = masked_attention(qc[b, h], xk, xv, M, scale)
    return oc


def ar_decode(q, k, v, pool_k, pool_v, slot, lens, layer: int,
              scale: float | None = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One autoregressive step of the retrieval model, reading and extending the slot.

    The retrieval side prefills the history and then decodes query tokens one at a time
    while the slot holds the K/V of everything so far ([review] section 2.4 and Figure 3;
    [notes] section 2: a 12-layer causal decoder that generates several query embeddings
    autoregressively, one token per step).  User b has N = lens[b] rows in slot[b] at
    `layer` (its history, then the tokens generated before); the new token q, k, v
    [B, H, 1, D] takes position N.  Its K/V are stored at row N, and it attends causally
    to rows 0..N, itself included: the last row of the N+1 by N+1 causal mask.
    Returns (o [B, H, 1, D], pool_k', pool_v').
    """
    q, k, v = (as_f64(t) for t in (q, k, v))
    pk, pv = as_f64(pool_k).copy(), as_f64(pool_v).copy()
    lens = [int(x) for x in np.asarray(as_f64(lens)).reshape(-1)]
    slot = [int(x) for x in np.asarray(as_f64(slot)).reshape(-1)]
    B, H, T, D = q.shape
    assert T == 1, "one new token per user and call"
    scale = default_scale(D) if scale is None else scale
    o = np.empty((B, H, 1, D))
    for b in range(B):
        N, s = lens[b], slot[b]
        pk[layer, s, :, N] = k[b, :, 0]
        pv[layer, s, :, N] = v[b, :, 0]
        M = mfalcon_mask(N + 1, 0)[N:N + 1]
        for h in range(H):
            o[b, h] = masked_attention(q[b, h], pk[layer, s, h, :N + 1], pv[layer, s, h, :N + 1], M, scale)
    return o, pk, pv


def rank_decode_rows(qc, kc, vc, hist_k, hist_v, rows: Sequence[int],
                     scale: float | None = None) -> np.ndarray:
    """Outputs of selected candidate rows only, for one (user, head).

    qc, kc, vc are [K, D]; hist_k, hist_v are the N history rows [N, D] of the slot.
    Used to check sampled outputs of very large calls one candidate at a time.
    """
    qc, kc, vc, hk, hv = (as_f64(t) for t in (qc, kc, vc, hist_k, hist_v))
    N, D = hk.shape
    K = qc.shape[0]
    scale = default_scale(D) if scale is None else scale
    M = mfalcon_mask(N, K)[N:, :]
    out = []
    for j in rows:
        xk = np.concatenate([hk, kc], axis=0)
        xv = np.concatenate([hv, vc], axis=0)
        out.append(masked_attention(qc[j : j + 1], xk, xv, M[j : j + 1], scale)[0])
    return np.stack(out) if out else np.zeros((0, D))


def prefill_rows(q, k, v, N: int, rows: Sequence[int], scale: float | None = None) -> np.ndarray:
    """Outputs of selected history rows only, for one (user, head); q, k, v are [>=N, D]."""
    q, k, v = (as_f64(t) for t in (q, k, v))
    D = q.shape[1]
    scale = default_scale(D) if scale is None else scale
    M = mfalcon_mask(N, 0)
    out = []
    for i in rows:
        out.append(masked_attention(q[i : i + 1], k[:N], v[:N], M[i : i + 1], scale)[0])
    return np.stack(out) if out else np.zeros((0, D))


# ----------------------------------------------------------------------------------
# Scalar brute force: nested loops, two-pass softmax, math.fsum.  It states the
# attention rule through loop bounds instead of a mask array, and is used only on
# tiny inputs to pin the vectorised functions above.
# ----------------------------------------------------------------------------------

def _softmax_average(query, keys, values, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(query, key)) for key in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    D = len(values[0])
    return [math.fsum(w * val[d] for w, val in zip(weights, values)) / total for d in range(D)]


def bruteforce_joint(q, k, v, qc, kc, vc, N: int, scale: float):
    """One (user, head): q, k, v are lists of N history rows; qc, kc, vc lists of K rows.

    Returns (history outputs, candidate outputs) as nested lists.
    """
    hist = []
    for i in range(N):
        visible = range(0, i + 1)                       # causal over history
        hist.append(_softmax_average(q[i], [k[t] for t in visible],
                                     [v[t] for t in visible], scale))
    cand = []
    for j in range(len(qc)):
        keys = [k[t] for t in range(N)] + [kc[j]]       # all history, then itself
        vals = [v[t] for t in range(N)] + [vc[j]]
        cand.append(_softmax_average(qc[j], keys, vals, scale))
    return hist, cand


class SlotRing:
    """Round-robin slot hand-out with per-slot generation counters ([review] section 2.4).

    The i-th acquisition (0-based) gets slot i mod S; a slot's generation is the
    number of times it has been handed out.
    """

    def __init__(self, S: int):
        self.S = S
        self.count = 0
        self.gen = [0] * S

    def acquire(self) -> Tuple[int, int]:
        s = self.count % self.S
        self.count += 1
        self.gen[s] += 1
        return s, self.gen[s]
