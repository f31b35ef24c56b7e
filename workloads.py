"""Seeded synthetic workloads for M-FALCON masked attention over a slotted KV pool.

This module only draws random inputs; it holds none of the attention arithmetic.
Both the HIP path (through the binding) and the CPU oracle consume what it draws.

Shapes and distributions follow the five workload descriptions used throughout the
tests and the benchmark (tiny fp32, bf16 single layer, bf16 ragged, the 12-layer
serving shape and the long-history shape).  The UniPinRec pages measure only on
internal Pinterest data (review page, section 3.1; reproduction notes, "experiment
setup"), which is not available; these seeded draws stand in for it.

Recipe (stated once, used everywhere):
  * seed of config i = 20260000 + i;
  * history lengths are drawn first, on a CPU ``torch.Generator`` seeded with the
    config seed, as integers uniform on the inclusive range [len_lo, len_hi];
  * the tensors of layer l are drawn on the requested device from a
    ``torch.Generator(device)`` seeded with ``seed * 100 + l``, in the order
    q, k, v, qc, kc, vc, each as float32 ``randn * std`` and then cast to the
    config dtype (bf16 casts round to nearest even);
  * history tensors are [B, H, n, D] with n the padded extent (rows >= len are
    ordinary random values, never meant to be read); candidate tensors are
    [B, H, k, D].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    dtype: torch.dtype
    L: int          # layers
    S: int          # pool slots
    B: int          # users (requests) per call
    H: int          # heads
    D: int          # head dim
    n: int          # padded history extent (= pool n_max)
    k: int          # candidates per user
    len_lo: int     # history length range, inclusive
    len_hi: int
    std: float = 1.0

    @property
    def seed(self) -> int:
        return 20260000 + self.index

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload(0, "tiny fp32: B=1 H=2 D=32 n=64 k=16", torch.float32,
             L=1, S=1, B=1, H=2, D=32, n=64, k=16, len_lo=64, len_hi=64),
    Workload(1, "bf16 single layer: B=32 H=8 D=64 n=256 k=128", torch.bfloat16,
             L=1, S=32, B=32, H=8, D=64, n=256, k=128, len_lo=256, len_hi=256),
    Workload(2, "bf16 ragged: B=64 H=8 D=64 n in [128,1024] k=512", torch.bfloat16,
             L=1, S=64, B=64, H=8, D=64, n=1024, k=512, len_lo=128, len_hi=1024),
    Workload(3, "bf16 12-layer serving shape: L=12 S=64 H=8 n=512 D=64, 64 requests x k=1000",
             torch.bfloat16, L=12, S=64, B=64, H=8, D=64, n=512, k=1000,
             len_lo=512, len_hi=512),
    Workload(4, "bf16 long history: B=16 H=16 D=128 n in [1024,4096] k=2048, std 0.5",
             torch.bfloat16, L=1, S=16, B=16, H=16, D=128, n=4096, k=2048,
             len_lo=1024, len_hi=4096, std=0.5),
]


def history_lengths(w: Workload) -> torch.Tensor:
    """int32 [B] history lengths, drawn on the CPU so every device sees the same values."""
    if w.len_lo == w.len_hi:
        return torch.full((w.B,), w.len_lo, dtype=torch.int32)
    g = torch.Generator("cpu").manual_seed(w.seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def layer_inputs(w: Workload, layer: int, device="cpu") -> Dict[str, torch.Tensor]:
    """q, k, v [B,H,n,D] and qc, kc, vc [B,H,k,D] of one layer, in the workload dtype."""
    dev = torch.device(device)
    g = torch.Generator(dev).manual_seed(w.seed * 100 + layer)
    out = {}
    for name in ("q", "k", "v"):
        t = torch.randn((w.B, w.H, w.n, w.D), generator=g, device=dev, dtype=torch.float32)
        out[name] = (t * w.std).to(w.dtype) if w.std != 1.0 else t.to(w.dtype)
    for name in ("qc", "kc", "vc"):
        t = torch.randn((w.B, w.H, w.k, w.D), generator=g, device=dev, dtype=torch.float32)
        out[name] = (t * w.std).to(w.dtype) if w.std != 1.0 else t.to(w.dtype)
    return out


def small_case(B: int, H: int, D: int, n: int, k: int, lens, dtype=torch.bfloat16,
               seed: int = 0, std: float = 1.0, device="cpu") -> Dict[str, torch.Tensor]:
    """A custom seeded case (used for edge cases: empty history, ragged tails, k=1 ...)."""
    w = Workload(-1, "custom", dtype, L=1, S=B, B=B, H=H, D=D, n=n, k=k,
                 len_lo=0, len_hi=n, std=std)
    w = replace(w, index=seed - 20260000)  # seed property then equals `seed`
    d = layer_inputs(w, 0, device)
    d["lens"] = torch.as_tensor(lens, dtype=torch.int32).reshape(B).clone()
    return d


def step_tokens(B: int, H: int, D: int, steps: int, dtype=torch.bfloat16, seed: int = 0,
                std: float = 1.0, device="cpu") -> Dict[str, torch.Tensor]:
    """q, k, v [steps, B, H, 1, D]: each user's new token for `steps` autoregressive steps.

    Drawn like layer_inputs: float32 randn * std on a generator of `device` seeded with
    `seed`, in the order q, k, v, then cast to `dtype`.
    """
    dev = torch.device(device)
    g = torch.Generator(dev).manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        t = torch.randn((steps, B, H, 1, D), generator=g, device=dev, dtype=torch.float32) * std
        out[name] = t.to(dtype)
    return out


def random_pool(L: int, S: int, H: int, n_max: int, D: int, dtype=torch.bfloat16, seed: int = 0,
                device="cpu"):
    """K and V pool arrays [L, S, H, n_max, D] filled with seeded randn values (stand-ins for
    rows an earlier call left in the slots)."""
    dev = torch.device(device)
    g = torch.Generator(dev).manual_seed(seed)
    k = torch.randn((L, S, H, n_max, D), generator=g, device=dev, dtype=torch.float32).to(dtype)
    v = torch.randn((L, S, H, n_max, D), generator=g, device=dev, dtype=torch.float32).to(dtype)
    return k, v


def poison_tail(x: torch.Tensor, lens: torch.Tensor, value=float("nan")) -> torch.Tensor:
    """Copy of a [B,H,n,D] tensor whose rows >= lens[b] hold `value` (used to prove they are never read)."""
    y = x.clone()
    for b, nb in enumerate(lens.tolist()):
        y[b, :, nb:, :] = value
    return y


BLOCK_WEIGHT_SHAPES = (("ln1_w", (1,)), ("ln1_b", (1,)), ("w_qkv", (1, 3)), ("b_qkv", (3,)), ("w_o", (1, 1)),
                       ("b_o", (1,)), ("ln2_w", (1,)), ("ln2_b", (1,)), ("w_fc", (1, 4)), ("b_fc", (4,)),
                       ("w_proj", (4, 1)), ("b_proj", (1,)))


def block_weights(C: int, dtype=torch.bfloat16, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Random weights of one transformer block of width C, drawn in the order of
    BLOCK_WEIGHT_SHAPES on a generator of `device` seeded with `seed` (shapes in units of
    C): matrices N(0, 1/fan_in) so projected values stay O(1), biases N(0, 0.02^2),
    LayerNorm gains 1 + N(0, 0.1^2) and shifts N(0, 0.02^2); then cast to `dtype`.
    Matrices are row-major "x @ W": [fan_in, fan_out]."""
    dev = torch.device(device)
    g = torch.Generator(dev).manual_seed(seed)
    out = {}
    for name, units in BLOCK_WEIGHT_SHAPES:
        shape = tuple(u * C for u in units)
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if name.startswith("w_"):
            t = t / math.sqrt(shape[0])
        elif name.endswith("_w"):
            t = 1.0 + 0.1 * t
        else:
            t = 0.02 * t
        out[name] = t.to(dtype)
    return out


def block_inputs(B: int, rows: int, C: int, dtype=torch.bfloat16, seed: int = 0, device="cpu") -> torch.Tensor:
    """Hidden states [B, rows, C] entering a block: float32 N(0, 1) on a generator of
    `device` seeded with `seed`, cast to `dtype`."""
    dev = torch.device(device)
    g = torch.Generator(dev).manual_seed(seed)
    return torch.randn((B, rows, C), generator=g, device=dev, dtype=torch.float32).to(dtype)
