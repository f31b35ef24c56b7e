"""Float64 oracle of the fp8 (E4M3) KV pool: the 8-bit format, and the pool writes and
reads that use it.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this module; the GPU library never calls it and shares no code
with it.

The pages run their forward pass in FP8 E4M3 (Transformer Engine's fused LayerNorm,
linear and activation layers; [review] section 3 and Table 2; [notes] section 7), and
attention itself stays bf16 there.  Storing the KV pool in E4M3, which halves the bytes
every ranking decode and retrieval step reads from it, is an extrapolation of that
choice to the cache.  The readings taken:
  * format: E4M3 of the OCP 8-bit floating point specification (the "fn" variant):
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
    the subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so the largest
    magnitude is 1.75 * 2^8 = 448;
  * encoding: the value is clamped to [-448, 448] (a saturating cast: an out-of-range
    K/V entry keeps its sign and the largest magnitude rather than turning into NaN),
    then rounded to the nearest E4M3 value, ties to the even mantissa; NaN stays NaN;
  * no scale factor: the pool stores the K/V values themselves (keys and values of a
    LayerNorm'd model are of order 1, well inside E4M3's range);
  * only what the pool holds is quantised.  Attention inside a call uses the call's
    own rows at their input precision (the prefill's history, the ranking decode's
    candidates, the retrieval step's new token); rows read back from the pool are the
    stored E4M3 values, which bf16 and fp32 represent exactly.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import as_f64, default_scale, masked_attention, mfalcon_mask

E4M3_MAX = 448.0          # 1.75 * 2^8
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
E4M3_NAN = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """The value of each E4M3 code (uint8) as float64: (-1)^s * 2^(e-7) * (1 + m/8) for
    exponent field e > 0, (-1)^s * 2^-6 * (m/8) for e = 0; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    out = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def _round_half_even(x: np.ndarray) -> np.ndarray:
    # numpy's rounding is half to even, and x here is exact (a binary scaling)
    return np.round(x)


def e4m3_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even encoding of values into E4M3 codes (uint8)."""
    x = as_f64(x)
    nan = np.isnan(x)
    sign = np.signbit(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    # the spacing of E4M3 values around a: 2^(E-3) in the binade [2^E, 2^(E+1)) for
    # E >= -6, and 2^-9 below 2^-6 (the subnormals share the spacing of the first binade)
    E = np.frexp(np.where(a > 0, a, 1.0))[1] - 1.0   # a = f * 2^E with f in [1, 2), exactly
    E = np.where(a >= E4M3_MIN_NORMAL, E, -6.0)
    step = np.ldexp(1.0, (E - 3).astype(np.int64))
    q = _round_half_even(a / step)            # integer count of steps, exact
    v = q * step                              # the rounded magnitude (may reach the next binade)
    v = np.minimum(v, E4M3_MAX)
    # bits of the rounded magnitude
    Ev = np.frexp(np.where(v > 0, v, 1.0))[1] - 1.0
    normal = v >= E4M3_MIN_NORMAL
    e_field = np.where(normal, Ev + 7, 0).astype(np.int64)
    m_field = np.where(normal, v / np.ldexp(1.0, Ev.astype(np.int64)) * 8 - 8, v / E4M3_SUBNORMAL_STEP)
    m_field = np.rint(m_field).astype(np.int64)
    code = (sign.astype(np.int64) << 7) | (e_field << 3) | m_field
    code = np.where(nan, E4M3_NAN | (sign.astype(np.int64) << 7), code)
    return code.astype(np.uint8)


def pool_write_e4m3(pool_k, pool_v, k, v, lens, slot, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """The E4M3 pool (uint8 codes [L, S, H, n_max, D]) after a prefill: rows 0..N-1 of
    slot[b] at `layer` hold the codes of k/v[b]; every other code is left as it was."""
    pk, pv = np.array(pool_k, dtype=np.uint8, copy=True), np.array(pool_v, dtype=np.uint8, copy=True)
    k, v = as_f64(k), as_f64(v)
    for b, (N, s) in enumerate(zip([int(x) for x in np.asarray(lens).reshape(-1)],
                                   [int(x) for x in np.asarray(slot).reshape(-1)])):
        pk[layer, s, :, :N] = e4m3_encode(k[b, :, :N])
        pv[layer, s, :, :N] = e4m3_encode(v[b, :, :N])
    return pk, pv


def ar_decode_e4m3(q, k, v, pool_k, pool_v, slot, lens, layer: int, scale: float | None = None
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One autoregressive step on an E4M3 pool: the new token (q, k, v [B, H, 1, D]) of
    user b attends to the decoded rows 0..N-1 of its slot and to itself at input
    precision, N = lens[b]; the codes of its k, v are stored at row N.
    Returns (o [B, H, 1, D], pool_k', pool_v') with the pools as uint8 codes."""
    q, k, v = (as_f64(t) for t in (q, k, v))
    pk, pv = np.array(pool_k, dtype=np.uint8, copy=True), np.array(pool_v, dtype=np.uint8, copy=True)
    B, H, T, D = q.shape
    assert T == 1, "one new token per user and call"
    scale = default_scale(D) if scale is None else scale
    o = np.empty((B, H, 1, D))
    for b in range(B):
        N, s = int(np.asarray(lens).reshape(-1)[b]), int(np.asarray(slot).reshape(-1)[b])
        M = mfalcon_mask(N + 1, 0)[N:N + 1]
        for h in range(H):
            keys = np.concatenate([e4m3_decode(pk[layer, s, h, :N]), k[b, h]], axis=0)
            vals = np.concatenate([e4m3_decode(pv[layer, s, h, :N]), v[b, h]], axis=0)
            o[b, h] = masked_attention(q[b, h], keys, vals, M, scale)
        pk[layer, s, :, N] = e4m3_encode(k[b, :, 0])
        pv[layer, s, :, N] = e4m3_encode(v[b, :, 0])
    return o, pk, pv
