"""Pins of the E4M3 oracle (oracle/fp8.py) to things other than itself.

* decoding of all 256 codes against torch's float8_e4m3fn;
* encoding of every finite bf16 value of magnitude below 464 against torch's cast
  (which rounds the same way but does not saturate: from 464 on it gives NaN);
* code points of the OCP format worked out by hand, ties to even in the normal and the
  subnormal range, and the saturation of large and infinite values;
* decode-encode round trip of every code and the order of the decoded values;
* the pool write stores exactly the codes of rows 0..N-1, and the retrieval step on an
  E4M3 pool reduces to the bf16 step when every value is already an E4M3 value;
* planted mistakes in the oracle are caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as OF

ALL_CODES = np.arange(256, dtype=np.uint8)


def _finite_bf16():
    b = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    return b[np.isfinite(b)]


def check_decode_vs_torch():
    t = torch.from_numpy(ALL_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(OF.e4m3_decode(ALL_CODES), t, equal_nan=True)


def check_encode_vs_torch():
    x = _finite_bf16()
    x = x[np.abs(x) < 464]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(OF.e4m3_encode(x), t)


def check_code_points():
    # value -> code, from the format's definition: bias 7, 3 mantissa bits
    table = {1.0: 0x38, 448.0: 0x7E, 2.0 ** -6: 0x08, 2.0 ** -9: 0x01, -2.0: 0xC0, 0.0: 0x00,
             1.125: 0x39, 0.875: 0x36, 240.0: 0x77, -448.0: 0xFE}
    got = OF.e4m3_encode(np.array(list(table)))
    assert got.tolist() == list(table.values())
    assert OF.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert OF.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    # ties go to the even mantissa
    ties = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 464.0: 0x7E, 1.8125: 0x3E}
    assert OF.e4m3_encode(np.array(list(ties))).tolist() == list(ties.values())
    # saturation
    big = OF.e4m3_encode(np.array([449.0, 500.0, 1e30, np.inf, -np.inf, -1e5]))
    assert big.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def check_round_trip_and_order():
    d = OF.e4m3_decode(ALL_CODES)
    ok = ~np.isnan(d)
    assert np.array_equal(OF.e4m3_encode(d[ok]), ALL_CODES[ok])
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])


def check_pool_write():
    rng = np.random.default_rng(5)
    L, S, H, n, D = 2, 3, 2, 9, 16
    pk0 = rng.integers(0, 256, size=(L, S, H, n, D), dtype=np.uint8)
    pv0 = rng.integers(0, 256, size=(L, S, H, n, D), dtype=np.uint8)
    k = rng.normal(size=(2, H, n, D))
    v = rng.normal(size=(2, H, n, D))
    pk, pv = OF.pool_write_e4m3(pk0, pv0, k, v, [9, 4], [2, 0], 1)
    exp_k, exp_v = pk0.copy(), pv0.copy()
    exp_k[1, 2] = OF.e4m3_encode(k[0])
    exp_v[1, 2] = OF.e4m3_encode(v[0])
    exp_k[1, 0, :, :4] = OF.e4m3_encode(k[1, :, :4])
    exp_v[1, 0, :, :4] = OF.e4m3_encode(v[1, :, :4])
    assert np.array_equal(pk, exp_k) and np.array_equal(pv, exp_v)


def check_ar_step_reduces_to_bf16_step():
    """With every value already an E4M3 value, quantising changes nothing: the step on
    the E4M3 pool equals the plain step on the decoded pool, and stores the same rows."""
    rng = np.random.default_rng(6)
    L, S, H, n, D, B = 1, 3, 2, 12, 8, 3
    grid = OF.e4m3_decode(np.arange(0x20, 0x50, dtype=np.uint8))   # a range of ordinary values
    pick = lambda *shape: rng.choice(np.concatenate([grid, -grid]), size=shape)
    pk = OF.e4m3_encode(pick(L, S, H, n, D))
    pv = OF.e4m3_encode(pick(L, S, H, n, D))
    q, k, v = pick(B, H, 1, D), pick(B, H, 1, D), pick(B, H, 1, D)
    slots, lens = [2, 0, 1], [5, 0, 11]
    o8, pk8, pv8 = OF.ar_decode_e4m3(q, k, v, pk, pv, slots, lens, 0)
    o, pkf, pvf = oracle.ar_decode(q, k, v, OF.e4m3_decode(pk), OF.e4m3_decode(pv), slots, lens, 0)
    assert np.allclose(o8, o, atol=1e-13, rtol=0)
    assert np.array_equal(OF.e4m3_decode(pk8), pkf) and np.array_equal(OF.e4m3_decode(pv8), pvf)


def check_ar_step_self_key_at_input_precision():
    """An empty slot: the step returns its own v exactly, not its quantised v."""
    q = np.ones((1, 1, 1, 4))
    v = np.array([0.3, -0.7, 1.3, 100.3]).reshape(1, 1, 1, 4)
    pk = np.zeros((1, 1, 1, 3, 4), dtype=np.uint8)
    o, pk2, pv2 = OF.ar_decode_e4m3(q, q, v, pk, pk.copy(), [0], [0], 0)
    assert np.array_equal(o, v)
    assert np.array_equal(pv2[0, 0, 0, 0], OF.e4m3_encode(v[0, 0, 0]))


ALL_CHECKS = [check_decode_vs_torch, check_encode_vs_torch, check_code_points, check_round_trip_and_order,
              check_pool_write, check_ar_step_reduces_to_bf16_step, check_ar_step_self_key_at_input_precision]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_fp8_pin(check):
    check()


# ---------------------------------------------------------------- planted mistakes

_orig_encode, _orig_decode, _orig_round = OF.e4m3_encode, OF.e4m3_decode, OF._round_half_even


def _truncating(x):
    return np.floor(x)


def _ties_away(x):
    return np.floor(x + 0.5)


def _no_saturation(x):
    x = OF.as_f64(x)
    code = _orig_encode(x).astype(np.int64)
    return np.where(np.abs(x) >= 464, 0x7F | (np.signbit(x).astype(np.int64) << 7), code).astype(np.uint8)


def _flush_subnormals(x):
    x = OF.as_f64(x)
    code = _orig_encode(x)
    return np.where(np.abs(x) < 2.0 ** -6, (np.signbit(x).astype(np.uint8) << 7), code).astype(np.uint8)


def _decode_bias_8(codes):
    return _orig_decode(codes) / 2.0


def _ar_self_key_quantised(q, k, v, pool_k, pool_v, slot, lens, layer, scale=None):
    return _orig_ar(q, OF.e4m3_decode(OF.e4m3_encode(k)), OF.e4m3_decode(OF.e4m3_encode(v)), pool_k, pool_v, slot,
                    lens, layer, scale)


_orig_ar = OF.ar_decode_e4m3

MUTANTS = {
    "rounding truncates": ("_round_half_even", _truncating),
    "ties round away from zero": ("_round_half_even", _ties_away),
    "no saturation": ("e4m3_encode", _no_saturation),
    "subnormals flushed to zero": ("e4m3_encode", _flush_subnormals),
    "exponent bias 8 in decoding": ("e4m3_decode", _decode_bias_8),
    "retrieval step quantises its own token": ("ar_decode_e4m3", _ar_self_key_quantised),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OF, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches: {name}"
