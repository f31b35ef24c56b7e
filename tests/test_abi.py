"""Host-side tests of the C ABI (no GPU needed: no call here reaches a kernel).

Every argument check of include/unipin.h runs before any HIP call, so these tests use
fake (aligned, never dereferenced) device addresses.
"""
import ctypes
import re
from pathlib import Path

import pytest

import falcon_attention_kv_amd as fa
import oracle

HEADER = Path(__file__).resolve().parents[1] / "include" / "unipin.h"
lib = fa.lib
vp = ctypes.c_void_p

FAKE = 0x10000          # aligned fake device address
FAKE_ODD = 0x10002      # misaligned


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(unipin_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == len(fa.EXPORTS)
    assert set(names) == set(fa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strerror():
    assert lib.unipin_version() == 10100
    for code in (fa.OK, fa.EINVAL, fa.ERANGE, fa.EDTYPE, fa.EALIGN, fa.EDEVICE, fa.EHIP, fa.ENOMEM, fa.EPERM,
                 fa.EIO, fa.ESCRATCH):
        text = lib.unipin_strerror(code).decode()
        assert text and text != "unknown status"
    assert lib.unipin_strerror(-99).decode() == "unknown status"


def test_binding_constants_match_the_header():
    # every UNIPIN_<NAME> = <value> of the header's enums has the same value in the binding
    text = HEADER.read_text()
    pairs = re.findall(r"\bUNIPIN_([A-Z0-9_]+)\s*=\s*(-?\d+)", text)
    assert len(pairs) >= 17
    for name, value in pairs:
        assert hasattr(fa, name), name
        assert getattr(fa, name) == int(value), (name, getattr(fa, name), value)


def make_pool(L=2, S=3, H=2, n_max=16, D=64, dtype=fa.BF16):
    h = vp()
    rc = lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE * 2, L, S, H, n_max, D, dtype)
    assert rc == fa.OK
    return h


@pytest.mark.parametrize("args,code", [
    ((0, FAKE, 1, 1, 1, 8, 64, fa.BF16), fa.EINVAL),        # null k pool
    ((FAKE, 0, 1, 1, 1, 8, 64, fa.BF16), fa.EINVAL),        # null v pool
    ((FAKE, FAKE, 0, 1, 1, 8, 64, fa.BF16), fa.EINVAL),     # L = 0
    ((FAKE, FAKE, 1, 0, 1, 8, 64, fa.BF16), fa.EINVAL),     # S = 0
    ((FAKE, FAKE, 1, 1, 0, 8, 64, fa.BF16), fa.EINVAL),     # H = 0
    ((FAKE, FAKE, 1, 1, 1, 0, 64, fa.BF16), fa.EINVAL),     # n_max = 0
    ((FAKE, FAKE, 1, 1, 1, 8, 48, fa.BF16), fa.EINVAL),     # unsupported D
    ((FAKE, FAKE, 1, 1, 1, 8, 64, 7), fa.EDTYPE),
    ((FAKE_ODD, FAKE, 1, 1, 1, 8, 64, fa.BF16), fa.EALIGN),
])
def test_pool_create_rejects(args, code):
    h = vp(123)
    assert lib.unipin_pool_create(ctypes.byref(h), *args) == code
    assert h.value is None


def test_pool_create_null_out():
    assert lib.unipin_pool_create(None, FAKE, FAKE, 1, 1, 1, 8, 64, fa.BF16) == fa.EINVAL


def test_pool_dims():
    h = make_pool(L=3, S=5, H=4, n_max=32, D=128, dtype=fa.FP32)
    out = [ctypes.c_int() for _ in range(6)]
    assert lib.unipin_pool_dims(h, *[ctypes.byref(x) for x in out]) == fa.OK
    assert [x.value for x in out] == [3, 5, 4, 32, 128, fa.FP32]
    assert lib.unipin_pool_dims(None, None, None, None, None, None, None) == fa.EINVAL
    lib.unipin_pool_destroy(h)


def test_acquire_matches_round_robin_oracle():
    S = 5
    h = make_pool(S=S)
    ring = oracle.SlotRing(S)
    for _ in range(3 * S + 2):
        s, g = ctypes.c_int32(), ctypes.c_uint64()
        assert lib.unipin_pool_acquire(h, ctypes.byref(s), ctypes.byref(g)) == fa.OK
        assert (s.value, g.value) == ring.acquire()
    for slot in range(S):
        assert lib.unipin_pool_generation(h, slot) == ring.gen[slot]
    # out of range and a null pool read as 0 (the value of a slot never handed out)
    assert lib.unipin_pool_generation(h, S) == 0
    assert lib.unipin_pool_generation(h, -1) == 0
    assert lib.unipin_pool_generation(None, 0) == 0
    s = ctypes.c_int32()
    assert lib.unipin_pool_acquire(h, ctypes.byref(s), None) == fa.OK   # generation optional
    assert lib.unipin_pool_acquire(None, ctypes.byref(s), None) == fa.EINVAL
    assert lib.unipin_pool_acquire(h, None, None) == fa.EINVAL
    lib.unipin_pool_destroy(h)


def test_acquire_is_thread_safe():
    import threading
    S, per, threads = 7, 500, 8
    h = make_pool(S=S)
    seen = []
    lock = threading.Lock()

    def work():
        mine = []
        for _ in range(per):
            s = ctypes.c_int32()
            assert lib.unipin_pool_acquire(h, ctypes.byref(s), None) == fa.OK
            mine.append(s.value)
        with lock:
            seen.extend(mine)

    ts = [threading.Thread(target=work) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    total = per * threads
    counts = [seen.count(s) for s in range(S)]
    # round-robin over `total` hand-outs: every slot gets floor or ceil of total / S
    assert sorted(counts) == sorted([total // S + (1 if i < total % S else 0) for i in range(S)])
    for s in range(S):
        assert lib.unipin_pool_generation(h, s) == counts[s]
    lib.unipin_pool_destroy(h)


def test_destroy_null_is_ok():
    assert lib.unipin_pool_destroy(None) == fa.OK


def _prefill(h, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, slot=FAKE, layer=0, B=1, n=8, scale=0.0, o=FAKE):
    return lib.unipin_prefill(q, k, v, lens, h, slot, layer, B, n, scale, o, None)


def _decode(h, qc=FAKE, kc=FAKE, vc=FAKE, slot=FAKE, lens=FAKE, layer=0, B=1, k=8, scale=0.0, oc=FAKE):
    return lib.unipin_rank_decode(qc, kc, vc, h, slot, lens, layer, B, k, scale, oc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.EINVAL), (dict(k=0), fa.EINVAL), (dict(v=0), fa.EINVAL),
    (dict(lens=0), fa.EINVAL), (dict(slot=0), fa.EINVAL), (dict(o=0), fa.EINVAL),
    (dict(B=0), fa.EINVAL), (dict(n=0), fa.EINVAL), (dict(n=17), fa.EINVAL),
    (dict(layer=-1), fa.ERANGE), (dict(layer=2), fa.ERANGE),
    (dict(q=FAKE_ODD), fa.EALIGN), (dict(o=FAKE_ODD), fa.EALIGN), (dict(lens=FAKE + 2), fa.EALIGN),
    (dict(scale=float("inf")), fa.EINVAL),
])
def test_prefill_host_checks(kw, code):
    h = make_pool(L=2, n_max=16)
    assert _prefill(h, **kw) == code
    lib.unipin_pool_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(qc=0), fa.EINVAL), (dict(kc=0), fa.EINVAL), (dict(vc=0), fa.EINVAL),
    (dict(lens=0), fa.EINVAL), (dict(slot=0), fa.EINVAL), (dict(oc=0), fa.EINVAL),
    (dict(B=0), fa.EINVAL), (dict(k=0), fa.EINVAL),
    (dict(layer=-1), fa.ERANGE), (dict(layer=2), fa.ERANGE),
    (dict(kc=FAKE_ODD), fa.EALIGN), (dict(slot=FAKE + 1), fa.EALIGN),
    (dict(scale=float("-inf")), fa.EINVAL),
])
def test_decode_host_checks(kw, code):
    h = make_pool(L=2, n_max=16)
    assert _decode(h, **kw) == code
    lib.unipin_pool_destroy(h)


def _ar(h, q=FAKE, k=FAKE, v=FAKE, slot=FAKE, lens=FAKE, layer=0, B=1, scale=0.0, o=FAKE, ws=None, ws_bytes=0):
    return lib.unipin_ar_decode(q, k, v, h, slot, lens, layer, B, scale, o, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.EINVAL), (dict(k=0), fa.EINVAL), (dict(v=0), fa.EINVAL),
    (dict(lens=0), fa.EINVAL), (dict(slot=0), fa.EINVAL), (dict(o=0), fa.EINVAL),
    (dict(B=0), fa.EINVAL), (dict(B=-3), fa.EINVAL),
    (dict(layer=-1), fa.ERANGE), (dict(layer=2), fa.ERANGE),
    (dict(v=FAKE_ODD), fa.EALIGN), (dict(o=FAKE + 8), fa.EALIGN), (dict(lens=FAKE + 2), fa.EALIGN),
    (dict(scale=float("inf")), fa.EINVAL),
])
def test_ar_decode_host_checks(kw, code):
    h = make_pool(L=2, n_max=16)
    assert _ar(h, **kw) == code
    # the allocation-free variant checks its arguments the same way
    a = dict(q=FAKE, k=FAKE, v=FAKE, slot=FAKE, lens=FAKE, layer=0, B=1, scale=0.0, o=FAKE)
    a.update(kw)
    assert lib.unipin_ar_decode_noalloc(a["q"], a["k"], a["v"], h, a["slot"], a["lens"], a["layer"], a["B"],
                                        a["scale"], a["o"], None) == code
    lib.unipin_pool_destroy(h)


def test_ar_decode_workspace_bytes():
    """A pair is split only when its slot at capacity holds at least 240 Ki elements per
    matrix (rows x D); then into parts of at least 4 chunks (64 rows each here), at most
    256 // (B*H) parts and 64, and only with 3 parts or more; the buffer holds one fp32
    state of D + 4 floats per (user, head, part)."""
    assert lib.unipin_ar_decode_workspace_bytes(None, 4) == 0
    h = make_pool(L=1, S=16, H=16, n_max=4106, D=128)   # 2 MiB of K/V per pair, 65 chunks
    assert lib.unipin_ar_decode_workspace_bytes(h, 0) == 0
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 16 * 16 * (128 + 4) * 4   # 256 // 16 parts
    assert lib.unipin_ar_decode_workspace_bytes(h, 4) == 64 * 4 * (128 + 4) * 4    # 256 // 64 parts
    assert lib.unipin_ar_decode_workspace_bytes(h, 5) == 80 * 3 * (128 + 4) * 4    # 256 // 80 = 3 parts
    assert lib.unipin_ar_decode_workspace_bytes(h, 8) == 0                         # 2 parts: one pass
    assert lib.unipin_ar_decode_workspace_bytes(h, 16) == 0                        # 256 pairs: one pass
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=2, n_max=1921, D=128)   # 1920 rows x 128: the smallest slot that splits
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) > 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=2, n_max=1920, D=128)   # one row fewer: one pass
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=2, n_max=3000, D=64)    # 750 KB of bf16 per pair, 192 Ki elements
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=2, n_max=4600, D=64, dtype=fa.FP8_E4M3)   # 294 Ki elements of codes
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) > 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=64, H=8, n_max=522, D=64)   # history 512 + a few steps: 130 KiB per pair
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 0
    assert lib.unipin_ar_decode_workspace_bytes(h, 64) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=1, n_max=4097, D=128)   # 64 chunks: 16 parts of 4
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 1 * 16 * (128 + 4) * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=1, n_max=40001, D=128)   # 625 chunks: capped at 64 parts
    assert lib.unipin_ar_decode_workspace_bytes(h, 1) == 64 * (128 + 4) * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=4, H=2, n_max=4097, D=64, dtype=fa.FP32)   # fp32 pools: fp64 one pass, no split
    assert lib.unipin_ar_decode_workspace_bytes(h, 3) == 0
    lib.unipin_pool_destroy(h)


def test_ar_decode_workspace_checks():
    h = make_pool(L=1, S=16, H=16, n_max=4106, D=128)
    need = lib.unipin_ar_decode_workspace_bytes(h, 1)
    assert need > 0
    assert _ar(h, B=1, ws=FAKE, ws_bytes=need - 1) == fa.EINVAL
    assert _ar(h, B=1, ws=FAKE + 4, ws_bytes=need) == fa.EALIGN
    lib.unipin_pool_destroy(h)


def test_block_workspace_bytes():
    """The block's workspace: 32 MiB for the GEMM library, then M x 4C and M x C bf16
    regions (M = B * rows), 4C x C + 4C bf16 values and 2 x 4C fp32 values for the GEMM
    tuner, each rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    h = make_pool(L=1, S=8, H=8, n_max=992, D=64)
    M, C = 8 * 656, 512
    assert lib.unipin_block_workspace_bytes(h, 8, 656) == (32 << 20) + up(M * 4 * C * 2) + up(M * C * 2) \
        + up((4 * C * C + 4 * C) * 2) + up(8 * C * 4)
    assert lib.unipin_block_workspace_bytes(h, 0, 656) == 0
    assert lib.unipin_block_workspace_bytes(None, 8, 656) == 0
    lib.unipin_pool_destroy(h)


def test_block_host_checks():
    h = make_pool(L=1, S=2, H=2, n_max=16, D=32)
    w = fa.BlockWeights(*([FAKE] * len(fa.BLOCK_WEIGHT_NAMES)))
    args = lambda ctx, wp, mode=fa.BLOCK_CANDIDATES: lib.unipin_block_forward(
        ctx, wp, mode, FAKE, h, FAKE, FAKE, 0, 1, 4, 0.0, FAKE, 1 << 30, None)
    assert args(None, ctypes.byref(w)) == fa.EINVAL          # no context
    assert lib.unipin_block_ctx_destroy(None) == fa.EINVAL
    assert lib.unipin_block_ctx_create(None) == fa.EINVAL
    assert lib.unipin_block_ctx_set_gemm(None, fa.GEMM_AUTO) == fa.EINVAL
    lib.unipin_pool_destroy(h)


def test_rank_decode_split_plan():
    """The split of the ranking decode: for histories of at least 16 tiles of 64 keys and
    few candidate tiles (items): at most half the resident workgroups (512 at D <= 64,
    256 at D = 128) and at most 2 (D <= 64) or 3 (D = 128) per history tile; parts of
    at least four tiles, as many as fit in one round of the resident workgroups; bf16
    and E4M3 pools.  The workspace holds (D + 2) fp32 per candidate row of every part of
    every 256-row tile."""
    h = make_pool(L=1, S=2, H=8, n_max=1024, D=64)
    # 8 pairs x 4 candidate tiles = 32 items: min(512 / 32, 16 tiles / 4) = 4 parts
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 1000) == 32 * 4 * 256 * 66 * 4
    assert lib.unipin_rank_decode_workspace_bytes(h, 64, 1000) == 0     # enough pairs: one pass
    assert lib.unipin_rank_decode_workspace_bytes(h, 0, 1000) == 0
    assert lib.unipin_rank_decode_workspace_bytes(None, 1, 1000) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=4, n_max=1024, D=128)
    # 4 pairs x 2 tiles = 8 items: min(256 / 8, 16 / 4) = 4 parts of 4 tiles
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 300) == 8 * 4 * 256 * 130 * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=8, n_max=1024, D=64)
    # 2 users: 64 items, more than 2 per history tile (16): one pass
    assert lib.unipin_rank_decode_workspace_bytes(h, 2, 1000) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=16, n_max=2048, D=128)
    # 2 x 16 pairs x 3 tiles = 96 items, 3 per history tile (32): floor(256 / 96) = 2 parts
    # of 16 tiles, all resident at once
    assert lib.unipin_rank_decode_workspace_bytes(h, 2, 656) == 96 * 2 * 256 * 130 * 4
    assert lib.unipin_rank_decode_workspace_bytes(h, 2, 1000) == 0     # 128 items: one pass
    lib.unipin_pool_destroy(h)
    h = make_pool(L=2, S=2, H=4, n_max=2048, D=32)
    # 4 pairs x 2 tiles = 8 items: min(512 / 8, 32 / 4) = 8 parts of 4 tiles
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 500) == 8 * 8 * 256 * 34 * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=4, n_max=2100, D=32)
    # 33 tiles: min(64, 33 / 4 = 8) parts of ceil(33 / 8) = 5 tiles, so 7 parts
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 500) == 8 * 7 * 256 * 34 * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=8, n_max=960, D=64)   # 15 tiles of history: one pass
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 1000) == 0
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=8, n_max=1024, D=64, dtype=fa.FP8_E4M3)   # E4M3: the same plan
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 1000) == 32 * 4 * 256 * 66 * 4
    lib.unipin_pool_destroy(h)
    h = make_pool(L=1, S=2, H=8, n_max=1024, D=64, dtype=fa.FP32)
    assert lib.unipin_rank_decode_workspace_bytes(h, 1, 1000) == 0      # fp32: one pass
    lib.unipin_pool_destroy(h)


def test_rank_decode_split_checks():
    """Argument checks of unipin_rank_decode_split before any device work."""
    h = make_pool(L=1, S=2, H=8, n_max=1024, D=64)
    need = lib.unipin_rank_decode_workspace_bytes(h, 1, 1000)
    call = lambda ws, nbytes, B=1: lib.unipin_rank_decode_split(FAKE, FAKE, FAKE, h, FAKE, FAKE, 0, B, 1000, 0.0,
                                                                FAKE, ws, nbytes, None)
    assert call(FAKE_ODD, need) == fa.EALIGN
    assert call(FAKE, need - 1) == fa.EINVAL
    assert call(FAKE, need, B=0) == fa.EINVAL
    assert lib.unipin_rank_decode_split(None, FAKE, FAKE, h, FAKE, FAKE, 0, 1, 1000, 0.0, FAKE, FAKE, need,
                                        None) == fa.EINVAL
    lib.unipin_pool_destroy(h)


def test_block_fold_layernorm_checks():
    """unipin_block_fold_layernorm rejects its arguments before any device work."""
    w = fa.BlockWeights(*([FAKE] * len(fa.BLOCK_WEIGHT_NAMES)))
    fold = lambda wp, C, a=FAKE, b=FAKE, c=FAKE, d=FAKE: lib.unipin_block_fold_layernorm(wp, C, a, b, c, d, None)
    assert fold(None, 512) == fa.EINVAL                       # no weights
    assert fold(ctypes.byref(w), 512, a=None) == fa.EINVAL    # an output missing
    assert fold(ctypes.byref(w), 512, d=None) == fa.EINVAL
    for C in (0, 4, 12, 2056):                                # C a multiple of 8 in [8, 2048]
        assert fold(ctypes.byref(w), C) == fa.EINVAL
    assert fold(ctypes.byref(w), 512, c=FAKE_ODD) == fa.EALIGN
    odd = fa.BlockWeights(*([FAKE] * 5 + [FAKE_ODD] + [FAKE] * 6))
    assert fold(ctypes.byref(odd), 512) == fa.EALIGN          # a misaligned weight
    part = fa.BlockWeights(*([FAKE] * 11 + [None]))
    assert fold(ctypes.byref(part), 512) == fa.EINVAL         # a weight missing


def test_e4m3_pool_dims():
    """E4M3 pools take D = 64 or 128; other element types keep D = 32 too."""
    h = vp()
    assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE * 2, 1, 1, 1, 8, 32, fa.FP8_E4M3) == fa.EINVAL
    assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE * 2, 1, 1, 1, 8, 64, 3) == fa.EDTYPE
    for D in (64, 128):
        assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE * 2, 1, 1, 1, 8, D, fa.FP8_E4M3) == fa.OK
        lib.unipin_pool_destroy(h)


def test_null_pool_rejected():
    assert _prefill(None) == fa.EINVAL
    assert _decode(None) == fa.EINVAL
    assert _ar(None) == fa.EINVAL


def test_binding_rejects_mismatched_tensors():
    import torch
    # host-side checks in the binding run before the library is called
    k = torch.empty((1, 1, 2, 8, 64), dtype=torch.bfloat16)
    pool = fa.Pool(k, torch.empty_like(k))
    q = torch.empty((1, 2, 8, 64), dtype=torch.float32)
    with pytest.raises(fa.UnipinError):
        fa.prefill(q, q, q, [8], pool, [0], 0)
    q = torch.empty((1, 3, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(fa.UnipinError):
        fa.prefill(q, q, q, [8], pool, [0], 0)
    with pytest.raises(fa.UnipinError):
        fa.Pool(k, torch.empty((1, 1, 2, 8, 32), dtype=torch.bfloat16))
    t = torch.empty((1, 2, 2, 64), dtype=torch.bfloat16)   # two new tokens per user: not a step
    with pytest.raises(fa.UnipinError):
        fa.ar_decode(t, t, t, pool, [0], [3], 0)
    pool.close()


def test_pool_status_host_checks():
    flags = ctypes.c_int(5)
    assert lib.unipin_pool_status(None, None, ctypes.byref(flags)) == fa.EINVAL
    assert flags.value == 0


def test_offsets_stay_within_32_bits():
    """One (user, head)'s rows of an operand, and one slot's rows of one head in the pool,
    are addressed with 32-bit byte offsets in the kernels: larger shapes are refused on the
    host instead of wrapping."""
    h = vp()
    # n_max * D * elem = 2^24 * 128 * 1 = 2^31 bytes (E4M3) -> refused; one row less fits
    assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE, 1, 1, 1, 1 << 24, 128, fa.FP8_E4M3) == fa.EINVAL
    assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE, 1, 1, 1, (1 << 23) - 1, 128, fa.BF16) == fa.OK
    lib.unipin_pool_destroy(h)
    assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE, 1, 1, 1, 1 << 23, 128, fa.BF16) == fa.EINVAL
    pool = make_pool(L=1, S=1, H=1, n_max=16, D=128)
    # k * D * 2 bytes = 2^23 * 128 * 2 = 2^31: the candidate rows of one (user, head)
    k = 1 << 23
    assert lib.unipin_rank_decode(FAKE, FAKE, FAKE, pool, FAKE, FAKE, 0, 1, k, 0.0, FAKE, None) == fa.EINVAL
    lib.unipin_pool_destroy(pool)


def test_pool_limit_and_flag_entries_are_reused():
    """4096 live descriptors per process; destroying one frees its flag entry."""
    hs = []
    try:
        while True:
            h = vp()
            rc = lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE, 1, 1, 1, 8, 64, fa.BF16)
            if rc != fa.OK:
                assert rc == fa.ENOMEM
                break
            hs.append(h)
            assert len(hs) <= 4096
        assert len(hs) >= 4000   # other tests may hold a few
        lib.unipin_pool_destroy(hs.pop())
        h = vp()
        assert lib.unipin_pool_create(ctypes.byref(h), FAKE, FAKE, 1, 1, 1, 8, 64, fa.BF16) == fa.OK
        hs.append(h)
    finally:
        for h in hs:
            lib.unipin_pool_destroy(h)


def test_share_host_checks(tmp_path):
    """Export/import argument and file checks that need no GPU."""
    h = vp()
    assert lib.unipin_pool_export(None, b"/tmp/x") == fa.EINVAL
    pool = make_pool()
    assert lib.unipin_pool_export(pool, None) == fa.EINVAL
    assert lib.unipin_pool_export(pool, b"") == fa.EINVAL
    lib.unipin_pool_destroy(pool)
    assert lib.unipin_pool_import(None, b"/tmp/x") == fa.EINVAL
    assert lib.unipin_pool_import(ctypes.byref(h), None) == fa.EINVAL
    assert lib.unipin_pool_import(ctypes.byref(h), str(tmp_path / "missing").encode()) == fa.EIO
    bad = tmp_path / "bad"
    bad.write_bytes(b"not a pool share file" * 40)
    assert lib.unipin_pool_import(ctypes.byref(h), str(bad).encode()) == fa.EIO
    short = tmp_path / "short"
    short.write_bytes(b"UNIPINP1")
    assert lib.unipin_pool_import(ctypes.byref(h), str(short).encode()) == fa.EIO
    assert h.value is None
