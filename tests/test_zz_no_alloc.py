"""The allocation-free autoregressive step (unipin_ar_decode_noalloc), called through the
C ABI, against the step with a caller workspace (unipin_ar_decode): two calls in a row,
the second with a smaller input, on shapes that take the split path (whose part states
the allocation-free variant keeps in the library's static array) and on one that does
not.  Outputs and pool contents must be bit for bit equal: both run the same kernels
with the same split."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import falcon_attention_kv_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def step(pool, tok, slots, lens, layer, noalloc):
    """One step through the C ABI; returns o."""
    dev = torch.device(DEV)
    q, k, v = tok["q"][0], tok["k"][0], tok["v"][0]
    B = q.shape[0]
    o = torch.full_like(q, float("nan"))
    s_t = torch.as_tensor(slots, dtype=torch.int32, device=dev)
    l_t = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        rc = fa.lib.unipin_ar_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), pool.handle, s_t.data_ptr(),
                                             l_t.data_ptr(), layer, B, 0.0, o.data_ptr(), stream)
    else:
        need = fa.ar_decode_workspace_bytes(pool, B)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        rc = fa.lib.unipin_ar_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), pool.handle, s_t.data_ptr(),
                                     l_t.data_ptr(), layer, B, 0.0, o.data_ptr(), ws.data_ptr(), need, stream)
    assert rc == fa.OK, fa.lib.unipin_strerror(rc)
    torch.cuda.synchronize()
    return o


# (pool dtype, D, H, n_max, [(slots, lens) of call 1, then of the smaller call 2])
CASES = [
    (torch.bfloat16, 128, 2, 4600, [([3, 0, 2, 1], [4100, 0, 2047, 4599]), ([1, 2], [3000, 65])]),
    (torch.bfloat16, 64, 4, 4600, [([0, 1, 2], [2999, 1024, 700]), ([2], [129])]),
    (torch.float8_e4m3fn, 64, 2, 4600, [([1, 3, 0], [4500, 100, 2600]), ([0, 3], [1500, 1])]),
    (torch.float32, 64, 2, 700, [([0, 1], [699, 5]), ([1], [3])]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{str(c[0])[6:]}-D{c[1]}-H{c[2]}-n{c[3]}")
def test_noalloc_step_matches_the_workspace_step(case):
    dtype, D, H, n_max, calls = case
    announce(f"ar_decode_noalloc {case[:4]}")
    L, S = 1, 4
    act = torch.float32 if dtype == torch.float32 else torch.bfloat16
    base_k, base_v = W.random_pool(L, S, H, n_max, D, torch.float32 if dtype != act else act, seed=61, device=DEV)
    base_k, base_v = base_k.to(dtype), base_v.to(dtype)
    pools = {}
    for noalloc in (False, True):
        pk, pv = base_k.clone(), base_v.clone()
        pools[noalloc] = (fa.Pool(pk, pv), pk, pv)
    for i, (slots, lens) in enumerate(calls):
        B = len(slots)
        tok = W.step_tokens(B, H, D, 1, act, seed=62 + i, device=DEV)
        ref_pool = pools[False][0]
        if dtype != torch.float32:
            assert fa.ar_decode_workspace_bytes(ref_pool, B) > 0 or i > 0, "the first call must split"
        outs = {}
        for noalloc in (False, True):
            outs[noalloc] = step(pools[noalloc][0], tok, slots, lens, 0, noalloc)
            assert pools[noalloc][0].status() == 0
        assert torch.equal(outs[True].view(torch.int16) if act == torch.bfloat16 else outs[True].view(torch.int32),
                           outs[False].view(torch.int16) if act == torch.bfloat16 else outs[False].view(torch.int32)), \
            f"call {i}: outputs differ"
        assert torch.equal(pools[True][1].view(torch.uint8), pools[False][1].view(torch.uint8)), f"call {i}: K pool"
        assert torch.equal(pools[True][2].view(torch.uint8), pools[False][2].view(torch.uint8)), f"call {i}: V pool"
        assert torch.isfinite(outs[True].float()).all()
    for p, _, _ in pools.values():
        p.close()
