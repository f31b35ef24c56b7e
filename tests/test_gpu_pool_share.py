"""Cross-process pool sharing on one GPU: a retrieval (owner) process prefills the pool
and exports it; a ranking process imports it and runs the ranking decode on the slots
in place ([notes] section 6, cross-process KV sharing; [review] section 2.4).

Both sides run as fresh subprocesses (tests/pool_share_roles.py), so neither inherits
this process's GPU state.  Checked here: the ranker's outputs equal the owner's own
single-process outputs bit for bit and the oracle within the bf16 tolerance; the
ranker's generation check sees the request's slots as current before and after its
decode and as stale once the owner has handed them out again; the ranker cannot write
the pool (every writing call is refused) and the pool bytes are unchanged.  Run with a
bf16 pool and with an E4M3 pool (the oracle then reads the history through the codes).
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import falcon_attention_kv_amd as fa
import oracle
import pool_share_roles as R

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_ranking_process_reads_the_owners_pool(tmp_path, fmt):
    sys.__stderr__.write(f"[gpu case] cross-process pool share ({fmt} pool): owner + ranker subprocesses\n")
    sys.__stderr__.flush()
    script = os.path.join(HERE, "pool_share_roles.py")
    procs = {role: subprocess.Popen([sys.executable, "-u", script, role, str(tmp_path), fmt],
                                    stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for role in ("owner", "ranker")}
    logs = {}
    try:
        for role, p in procs.items():
            logs[role], _ = p.communicate(timeout=240)
    finally:
        for p in procs.values():
            if p.poll() is None:
                p.kill()
                p.wait()
    for role, p in procs.items():
        assert p.returncode == 0, f"{role} failed ({p.returncode}):\n{logs.get(role, '')}"

    ranked = json.loads((tmp_path / "ranked.json").read_text())
    checked = json.loads((tmp_path / "checked.json").read_text())
    done = json.loads((tmp_path / "owner_done.json").read_text())
    assert ranked["fresh_before"] == [True] * R.B and ranked["fresh_after"] == [True] * R.B
    assert ranked["status"] == 0
    assert ranked["denied"] == {"prefill": fa.EPERM, "ar_decode": fa.EPERM, "acquire": fa.EPERM}
    assert checked["stale"] == [True] * R.B, "a recycled slot must be detected through its generation"
    assert done["pool_unchanged"], "the ranking process must not write the pool"

    mine = np.load(tmp_path / "owner_out.npz")
    theirs = np.load(tmp_path / "ranker_out.npz")
    dev = torch.device("cuda")
    for layer in range(R.SHAPE["L"]):
        a, b = mine[f"oc{layer}"], theirs[f"oc{layer}"]
        assert np.array_equal(a, b), f"layer {layer}: cross-process outputs differ from the single-process run"
        x = {k: v.cpu() for k, v in R.layer_case(layer, dev).items()}
        got = torch.from_numpy(b).view(torch.bfloat16).double().numpy()
        hk, hv = x["k"], x["v"]
        if fmt == "e4m3":   # the history as the pool holds it: the codes of its rows
            hk, hv = oracle.e4m3_decode(oracle.e4m3_encode(hk)), oracle.e4m3_decode(oracle.e4m3_encode(hv))
        _, ref = oracle.joint(x["q"], hk, hv, x["qc"], x["kc"], x["vc"], R.LENS)
        err = np.abs(got - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (layer, err.max(), err.mean())
