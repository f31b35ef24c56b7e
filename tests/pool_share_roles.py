"""The two processes of the cross-process pool test (run as fresh subprocesses by
tests/test_gpu_pool_share.py; not collected by pytest).

    python tests/pool_share_roles.py owner  DIR [bf16|e4m3]
    python tests/pool_share_roles.py ranker DIR [bf16|e4m3]

The last argument is the pool's format (bf16 by default; e4m3: the pool holds E4M3
codes, the activations stay bf16).

owner:  the retrieval side.  Allocates a pool, hands out a slot per request, prefills two
        layers into the slots, runs the ranking decode itself once (the single-process
        result), exports the pool to DIR/pool.share and posts the request (slots,
        generations, lengths) to DIR/request.json.  After the ranker's first answer it
        hands out S more slots, so that the requests' slots are recycled, and posts
        DIR/recycled.json.  At the end it checks that the pool bytes are unchanged by
        the ranker.
ranker: the ranking side.  Imports the pool read-only, checks the request's generations,
        runs the ranking decode on the slots in place, checks the generations again
        (still current), saves its outputs, and after the recycling reports which
        requests it now detects as stale.

Files are written through a temporary name and a rename; each side polls for the
other's file with a time limit.  Every step prints what it does.
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SHAPE = dict(L=2, S=4, H=2, n_max=96, D=64)
B, K = 3, 40
LENS = [96, 50, 1]
SEED = 7100


def say(msg):
    print(f"[{sys.argv[1]}] {msg}", flush=True)


def post(path, obj):
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(obj, f)
    os.replace(tmp, path)


def wait_for(path, limit=120.0):
    t0 = time.time()
    while not os.path.exists(path):
        if time.time() - t0 > limit:
            raise TimeoutError(f"no {os.path.basename(path)} after {limit:.0f} s")
        time.sleep(0.05)
    with open(path) as f:
        return json.load(f)


def layer_case(layer, device):
    import workloads as W
    return W.small_case(B, SHAPE["H"], SHAPE["D"], SHAPE["n_max"], K, LENS, seed=SEED + layer, device=device)


def owner(d):
    import numpy as np
    import torch
    import falcon_attention_kv_amd as fa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    e4m3 = len(sys.argv) > 3 and sys.argv[3] == "e4m3"
    pool = fa.Pool.allocate(SHAPE["L"], SHAPE["S"], SHAPE["H"], SHAPE["n_max"], SHAPE["D"],
                            torch.float8_e4m3fn if e4m3 else torch.bfloat16, dev)
    if not e4m3:
        pool.k.fill_(float("nan"))
        pool.v.fill_(float("nan"))
    got = [pool.acquire() for _ in range(B)]
    slots, gens = [s for s, _ in got], [g for _, g in got]
    say(f"slots {slots} generations {gens}")
    refs = {}
    for layer in range(SHAPE["L"]):
        x = layer_case(layer, dev)
        fa.prefill(x["q"], x["k"], x["v"], LENS, pool, slots, layer)
        oc = fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, LENS, layer)
        refs[f"oc{layer}"] = oc.view(torch.int16).cpu().numpy()
    torch.cuda.synchronize()
    assert pool.status() == 0
    np.savez(os.path.join(d, "owner_out.npz"), **refs)
    snap_k, snap_v = pool.k.cpu().clone(), pool.v.cpu().clone()
    pool.export(os.path.join(d, "pool.share"))
    say("exported")
    post(os.path.join(d, "request.json"), {"slots": slots, "generations": gens, "lens": LENS})
    wait_for(os.path.join(d, "ranked.json"))
    say("ranker answered; recycling every slot")
    for _ in range(SHAPE["S"]):
        pool.acquire()
    post(os.path.join(d, "recycled.json"), {"generations": [pool.generation(s) for s in slots]})
    wait_for(os.path.join(d, "checked.json"))
    same = bool(torch.equal(pool.k.cpu().view(torch.uint8), snap_k.view(torch.uint8)) and
                torch.equal(pool.v.cpu().view(torch.uint8), snap_v.view(torch.uint8)))
    post(os.path.join(d, "owner_done.json"), {"pool_unchanged": same})
    say(f"pool bytes unchanged by the ranker: {same}")
    pool.close()


def ranker(d):
    import numpy as np
    req = wait_for(os.path.join(d, "request.json"))
    import torch
    import falcon_attention_kv_amd as fa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pool = fa.Pool.import_shared(os.path.join(d, "pool.share"), dev)
    say(f"imported pool L={pool.L} S={pool.S} H={pool.H} n_max={pool.n_max} D={pool.D} {pool.dtype}")
    slots, gens, lens = req["slots"], req["generations"], req["lens"]
    fresh_before = [pool.generation(s) == g for s, g in zip(slots, gens)]
    # the imported pool is read-only
    denied = {}
    x0 = layer_case(0, dev)
    for name, call in (("prefill", lambda: fa.prefill(x0["q"], x0["k"], x0["v"], lens, pool, slots, 0)),
                       ("ar_decode", lambda: fa.ar_decode(x0["q"][:, :, :1].contiguous(), x0["k"][:, :, :1].contiguous(),
                                                          x0["v"][:, :, :1].contiguous(), pool, slots, lens, 0)),
                       ("acquire", pool.acquire)):
        try:
            call()
            denied[name] = None
        except fa.UnipinError as e:
            denied[name] = e.status
    outs = {}
    for layer in range(pool.L):
        x = layer_case(layer, dev)
        oc = fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens, layer)
        outs[f"oc{layer}"] = oc
    torch.cuda.synchronize()
    status = pool.status()
    fresh_after = [pool.generation(s) == g for s, g in zip(slots, gens)]
    np.savez(os.path.join(d, "ranker_out.npz"), **{k: v.view(torch.int16).cpu().numpy() for k, v in outs.items()})
    post(os.path.join(d, "ranked.json"), {"fresh_before": fresh_before, "fresh_after": fresh_after,
                                          "denied": denied, "status": status})
    say(f"ranked: fresh before {fresh_before}, after {fresh_after}, denied {denied}")
    wait_for(os.path.join(d, "recycled.json"))
    stale = [pool.generation(s) != g for s, g in zip(slots, gens)]
    post(os.path.join(d, "checked.json"), {"stale": stale, "now": [pool.generation(s) for s in slots]})
    say(f"after recycling, stale: {stale}")
    pool.close()


if __name__ == "__main__":
    role, d = sys.argv[1], sys.argv[2]
    {"owner": owner, "ranker": ranker}[role](d)
