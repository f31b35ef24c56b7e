"""Throughput of the M-FALCON attention hot path on one MI355X.

One step = one batch of 64 requests through the 12-layer serving shape
(L=12 layers, S=64 pool slots, H=8 heads, history n=512, D=64, k=1000 candidates per
request, bf16): acquire a slot per request (round-robin), 12 causal prefills that
write each layer's history K/V into the slots, then 12 ranking decodes in which every
candidate attends to its request's cached history plus itself.  Inputs are seeded
synthetic draws resident in HBM before timing starts.

Prints one JSON line.  `value` = ranked candidates per second through the whole step
(64 x 1000 candidates per step).  The roofline object describes the dominant kernel
(the ranking decode), its algorithmic bytes per launch over its average launch time
(HIP events on the launch stream around the step's 12 decode launches, gaps included).  The CPU baseline is the float64 oracle timed on a
bounded sample of the same work on the host cores.

After the timed steps, `block_table2` reports the 12-layer transformer around the
attention (projections, LayerNorm, MLP) at the pages' Table 2 shape, `e4m3_pool` the
serving step and the retrieval step with the pool stored as E4M3 codes, and `ar_step` reports the autoregressive retrieval step (one new
token per user and head appended to its slot) on the serving shape and on the long
history shape; it is a secondary figure and does not enter `value`.

`long_history` times one layer of the long-history workload (B=16, H=16, D=128, histories
1024..4096, 2048 candidates: the workload bound by the matrix cores), cold.  `probes`
reports the matrix-core rate a plain MFMA loop reaches and whether a SIMD overlaps
matrix-core with exponential work (libunipin_probe.so), beside `hbm_copy_reference`.

`--block-only` runs only the Table 2 transformer measurement (3 timed passes).
`--probes` runs only the probes.
`--sweep-splits` runs only the sweeps behind the two split plans: the ranking decode and
the retrieval step, one pass against split, over request counts, history lengths and head
dimensions (bf16 and E4M3 pools), each with the plan's choice.
`--workloads` replaces all of this with a per-kernel table over every bf16 workload
(one layer each, cold and back to back), with the ragged/full time ratios of the two
ragged workloads beside the ratios of their algorithmic work.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-ar-step] [--no-block] [--no-e4m3]
                       [--no-long-history] [--workloads] [--block-only] [--probes] [--sweep-splits]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ranked candidates/sec + TFLOP/s (frac of MFMA/HBM roofline), 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published (no sparsity)
CSRC = os.path.join(ROOT, "falcon_attention_kv_amd", "csrc")
# The sources each committed profile summary depends on.  A summary records the hash of
# its set (fields `sources:` and `kernel_source_sha256:`); it is current while that hash
# matches the tree (`profiles` in the output line), and the decode traffic it holds
# enters `roofline.traffic` only then.
PROFILE_SOURCES = {
    "attention": ["attn_bf16.hip", "lds_dma.h", "e4m3.h", "attn_launch.h"],
    "ar": ["attn_ar.hip", "attn_fp32.hip", "e4m3.h", "attn_launch.h"],
    "block": ["block.cpp", "block_kernels.hip", "gemm_bf16.hip", "block_launch.h", "lds_dma.h", "attn_bf16.hip",
              "e4m3.h", "attn_launch.h"],
    "probe": ["probe.hip"],
}
KERNEL_SRC = [os.path.join(CSRC, f) for f in PROFILE_SOURCES["attention"]]
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "rank_decode_serving_shape_pmc.txt")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-ar-step", action="store_true",
                   help="skip the secondary measurement of the autoregressive retrieval step")
    p.add_argument("--no-block", action="store_true",
                   help="skip the secondary measurement of the 12-layer transformer at the Table 2 shape")
    p.add_argument("--no-e4m3", action="store_true",
                   help="skip the secondary measurements on an E4M3 pool")
    p.add_argument("--no-long-history", action="store_true",
                   help="skip the secondary one-layer measurement of the long-history workload (D = 128)")
    p.add_argument("--probes", action="store_true",
                   help="instead of the serving step, run only the matrix-core and overlap probes")
    p.add_argument("--workloads", action="store_true",
                   help="instead of the serving step, time one layer's prefill and decode on every bf16 "
                        "workload, cold (a 512 MiB overwrite before each launch) and back to back")
    p.add_argument("--block-only", action="store_true",
                   help="instead of the serving step, run only the Table 2 transformer measurement "
                        "(3 timed passes after 1 warm-up; a short program for a kernel trace)")
    p.add_argument("--sweep-splits", action="store_true",
                   help="instead of the serving step, time the ranking decode and the retrieval step "
                        "one pass against split over the grids their split plans were set from")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="after timing, run 3 plain device copies of this many MiB (a known-size "
                        "reference for the HBM byte counters of a profiler run)")
    return p.parse_args()


def algorithmic(w, lens):
    """Algorithmic FLOPs and bytes of one prefill and one decode launch (one layer).

    Prefill: per (user, head) with N history rows, N(N+1)/2 allowed pairs, 4D FLOPs per
    pair (QK and PV); bytes read q, k, v and write o and the two pool rows: 6 N D e.
    Decode: k(N+1) allowed pairs per (user, head), 4D FLOPs each; bytes read the slot's
    K and V once (2 N D e) and the candidates' q, k, v and write o (4 k D e).
    """
    e = 2
    pf = sum(4 * w.D * N * (N + 1) // 2 for N in lens) * w.H
    pb = sum(6 * N * w.D * e for N in lens) * w.H
    df = sum(4 * w.D * w.k * (N + 1) for N in lens) * w.H
    db = sum((2 * N + 4 * w.k) * w.D * e for N in lens) * w.H
    return pf, pb, df, db


def ar_step(fa, W, torch, dev, w, lens, steps: int, warmup: int, pool_dtype=None):
    """The autoregressive retrieval step on the shape w: every user's slot holds lens[b]
    rows in each of the w.L layers; one step appends one token per (user, head) in every
    layer (w.L launches), the next step sees one row more.  Returns per-launch figures;
    algorithmic bytes per (user, head) are the slot's K and V rows read once (2 N D e,
    e the pool's element size) plus the token's q, k, v read and o and its two pool rows
    written (6 D e_act, counted at the activation size)."""
    pool_dtype = pool_dtype or w.dtype
    e = torch.tensor([], dtype=pool_dtype).element_size()   # bytes of one pool element
    ea = torch.tensor([], dtype=w.dtype).element_size()     # bytes of one activation element
    T = warmup + steps
    n_max = max(lens) + T
    pk, pv = W.random_pool(w.L, w.B, w.H, n_max, w.D, torch.float32 if pool_dtype != w.dtype else w.dtype,
                           seed=41, device=dev)
    pk, pv = pk.to(pool_dtype), pv.to(pool_dtype)
    pool = fa.Pool(pk, pv)
    tok = W.step_tokens(w.B, w.H, w.D, T, w.dtype, seed=42, device=dev)
    o = torch.empty_like(tok["q"][0])
    slots = torch.arange(w.B, dtype=torch.int32, device=dev)
    lens_t = [torch.as_tensor(lens, dtype=torch.int32, device=dev) + j for j in range(T)]
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for j in range(T):
        if j >= warmup:
            ev[2 * (j - warmup)].record(stream)
        for l in range(w.L):
            fa.ar_decode(tok["q"][j], tok["k"][j], tok["v"][j], pool, slots, lens_t[j], l, o=o)
        if j >= warmup:
            ev[2 * (j - warmup) + 1].record(stream)
    torch.cuda.synchronize()
    if pool.status() != 0:
        raise RuntimeError("the autoregressive step flagged an invalid slot or length")
    avg_ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / (steps * w.L)
    rows = sum(lens) + w.B * (warmup + (steps - 1) / 2)   # mean slot fill over the timed steps
    nbytes = (2 * rows * e + 6 * w.B * ea) * w.H * w.D
    gbs = nbytes / (avg_ms / 1e3) / 1e9
    ws_bytes = fa.ar_decode_workspace_bytes(pool, w.B)
    pool.close()
    del pk, pv
    return {"avg_ms": round(avg_ms, 5), "split_workspace_bytes": ws_bytes,
            "algorithmic_bytes_per_launch": int(nbytes), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tokens_per_s": round(w.B * w.H / (avg_ms / 1e3), 1),
            "shape": f"B={w.B} H={w.H} D={w.D} history {min(lens)}..{max(lens)}, {w.L} layer(s), "
                     f"{steps} timed steps"}


def one_request_decode(fa, W, torch, dev, H: int, D: int, N: int, k: int, launches: int = 20, warmup: int = 3,
                       e4m3: bool = False):
    """The ranking decode of a single request (B = 1, one layer): one user's history of N
    rows in its slot and k candidates, timed as the one-pass kernel and as the split over
    the history (rank_decode(split=True)), `launches` back-to-back launches each after
    `warmup`.  FLOPs per head 4 D k (N + 1); bytes per head the slot's K and V read once
    (2 N D e, e = 2 for a bf16 pool, 1 for an E4M3 pool) and the candidates' q, k, v, o
    (4 k D 2)."""
    if e4m3:
        pk, pv = W.random_pool(1, 1, H, N, D, torch.float32, seed=51, device=dev)
        pool = fa.Pool(pk.to(torch.float8_e4m3fn), pv.to(torch.float8_e4m3fn))
        del pk, pv
    else:
        pk, pv = W.random_pool(1, 1, H, N, D, torch.bfloat16, seed=51, device=dev)
        pool = fa.Pool(pk, pv)
    g = torch.Generator(device="cpu").manual_seed(52)
    qc, kc, vc = (torch.randn((1, H, k, D), generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
    oc = torch.empty_like(qc)
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    lens = torch.full((1,), N, dtype=torch.int32, device=dev)
    ws = torch.empty(max(fa.rank_decode_workspace_bytes(pool, 1, k), 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, split in (("one_pass", False), ("split", True)):
        for _ in range(warmup):
            fa.rank_decode(qc, kc, vc, pool, slot, lens, 0, oc=oc, split=split, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fa.rank_decode(qc, kc, vc, pool, slot, lens, 0, oc=oc, split=split, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / launches * 1e3
    if pool.status() != 0:
        raise RuntimeError("the one-request decode flagged an invalid slot or length")
    flop = 4.0 * D * k * (N + 1) * H
    nbytes = (2 * N * D * (1 if e4m3 else 2) + 4 * k * D * 2) * H
    out = {"shape": f"B=1 H={H} D={D} history {N} k={k}, one layer" + (", E4M3 pool" if e4m3 else ""),
           "split_workspace_bytes": fa.rank_decode_workspace_bytes(pool, 1, k)}
    for name, us in res.items():
        out[name] = {"avg_us": round(us, 2), "candidates_per_s": round(k / (us / 1e6), 1),
                     "tflops": round(flop / us / 1e6, 1), "gbs": round(nbytes / us / 1e3, 1)}
    out["split_speedup"] = round(res["one_pass"] / res["split"], 3)
    pool.close()
    return out


def serving_step_e4m3(fa, torch, dev, w, layers, lens, steps: int, warmup: int):
    """The serving-shape step of the headline (12 prefills, then 12 ranking decodes over
    the same layer inputs) with the pool stored as E4M3 codes.  Decode bytes per (user,
    head): the slot's K and V codes (2 N D) plus the candidates' bf16 q, k, v, o
    (4 k D 2)."""
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, torch.float8_e4m3fn, dev)
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    outs = [torch.empty_like(x["q"]) for x in layers]
    outc = [torch.empty_like(x["qc"]) for x in layers]
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup + steps):
        slots = torch.tensor(pool.acquire_many(w.B), dtype=torch.int32).pin_memory().to(dev, non_blocking=True)
        e = ev[i - warmup] if i >= warmup else None
        if e:
            e[0].record(stream)
        for l, x in enumerate(layers):
            fa.prefill(x["q"], x["k"], x["v"], lens_d, pool, slots, l, o=outs[l])
        if e:
            e[1].record(stream)
        for l, x in enumerate(layers):
            fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens_d, l, oc=outc[l])
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    if pool.status() != 0:
        raise RuntimeError("a kernel flagged an invalid slot or length")
    pf = sum(e[0].elapsed_time(e[1]) for e in ev) / (steps * w.L)
    dc = sum(e[1].elapsed_time(e[2]) for e in ev) / (steps * w.L)
    step_ms = sum(e[0].elapsed_time(e[2]) for e in ev) / steps
    dbytes = sum((2 * N * 1 + 4 * w.k * 2) * w.D for N in lens) * w.H
    pool.close()
    return {"candidates_per_s": round(w.B * w.k / (step_ms / 1e3), 1), "step_ms": round(step_ms, 4),
            "prefill_avg_ms": round(pf, 5), "rank_decode_avg_ms": round(dc, 5),
            "rank_decode_bytes_per_launch": int(dbytes),
            "rank_decode_hbm_frac": round(dbytes / (dc / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}


def block_table2(fa, W, torch, dev, steps: int, warmup: int):
    """The 12-layer transformer around the attention at the Table 2 shape of the pages
    (B=8 requests, history 992, 656 candidates, 12 layers), width 512 = 8 heads x 64:
    the history forward that fills the pool and the ranking stage's candidate-only
    forward (the pages' "decode with KV reuse"), each timed over its 12 layers with HIP
    events.  FLOPs per layer: 24 M C^2 in the four projections (M hidden rows) plus the
    attention's 2 D N (N + 1) per (user, head) for the history, 4 D k (N + 1) for the
    candidates.  Each layer's LayerNorms are folded into its weights once, before the
    timing (fold_layernorm); the tuner then chooses per projection between the GEMM on
    the hidden state with the statistics applied in its epilogue and the LayerNorm
    kernel followed by the best plain GEMM."""
    L, B, n, K, H, D = 12, 8, 992, 656, 8, 64
    C = H * D
    ws = [fa.fold_layernorm(W.block_weights(C, torch.bfloat16, seed=300 + l, device=dev)) for l in range(L)]
    xh0 = W.block_inputs(B, n, C, torch.bfloat16, seed=298, device=dev)
    xc0 = W.block_inputs(B, K, C, torch.bfloat16, seed=299, device=dev)
    xh, xc = xh0.clone(), xc0.clone()
    pool = fa.Pool.allocate(L, B, H, n, D, torch.bfloat16, dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    ctx = fa.BlockContext()
    work = torch.empty(max(fa.block_workspace_bytes(pool, B, n), fa.block_workspace_bytes(pool, B, K)),
                       dtype=torch.uint8, device=dev)
    ctx.tune(pool, B, n, work)   # choose the GEMM kernels for both shapes, before any timing
    ctx.tune(pool, B, K, work)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup + steps):
        xh.copy_(xh0)
        xc.copy_(xc0)
        e = ev[i - warmup] if i >= warmup else None
        if e:
            e[0].record(stream)
        for l in range(L):
            fa.block_forward(ctx, ws[l], fa.BLOCK_HISTORY, xh, pool, slots, lens, l, workspace=work)
        if e:
            e[1].record(stream)
        for l in range(L):
            fa.block_forward(ctx, ws[l], fa.BLOCK_CANDIDATES, xc, pool, slots, lens, l, workspace=work)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    if pool.status() != 0:
        raise RuntimeError("a block flagged an invalid slot or length")
    hist_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    cand_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    hist_flop = L * (24 * B * n * C * C + 2 * D * n * (n + 1) * B * H)
    cand_flop = L * (24 * B * K * C * C + 4 * D * K * (n + 1) * B * H)
    pool.close()
    ctx.close()
    return {"shape": "B=8 history 992 candidates 656, 12 layers, C=512 (H=8, D=64), bf16",
            "history_forward_ms": round(hist_ms, 4), "history_tflops": round(hist_flop / hist_ms / 1e9, 1),
            "candidate_forward_ms": round(cand_ms, 4), "candidate_tflops": round(cand_flop / cand_ms / 1e9, 1),
            "candidate_mfma_frac": round(cand_flop / cand_ms / 1e9 / BF16_PEAK_TFLOPS, 4)}


def layer_kernels(fa, W, torch, dev, w, lens, flush, launches: int = 10, warmup: int = 3):
    """One layer's prefill and rank decode of workload w with history lengths `lens`.
    Cold: before each launch the 512 MiB `flush` buffer is overwritten, so inputs and pool
    come from HBM, and HIP events bracket the launch alone (median reported).  Warm:
    `launches` back-to-back launches on the same inputs (mean reported)."""
    stream = torch.cuda.current_stream(dev)
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    x = W.layer_inputs(w, 0, dev)
    pool = fa.Pool.allocate(1, w.S, w.H, w.n, w.D, w.dtype, dev)
    slots = torch.tensor(pool.acquire_many(w.B), dtype=torch.int32, device=dev)
    o, oc = torch.empty_like(x["q"]), torch.empty_like(x["qc"])
    calls = {
        "prefill": lambda: fa.prefill(x["q"], x["k"], x["v"], lens_d, pool, slots, 0, o=o),
        "rank_decode": lambda: fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots, lens_d, 0, oc=oc),
    }
    pf, pb, df, db = algorithmic(w, lens)
    work = {"prefill": (pf, pb), "rank_decode": (df, db)}
    entry = {}
    for name, call in calls.items():
        for _ in range(warmup):
            call()
        cold = []
        for _ in range(launches):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            cold.append(e0.elapsed_time(e1))
        cold.sort()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            call()
        e1.record(stream)
        e1.synchronize()
        warm = e0.elapsed_time(e1) / launches
        flop, byts = work[name]
        t = cold[len(cold) // 2]
        entry[name] = {"cold_median_ms": round(t, 5), "warm_mean_ms": round(warm, 5),
                       "algorithmic_gflop": round(flop / 1e9, 3), "algorithmic_mb": round(byts / 1e6, 2),
                       "cold_tflops": round(flop / (t / 1e3) / 1e12, 1),
                       "cold_mfma_frac": round(flop / (t / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                       "cold_gbs": round(byts / (t / 1e3) / 1e9, 1),
                       "cold_hbm_frac": round(byts / (t / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    if pool.status() != 0:
        raise RuntimeError("a kernel flagged an invalid slot or length")
    pool.close()
    del x, o, oc
    return entry


def workload_kernels(fa, W, torch, dev, launches: int = 10, warmup: int = 3):
    """One layer's prefill and rank decode on each bf16 workload (the parity shapes and
    the serving shape's first layer), cold and warm (layer_kernels).  For the two ragged
    workloads the same launches also run with every history at full length, and the
    ragged/full time ratios are reported beside the ratios of the algorithmic FLOPs
    (decode: sum(len + 1) / (B (n + 1)); prefill: sum(len (len + 1)) / (B n (n + 1))) and
    bytes (the candidates' rows do not shrink with the history), with the roof that binds
    the full-length launch: a kernel whose time follows the real work, not the padded
    extent, matches the ratio of that roof."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {}
    for w in W.WORKLOADS[1:]:
        lens = W.history_lengths(w).tolist()
        entry = layer_kernels(fa, W, torch, dev, w, lens, flush, launches, warmup)
        if w.len_lo != w.len_hi:
            full = layer_kernels(fa, W, torch, dev, w, [w.n] * w.B, flush, launches, warmup)
            flen = [w.n] * w.B
            (pf, pb, df, db), (fpf, fpb, fdf, fdb) = algorithmic(w, lens), algorithmic(w, flen)
            entry["full_length"] = full
            ratios = {}
            for name, flop, byts, fflop, fbyts in (("prefill", pf, pb, fpf, fpb), ("rank_decode", df, db, fdf, fdb)):
                # the roof that binds the full-length launch decides which work ratio applies
                bound = "mfma" if fflop / BF16_PEAK_TFLOPS / 1e12 > fbyts / HBM_PEAK_GBS / 1e9 else "hbm"
                ratios[name] = {"cold": round(entry[name]["cold_median_ms"] / full[name]["cold_median_ms"], 4),
                                "flop_ratio": round(flop / fflop, 4), "byte_ratio": round(byts / fbyts, 4),
                                "bound": bound}
            entry["ragged_over_full"] = ratios
        res[w.name] = entry
    return res


def probes(torch, dev) -> dict:
    """The chip's achievable matrix-core rate, whether a SIMD overlaps matrix-core and
    exponential work (two waves per SIMD on every CU), and the LDS read rate of the
    attention tiles' two operand reads (16 waves per CU), from libunipin_probe.so."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "falcon_attention_kv_amd", "libunipin_probe.so"))
    lib.unipin_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.unipin_probe_overlap.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.unipin_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_double)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.empty(2 * cus * 512, dtype=torch.float32, device=dev)
    tf = ctypes.c_double()
    if lib.unipin_probe_mfma(buf.data_ptr(), cus, 20000, ctypes.byref(tf)) != 0:
        raise RuntimeError("unipin_probe_mfma failed")
    ns = (ctypes.c_double * 6)()
    if lib.unipin_probe_overlap(buf.data_ptr(), cus, 20000, ns) != 0:
        raise RuntimeError("unipin_probe_overlap failed")
    m, e, both, split, m16, both16 = (round(v, 2) for v in ns)
    lds = (ctypes.c_double * 2)()
    if lib.unipin_probe_lds(buf.data_ptr(), 2 * cus, 1000, cus, lds) != 0:
        raise RuntimeError("unipin_probe_lds failed")
    return {"mfma_loop": {"tflops": round(tf.value, 1), "frac_of_peak": round(tf.value / BF16_PEAK_TFLOPS, 4),
                          "what": f"{cus} CUs x 8 waves of independent 32x32x16 bf16 MFMAs"},
            "lds_read_bytes_per_ns_per_cu": {
                "ds_read_b128": round(lds[0], 1), "ds_read_b64_tr_b16": round(lds[1], 1),
                "what": f"{2 * cus} blocks of 8 waves (16 waves per CU), each wave 8 KiB per loop iteration in "
                        "reads that are 1 KiB (b128) or 512 B (tr_b64) in a row per instruction"},
            "mfma_exp_overlap_ns_per_iter": {
                "mfma_only": m, "exp_only": e, "both_in_each_wave": both, "mfma_wave_beside_exp_wave": split,
                "mfma_only_16x16x32": m16, "both_in_each_wave_16x16x32": both16,
                "what": "per SIMD and loop iteration, two waves: 8 MFMAs and/or 32 (v_exp_f32 + subtract) "
                        "per wave; full overlap would give max(mfma_only, exp_only), none their sum; the "
                        "16x16x32 entries issue the same matrix work as 16 MFMAs of 16x16x32 bf16"}}


def _best_us(fn, launches: int = 20, reps: int = 2) -> float:
    """Mean launch time of `launches` back-to-back calls, the best of `reps` runs."""
    import torch
    for _ in range(3):
        fn()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / launches * 1e3)
    return best


def sweep_splits(fa, W, torch, dev) -> dict:
    """The two split plans' choices over the grids they were set from: the ranking decode
    (1-8 requests of 8 heads at D = 64 and 16 at D = 128, histories 1024, 2048 and 4000,
    656-2048 candidates; only where the candidate tiles fill at most half the resident
    workgroups) and the retrieval step (1-16 requests, slots of 1024-8192 rows, bf16 and
    E4M3 pools).  Each entry gives whether the plan splits, the one-pass time and, where it
    splits, the split time and the ratio."""
    F8 = torch.float8_e4m3fn
    out = {"rank_decode": [], "ar_step": []}
    for D, H in ((64, 8), (128, 16)):
        for N in (1024, 2048, 4000):
            for B in (1, 2, 4, 8):
                for k in (656, 1000, 2048):
                    if B * H * ((k + 255) // 256) * 2 > (512 if D <= 64 else 256):
                        continue
                    pk, pv = W.random_pool(1, B, H, N, D, torch.bfloat16, seed=51, device=dev)
                    pool = fa.Pool(pk, pv)
                    g = torch.Generator(device="cpu").manual_seed(52)
                    qc, kc, vc = (torch.randn((B, H, k, D), generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
                    oc = torch.empty_like(qc)
                    slot = torch.arange(B, dtype=torch.int32, device=dev)
                    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
                    plan = fa.rank_decode_workspace_bytes(pool, B, k)
                    # the split entry point runs the one-pass kernel wherever the plan
                    # declines, so only the planned splits get a split time
                    one = _best_us(lambda: fa.rank_decode(qc, kc, vc, pool, slot, lens, 0, oc=oc))
                    entry = {"D": D, "H": H, "history": N, "requests": B, "candidates": k, "plan_splits": plan > 0,
                             "one_pass_us": round(one, 1)}
                    if plan:
                        ws = torch.empty(plan, dtype=torch.uint8, device=dev)
                        sp = _best_us(lambda: fa.rank_decode(qc, kc, vc, pool, slot, lens, 0, oc=oc, split=True,
                                                             workspace=ws))
                        entry.update(split_us=round(sp, 1), speedup=round(one / sp, 3))
                    out["rank_decode"].append(entry)
                    pool.close()
                    del pk, pv, qc, kc, vc, oc
    for fmt, D, H in (("bf16", 64, 8), ("bf16", 128, 16), ("e4m3", 64, 8), ("e4m3", 128, 16)):
        for n in (1024, 2048, 4096, 8192):
            for B in (1, 4, 8, 16):
                if fmt == "e4m3":
                    pk, pv = W.random_pool(1, B, H, n, D, torch.float32, seed=61, device=dev)
                    pool = fa.Pool(pk.to(F8), pv.to(F8))
                else:
                    pk, pv = W.random_pool(1, B, H, n, D, torch.bfloat16, seed=61, device=dev)
                    pool = fa.Pool(pk, pv)
                del pk, pv
                tok = W.step_tokens(B, H, D, 1, torch.bfloat16, seed=62, device=dev)
                q, k, v = tok["q"][0], tok["k"][0], tok["v"][0]
                o = torch.empty_like(q)
                slot = torch.arange(B, dtype=torch.int32, device=dev)
                lens = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
                plan = fa.ar_decode_workspace_bytes(pool, B)
                one = _best_us(lambda: fa.ar_decode(q, k, v, pool, slot, lens, 0, o=o, split=False))
                entry = {"pool": fmt, "D": D, "H": H, "slot_rows": n, "requests": B, "plan_splits": plan > 0,
                         "one_pass_us": round(one, 1)}
                if plan:
                    ws = torch.empty(plan, dtype=torch.uint8, device=dev)
                    sp = _best_us(lambda: fa.ar_decode(q, k, v, pool, slot, lens, 0, o=o, workspace=ws))
                    entry.update(split_us=round(sp, 1), speedup=round(one / sp, 3))
                out["ar_step"].append(entry)
                pool.close()
    return out


def copy_calibration(torch, dev, mib: int) -> int:
    """Three plain device copies of `mib` MiB: a known-size reference for the HBM byte
    counters of a profiler run.  Returns the bytes one copy reads."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return n * 4


def hbm_copy_reference(torch, dev, mib: int = 1024, launches: int = 10) -> dict:
    """What a plain device copy reaches on this GPU: `launches` copies of `mib` MiB, timed
    with events, (bytes read + bytes written) / time.  Context for the roofline fractions,
    which are taken against the published 8 TB/s."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / launches
    gbs = 2 * n * 4 / (ms / 1e3) / 1e9
    del src, dst
    return {"bytes_read_plus_written": 2 * n * 4, "avg_ms": round(ms, 4), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def source_hash(kind: str) -> str:
    """sha256[:16] over the sources of PROFILE_SOURCES[kind], in order."""
    h = hashlib.sha256()
    for name in PROFILE_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash("attention")


def summary_fields(path: str) -> dict:
    """The `key: value` lines of a profile summary (comment lines start with '#')."""
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    return fields


def profile_status() -> dict:
    """Every committed profile summary with the source set it was taken on and whether
    that set is unchanged since."""
    out = {}
    for name in sorted(os.listdir(PROFILES)):
        try:
            fields = summary_fields(os.path.join(PROFILES, name))
            kind = fields.get("sources")
            out[name] = {"sources": kind,
                         "current": bool(kind in PROFILE_SOURCES and
                                         fields.get("kernel_source_sha256") == source_hash(kind))}
        except OSError:
            out[name] = {"sources": None, "current": False}
    return out


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different kernel source."""
    try:
        fields = summary_fields(PMC_SUMMARY)
        if fields.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, layers_cpu, lens, budget_s):
    """The oracle, as it stands, on (layer, user, head) units of the step until the budget
    is spent; scaled to candidates/s of a whole step."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    rng = np.random.default_rng(0)
    units, t_pre, t_dec = 0, 0.0, 0.0
    while t_pre + t_dec < budget_s and units < w.L * w.B * w.H:
        l, b, h = int(rng.integers(w.L)), int(rng.integers(w.B)), int(rng.integers(w.H))
        x = layers_cpu[l]
        N = lens[b]
        t0 = time.perf_counter()
        oracle.prefill(x["q"][b:b + 1, h:h + 1], x["k"][b:b + 1, h:h + 1], x["v"][b:b + 1, h:h + 1], [N])
        t1 = time.perf_counter()
        pk = oracle.as_f64(x["k"][b:b + 1, h:h + 1, :N]).reshape(1, 1, 1, N, w.D)
        pv = oracle.as_f64(x["v"][b:b + 1, h:h + 1, :N]).reshape(1, 1, 1, N, w.D)
        oracle.rank_decode(x["qc"][b:b + 1, h:h + 1], x["kc"][b:b + 1, h:h + 1],
                           x["vc"][b:b + 1, h:h + 1], pk, pv, [0], [N], 0)
        t_pre += t1 - t0
        t_dec += time.perf_counter() - t1
        units += 1
    t_total = t_pre + t_dec
    per_unit = t_total / units
    step_s = per_unit * w.L * w.B * w.H
    # algorithmic FLOPs of one (layer, user, head) unit: prefill N(N+1)/2 pairs, decode
    # k(N+1) pairs, 4D FLOPs each (all lens are equal at this shape)
    N = lens[0]
    unit_flop = 4 * w.D * (N * (N + 1) // 2 + w.k * (N + 1))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": w.B * w.k / step_s, "unit": "candidates/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} (layer, user, head) units of prefill + rank decode "
                      f"(float64 numpy, {t_total:.1f} s), scaled x{w.L * w.B * w.H} to one step",
            "algorithmic_gflops": round(unit_flop / per_unit / 1e9, 2), "cpu_model": model,
            # the two oracle calls timed apart, per (layer, user, head) unit; the oracle
            # evaluates its dense masked blocks (N x N for the prefill, k x (N + k) for the
            # decode), this many times the algorithmic pairs
            "prefill_ms_per_unit": round(t_pre / units * 1e3, 3), "decode_ms_per_unit": round(t_dec / units * 1e3, 3),
            "dense_over_algorithmic": {"prefill": round(2 * N / (N + 1), 3),
                                       "decode": round((N + w.k) / (N + 1), 3)}}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one process drives one GPU here; --gpus must be 1 (sharding over GPUs is a design, not code)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import falcon_attention_kv_amd as fa
    import workloads as W

    w = W.WORKLOADS[3]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probes:
        print(json.dumps({"probes": probes(torch, dev)}), flush=True)
        return
    if args.sweep_splits:
        print(json.dumps({"sweep_splits": sweep_splits(fa, W, torch, dev)}), flush=True)
        return
    if args.block_only:
        print(json.dumps({"block_table2": block_table2(fa, W, torch, dev, steps=3, warmup=1)}), flush=True)
        return
    if args.workloads:
        out = {"workload_kernels": workload_kernels(fa, W, torch, dev)}
        if args.copy_calib_mib:
            out["copy_calibration_bytes"] = copy_calibration(torch, dev, args.copy_calib_mib)
        print(json.dumps(out), flush=True)
        return
    lens = W.history_lengths(w).tolist()
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    layers = [W.layer_inputs(w, l, dev) for l in range(w.L)]
    outs = [torch.empty_like(x["q"]) for x in layers]
    outc = [torch.empty_like(x["qc"]) for x in layers]
    pool = fa.Pool.allocate(w.L, w.S, w.H, w.n, w.D, w.dtype, dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        slots = torch.tensor(pool.acquire_many(w.B), dtype=torch.int32).pin_memory()
        slots_d = slots.to(dev, non_blocking=True)
        if events is not None:
            events[0].record(stream)
        for l, x in enumerate(layers):
            fa.prefill(x["q"], x["k"], x["v"], lens_d, pool, slots_d, l, o=outs[l])
        if events is not None:
            events[1].record(stream)
        for l, x in enumerate(layers):
            fa.rank_decode(x["qc"], x["kc"], x["vc"], pool, slots_d, lens_d, l, oc=outc[l])
        if events is not None:
            events[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Three HIP events per step on the launch stream: before the prefills, between the
    # prefills and the decodes, after the decodes.  A kernel's average launch time is its
    # span over the step divided by the 12 launches (launch gaps included).
    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(all_events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if pool.status() != 0:
        raise RuntimeError("a kernel flagged an invalid slot or length")

    pf_per_step = sorted(ev[0].elapsed_time(ev[1]) / w.L for ev in all_events)
    dc_per_step = sorted(ev[1].elapsed_time(ev[2]) / w.L for ev in all_events)
    pf_avg = sum(pf_per_step) / args.steps
    dc_avg = sum(dc_per_step) / args.steps

    def spread(xs):
        # per-launch time of the steps (each step's span / its 12 launches): median, p10, p90
        q = lambda f: xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]
        return {"median_ms": round(q(0.5), 5), "p10_ms": round(q(0.1), 5), "p90_ms": round(q(0.9), 5)}

    pflop, pbytes, dflop, dbytes = algorithmic(w, lens)
    ms_per_step = wall * 1e3 / args.steps
    cand_per_step = w.B * w.k
    value = cand_per_step / (ms_per_step / 1e3)
    step_tflops = w.L * (pflop + dflop) / (ms_per_step / 1e3) / 1e12

    dc_gbs = dbytes / (dc_avg / 1e3) / 1e9
    traffic = measured_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "12-layer serving shape: L=12 S=64 H=8 n=512 D=64, "
                               "64 requests x k=1000 candidates, bf16",
                   "L": w.L, "S": w.S, "B": w.B, "H": w.H, "n": w.n, "D": w.D, "k": w.k},
        "tflops": round(step_tflops, 2),
        "roofline": {"bound": "hbm", "achieved": round(dc_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dc_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "rank_decode (one layer, 64 users x 8 heads)",
                     "algorithmic_bytes_per_launch": dbytes,
                     "avg_launch_ms": round(dc_avg, 5)},
        "kernels": {
            "prefill": {"avg_ms": round(pf_avg, 5), "per_step": spread(pf_per_step),
                        "tflops": round(pflop / (pf_avg / 1e3) / 1e12, 2),
                        "gbs": round(pbytes / (pf_avg / 1e3) / 1e9, 1),
                        "hbm_frac": round(pbytes / (pf_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_frac": round(pflop / (pf_avg / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "rank_decode": {"avg_ms": round(dc_avg, 5), "per_step": spread(dc_per_step),
                            "tflops": round(dflop / (dc_avg / 1e3) / 1e12, 2),
                            "gbs": round(dc_gbs, 1), "hbm_frac": round(dc_gbs / HBM_PEAK_GBS, 4),
                            "mfma_frac": round(dflop / (dc_avg / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                            "decode_candidates_per_s": round(cand_per_step / (w.L * dc_avg / 1e3), 1)},
        },
    }
    out["profiles"] = profile_status()
    if not args.no_block:
        out["block_table2"] = block_table2(fa, W, torch, dev, steps=5, warmup=2)
    if args.copy_calib_mib:
        out["copy_calibration_bytes"] = copy_calibration(torch, dev, args.copy_calib_mib)
    else:  # kept out of the counter runs, whose calibration picks the run's largest copies
        out["hbm_copy_reference"] = hbm_copy_reference(torch, dev)
        out["probes"] = probes(torch, dev)
    if not args.no_long_history:
        # the matrix-core-bound workload (D = 128, long ragged histories), one layer, cold
        wl = W.WORKLOADS[4]
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        lh = layer_kernels(fa, W, torch, dev, wl, W.history_lengths(wl).tolist(), flush, launches=5, warmup=2)
        del flush
        out["long_history"] = {"workload": wl.name, **lh}
    if not args.no_cpu_baseline:
        layers_cpu = [{k: v.cpu() for k, v in x.items()} for x in layers]
        out["cpu_baseline"] = cpu_baseline(w, layers_cpu, lens, args.cpu_seconds)
    if not args.no_e4m3:
        pool.close()
        e8 = {"serving_step": serving_step_e4m3(fa, torch, dev, w, layers, lens, steps=10, warmup=3)}
        wl4 = W.WORKLOADS[4]
        e8["ar_step_serving_shape"] = ar_step(fa, W, torch, dev, w, lens, steps=8, warmup=2,
                                             pool_dtype=torch.float8_e4m3fn)
        e8["ar_step_long_history"] = ar_step(fa, W, torch, dev, wl4, W.history_lengths(wl4).tolist(), steps=8,
                                            warmup=2, pool_dtype=torch.float8_e4m3fn)
        out["e4m3_pool"] = e8
    if not args.no_ar_step:
        del layers, outs, outc
        pool.close()
        wl = W.WORKLOADS[4]
        out["ar_step"] = {
            "serving_shape": ar_step(fa, W, torch, dev, w, lens, steps=8, warmup=2),
            "long_history": ar_step(fa, W, torch, dev, wl, W.history_lengths(wl).tolist(), steps=8, warmup=2),
            "one_request_long_history": ar_step(fa, W, torch, dev, replace(wl, B=1, S=1), [4000], steps=8,
                                                warmup=2),
        }
        # the ranking side of a single request, one-pass against split over the history
        out["rank_decode_one_request"] = {
            "serving_shape": one_request_decode(fa, W, torch, dev, H=w.H, D=w.D, N=w.n, k=w.k),
            "long_history": one_request_decode(fa, W, torch, dev, H=wl.H, D=wl.D, N=4000, k=wl.k),
            "long_history_e4m3": one_request_decode(fa, W, torch, dev, H=wl.H, D=wl.D, N=4000, k=wl.k, e4m3=True),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
