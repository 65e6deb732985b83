"""Verify-step benchmark on one MI355X.

One step = the whole verify hot path over one batch of synthetic input
(mtp_verify_step): the split-K verify-attention partial kernel, then one
launch running the combine beside greedy acceptance and KV commit.  Inputs
are resident in HBM before timing.
Cold-cache by default: the KV page pool is replicated R times (R * KV >= 1 GB,
well above the 256 MB Infinity Cache) and step i reads replica i % R.

Prints ONE JSON line.  `value` is committed-KV GB/s of the whole step;
`roofline` is the split-K partial kernel's algorithmic bytes per launch over
its mean duration from HIP events recorded around each launch in the timed
region; `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from speculative_decoding_verify_mtp_amd import inputs as I  # noqa: E402
from speculative_decoding_verify_mtp_amd import lib  # noqa: E402

HBM_PEAK_GBS = 8000.0
# The headline: the 64-sequence ragged batch (4.9 GB of paged KV), the largest
# workload and the one whose step is bound by HBM bandwidth.
DEFAULT_WORKLOAD = "ragged_batch"
# The first launches of a process over a multi-GB pool run slower, and not
# only the first few: on the ragged batch (kernel trace) launches 0-20 take
# 0.94-1.22 ms, 20-40 about 0.90-0.94 ms, and the partial kernel settles near
# 0.87-0.89 ms only after about 150 ms of work (clocks and page-table / TLB
# warm-up).  So at least MIN_WARMUP_STEPS untimed steps run first, and the
# untimed steps continue until MIN_WARMUP_SECONDS of them have run.
MIN_WARMUP_STEPS = 24
MIN_WARMUP_SECONDS = 0.5
# Bytes that stay resident between two reads of one KV replica only if they
# fit the 256 MB Infinity Cache; a step whose replicas exceed it reads cold.
MALL_BYTES = 256 << 20
# The partial kernels and their launch plan: traffic counters taken on other
# sources are not reported.
KERNEL_SOURCES = ["attn_lds.hpp", "attn_mfma.hpp", "attn_stream.hpp", "attn_valu.hpp",
                  "common.hpp", "plan.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_decoding_verify_mtp_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def elem_bytes(wl: I.Workload) -> int:
    return 4 if wl.dtype == "f32" else 2


def algorithmic_bytes(wl: I.Workload, ctx: np.ndarray) -> dict:
    """Bytes the method must move per step (not what the kernels happen to move)."""
    e = elem_bytes(wl)
    B, W, Hq, Hkv, D = wl.B, wl.W, wl.Hq, wl.Hkv, wl.D
    kv = int(np.sum(ctx.astype(np.int64))) * Hkv * D * 2 * e
    q = B * W * Hq * D * e
    new_kv = B * W * Hkv * D * 2 * e
    out = B * W * Hq * D * 4 + B * W * Hq * 4
    table = int(np.sum((ctx.astype(np.int64) + 15) // 16)) * 4
    logits = B * W * wl.vocab * 4
    return dict(kv=kv, partial=kv + q + new_kv + table, step=kv + q + new_kv + out + table + logits)


def traffic_from_profile(workload: str, launch_bytes: int) -> float | None:
    """HBM bytes per partial launch from the committed rocprofv3 counter summary,
    scaled by the copy-kernel calibration, if it was taken on the current kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return float(rec["bytes_per_launch"])


PARTIAL_KERNELS = ("attn_partial_lds", "attn_partial_stream", "attn_partial_mfma",
                   "attn_partial_valu")


def _median_counter(csv_dir: str, counter: str, match) -> tuple[float, int]:
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} values for the kernel under {csv_dir}")
    return float(np.median(vals)), len(vals)


def write_traffic(workload: str, ctr_dir: str) -> int:
    """profiles/traffic_<workload>.json from two rocprofv3 --pmc runs of the
    bench (FETCH_SIZE, WRITE_SIZE) and the same two counters of the copy
    calibration kernel, under ctr_dir/{<workload>,copy}_{FETCH_SIZE,WRITE_SIZE}.
    Runs on the CPU."""
    is_partial = lambda name: any(k in name for k in PARTIAL_KERNELS)  # noqa: E731
    is_copy = lambda name: "copyBuffer" in name  # the runtime's device-to-device copy  # noqa: E731
    fetch, nf = _median_counter(os.path.join(ctr_dir, f"{workload}_FETCH_SIZE"), "FETCH_SIZE",
                                is_partial)
    write, nw = _median_counter(os.path.join(ctr_dir, f"{workload}_WRITE_SIZE"), "WRITE_SIZE",
                                is_partial)
    cf, _ = _median_counter(os.path.join(ctr_dir, "copy_FETCH_SIZE"), "FETCH_SIZE", is_copy)
    cw, _ = _median_counter(os.path.join(ctr_dir, "copy_WRITE_SIZE"), "WRITE_SIZE", is_copy)
    copy_kib = 512e6 / 1024
    ff, fw = copy_kib / cf, copy_kib / cw
    steps = "--steps 3 --warmup 1" if workload == "ragged_batch" else "--steps 100 --warmup 2"
    rec = {
        "workload": workload, "kernel": "partial kernel of the step",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": fetch, "write_size_kib_per_dispatch": write,
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": 512000000, "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
        "fetch_bytes_per_launch": int(fetch * 1024 * ff),
        "write_bytes_per_launch": int(write * 1024 * fw),
        "bytes_per_launch": int(fetch * 1024 * ff + write * 1024 * fw),
        "commands": [
            f"timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d {ctr_dir}/{t}_{c} -o run "
            f"-- python3 bench.py " + (f"--workload {workload} {steps} --no-cpu-baseline"
                                      if t == workload else "--copy-calibration 512")
            for t in (workload, "copy") for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
            f"python3 bench.py --write-traffic {workload} --ctr-dir {ctr_dir}"],
        "note": "medians over dispatches of the partial kernel; the copy kernel moves 512 MB "
                "each way, so factor = 500000 KiB / counter reading",
    }
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"wrote": f"profiles/traffic_{workload}.json",
                      "bytes_per_launch": rec["bytes_per_launch"]}))
    return 0


def _oracle_steps(wl: I.Workload, seed: int, budget_s: float, threads: int) -> dict:
    """Whole oracle steps (attention + acceptance + commit) on a bounded sample
    of the workload, repeated for about budget_s with `threads` BLAS threads."""
    from threadpoolctl import threadpool_limits

    from oracle import verify_oracle as O

    sample = wl if wl.B <= 4 else wl.scaled(B=4)  # bounded sample: at most 4 sequences
    inp = I.make_inputs(sample, seed, device="cpu")
    host = inp["host"]
    f64 = lambda t: t.double().numpy()  # noqa: E731
    q, kc, vc = f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"])
    kn, vn = f64(inp["k_new"]), f64(inp["v_new"])
    logits = inp["logits"].numpy()
    steps = 0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        while True:
            O.verify_attention(q, kc, vc, host["block_table"], host["ctx_lens"], kn, vn,
                               host["mask_kind"], host["mask_ids"], inp["scale"], wl.seg_lookback)
            n, path, _ = O.accept(logits, host["draft_ids"], host["mask_kind"], host["mask_ids"])
            O.kv_commit(kc, vc, kn, vn, n, path, host["block_table"], host["ctx_lens"])
            steps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    kv = algorithmic_bytes(sample, host["ctx_lens"])["kv"]
    return {"value": kv * steps / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole oracle steps of {sample.B} sequence(s) of {wl.name} "
                      f"(ctx {host['ctx_lens'].tolist()}) in {dt:.1f} s, fp64 numpy"}


def host_cores() -> int:
    """Cores this process may run on (its affinity mask), at most 16: the
    share of the host one GPU's job gets."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # not Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl: I.Workload, seed: int, budget_s: float) -> dict:
    """The fp64 oracle on the host cores: its matmuls and reductions run on a
    BLAS pool of one thread per core of this process's affinity mask; the
    paged-cache gather into dense arrays is a single-threaded Python loop."""
    rec = _oracle_steps(wl, seed, budget_s, host_cores())
    rec["note"] = ("cores = BLAS threads (the affinity mask, at most 16); the oracle's gather "
                   "of the paged cache into dense fp64 arrays is single-threaded")
    return rec


def timed_graph(launch, steps: int, warmup: int) -> float:
    """Milliseconds per launch of `launch()`, from HIP events around replays of
    a graph that holds 100 launches."""
    launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    n = 100
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for _ in range(n):
                launch()
    torch.cuda.synchronize()
    for _ in range(max(1, warmup // n)):
        g.replay()
    reps = max(1, steps // n)
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    z.record()
    torch.cuda.synchronize()
    return a.elapsed_time(z) / (reps * n)


def bench_accept_hybrid(wl: I.Workload, inp: dict, args) -> int:
    """Confidence / hybrid acceptance on its own: one launch per step over the
    batch, with the verifier logits (hybrid) and without (confidence only).
    Algorithmic bytes: the logits rows read (W - 1 drafter rows, plus W
    verifier rows when given) and the int32 inputs and outputs."""
    B, W, V = inp["draft_logits"].shape
    out = [torch.empty(B, dtype=torch.int32, device="cuda"),
           torch.empty((B, W), dtype=torch.int32, device="cuda"),
           torch.empty(B, dtype=torch.int32, device="cuda"),
           torch.empty(B, dtype=torch.int32, device="cuda")]
    res = {}
    for name, logits in (("hybrid", inp["logits"]), ("confidence_only", None)):
        def launch(logits=logits):
            lib.accept_hybrid(inp["draft_logits"], logits, inp["draft_ids"], inp["mask_kind"],
                              inp["mask_ids"], args.tau, args.min_prefix, accept_len=out[0],
                              accept_path=out[1], bonus_id=out[2], conf_len=out[3])
        ms = timed_graph(launch, args.steps, args.warmup)
        rows = (W - 1) + (W if logits is not None else 0)
        nbytes = B * (rows * V * 4 + W * 4 * 3 + 1 + 4 * 3)
        res[name] = {"us": round(ms * 1e3, 3), "bytes": nbytes,
                     "GBs": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    if lib.device_status(clear=True) != 0:
        print("bench.py: the device reported a data error", file=sys.stderr)
        return 3
    h = res["hybrid"]
    rec = {
        "metric": "hybrid acceptance launches/s at 1 GPU (confidence prefix + greedy fallback)",
        "value": round(1e6 / h["us"], 1), "unit": "launches/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["us"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded drafter and verifier logits)",
        "config": {"workload": wl.name, "B": B, "W": W, "V": V, "tau": args.tau,
                   "min_prefix": args.min_prefix},
        "roofline": {"bound": "hbm", "achieved": h["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(h["GBs"] / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "accept_hybrid_kernel", "kernel_us": h["us"],
                     "algorithmic_bytes": h["bytes"]},
        "confidence_only": res["confidence_only"],
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def nested_kv_bytes(wl: I.Workload, ctx: np.ndarray, kv8_recent: int) -> int:
    """Committed K + V bytes a nested-cache read must move: per token and KV
    head, D/2 base bytes and a 4-byte scale per tensor, plus D/2 refinement
    bytes for tokens read in KV8."""
    ctx = ctx.astype(np.int64)
    n8 = ctx if kv8_recent < 0 else np.minimum(ctx, kv8_recent)
    per_tensor = int(np.sum(ctx)) * (wl.D // 2 + 4) + int(np.sum(n8)) * (wl.D // 2)
    return per_tensor * wl.Hkv * 2


def bench_nested_attn(wl: I.Workload, inp: dict, args) -> int:
    """Verify attention over the nested cache: the bf16 pool (replicated for a
    cold cache, as for the step) is quantized once, untimed; then graphs of
    R partial-kernel launches and of R whole attentions are replayed."""
    host = inp["host"]
    ctx = host["ctx_lens"]
    if wl.D != 128 or wl.dtype != "bf16":
        print("bench.py: the nested cache is built for bf16 heads of 128", file=sys.stderr)
        return 2
    nb = algorithmic_bytes(wl, ctx)
    kvb = nested_kv_bytes(wl, ctx, args.kv8_recent)
    part_bytes = nb["partial"] - nb["kv"] + kvb
    pool = inp["k_cache"].shape[0]
    R = 1 if args.warm else (args.replicas or max(1, math.ceil(1.0e9 / max(kvb, 1))))
    R = min(R, max(1, (2**31 - 1) // pool))
    kv = lib.NestedKV(pool * R, wl.Hkv, wl.D)
    for r in range(R):
        slots = torch.arange(pool * 16, dtype=torch.int32, device="cuda") + r * pool * 16
        lib.kv_quantize(inp["k_cache"].reshape(pool * 16, wl.Hkv, wl.D),
                        inp["v_cache"].reshape(pool * 16, wl.Hkv, wl.D), slots, kv)
    bt = inp["block_table"]
    tables = [torch.where(bt >= 0, bt + r * pool, bt).contiguous() for r in range(R)]
    del inp["k_cache"], inp["v_cache"]
    mc = int(ctx.max())
    B, W, Hq, D = inp["q"].shape
    shape = lib.VerifyShape(B, W, Hq, wl.Hkv, D, pool * R, bt.shape[1], mc, lib.MTP_BF16,
                            inp["scale"], wl.seg_lookback, args.split_tokens)
    ws = torch.empty(max(lib.nested_workspace_bytes(shape), 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, W, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, W, Hq), dtype=torch.float32, device="cuda")

    def run(r, phase):
        lib.verify_attn_nested(inp["q"], kv, tables[r], inp["ctx_lens"], inp["k_new"],
                               inp["v_new"], inp["mask_kind"], inp["mask_ids"],
                               kv8_recent=args.kv8_recent, out=out, lse=lse, workspace=ws,
                               shape=shape, phase=phase)

    res = {}
    for phase in ("both", "partial"):
        for r in range(R):
            run(r, phase)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for r in range(R):
                    run(r, phase)
        torch.cuda.synchronize()
        reps = max(1, math.ceil(args.steps / R))
        tw = time.perf_counter()
        for _ in range(max(1, math.ceil(args.warmup / R))):
            g.replay()
        torch.cuda.synchronize()
        while time.perf_counter() - tw < MIN_WARMUP_SECONDS:  # until the clocks have settled
            for _ in range(4):
                g.replay()
            torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        z.record()
        torch.cuda.synchronize()
        res[phase] = a.elapsed_time(z) / (reps * R)
    if lib.device_status(clear=True) != 0:
        print("bench.py: the device reported a data error", file=sys.stderr)
        return 3
    ms, pms = res["both"], res["partial"]
    achieved = part_bytes / (pms * 1e-3) / 1e9
    mode = {-1: "KV8"}.get(args.kv8_recent, "KV4" if args.kv8_recent == 0
                           else f"Recent-{args.kv8_recent}")
    rec = {
        "metric": "nested-KV verify attention: committed KV GB/s at 1 GPU; % of HBM roofline",
        "value": round(kvb / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": reps * R, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q quantized to nested KV4/KV8 planes)",
        "config": {"workload": wl.name, "B": wl.B, "W": wl.W, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "D": wl.D, "ctx": [int(ctx.min()), int(ctx.max())], "read": mode,
                   "kv_replicas": R, "cache": "warm" if R == 1 else "cold"},
        "kv_bytes_per_step": kvb,
        "bf16_kv_bytes_same_tokens": nb["kv"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_partial_nested", "kernel_us": round(pms * 1e3, 3),
                     "algorithmic_bytes": part_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_tree(wl: I.Workload, args) -> int:
    """The dynamic tree builder on its own: B sequences of the workload, K = 8
    probed depths over its vocabulary, a block of its width with 4 mask rows.
    Algorithmic bytes: the probability rows read plus the int32 outputs."""
    K, n_mask = 8, min(4, wl.W - 1)
    tin = I.make_tree_inputs(wl.B, K, wl.vocab, I.workload_seed(wl.name), device="cuda")

    B, W = wl.B, wl.W
    out = tuple(torch.empty(sz, dtype=torch.int32, device="cuda")
                for sz in ((B, W), (B, W), (B, W), (B,)))
    ws = torch.empty(B * K * W * 8 + 1024, dtype=torch.uint8, device="cuda")

    def launch():
        lib.build_tree(tin["probs"], tin["root"], wl.W, n_mask, workspace=ws, out=out)

    ms = timed_graph(launch, args.steps, args.warmup)
    nbytes = wl.B * (K * wl.vocab * 4 + 4 + wl.W * 12 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "dynamic tree builds/s at 1 GPU", "value": round(1e3 / ms, 1),
        "unit": "launches/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded heavy-tailed drafter probabilities)",
        "config": {"workload": wl.name, "B": wl.B, "K": K, "V": wl.vocab, "W": wl.W,
                   "n_mask": n_mask},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "tree_build_kernel", "kernel_us": round(ms * 1e3, 3),
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_loop(wl: I.Workload, args) -> int:
    """A device-resident decode loop: N dependent steps (block positions, then
    the verify step reading the context lengths the previous commit wrote)
    replayed from one graph (with a reset of the first context buffer at its
    head), against the same N steps launched eagerly.  Warm cache (the loop
    rereads one pool)."""
    N = args.loop_steps
    wl = wl.scaled(commit_steps=N + 1)
    seed = I.workload_seed(wl.name)
    base = I.make_inputs(wl, seed, device="cuda")
    steps = [I.make_inputs(wl, seed + 1000 * (k + 1), device="cuda") for k in range(N)]
    bt, kc, vc = base["block_table"], base["k_cache"], base["v_cache"]
    ctx0 = base["ctx_lens"].clone()
    ctx = [base["ctx_lens"].clone(), torch.empty_like(ctx0)]
    mc = int(base["host"]["ctx_lens"].max()) + N * wl.W
    shape = lib.shape_of(steps[0]["q"], kc, bt, max_ctx_len=mc, scale=base["scale"],
                         seg_lookback=wl.seg_lookback)
    ws = torch.empty(max(lib.workspace_bytes(shape), 16), dtype=torch.uint8, device="cuda")
    B, W, Hq, D = steps[0]["q"].shape
    out = torch.empty((B, W, Hq, D), device="cuda")
    lse = torch.empty((B, W, Hq), device="cuda")
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    apath = torch.empty((B, W), dtype=torch.int32, device="cuda")
    bonus = torch.empty(B, dtype=torch.int32, device="cuda")
    pos = torch.empty((B, W), dtype=torch.int32, device="cuda")

    def loop():
        ctx[0].copy_(ctx0)
        for k in range(N):
            s = steps[k]
            cin, cout = ctx[k % 2], ctx[(k + 1) % 2]
            lib.block_positions(cin, s["mask_kind"], s["mask_ids"], positions=pos)
            lib.verify_step(s["q"], kc, vc, bt, cin, s["k_new"], s["v_new"], s["mask_kind"],
                            s["mask_ids"], s["logits"], s["draft_ids"], out=out, lse=lse,
                            accept_len=alen, accept_path=apath, bonus_id=bonus,
                            ctx_lens_out=cout, workspace=ws, shape=shape)

    loop()
    torch.cuda.synchronize()
    reps = max(1, args.steps // N)
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        loop()
    z.record()
    torch.cuda.synchronize()
    eager_ms = a.elapsed_time(z) / (reps * N)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            loop()
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup // N)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        g.replay()
    z.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    graph_ms = a.elapsed_time(z) / (reps * N)
    if lib.device_status(clear=True) != 0:
        print("bench.py: the device reported a data error", file=sys.stderr)
        return 3
    kvb = algorithmic_bytes(wl, base["host"]["ctx_lens"])["kv"]
    rec = {
        "metric": "device-resident decode loop: verify steps/s at 1 GPU",
        "value": round(1e3 / graph_ms, 1), "unit": "steps/s", "n_gpus": 1,
        "steps": reps * N, "warmup": args.warmup, "ms_per_step": round(graph_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; a different block per step, one pool)",
        "config": {"workload": wl.name, "B": wl.B, "W": wl.W, "loop_steps": N, "cache": "warm"},
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_wall_ms_per_step": round((t1 - t0) * 1e3 / (reps * N), 5),
        "kv_GBs_first_step": round(kvb / (graph_ms * 1e-3) / 1e9, 1),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(I.WORKLOADS))
    ap.add_argument("--seg-lookback", type=int, default=None)
    ap.add_argument("--replicas", type=int, default=0, help="KV pool replicas (0 = auto, >= 1 GB)")
    ap.add_argument("--warm", action="store_true", help="one replica (cache-warm numbers)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--linear-pages", action="store_true",
                    help="identity page order instead of the shuffled pool (comparison only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only time a plain device copy of MB megabytes (HBM reference and "
                         "the FETCH_SIZE/WRITE_SIZE calibration kernel), then exit")
    ap.add_argument("--kernel", default="step",
                    choices=["step", "accept_hybrid", "nested_attn", "tree", "loop"],
                    help="step: the whole verify step (default); accept_hybrid: only the "
                         "confidence/hybrid acceptance kernel; nested_attn: verify attention "
                         "over the nested KV4/KV8 cache; tree: the dynamic tree builder for "
                         "the workload's B and W (K = 8 probed depths, 4 mask rows); loop: "
                         "--loop-steps dependent steps (positions + verify step, each step's "
                         "context lengths from the previous commit) in one graph vs eager")
    ap.add_argument("--loop-steps", type=int, default=8)
    ap.add_argument("--kv8-recent", type=int, default=-1,
                    help="nested_attn: -1 all KV8, 0 all KV4, N the N newest tokens in KV8")
    ap.add_argument("--tau", type=float, default=0.9)
    ap.add_argument("--min-prefix", type=int, default=2)
    ap.add_argument("--write-traffic", metavar="WORKLOAD", default=None,
                    help="only write profiles/traffic_WORKLOAD.json from rocprofv3 counter "
                         "CSVs under --ctr-dir (no GPU needed), then exit")
    ap.add_argument("--ctr-dir", default=None,
                    help="directory holding the counter runs (required with --write-traffic)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.write_traffic:
        if not args.ctr_dir:
            ap.error("--write-traffic needs --ctr-dir")
        return write_traffic(args.write_traffic, args.ctr_dir)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the verify step is measured on one GPU (its share of a sharded "
              "batch is the same kernel at its own shape); --gpus must be 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * 1000 * 1000
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        z.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(z) / reps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                          "read_plus_write_GBs": 2 * n / ms / 1e6}), flush=True)
        return 0

    wl = I.WORKLOADS[args.workload]
    if args.linear_pages:
        wl = wl.scaled(shuffle_pages=False)
    if args.seg_lookback is not None:
        wl = wl.scaled(seg_lookback=args.seg_lookback)
    seed = I.workload_seed(args.workload)
    inp = I.make_inputs(wl, seed, device=dev)
    if args.kernel == "accept_hybrid":
        return bench_accept_hybrid(wl, inp, args)
    if args.kernel == "nested_attn":
        return bench_nested_attn(wl, inp, args)
    if args.kernel == "tree":
        return bench_tree(wl, args)
    if args.kernel == "loop":
        return bench_loop(wl, args)
    host = inp["host"]
    ctx = host["ctx_lens"]
    nbytes = algorithmic_bytes(wl, ctx)
    pool = inp["k_cache"].shape[0]

    # cold-cache replicas of the page pool
    if args.warm:
        R = 1
    elif args.replicas > 0:
        R = args.replicas
    else:
        R = max(1, math.ceil(1.0e9 / max(nbytes["kv"], 1)))
    R = min(R, max(1, (2**31 - 1) // pool))
    k_all = inp["k_cache"].repeat(R, 1, 1, 1)
    v_all = inp["v_cache"].repeat(R, 1, 1, 1)
    bt = inp["block_table"]
    tables = [torch.where(bt >= 0, bt + r * pool, bt).contiguous() for r in range(R)]
    del inp["k_cache"], inp["v_cache"]

    max_ctx = int(ctx.max())
    shape = lib.shape_of(inp["q"], k_all, bt, max_ctx_len=max_ctx, scale=inp["scale"],
                         seg_lookback=wl.seg_lookback, split_tokens=args.split_tokens)
    workspace = torch.empty(max(lib.workspace_bytes(shape), 16), dtype=torch.uint8, device=dev)
    B, W, Hq, D = inp["q"].shape
    out = torch.empty((B, W, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, W, Hq), dtype=torch.float32, device=dev)
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    apath = torch.empty((B, W), dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    ctx_out = torch.empty_like(inp["ctx_lens"])

    def launch_step(r: int, partial_only: bool = False):
        common = (inp["q"], k_all, v_all, tables[r], inp["ctx_lens"], inp["k_new"], inp["v_new"],
                  inp["mask_kind"], inp["mask_ids"])
        if partial_only:
            lib.verify_attn(*common, out=out, lse=lse, workspace=workspace, shape=shape,
                            phase="partial")
            return
        lib.verify_step(*common, inp["logits"], inp["draft_ids"], out=out, lse=lse,
                        accept_len=alen, accept_path=apath, bonus_id=bonus,
                        ctx_lens_out=ctx_out, workspace=workspace, shape=shape)

    # Steps are replayed from HIP graphs: one graph holds NG whole steps (step
    # j reads replica j % R; at least 4 steps, so that the host's graph launch
    # is not counted once per step when a single replica is already cold), a
    # tail graph the remaining steps % NG, so that exactly --steps steps are
    # timed.  A third graph holds NG partial-kernel launches alone, for the
    # per-launch duration of the dominant kernel.
    NG = max(R, 4)
    reps, tail = divmod(args.steps, NG)
    for r in range(R):  # eager warm-up (also loads the code objects)
        launch_step(r)
    torch.cuda.synchronize()
    g_step, g_part = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    g_tail = torch.cuda.CUDAGraph() if tail else None
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g_step, stream=cap):
            for j in range(NG):
                launch_step(j % R)
        if g_tail is not None:
            with torch.cuda.graph(g_tail, stream=cap):
                for j in range(tail):
                    launch_step(j % R)
        with torch.cuda.graph(g_part, stream=cap):
            for j in range(NG):
                launch_step(j % R, partial_only=True)
    torch.cuda.synchronize()

    warm_steps = max(args.warmup, MIN_WARMUP_STEPS)
    wreps = math.ceil(warm_steps / NG)
    tw = time.perf_counter()
    for _ in range(wreps):
        g_step.replay()
    torch.cuda.synchronize()
    while time.perf_counter() - tw < MIN_WARMUP_SECONDS:  # until the clocks have settled
        for _ in range(4):
            g_step.replay()
        wreps += 4
        torch.cuda.synchronize()
    # one event after each replay: per-replay step times give the spread
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(reps):
        g_step.replay()
        marks[i + 1].record()
    if g_tail is not None:
        g_tail.replay()
    marks[-1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms_events = marks[0].elapsed_time(marks[-1]) / args.steps
    per_replay = [marks[i].elapsed_time(marks[i + 1]) / NG for i in range(reps)]

    # dominant kernel: HIP events around replays of the partial-only graph
    preps = max(1, math.ceil(args.steps / NG))
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(math.ceil(warm_steps / NG)):  # the device is warm by now
        g_part.replay()
    p0.record()
    for _ in range(preps):
        g_part.replay()
    p1.record()
    torch.cuda.synchronize()
    if lib.device_status(clear=True) != 0:
        print("bench.py: the device reported a data error", file=sys.stderr)
        return 3

    sec_per_step = (t1 - t0) / args.steps
    partial_ms = p0.elapsed_time(p1) / (preps * NG)
    achieved = nbytes["partial"] / (partial_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(wl.name, nbytes["partial"])
    spread = None
    if per_replay:
        q = np.percentile(np.array(per_replay), [10, 50, 90])
        spread = {"p10": round(float(q[0]), 5), "median": round(float(q[1]), 5),
                  "p90": round(float(q[2]), 5), "replays": len(per_replay),
                  "steps_per_replay": NG}
    reference = achievable_bandwidth(dev, k_all)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, seed, args.cpu_seconds)
        if wl.B == 1:  # the single-sequence workloads: also one thread
            cpu["one_thread"] = _oracle_steps(wl, seed, args.cpu_seconds, 1)

    mask_desc = {"chain": "chain", "tree": "tree", "segment": f"segment(lookback={wl.seg_lookback})",
                 "mixed": "half chain, half tree"}[wl.masks]
    cold = R * nbytes["kv"] > MALL_BYTES
    rec = {
        "metric": "verify-step KV GB/s and W-token blocks/sec at 1 GPU; % of HBM roofline",
        "value": round(nbytes["kv"] / sec_per_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": R + wreps * NG,
        "warmup_requested": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) K/V/Q, paged KV, shuffled pages)",
        "config": {"workload": wl.name, "B": wl.B, "W": wl.W, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "D": wl.D, "ctx": [int(ctx.min()), int(ctx.max())], "mask": mask_desc,
                   "page_size": 16, "kv_replicas": R, "cache": "cold" if cold else "warm",
                   "split_tokens": args.split_tokens or "auto"},
        "blocks_per_s": round(wl.B / sec_per_step, 1),
        "ms_per_step_gpu_events": round(step_ms_events, 5),
        "ms_per_step_spread": spread,
        "timing": f"{args.steps} steps: {reps} HIP graph replays of {NG} steps (step j reads KV "
                  f"replica j % {R}) + a graph of {tail}, after {R} eager and {wreps * NG} graph-replayed "
                  f"untimed steps; "
                  f"wall clock around the timed replays; partial kernel from events around "
                  f"{preps} replays of a graph of {NG} partial launches",
        "kv_bytes_per_step": nbytes["kv"],
        "hbm_frac_step": round(nbytes["kv"] / sec_per_step / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "attn_partial (split-K verify attention)",
                     "kernel_us": round(partial_ms * 1e3, 3),
                     "algorithmic_bytes": nbytes["partial"],
                     "launches_timed": preps * NG},
        "achievable_bandwidth": reference,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def achievable_bandwidth(dev, pool: torch.Tensor) -> dict:
    """What plain streaming kernels reach on this device, as a reference beside
    the 8 TB/s peak: a one-pass 16-byte-load read of up to 4 GB of the KV pool
    (mtp_probe_stream_read, libmtpprobe.so) and a 1 GB device copy (torch's
    copy_, read + write)."""
    import ctypes

    from speculative_decoding_verify_mtp_amd import build as B

    probe = ctypes.CDLL(B.PROBE_LIB)
    probe.mtp_probe_stream_read.restype = ctypes.c_int32
    probe.mtp_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_void_p]
    flat = pool.view(-1)
    nbytes = min(flat.numel() * flat.element_size(), 4 << 30) // 16 * 16
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    strm = torch.cuda.current_stream().cuda_stream

    def read():
        if probe.mtp_probe_stream_read(flat.data_ptr(), nbytes, sink.data_ptr(), strm) != 0:
            raise RuntimeError("mtp_probe_stream_read failed")

    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
        read()
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    z.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * reps / (a.elapsed_time(z) * 1e-3) / 1e9
    a.record()
    for _ in range(reps):
        read()
    z.record()
    torch.cuda.synchronize()
    read_gbs = nbytes * reps / (a.elapsed_time(z) * 1e-3) / 1e9
    del src, dst
    return {"stream_read_GBs": round(read_gbs, 1), "stream_read_frac": round(read_gbs / HBM_PEAK_GBS, 4),
            "read_bytes": nbytes, "copy_read_plus_write_GBs": round(copy_gbs, 1),
            "note": "one-pass 16-byte-load read of the KV pool (libmtpprobe.so) and torch copy_ "
                    "of 1 GB, same process, HIP events; what plain streaming kernels reach, "
                    "not a peak"}


if __name__ == "__main__":
    sys.exit(main())
