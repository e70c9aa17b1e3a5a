#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify-and-resample step on one MI355X.

A step is one spec_verify_sample call over one batch of the headline
workload: sampling verify, B=64 requests, K=8 draft positions, V=128256,
bf16 logits, temperature 0.7 (target logits ~ N(0, 3^2), draft = target +
N(0, 0.5^2), tokens drawn from the tempered draft).  Inputs are synthetic,
seeded, resident in HBM before the timed region, and three independent input
sets are rotated so the 256 MB memory-side cache cannot hold a step's inputs.

Prints one JSON line: verified logit-positions/s (B * (K+1) per call) over the
timed steps (HIP events on the launch stream around the whole region), the
roofline of the logit-streaming kernel (its duration against the algorithmic
bytes, every logit once; a step that is that one launch takes the timed
region's per-step time, an upper bound on the kernel), and the CPU oracle
timed on this host as a reported baseline.

  python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload c3]
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified logit-positions/s and % peak HBM GB/s at B=64 K=8 V=128256 bf16"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MALL_BYTES = 256 << 20  # MI355X memory-side (Infinity) cache
WORKLOADS = {"c1": 0, "c2": 1, "c3": 2, "c4": 3, "c5": 4, "mixed": 2}
# the mixed batch: the headline inputs, one request in four greedy, the others
# at temperatures 0.7, 1.0, 0.5 in turn (spec_verify_mixed)
MIXED_TEMPS = (0.0, 0.7, 1.0, 0.5)
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and blank space, so that the digest below
    changes with the code and not with its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# The sources each kernel's code comes from: its own file and the device
# headers it includes (declaration-only headers and the host-side ABI file
# hold no device code).
KERNEL_SOURCES = {
    "k_sample_fused": ("sv_sample.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_topp_gather": ("sv_topp.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_topp_band": ("sv_topp.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_topp_cut": ("sv_topp.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_topp_decide": ("sv_sample.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_resid_mass": ("sv_sample.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_resid_draw": ("sv_sample.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_argmax_fused": ("sv_stream.hip", "sv_tiles.hpp", "sv_device.hpp", "sv_layout.hpp"),
    "k_kv_commit": ("sv_kv.hip", "sv_device.hpp", "sv_layout.hpp"),
    "k_tree_merge": ("sv_merge.hip", "sv_device.hpp", "sv_layout.hpp"),
    "k_lmhead_argmax": ("sv_lmhead.hip", "sv_device.hpp", "sv_layout.hpp"),
}


def source_digest(kernel: str) -> str:
    """sha256 over the code of the sources `kernel` is built from: hardware
    counters are only quoted for the kernel code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_sample_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def counters_for(workload: str, kernel: str):
    """HBM traffic per launch of `kernel` on `workload` from committed
    rocprofv3 --pmc summaries, or None when absent or taken on other kernel
    code."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(kernel)
    if not entry or entry.get("source_sha256") != source_digest(kernel):
        return None
    return entry.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep warming up until this many seconds have passed")
    ap.add_argument("--workload", default="c3",
                    choices=sorted(WORKLOADS) + ["kv", "merge", "lmhead", "lmhead_sample"],
                    help="c1..c5: the five settings; mixed: the headline inputs with "
                         "per-request temperatures; kv: the KV-cache commit; "
                         "merge: two drafters' trees merged with confidence routing; "
                         "lmhead: greedy verify with the LM head fused in front")
    ap.add_argument("--sets", type=int, default=3,
                    help="input sets rotated across steps (2 when one set is >= 512 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 20 times (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.workload in ("kv", "merge", "lmhead", "lmhead_sample"):
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            sys.exit(2)
        {"kv": kv_bench, "merge": merge_bench, "lmhead": lmhead_bench,
         "lmhead_sample": lmhead_sample_bench}[args.workload](args)
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "the verify step shards over requests, with no exchange between GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_verification_sample_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    cfg = WORKLOADS[args.workload]
    sets = []
    n_sets = max(1, args.sets)
    s = 0
    while s < n_sets:
        t0 = time.time()
        w = W.make_config(cfg, seed=s)
        log(f"input set {s}: {w.name} generated in {time.time() - t0:.1f}s")
        sets.append(w)
        if w.logit_bytes >= 2 * MALL_BYTES:
            # a set that overflows the memory-side cache twice: two sets, so
            # that what one call leaves in that cache (the last lines it
            # read) is not the next call's input
            n_sets = min(n_sets, 2)
        s += 1
    w0 = sets[0]

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    dt = sv.SPEC_BF16 if w0.dtype == "bf16" else sv.SPEC_F32
    op = {"sample": sv.SPEC_OP_SAMPLE, "greedy": sv.SPEC_OP_GREEDY, "tree": sv.SPEC_OP_TREE}[w0.kind]
    nbytes = sv.verify_workspace_bytes(op, w0.B, w0.K, w0.V, dt, w0.top_p < 1.0)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    calls = []
    for w in sets:
        if args.workload == "mixed":
            a = (up(w.target), up(w.draft), up(w.tokens), up(w.u_accept), up(w.u_sample))
            temps = up(np.array([MIXED_TEMPS[b % 4] for b in range(w.B)], np.float32))
            out = dict(accepted=torch.empty(w.B, dtype=torch.int32, device=dev),
                       tokens=torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev))
            calls.append(lambda a=a, temps=temps, out=out: sv.verify_mixed(
                *a, temps, None, diagnostics=False, workspace=ws, out=out))
        elif w.kind == "sample":
            a = (up(w.target), up(w.draft), up(w.tokens), up(w.u_accept), up(w.u_sample))
            out = dict(accepted=torch.empty(w.B, dtype=torch.int32, device=dev),
                       tokens=torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev))
            calls.append(lambda a=a, w=w, out=out: sv.verify_sample(
                *a, w.temperature, w.top_p, diagnostics=False, workspace=ws, out=out))
        elif w.kind == "greedy":
            a = (up(w.target), up(w.tokens))
            out = dict(accepted=torch.empty(w.B, dtype=torch.int32, device=dev),
                       tokens=torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev))
            calls.append(lambda a=a, out=out: sv.verify_greedy(*a, workspace=ws, out=out))
        else:
            a = (up(w.target), up(w.parents), up(w.tokens), up(w.anc_mask))
            out = dict(path_len=torch.empty(w.B, dtype=torch.int32, device=dev),
                       path_nodes=torch.empty((w.B, w.K), dtype=torch.int32, device=dev),
                       tokens=torch.empty((w.B, w.K), dtype=torch.int32, device=dev))
            calls.append(lambda a=a, out=out: sv.verify_tree(*a, workspace=ws, out=out))
    torch.cuda.synchronize()

    first = calls[0]()
    torch.cuda.synchronize()
    mean_accepted = float(first["accepted" if w0.kind != "tree" else "path_len"].float().mean())

    # warmup: the W steps asked for, and at least --min-warmup-s of steps in
    # all (the GPU clocks ramp up over the first tens of milliseconds of work)
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < args.min_warmup_s:
        calls[i % len(calls)]()
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_done = i

    # timed region: K steps between two HIP events on the stream the library
    # launches on (torch's current stream); nothing else is enqueued there
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        calls[i % len(calls)]()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # the streaming kernel alone: when a step is that one launch, the timed
    # region above is its duration (an upper bound: it includes the gaps
    # between launches); otherwise (top-p: the streaming launch of each chunk
    # of requests, then the top-p and residual launches) a second loop
    # brackets each streaming launch with HIP events (which themselves add
    # about a microsecond to what they bracket)
    single_launch = not (w0.kind == "sample" and w0.top_p < 1.0)
    launches_per_call = 1
    if single_launch:
        kern_us = 1000.0 * total_ms / args.steps
        kern_src = "timed region / steps"
    else:
        n_iso = min(args.steps, 50)
        sv.profile_begin(8 * n_iso)
        for i in range(n_iso):
            calls[i % len(calls)]()
        kern_ms, launches = sv.profile_end()
        launches_per_call = max(1, launches // n_iso)
        kern_us = 1000.0 * kern_ms / max(1, launches)
        kern_src = (f"HIP events around each streaming launch, {launches} launches "
                    f"({launches_per_call} per call, one per chunk of requests)")

    # per-call distribution: each call bracketed by its own pair of events
    n_call = min(args.steps, 100)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_call)]
    torch.cuda.synchronize()
    for i in range(n_call):
        ev[i][0].record()
        calls[i % len(calls)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    per_call = np.array([1000.0 * a.elapsed_time(b) for a, b in ev])
    call_us = {"median": float(np.median(per_call)), "p10": float(np.percentile(per_call, 10)),
               "p90": float(np.percentile(per_call, 90)), "calls": n_call,
               "note": "each call between its own two HIP events"}

    ms_per_step = total_ms / args.steps
    positions = w0.positions
    value = positions / (ms_per_step / 1000.0)
    algo_bytes = w0.logit_bytes  # every logit read once
    if args.workload == "mixed":  # a greedy request reads only its target rows
        row = w0.V * (2 if w0.dtype == "bf16" else 4)
        n_greedy = sum(1 for b in range(w0.B) if MIXED_TEMPS[b % 4] == 0.0)
        algo_bytes -= n_greedy * w0.K * row
    # the residual pass re-reads one row pair per request (the bonus draw: one
    # row); counted here from the first call's outcomes, never in `achieved`
    resample_bytes = 0
    if w0.kind == "sample":
        row = w0.V * (2 if w0.dtype == "bf16" else 4)
        acc = first["accepted"].cpu().numpy()
        greedy_req = ([MIXED_TEMPS[b % 4] == 0.0 for b in range(w0.B)]
                      if args.workload == "mixed" else [False] * w0.B)
        resample_bytes = int(sum(0 if g else (row if n == w0.K else 2 * row)
                                 for n, g in zip(acc, greedy_req)))
    kernel = "k_sample_fused" if w0.kind == "sample" else "k_argmax_fused"
    algo_launch = algo_bytes / launches_per_call  # the chunks are of equal size
    achieved = algo_launch / (kern_us * 1e-6) / 1e9
    step_gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    cpu = cpu_baseline(w0, args.cpu_seconds) if args.cpu_seconds > 0 else None
    outcomes = {}
    cpu_pool = (cpu_baseline_threads(w0, args.cpu_seconds, outcomes)
                if args.cpu_seconds > 0 else None)
    agreement = (oracle_agreement(w0, first, outcomes)
                 if args.cpu_seconds > 0 and args.workload != "mixed" else None)
    traffic = counters_for(args.workload, kernel)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_done,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w0.name + (" per-request T (1 in 4 greedy)"
                                          if args.workload == "mixed" else ""),
                   "B": w0.B, "K": w0.K, "V": w0.V,
                   "logits": w0.dtype, "temperature": w0.temperature, "top_p": w0.top_p,
                   "input_sets": len(sets), "parallelism": "none (1 GPU)"},
        "requests_per_s": w0.B / (ms_per_step / 1000.0),
        "step_pct_peak_hbm": 100.0 * step_gbs / HBM_PEAK_GBS,
        "mean_accepted": mean_accepted,
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_over_algorithmic": (traffic / algo_launch) if traffic else None,
                     "kernel_us": kern_us, "kernel_us_from": kern_src,
                     "launches_per_call": launches_per_call,
                     "algorithmic_bytes_per_launch": algo_launch,
                     "algorithmic_bytes": algo_bytes,
                     "algorithmic_bytes_with_resample": algo_bytes + resample_bytes},
        "call_us": call_us,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_pool,
        "oracle_agreement": agreement,
    }
    if not single_launch:
        # several launches per call: the whole call against the same bytes
        call_gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
        result["roofline"]["whole_call"] = {
            "achieved": call_gbs, "frac": call_gbs / HBM_PEAK_GBS, "us": ms_per_step * 1000.0,
            "note": "algorithmic bytes over the timed region's per-step time (all launches)"}
    print(json.dumps(result), flush=True)


def kv_bench(args):
    """KV-cache commit after a cycle (spec_kv_commit): a Llama-3-8B-shaped
    cache (32 layers, 8 KV heads of 128, bf16), B=32 requests with merged
    trees of 63 nodes, accepted paths of random tree nodes, and a mirror (the
    drafter's copy).  A step is one commit; it moves the same rows each time
    (the cache contents change, the work does not)."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sample_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.kv_commit_workload(seed=0)
    L, _, B, H, S, D = w.kv.shape
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)
                                    if a.dtype == np.uint16 else np.ascontiguousarray(a)).to(dev)
    kv, mir = up(w.kv), up(w.mirror)
    cl, pl, pn = up(w.cache_len), up(w.path_len), up(w.path_nodes)
    new_len = torch.empty(B, dtype=torch.int32, device=dev)
    call = lambda: sv.kv_commit(kv, cl, pl, pn, mirror=mir, out=new_len)
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < args.min_warmup_s:
        call()
        i += 1
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # algorithmic bytes: every path row read once, written where it moves,
    # and written to the mirror
    row = D * 2 * L * 2 * H
    moved = sum(int((w.path_nodes[b, :w.path_len[b]] != np.arange(1, w.path_len[b] + 1)).sum())
                for b in range(B))
    rows_read = int((w.path_len + 1).sum())
    algo = row * (rows_read + moved + rows_read)
    achieved = algo / (ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.lib()
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            oracle.kv_commit(w.kv, w.cache_len, w.path_len, w.path_nodes, mirror=w.mirror)
            n += 1
        el = time.perf_counter() - t1
        cpu = {"value": n * B / el, "unit": "requests/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} full commits of B={B} (whole-cache copies included), {el:.1f}s"}
    print(json.dumps({
        "metric": "KV-cache commit: requests/s and % peak HBM GB/s", "value": B / (ms * 1e-3),
        "unit": "requests/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": i, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"kv commit L{L} H{H} D{D} bf16 B{B} S{S} tree N{w.N} + mirror",
                   "mean_path_len": float(w.path_len.mean()), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "k_kv_commit", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counters_for("kv", "k_kv_commit"), "kernel_us": ms * 1000.0,
                     "kernel_us_from": "timed region / steps", "algorithmic_bytes": algo},
        "cpu_baseline": cpu}), flush=True)


def merge_bench(args):
    """Two drafters' trees merged under one root with confidence routing
    (spec_tree_merge): B=64 requests, two random trees of 31 non-root nodes
    each (the merged 63-node tree of the greedy tree workload).  A step is
    one merge."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sample_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(0)
    B, n = 64, 31
    host = []
    for _ in range(2):
        host += [np.stack([W.grow_tree(rng, n) for _ in range(B)]).astype(np.int32),
                 rng.integers(0, 128256, (B, n + 1)).astype(np.int32),
                 rng.random((B, n + 1)).astype(np.float32)]
    d = [torch.from_numpy(a).to(dev) for a in host]
    N = 2 * n + 1
    out = dict(parents=torch.empty((B, N), dtype=torch.int32, device=dev),
               tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
               mask=torch.empty((B, N, N), dtype=torch.uint8, device=dev),
               conf=torch.empty((B, 2), dtype=torch.float32, device=dev),
               route=torch.empty(B, dtype=torch.int32, device=dev))
    call = lambda: sv.tree_merge(*d, out=out)
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < args.min_warmup_s:
        call()
        i += 1
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # algorithmic bytes: both trees' parents, tokens, confidences read once;
    # merged parents, tokens, mask, means and route written once
    algo = B * (2 * (n + 1) * 12 + N * 8 + N * N + 12)
    achieved = algo / (ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.lib()
        k, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            oracle.tree_merge(*host)
            k += 1
        el = time.perf_counter() - t1
        cpu = {"value": k * B / el, "unit": "requests/s", "cores": 1, "kind": "oracle",
               "sample": f"{k} full merges of B={B}, {el:.1f}s"}
    print(json.dumps({
        "metric": "tree merge with confidence routing: requests/s", "value": B / (ms * 1e-3),
        "unit": "requests/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": i, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"tree merge B{B} two trees of {n} nodes -> N{N}",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "k_tree_merge", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counters_for("merge", "k_tree_merge"), "kernel_us": ms * 1000.0,
                     "kernel_us_from": "timed region / steps", "algorithmic_bytes": algo},
        "cpu_baseline": cpu}), flush=True)


def lmhead_bench(args):
    """Greedy verification with the target's LM head fused in front
    (spec_lmhead_greedy): B=64 requests of K=5 drafts, hidden size 4096,
    vocabulary 128256 (a Llama-3-8B-sized head, bf16, random weights).  A
    step is one call (the GEMM-with-argmax launch and the decide launch).
    Also timed: the unfused path on the same inputs (torch's bf16 matmul
    writing the logits, then spec_verify_greedy)."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sample_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    wl = W.lmhead_workload(seed=0)
    B, K, d, V = wl.B, wl.K, wl.d, wl.V
    M = B * (K + 1)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    hid, wgt = up(wl.hidden), up(wl.weight)
    tok = torch.from_numpy(wl.tokens).to(dev)
    ws = torch.empty(sv.load().spec_lmhead_workspace_bytes(B, K, d, V) + 256, dtype=torch.uint8,
                     device=dev)
    out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    call = lambda: sv.lmhead_greedy(hid, wgt, tok, workspace=ws, out=out)

    def timed(fn, steps, warmup_s):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while n < args.warmup or time.perf_counter() - t0 < warmup_s:
            fn()
            n += 1
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, n

    ms, nwarm = timed(call, args.steps, args.min_warmup_s)
    mean_acc = float(out["accepted"].float().mean())
    # unfused comparison: logits materialised by torch's bf16 matmul
    hb, wb = hid.view(torch.bfloat16).view(M, d), wgt.view(torch.bfloat16)
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    gout = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))

    def unfused():
        torch.mm(hb, wb.t(), out=logits)
        sv.verify_greedy(logits.view(B, K + 1, V), tok, out=gout)

    ums, _ = timed(unfused, max(10, args.steps // 4), 0.1)
    flops = 2.0 * M * d * V
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.lib()
        rows, t1 = 0, time.perf_counter()
        h2 = wl.hidden.reshape(M, d)
        while time.perf_counter() - t1 < args.cpu_seconds:
            oracle.lmhead_logits(h2[rows % M:rows % M + 1], wl.weight)
            rows += 1
        el = time.perf_counter() - t1
        cpu = {"value": rows / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{rows} rows of logits (d {d} x V {V}, fp64) in {el:.1f}s; the argmax "
                         "and greedy rule on top are negligible"}
    print(json.dumps({
        "metric": "verified logit-positions/s (fused LM head + greedy verify)",
        "value": M / (ms * 1e-3), "unit": "positions/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": nwarm, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {"workload": f"lmhead greedy B{B} K{K} d{d} V{V} bf16",
                   "mean_accepted": mean_acc, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "k_lmhead_argmax", "achieved": tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": counters_for("lmhead", "k_lmhead_argmax"),
                     "kernel_us": ms * 1000.0,
                     "kernel_us_from": "timed region / steps (both launches of the call)",
                     "algorithmic_flops": flops, "weight_bytes": V * d * 2,
                     "algorithmic_bytes": V * d * 2 + M * d * 2,
                     "hbm_gbs_weight_stream": V * d * 2 / (ms * 1e-3) / 1e9},
        "unfused": {"us_per_step": ums * 1000.0,
                    "what": "torch.mm bf16 logits [M, V] (hipBLASLt) + spec_verify_greedy"},
        "cpu_baseline": cpu}), flush=True)


def lmhead_sample_bench(args):
    """What fusing the LM head in front of sampling verification could save,
    measured at the sampling workload's shape: B=64 requests of K=8 drafts (576 target
    positions), hidden size 4096, V=128256, bf16, T=0.7.  Timed on the same
    inputs: (1) torch's bf16 matmul writing the target logits (hipBLASLt);
    (2) spec_verify_sample on those logits and draft logits (the unfused
    path is 1 + 2); (3) the library's matrix-core pass over the vocabulary
    matrix with a per-row reduction epilogue (spec_lmhead_greedy at this
    shape), the floor of any fused front end, which would still have to
    stream the draft rows and re-read the drawn row pairs and would add an
    exponential per logit to its epilogue; (4) the target rows' share of
    the verify's streamed bytes at the verify's own rate, the most a fused
    front end could take off (2)."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sample_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    B, K, T = 64, 8, 0.7
    wl = W.lmhead_workload(seed=0, B=B, K=K)
    d, V = wl.d, wl.V
    M = B * (K + 1)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    hid, wgt = up(wl.hidden), up(wl.weight)
    hb, wb = hid.view(torch.bfloat16).view(M, d), wgt.view(torch.bfloat16)
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    torch.mm(hb, wb.t(), out=logits)
    g = torch.Generator(device=dev).manual_seed(5)
    draft = (logits.view(B, K + 1, V)[:, :K].float()
             + 0.5 * torch.randn((B, K, V), generator=g, device=dev)).to(torch.bfloat16)
    # draft tokens drawn from the drafter's own distribution (as a drafter
    # does), so that the residual mass is never negligible by construction
    probs = torch.softmax(draft.float().view(B * K, V) / T, dim=-1)
    tok = torch.multinomial(probs, 1, generator=g).view(B, K).to(torch.int32)
    del probs
    ua = torch.rand((B, K), generator=g, device=dev)
    us = torch.rand((B,), generator=g, device=dev)
    tgt16, dft16 = logits.view(torch.int16).view(B, K + 1, V), draft.view(torch.int16)
    ws = torch.empty(sv.verify_workspace_bytes(sv.SPEC_OP_SAMPLE, B, K, V, sv.SPEC_BF16) + 256,
                     dtype=torch.uint8, device=dev)
    out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    lws = torch.empty(sv.load().spec_lmhead_workspace_bytes(B, K, d, V) + 256, dtype=torch.uint8,
                      device=dev)
    gout = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))

    def timed(fn, steps):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.min_warmup_s:
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / steps

    steps = max(20, args.steps)
    ver = lambda: sv.verify_sample(tgt16, dft16, tok, ua, us, T, 1.0, diagnostics=False,
                                   workspace=ws, out=out)
    ver_us = timed(ver, steps)
    mm_us = timed(lambda: torch.mm(hb, wb.t(), out=logits), steps)
    unfused_us = timed(lambda: (torch.mm(hb, wb.t(), out=logits), ver()), steps)
    fused_gemm_us = timed(lambda: sv.lmhead_greedy(hid, wgt, tok, workspace=lws, out=gout), steps)
    share = (K + 1) / (2 * K + 1)
    print(json.dumps({
        "metric": "LM head + sampling verify: unfused path and the fused bound, us per call",
        "value": unfused_us, "unit": "us", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": unfused_us / 1000.0, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (random weights)",
        "config": {"workload": f"lmhead + sample B{B} K{K} d{d} V{V} bf16 T{T}",
                   "parallelism": "none (1 GPU)"},
        "torch_mm_logits_us": mm_us, "verify_sample_us": ver_us, "unfused_us": unfused_us,
        "matrix_core_pass_us": fused_gemm_us,
        "target_rows_share_of_verify_us": share * ver_us,
        "fused_bound_us": fused_gemm_us + (1 - share) * ver_us,
        "note": "fused_bound = the library's matrix-core pass at this shape + the verify's "
                "draft-row share; a fused front end would also re-read the drawn row pairs "
                "and add an exponential per logit, so this bound is optimistic"}), flush=True)


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(20):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 20}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, seconds):
    """The CPU oracle, single-threaded and pinned to one core, on consecutive
    requests of the same workload (whole-call arithmetic per request), for
    about `seconds`."""
    import oracle
    import workloads as W
    oracle.lib()
    cores = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {cores[0]})
    try:
        return _cpu_single(w, seconds)
    finally:
        os.sched_setaffinity(0, set(cores))


def _cpu_single(w, seconds):
    import oracle
    import workloads as W
    t0 = time.perf_counter()
    oracle.verify_workload(W.subset(w, [0]))
    one = max(time.perf_counter() - t0, 1e-6)
    n = int(min(w.B, max(1, seconds / 4.0 / one)))  # requests per oracle call
    done, i, t0 = 0, 0, time.perf_counter()
    while True:
        reqs = [(i + j) % w.B for j in range(n)]
        oracle.verify_workload(W.subset(w, reqs))
        done += n
        i = (i + n) % w.B
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_req = w.positions // w.B
    return {"value": done * per_req / el, "unit": "positions/s", "cores": 1,
            "kind": "oracle",
            "requests_per_s": done / el,
            "sample": f"{done} requests of {w.name} in oracle calls of {n} request(s), "
                      f"{el:.1f}s single-threaded on one core of {cpu_model()} "
                      f"({os.cpu_count()} cpus visible)"}


def cpu_baseline_threads(w, seconds, outcomes=None):
    """The same oracle fanned out over requests on every core this process
    may use (one thread per core; the oracle's C code runs outside the
    interpreter lock), for about `seconds`.  `outcomes` (a dict) receives
    the oracle's result for each request index it verified."""
    import concurrent.futures as cf
    import oracle
    import workloads as W
    oracle.lib()
    n_thr = max(1, min(len(os.sched_getaffinity(0)), 16, w.B))
    done = [0] * n_thr
    t0 = time.perf_counter()

    def worker(k):
        i = k
        while time.perf_counter() - t0 < seconds:
            r = oracle.verify_workload(W.subset(w, [i % w.B]))
            if outcomes is not None and (i % w.B) not in outcomes:
                outcomes[i % w.B] = r
            done[k] += 1
            i += n_thr

    with cf.ThreadPoolExecutor(n_thr) as ex:
        list(ex.map(worker, range(n_thr)))
    el = time.perf_counter() - t0
    per_req = w.positions // w.B
    total = sum(done)
    return {"value": total * per_req / el, "unit": "positions/s", "cores": n_thr,
            "kind": "oracle", "requests_per_s": total / el,
            "sample": f"{total} requests of {w.name}, one request per oracle call, "
                      f"{el:.1f}s on {n_thr} threads of {cpu_model()}"}


def oracle_agreement(w, first, outcomes):
    """The first timed call's outputs against the oracle's, on the requests
    the CPU baseline verified: per-flag request counts (a uniform within 1e-6
    relative of its threshold or CDF step; a nucleus edge within 1e-6 of
    top_p) and the requests, outside the flagged ones, whose accepted length
    or tokens differ."""
    import numpy as np
    import oracle
    if not outcomes:
        return None
    idx = sorted(outcomes)
    key = "accepted" if w.kind != "tree" else "path_len"
    acc = first[key].cpu().numpy()
    tok = first["tokens"].cpu().numpy()
    flags = np.array([int(outcomes[i]["flags"][0]) if "flags" in outcomes[i] else 0 for i in idx])
    amb = (flags & (oracle.FLAG_ACCEPT_NEAR | oracle.FLAG_CDF_NEAR | oracle.FLAG_S_NEAR)) != 0
    near = (flags & oracle.FLAG_TOPP_NEAR) != 0
    mism = 0
    for j, i in enumerate(idx):
        same = acc[i] == outcomes[i][key][0] and (tok[i] == outcomes[i]["tokens"][0]).all()
        if not same and not amb[j] and not near[j]:
            mism += 1
    return {"requests_compared": len(idx), "unflagged_mismatches": mism,
            "flagged": {"accept_near": int(((flags & oracle.FLAG_ACCEPT_NEAR) != 0).sum()),
                        "cdf_near": int(((flags & oracle.FLAG_CDF_NEAR) != 0).sum()),
                        "s_near": int(((flags & oracle.FLAG_S_NEAR) != 0).sum()),
                        "topp_near": int(near.sum()),
                        "topp_edge": int(((flags & oracle.FLAG_TOPP_EDGE) != 0).sum())},
            "note": "oracle outcomes from the CPU baseline's own runs; topp_near requests "
                    "may take either nucleus membership"}


if __name__ == "__main__":
    main()
