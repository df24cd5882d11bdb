"""Benchmark of the batched verify step on one MI355X.

One step = one call of spec_verify_sample over one batch of the
chain_bf16_llama workload (B=256 sequences, gamma=8 drafts, V=128256, bf16
logits, temperatures drawn from {0, 0.7, 1.0}), inputs resident in HBM. Prints
one JSON line: verified positions/s (B * gamma per step) as `value`, the
logit-read bandwidth against the HBM roofline of one verify call (the kernels
it launches back to back on one stream, timed with one pair of HIP events on
that stream around the timed steps), and the CPU oracle timed on the host as a
baseline (every host thread the process may use, and one). Before the warmup
steps the GPU reads a buffer for about 50 ms, so that the timed steps do not
start on idle clocks.
Beside the roofline it reports the GPU's streaming-read rate measured in the
same run (the library's read yardstick over a 2 GiB buffer) and the call's
fraction of it, and a warm-cache launch time (the same input copy every step,
labelled as such; the timed steps rotate over copies of the inputs that
together exceed the 256 MB MALL).

Other workloads (--workload): the four other verify configurations
(chain_f32_small, chain_bf16_peaked, onehot_bf16_qwen, tree_bf16_llama),
sampled trees (tree_sample_bf16_llama), and the steps around the verify, each
with its own metric and the same roofline / cpu_baseline fields:
kv_rollback_bf16_llama (sequences rolled back per second), ngram_draft_qwen
(drafts per second) and tree_mask_b256 (masks per second).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified positions/s + logit-read GB/s (% of HBM peak), B=256 γ=8 V=128256"
HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 30
DEFAULT_WORKLOAD = "chain_bf16_llama"
KERNEL_SOURCES = ["rejection_sampling_verify_amd/csrc/sv_chain.hip", "rejection_sampling_verify_amd/csrc/sv_tree.hip",
                  "rejection_sampling_verify_amd/csrc/sv_device.h", "rejection_sampling_verify_amd/csrc/sv_internal.h",
                  "rejection_sampling_verify_amd/csrc/sv_api.hip"]
KV_KERNEL_SOURCES = ["rejection_sampling_verify_amd/csrc/sv_kv.hip"]
NGRAM_KERNEL_SOURCES = ["rejection_sampling_verify_amd/csrc/sv_ngram.hip"]
TREE_MASK_KERNEL_SOURCES = ["rejection_sampling_verify_amd/csrc/sv_treemask.hip"]


def kernel_source_hash(workload: str = DEFAULT_WORKLOAD) -> str:
    """Hash of the sources of the kernels a workload runs (verify, KV rollback,
    n-gram drafting or the tree mask)."""
    h = hashlib.sha256()
    srcs = (KV_KERNEL_SOURCES if workload.startswith("kv_rollback") else
            NGRAM_KERNEL_SOURCES if workload.startswith("ngram") else
            TREE_MASK_KERNEL_SOURCES if workload.startswith("tree_mask") else KERNEL_SOURCES)
    for rel in srcs:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def to_dev(a, torch, dev):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def host_threads() -> int:
    """The host threads this process may use: the CPUs it is allowed to run on,
    within the OpenMP thread budget of its environment when one is set (a GPU
    host shares its cores between its GPUs' jobs that way)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    budget = os.environ.get("OMP_NUM_THREADS", "")
    if budget.isdigit() and int(budget) > 0:
        n = min(n, int(budget))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, is_tree: bool, positions_per_step: int, threads: int | None = None, max_runs: int = 3):
    """The oracle as it stands, on every host thread this process may use
    unless told otherwise, over the whole workload; repeated until about 10 s
    of CPU time or max_runs runs."""
    import oracle
    import workloads
    threads = threads or host_threads()
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs and (not times or time.perf_counter() - t_start < 10.0):
        t0 = time.perf_counter()
        if isinstance(inp, workloads.TreeSampleInputs):
            oracle.verify_tree_sample(inp.target, inp.draft, inp.parents, inp.depth, inp.node_tokens,
                                      inp.temperature, inp.max_depth, seed=inp.seed, offset=inp.offset,
                                      nthreads=threads,
                                      without_replacement=inp.meta.get("without_replacement", False))
        elif is_tree:
            oracle.verify_tree(inp.target, inp.parents, inp.depth, inp.node_tokens, inp.max_depth, nthreads=threads)
        else:
            oracle.verify_sample(inp.target, inp.draft, inp.draft_ids, inp.temperature, seed=inp.seed,
                                 offset=inp.offset, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": positions_per_step / t, "unit": "verified positions/s", "cores": threads, "kind": "oracle",
            "sample": "the whole workload (one step), %d run(s), median %.3f s, fp64 plain loops" % (len(times), t),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def read_ceiling(torch, dev, rsv, nbytes: int = 2 << 30, launches: int = 10):
    """Streaming-read rate of this GPU: one plain read of a 2 GiB buffer per
    launch (the library's read yardstick), HIP events around each launch."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    nblocks = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(4 * nblocks, dtype=torch.int32, device=dev)
    for _ in range(2):
        rsv.sv_debug_read_stream(buf, nblocks, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record()
        rsv.sv_debug_read_stream(buf, nblocks, out=out)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def copy_calibration(torch, dev, steps: int):
    """Copies of a 1 GiB buffer into another: each launch reads and writes
    exactly COPY_BYTES, the yardstick for the HBM byte counters."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": steps}), flush=True)


def settle(torch, dev, rsv, seconds: float = 0.05):
    """Untimed, before the warmup steps: plain reads of a 512 MiB buffer for
    about `seconds` of wall-clock time, so that the timed steps do not begin
    while the GPU is still leaving its idle clocks (the first tens of calls
    after an idle spell run several percent slower otherwise)."""
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    nblocks = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(4 * nblocks, dtype=torch.int32, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            rsv.sv_debug_read_stream(buf, nblocks, out=out)
        torch.cuda.synchronize()
    del buf


def timed_region(torch, step, steps: int, stream, per_call: bool = False):
    """The timed steps: synchronize, `steps` calls on `stream`, synchronize.
    Returns (wall-clock seconds, mean ms per call from HIP events on `stream`,
    per-call ms or None).

    By default one event goes before the first call and one after the last, and
    nothing else is queued between the calls: an event pair around every call
    would put its own markers (several microseconds a call) into the timed
    region. With per_call, an event pair goes around each call instead: for
    kernels shorter than the host's time to issue a call, where back-to-back
    calls leave the GPU waiting on the host and the mean of the whole region
    would time the host."""
    torch.cuda.synchronize()
    if per_call:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for k, (a, b) in enumerate(ev):
            a.record(stream)
            step(k)
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        each = np.array([a.elapsed_time(b) for a, b in ev])
        return wall, float(each.mean()), each
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for k in range(steps):
        step(k)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, a.elapsed_time(b) / steps, None


def launch_spread(torch, step, steps: int, stream):
    """Untimed, after a timed region without per-call events: the same calls
    with an event pair around each one, for the spread of a single call's time
    (each figure includes the markers of its own pair)."""
    return timed_region(torch, step, steps, stream, per_call=True)[2]


def launch_stats(mean_ms: float, spread, per_call: bool = False):
    note = ("an event pair around each timed call" if per_call else
            "mean: two HIP events around the timed calls on the kernels' stream, divided by the calls; "
            "p10/p50/p90: a second pass with an event pair around each call")
    return {"mean": mean_ms, "p10": float(np.percentile(spread, 10)), "p50": float(np.median(spread)),
            "p90": float(np.percentile(spread, 90)), "note": note}


def run_kv(args, torch, rsv, workloads, dev):
    """KV-cache rollback after a tree verify step: one sv_kv_rollback call over
    the resident K and V caches of every layer. Successive steps move the root
    positions on by 64 (16 distinct sets, as decoding advances), so the rows a
    step touches are not left in the caches by the step before."""
    inp = workloads.make_extra(args.workload)
    L, B, H, S, D = inp.shape
    k = workloads.fill_kv_device(torch, torch.empty(inp.shape, dtype=torch.int16, device=dev), inp.seed, 0)
    v = workloads.fill_kv_device(torch, torch.empty(inp.shape, dtype=torch.int16, device=dev), inp.seed, 1)
    roots = [torch.from_numpy(inp.root + 64 * j).to(dev) for j in range(16)]
    path = torch.from_numpy(inp.path).to(dev)
    plen = torch.from_numpy(inp.path_len).to(dev)
    out = torch.empty(B, dtype=torch.int32, device=dev)
    print("[bench] workload %s resident" % args.workload, file=sys.stderr, flush=True)

    def step(j):
        rsv.sv_kv_rollback(k, v, roots[j % 16], path, plen, cache_len=out)

    stream = torch.cuda.current_stream()
    settle(torch, dev, rsv)
    for j in range(args.warmup):
        step(j)
    wall, mean_ms, launch_ms = timed_region(torch, step, args.steps, stream, per_call=True)
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)
    ms_per_step = wall * 1e3 / args.steps
    alg_bytes = inp.algorithmic_bytes()
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    rec = {
        "metric": "KV-cache rollback sequences/s (every layer's K and V moved to the accepted path)",
        "value": B / (ms_per_step * 1e-3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "L": L, "B": B, "H": H, "S": S, "D": D, "cache_dtype": "bf16",
                   "paths": "walks in the 65-node tree, 1 to 4 nodes"},
        "moved_rows_per_layer_head": int(inp.moved_rows().sum()),
        "algorithmic_bytes_per_step": int(alg_bytes),
        "launch_ms": launch_stats(mean_ms, launch_ms, per_call=True),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = kv_cpu_baseline(inp)
    print(json.dumps(rec), flush=True)


def run_ngram(args, torch, rsv, workloads, dev):
    """Prompt-lookup drafting: one sv_ngram_draft call over the batch of token
    histories. The histories (33.5 MB) would sit in the 256 MB MALL if one copy
    were reused, so 16 resident copies are used in turn."""
    inp = workloads.make_extra(args.workload)
    copies = [torch.from_numpy(inp.tokens).to(dev) for _ in range(16)]
    lengths = torch.from_numpy(inp.lengths).to(dev)
    B, gamma = inp.B, inp.gamma
    out = (torch.empty((B, gamma), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
           torch.empty(B, dtype=torch.int32, device=dev))
    print("[bench] workload %s resident" % args.workload, file=sys.stderr, flush=True)

    def step(j):
        rsv.sv_ngram_draft(copies[j % 16], lengths, inp.ngram, gamma, inp.pad, out_draft=out[0], out_count=out[1],
                           out_match=out[2])

    stream = torch.cuda.current_stream()
    settle(torch, dev, rsv)
    for j in range(args.warmup):
        step(j)
    wall, mean_ms, launch_ms = timed_region(torch, step, args.steps, stream, per_call=True)
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)
    ms_per_step = wall * 1e3 / args.steps
    match = out[2].cpu().numpy()
    alg_bytes = inp.algorithmic_bytes(match)
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    rec = {
        "metric": "n-gram (prompt-lookup) drafts/s: one-hot gamma-token proposals per second",
        "value": B / (ms_per_step * 1e-3), "unit": "drafts/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": [int(inp.lengths.min()), int(inp.lengths.max())],
                   "stride": int(inp.tokens.shape[1]), "ngram": inp.ngram, "gamma": gamma,
                   "pad_with_last": bool(inp.pad), "V": inp.meta["V"]},
        "matched_fraction": float(np.mean(match >= 0)),
        "algorithmic_bytes_per_step": int(alg_bytes),
        "algorithmic_bytes_note": "each sequence's tokens from its match's start to its end (all of them "
                                  "without a match), plus lengths and outputs",
        "launch_ms": launch_stats(mean_ms, launch_ms, per_call=True),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        from oracle import ngram as og
        times = []
        t_start = time.perf_counter()
        while len(times) < 3 and time.perf_counter() - t_start < 10.0:
            t1 = time.perf_counter()
            og.ngram_draft(inp.tokens, inp.lengths, inp.ngram, gamma, inp.pad)
            times.append(time.perf_counter() - t1)
        t = float(np.median(times))
        rec["cpu_baseline"] = {"value": B / t, "unit": "drafts/s", "cores": 1, "kind": "oracle",
                               "sample": "the whole workload (one step), %d run(s), median %.3f s, Python loops"
                                         % (len(times), t)}
    print(json.dumps(rec), flush=True)


def run_tree_mask(args, torch, rsv, workloads, dev):
    """Tree attention mask and position ids for a batch of per-sequence trees:
    one sv_tree_mask call (bool mask and position ids)."""
    inp = workloads.make_extra(args.workload)
    B, N = inp.B, inp.N
    par = torch.from_numpy(inp.parents).to(dev)
    off = torch.from_numpy(inp.offsets).to(dev)
    out_mask = torch.empty((B, N, N), dtype=torch.bool, device=dev)
    out_pos = torch.empty((B, N), dtype=torch.int32, device=dev)
    print("[bench] workload %s resident" % args.workload, file=sys.stderr, flush=True)

    def step(j):
        rsv.sv_tree_mask(par, off, out_mask=out_mask, out_position_ids=out_pos)

    stream = torch.cuda.current_stream()
    settle(torch, dev, rsv)
    for j in range(args.warmup):
        step(j)
    wall, mean_ms, launch_ms = timed_region(torch, step, args.steps, stream, per_call=True)
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)
    ms_per_step = wall * 1e3 / args.steps
    alg_bytes = inp.algorithmic_bytes()
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    rec = {
        "metric": "tree attention masks/s (ancestor mask and depth position ids per sequence)",
        "value": B / (ms_per_step * 1e-3), "unit": "masks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "nodes": N, "mask": "bool [B, N, N]",
                   "trees": "one per sequence, breadth-first, 1 to 4 children per node"},
        "algorithmic_bytes_per_step": int(alg_bytes),
        "launch_ms": launch_stats(mean_ms, launch_ms, per_call=True),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        from oracle import trees
        times = []
        t_start = time.perf_counter()
        while len(times) < 20 and time.perf_counter() - t_start < 10.0:
            t1 = time.perf_counter()
            trees.tree_attn_batch(inp.parents, inp.offsets)
            times.append(time.perf_counter() - t1)
        t = float(np.median(times))
        rec["cpu_baseline"] = {"value": B / t, "unit": "masks/s", "cores": 1, "kind": "oracle",
                               "sample": "the whole workload (one step), %d run(s), median %.4f s, Python loops"
                                         % (len(times), t)}
    print(json.dumps(rec), flush=True)


def kv_cpu_baseline(inp, max_runs: int = 5):
    """The oracle on one layer of K and V for every sequence (numpy, one
    thread), scaled to whole sequences (all layers)."""
    from oracle import kv as okv
    L, B, H, S, D = inp.shape
    rng = np.random.default_rng(inp.seed)
    kc = rng.integers(-32768, 32767, size=(1, B, H, S, D), dtype=np.int16)
    vc = rng.integers(-32768, 32767, size=(1, B, H, S, D), dtype=np.int16)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs and time.perf_counter() - t_start < 10.0:
        t0 = time.perf_counter()
        okv.kv_rollback(kc, inp.root, inp.path, inp.path_len)
        okv.kv_rollback(vc, inp.root, inp.path, inp.path_len)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": B / L / t, "unit": "sequences/s", "cores": 1, "kind": "oracle",
            "sample": "one of %d layers, K and V, all %d sequences; %d run(s), median %.3f s" % (L, B, len(times), t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run device-to-device copies of a known size (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import rejection_sampling_verify_amd as rsv
    import workloads

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev, args.steps)
        return
    rsv.lib()
    if args.workload.startswith("kv_rollback"):
        run_kv(args, torch, rsv, workloads, dev)
        return
    if args.workload.startswith("ngram"):
        run_ngram(args, torch, rsv, workloads, dev)
        return
    if args.workload.startswith("tree_mask"):
        run_tree_mask(args, torch, rsv, workloads, dev)
        return
    inp = workloads.make_extra(args.workload) if args.workload in workloads.EXTRA else workloads.make(args.workload)
    is_tree = args.workload.startswith("tree")
    sampled_tree = isinstance(inp, workloads.TreeSampleInputs)
    print("[bench] workload %s generated" % args.workload, file=sys.stderr, flush=True)

    # Resident copies of the inputs, used in turn, so that no step finds its
    # logits in the 256 MB Infinity Cache (MALL) from the steps before: as
    # many as make the rotation at least 512 MiB (two for the large
    # workloads, twelve for chain_bf16_peaked's 45 MB), at most 16.
    per_copy = inp.target.nbytes + (inp.draft.nbytes if getattr(inp, "draft", None) is not None else 0)
    ncopies = int(min(16, max(2, -(-(512 << 20) // per_copy))))
    copies = []
    for _ in range(ncopies):
        if is_tree:
            copies.append(dict(t=to_dev(inp.target, torch, dev), par=torch.from_numpy(inp.parents).to(dev),
                               dep=torch.from_numpy(inp.depth).to(dev), tok=torch.from_numpy(inp.node_tokens).to(dev)))
            if sampled_tree:
                copies[-1].update(d=to_dev(inp.draft, torch, dev), temp=torch.from_numpy(inp.temperature).to(dev))
        else:
            copies.append(dict(t=to_dev(inp.target, torch, dev), d=to_dev(inp.draft, torch, dev),
                               ids=torch.from_numpy(inp.draft_ids).to(dev),
                               temp=torch.from_numpy(inp.temperature).to(dev)))
    ws = rsv.Workspace(dev)
    if is_tree:
        B, N = inp.node_tokens.shape
        wbuf = ws.get(B, N, inp.V)
        out = (torch.empty((B, inp.max_depth + 1), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
        positions = B * (N - 1)

        def step(k):
            c = copies[k % ncopies]
            if sampled_tree:
                rsv.spec_verify_tree_sample(c["t"], c["d"], c["par"], c["dep"], c["tok"], c["temp"], inp.max_depth,
                                            seed=inp.seed, offset=inp.offset, out_path=out[0], out_path_len=out[1],
                                            out_token=out[2], workspace=wbuf,
                                            without_replacement=inp.meta.get("without_replacement", False))
            else:
                rsv.spec_verify_tree(c["t"], c["par"], c["dep"], c["tok"], inp.max_depth, out_path=out[0],
                                     out_path_len=out[1], out_bonus=out[2], workspace=wbuf)
    else:
        B, G = inp.draft_ids.shape
        wbuf = ws.get(B, G + 1, inp.V)
        out = (torch.empty((B, G + 1), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
        positions = B * G

        def step(k):
            c = copies[k % ncopies]
            rsv.spec_verify_sample(c["t"], c["d"], c["ids"], c["temp"], seed=inp.seed, offset=inp.offset,
                                   out_tokens=out[0], out_num_accepted=out[1], workspace=wbuf)

    stream = torch.cuda.current_stream()
    settle(torch, dev, rsv)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    wall, mean_ms, _ = timed_region(torch, step, args.steps, stream)
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)
    launch_ms = launch_spread(torch, step, args.steps, stream)

    # Warm cache, labelled as such: the same input copy every step, so that
    # part of it is still in the 256 MB MALL from the step before.
    warm = []
    for k in range(max(5, args.steps // 5)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(0)
        b.record(stream)
        warm.append((a, b))
    torch.cuda.synchronize()
    warm_ms = np.array([a.elapsed_time(b) for a, b in warm])
    ceiling = read_ceiling(torch, dev, rsv)
    print("[bench] warm-cache steps and read ceiling done", file=sys.stderr, flush=True)

    ms_per_step = wall * 1e3 / args.steps
    if sampled_tree:
        # Data-dependent: the walk reads only the nodes on each sequence's path.
        inp.paths = (out[0].cpu().numpy(), out[1].cpu().numpy())
    alg_bytes = inp.algorithmic_bytes()
    t_launch = mean_ms * 1e-3
    achieved = alg_bytes / t_launch / 1e9
    traffic = measured_traffic(args.workload)

    if is_tree:
        cfg = {"workload": args.workload, "B": int(B), "nodes": int(inp.node_tokens.shape[1]), "V": int(inp.V),
               "input_dtype": str(inp.target.dtype).replace("uint16", "bf16"), "verify": "greedy tree"}
        extra = {}
        if sampled_tree:
            cfg["verify"] = "sampled tree (multi-round rejection sampling)"
            if inp.meta.get("without_replacement"):
                cfg["verify"] += ", siblings drawn without replacement"
            cfg["temperatures"] = sorted(set(float(x) for x in inp.temperature))
            plen = out[1].cpu().numpy()
            extra = {"mean_accepted_depth": float(np.mean(plen[plen >= 1] - 1)),
                     "algorithmic_bytes_note": "rows the walk must read: target and draft row of every inner "
                                               "node on the accepted path, plus the leaf row of a bonus draw"}
    else:
        n = out[1].cpu().numpy()
        cfg = {"workload": args.workload, "B": int(B), "gamma": int(G), "V": int(inp.V),
               "input_dtype": "bf16" if inp.is_bf16 else "f32",
               "temperatures": sorted(set(float(x) for x in inp.temperature)),
               "draft": "one-hot" if inp.draft is None else "dense"}
        valid = n[n >= 0]
        extra = {"mean_accepted": float(valid.mean()),
                 "emitted_tokens_per_s": float((valid + 1).sum() / (ms_per_step * 1e-3)),
                 "per_position_acceptance": [float(np.mean(n[n >= i] > i)) if np.any(n >= i) else None
                                             for i in range(G)]}
    rec = {
        "metric": METRIC, "value": positions / (ms_per_step * 1e-3), "unit": "verified positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": cfg,
        "logit_read_GBps": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": int(alg_bytes),
        "launch_ms": launch_stats(mean_ms, launch_ms),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "hbm_read_ceiling_GBps": ceiling,
        "frac_of_read_ceiling": achieved / ceiling,
        "warm_cache_launch_ms": {"p50": float(np.median(warm_ms)), "note": "same input copy every step"},
        "input_copies": {"count": ncopies, "bytes_each": int(per_copy),
                         "note": "used in turn, so that the timed steps read their logits from HBM"},
        **extra,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, is_tree, positions)
        rec["cpu_baseline_1thread"] = cpu_baseline(inp, is_tree, positions, threads=1, max_runs=1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
