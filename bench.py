#!/usr/bin/env python3
"""Throughput of the per-cycle draft -> schedule -> verify step on one MI355X.

One step = dspark_draft + dspark_schedule + dspark_verify over one batch of
synthetic input (the high-concurrency workload by default: B=256 requests,
K=16 draft positions, V=151,936, rank 256, d=4096, bf16), with the inputs
resident in HBM.  Three input sets (the generated one and two copies rolled
along the vocabulary) rotate so that consecutive steps do not find their
logits in the 256 MB Infinity Cache.

Prints one JSON line: positions/s (B*K per step), the cycle's algorithmic HBM
bandwidth, a roofline entry for the dominant kernel (the vocabulary-stream
kernel of the draft steps, timed with HIP events recorded on the library's
stream), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "draft+verify positions/sec and achieved HBM GB/s (% peak), B=256 K=16 V=152k"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["draft_sampling_verification_markov_amd/csrc/k_stream.hip",
                  "draft_sampling_verification_markov_amd/csrc/dspark_device.hpp",
                  "draft_sampling_verification_markov_amd/csrc/dspark_internal.hpp"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(all_sources: bool = False) -> str:
    """sha256 of the draft-stream kernel's sources (or of every library source)."""
    rels = KERNEL_SOURCES
    if all_sources:
        csrc = os.path.join(ROOT, "draft_sampling_verification_markov_amd", "csrc")
        rels = sorted(os.path.relpath(os.path.join(csrc, f), ROOT) for f in os.listdir(csrc)
                      if f.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def element_size(dt: str) -> int:
    return 2 if dt == "bf16" else 4


def cycle_bytes(cfg, N: int, R: int) -> float:
    """Algorithmic HBM bytes of one cycle: Z once, Wt once, E gathers, h, the N
    verified target rows, and the Z rows re-read at the R rejections."""
    sz, sw, sh = element_size(cfg.logits_dtype), element_size(cfg.weight_dtype), element_size(cfg.hidden_dtype)
    B, K, V, r, d = cfg.B, cfg.K, cfg.V, cfg.r, cfg.d
    return (B * K * V * sz + r * V * sw + 2 * B * K * r * sw + B * K * d * sh + N * V * sz + R * V * sz)


def stream_launch_bytes(cfg) -> float:
    """Algorithmic bytes of one draft step: the step's Z slab, the gathered E rows
    of the previous tokens, and 1/K of Wt.  The cycle reads Wt once
    (B*K*V*s_z + r*V*s_w + B*K*r*s_w ... per cycle): a re-read of Wt at each of the K
    steps is traffic, not algorithmic bytes, so a step is charged Wt / K."""
    sz, sw = element_size(cfg.logits_dtype), element_size(cfg.weight_dtype)
    return cfg.B * cfg.V * sz + cfg.V * cfg.r * sw / cfg.K + cfg.B * cfg.r * sw


def stream_launch_bytes_full_wt(cfg, G: int) -> float:
    """The same launch charged a whole Wt read (what the launch streams when Wt
    does not stay on chip across the steps) plus the partials it writes."""
    sz, sw = element_size(cfg.logits_dtype), element_size(cfg.weight_dtype)
    return cfg.B * cfg.V * sz + cfg.V * cfg.r * sw + cfg.B * cfg.r * sw + cfg.B * G * 16


class Hip:
    """Raw HIP events through the runtime library (events recorded on the library's stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n: int):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(h)) == 0
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, arr) -> None:
        for h in arr:
            self.lib.hipEventDestroy(h)


PERSIST_MAX_B = {"bf16": 192, "f32": 256}  # dspark_draft's batch limits for the persistent schedule, by logits dtype


def draft_persistent(cfg) -> bool:
    """Whether dspark_draft takes the persistent draft schedule for this workload
    (the library's rule, which dspark_draft_path reports on the GPU: bf16 or fp32
    logits, bf16 factors, rank 256, at most 5 vocabulary chunks per workgroup, and
    at most PERSIST_MAX_B requests)."""
    nc = (cfg.V + 127) // 128
    G = min(nc, 256)
    return (cfg.logits_dtype in ("bf16", "f32") and cfg.weight_dtype == "bf16" and cfg.r == 256
            and cfg.B <= PERSIST_MAX_B[cfg.logits_dtype] and -(-nc // G) <= 5)


DOMINANT = "k_draft_persist"  # the kernel of the draft phase (all K positions in one launch)
DOMINANT_STEPWISE = "k_draft"  # the per-position stream kernel where the persistent one does not apply


def dominant(cfg) -> str:
    return DOMINANT if draft_persistent(cfg) else DOMINANT_STEPWISE


def _profile_record(workload: str):
    """The counter record of the workload's dominant draft kernel (whichever
    schedule the profile run took: the file is named for that kernel)."""
    path = None
    for k in (DOMINANT, DOMINANT_STEPWISE):
        q = os.path.join(PROFILE_DIR, f"{k}_{workload}_pmc.json")
        if os.path.exists(q):
            path = q
            break
    if path is None:
        return None
    with open(path) as f:
        return json.load(f)


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the draft phase's dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source; else None."""
    rec = _profile_record(workload)
    if rec is None or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(rec["hbm_bytes_per_launch"])


def mfma_from_profile(workload: str):
    """MFMA counters of the draft-step kernel (bf16 MFMA flops per launch, MFMA busy
    share of the SIMD cycles) from the committed profile record, if it was taken on
    the current kernel source; else None."""
    rec = _profile_record(workload)
    if rec is None or rec.get("kernel_source_sha256") != kernel_source_hash() or not rec.get("mfma"):
        return None
    return rec["mfma"].get(rec.get("kernel", DOMINANT))


def step_kernels(cfg) -> dict:
    """The kernels of one step of the first-drop cycle (dspark_draft, dspark_schedule,
    dspark_verify with bf16 logits and factors) and how often each runs per step."""
    n = cfg.B * cfg.K
    sched = {"k_sched_rank": 1, "k_sched_greedy_lds": 1} if n <= 8192 else \
        {"k_sched_rank": 1, "k_sched_scatter": 1, "k_sched_greedy_global": 1}
    rowlist = {} if (cfg.B <= 1024 and n <= 8192) else {"k_rowlist": 1}  # else built inside k_vlse
    draft = {"k_persist_init": 1, DOMINANT: 1} if draft_persistent(cfg) else \
        {"k_draft_first": 1, DOMINANT_STEPWISE: cfg.K - 1, "k_select_b16": cfg.K}
    return {**draft, "k_conf": 1, **sched, **rowlist,
            "k_vlse": 1, "k_accept": 1, "k_verify64": 1, "k_finish_b16": 1}


def step_traffic_from_profile(cfg):
    """HBM bytes of one whole step: each kernel of the step (counter-measured per
    dispatch in a profiling run of the step alone, bench.py --main-only) times its
    calls per step; None unless the counters were taken on the current library
    sources and cover every kernel of the step."""
    rec = _profile_record(cfg.name)
    if rec is None or rec.get("all_sources_sha256") != kernel_source_hash(all_sources=True):
        return None
    per = rec.get("per_kernel_bytes", {})
    kern = step_kernels(cfg)
    if not rec.get("main_only") or any(k not in per for k in kern):
        return None
    return float(sum(per[k] * c for k, c in kern.items()))


def cpu_baseline(cfg, inp, n_req: int, min_seconds: float = 10.0):
    """The oracle, as it stands, on a bounded sample: all K draft steps, the
    confidence head and verification for n_req requests, and the scheduler over
    a whole batch of candidates (the sample's own survivals, the other requests'
    from the seeded survival generator).  Nothing the GPU computed enters it."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import conf as oconf
    from oracle import draft as odraft
    from oracle import sched as osched
    from oracle import verify as overify

    reqs = np.arange(n_req)
    S_rest = synth.make_survivals(cfg.B, cfg.K, seed=cfg.seed).astype(np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:  # the sample, repeated until at least min_seconds of CPU work
        d = odraft.draft(inp["Z"], inp["E"], inp["Wt"], inp["anchor"], cfg.T_s, cfg.seed, requests=reqs)
        _, S = oconf.confidence(inp["h"][reqs], inp["E"], inp["w_c"], inp["b_c"], inp["tau"], inp["anchor"][reqs],
                                d["x"])
        S_all = S_rest.copy()
        S_all[reqs] = S
        sc = osched.schedule(S_all, inp["T"])
        x = np.zeros((cfg.B, cfg.K), np.int64)
        x[reqs] = d["x"]
        overify.verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], x, sc["n"], cfg.T_s, cfg.seed,
                       requests=reqs)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    t = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": reps * n_req * cfg.K / t, "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_req} of {cfg.B} requests x all {cfg.K} positions (draft, confidence, verify) "
                      f"+ full-batch schedule, {reps} pass(es); {t:.1f} s wall; host "
                      f"{platform.processor() or platform.machine()}, {os.cpu_count()} logical CPUs"}


def _short_kernel_name(name: str) -> str:
    """'void dspark::(anonymous namespace)::k_draft<256>(dspark::StreamArgs)' -> 'k_draft'."""
    n = name.replace("(anonymous namespace)", "")
    n = n.split("(")[0].split("<")[0]
    return n.split("::")[-1].split()[-1] if n.strip() else name


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _pmc_means(directory: str, counter: str):
    """Mean counter value per dispatch, by short kernel name (rows of one dispatch,
    if the counter is reported per hardware instance, are summed first)."""
    per_dispatch = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = (_short_kernel_name(r["Kernel_Name"]), r.get("Dispatch_Id", id(r)))
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    acc = {}
    for (k, _), v in per_dispatch.items():
        acc.setdefault(k, []).append(v)
    return {k: sum(v) / len(v) for k, v in acc.items()}


PROFILE_COMMANDS = """cd /tmp && export TMPDIR=/tmp; R=<repository root>; OUT=<output directory>
rocprofv3 --kernel-trace --stats -T -d $OUT/trace -o trace --output-format csv -- python3 $R/bench.py --main-only --steps 5 --warmup 2 --no-cpu-baseline --no-schedule-compare
rocprofv3 --pmc FETCH_SIZE -d $OUT/fetch -o fetch --output-format csv -- python3 $R/bench.py --main-only --steps 2 --warmup 1 --no-cpu-baseline --no-schedule-compare
rocprofv3 --pmc WRITE_SIZE -d $OUT/write -o write --output-format csv -- python3 $R/bench.py --main-only --steps 2 --warmup 1 --no-cpu-baseline --no-schedule-compare
rocprofv3 --pmc FETCH_SIZE -d $OUT/cfetch -o cfetch --output-format csv -- python3 $R/bench.py --calibrate-copy
rocprofv3 --pmc WRITE_SIZE -d $OUT/cwrite -o cwrite --output-format csv -- python3 $R/bench.py --calibrate-copy
rocprofv3 --pmc MfmaFlopsBF16 MfmaUtil -d $OUT/mfma -o mfma --output-format csv -- python3 $R/bench.py --main-only --steps 2 --warmup 1 --no-cpu-baseline --no-schedule-compare
python3 $R/bench.py --summarize-profiles $OUT"""


def summarize_profiles(prof_dir: str, workload: str) -> None:
    """Writes the kernel-trace and HBM-counter summaries of one profiling run
    (the commands in PROFILE_COMMANDS) under profiles/, and the per-launch
    traffic record of the dominant kernel that the roofline entry reads."""
    import subprocess
    try:
        commit = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"], capture_output=True,
                                text=True).stdout.strip() or "unknown"
    except OSError:
        commit = "unknown"
    src = kernel_source_hash()
    # kernel trace
    rows = _csv_rows(os.path.join(prof_dir, "trace"), "kernel_stats.csv")
    cmd = PROFILE_COMMANDS if workload == "high_concurrency" else "\n".join(
        l.replace("bench.py --main-only", f"bench.py --config {workload} --main-only")
        for l in PROFILE_COMMANDS.splitlines() if "--kernel-trace" in l or "summarize" in l or l.startswith("cd "))
    if workload != "high_concurrency":
        cmd = cmd.replace("--summarize-profiles $OUT", f"--config {workload} --summarize-profiles $OUT")
    lines = [f"# Kernel trace: {workload} workload, bench.py --config {workload} --main-only --steps 5 --warmup 2", "",
             "Command (one of the sequence below; trace run first):", "", "```", cmd, "```", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {_short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"Library source: commit {commit} (kernel sources sha256 {src[:16]}...).",
              "roll_cuda_kernel is torch.roll building the rotated input sets before the timed region.",
              "The run (--main-only) holds only first-drop cycles of the workload and draft calls, so every "
              "verify kernel average is at the step's own schedule."]
    with open(os.path.join(PROFILE_DIR, f"cycle_{workload}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if not os.path.isdir(os.path.join(prof_dir, "fetch")):
        return  # a kernel-trace run only (no counter passes)
    # HBM counters, scaled by what the same counters read for a plain 1 GiB copy
    fetch, write = _pmc_means(os.path.join(prof_dir, "fetch"), "FETCH_SIZE"), _pmc_means(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    cf, cw = _pmc_means(os.path.join(prof_dir, "cfetch"), "FETCH_SIZE"), _pmc_means(os.path.join(prof_dir, "cwrite"), "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0
    ck = [k for k in cf if "copy" in k.lower()]
    fscale, wscale = copy_kib / cf[ck[0]], copy_kib / cw[ck[0]]
    lines = [f"# HBM counters per dispatch: {workload} workload", "", "Commands:", "", "```", PROFILE_COMMANDS, "```", "",
             f"Calibration: a plain 1 GiB device copy ({ck[0]}) reads FETCH_SIZE = {cf[ck[0]]:.1f} KiB and "
             f"WRITE_SIZE = {cw[ck[0]]:.1f} KiB per dispatch against {copy_kib:.0f} KiB moved each way, so "
             f"FETCH_SIZE is scaled by {fscale:.4f} and WRITE_SIZE by {wscale:.4f} below.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MB per dispatch |", "|---|---:|---:|---:|"]
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if "roll" in k or "copy" in k.lower():
            continue
        w = write.get(k, 0.0)
        lines.append(f"| {k} | {fetch[k]:.1f} | {w:.1f} | {(fetch[k] * fscale + w * wscale) * 1024 / 1e6:.1f} |")
    # MFMA work of the kernels that use the matrix cores: bf16 MFMA flops per
    # dispatch, and the MFMA busy cycles over the active cycles of all SIMDs
    mfma = None
    if os.path.isdir(os.path.join(prof_dir, "mfma")):
        flops = _pmc_means(os.path.join(prof_dir, "mfma"), "MfmaFlopsBF16")
        util = _pmc_means(os.path.join(prof_dir, "mfma"), "MfmaUtil")
        avg_us = {_short_kernel_name(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}
        mfma = {}
        lines += ["", "## MFMA work (bf16), per dispatch", "",
                  "| kernel | MFMA GFLOP | MFMA busy % of SIMD cycles | TFLOP/s over the traced average | "
                  "% of the 2.5 PFLOP/s bf16 peak |", "|---|---:|---:|---:|---:|"]
        for k in sorted(flops, key=lambda k: -flops[k]):
            if flops[k] <= 0 or not k.startswith("k_"):
                continue
            tf = flops[k] / (avg_us[k] * 1e-6) / 1e12 if k in avg_us else float("nan")
            mfma[k] = {"gflop": flops[k] / 1e9, "busy_pct": util.get(k), "tflops": tf}
            lines.append(f"| {k} | {flops[k] / 1e9:.2f} | {util.get(k, float('nan')):.1f} | {tf:.0f} | "
                         f"{100 * tf / 2500:.1f} |")
    lines += ["", f"Library source: commit {commit} (kernel sources sha256 {src[:16]}...)."]
    with open(os.path.join(PROFILE_DIR, f"cycle_{workload}_hbm_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    per_kernel = {k: (fetch[k] * fscale + write.get(k, 0.0) * wscale) * 1024 for k in fetch
                  if k.startswith("k_")}
    dom = DOMINANT if DOMINANT in fetch else DOMINANT_STEPWISE
    rec = {"kernel": dom, "workload": workload, "main_only": True, "commit": commit, "kernel_source_sha256": src,
           "all_sources_sha256": kernel_source_hash(all_sources=True), "per_kernel_bytes": per_kernel,
           "fetch_kib_per_launch": fetch[dom], "write_kib_per_launch": write.get(dom, 0.0),
           "fetch_scale": fscale, "write_scale": wscale,
           "hbm_bytes_per_launch": (fetch[dom] * fscale + write.get(dom, 0.0) * wscale) * 1024,
           "mfma": mfma,
           "source": f"profiles/cycle_{workload}_hbm_counters.md"}
    with open(os.path.join(PROFILE_DIR, f"{dom}_{workload}_pmc.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="high_concurrency")
    ap.add_argument("--cpu-requests", type=int, default=0,
                    help="requests in the oracle's timed sample (default: the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule-compare", action="store_true",
                    help="skip timing the draft schedule dspark_draft does not take (profiled runs: rocprofv3 "
                         "ends with a fault after a cooperative launch and then writes no results)")
    ap.add_argument("--main-only", action="store_true",
                    help="time the first-drop step alone (no graph replay, asynchronous scheduler, baselines, "
                         "STS fit or RNN head): the run the profiling commands use")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (scale for HBM counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries of a rocprofv3 run laid out as in PROFILE_COMMANDS")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.config)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this step has no multi-GPU path; "
              "each GPU would run its own batch, table and scheduler independently.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from draft_sampling_verification_markov_amd import dspark, runner

    if not os.path.exists(dspark.LIB_PATH):
        from draft_sampling_verification_markov_amd import build as _b
        _b.build()
    dspark.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": src.numel() * 4}), flush=True)
        return 0

    cfg = synth.get_config(args.config)
    P = dspark.Problem.from_config(cfg)
    log(f"workload {cfg.name}: B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r} d={cfg.d} {cfg.logits_dtype}")
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    log(f"inputs generated in {time.time() - t0:.1f} s")
    x0 = runner.CycleInputs.upload(inp, dev)
    sets = [x0]
    for shift in (cfg.V // 3, 2 * cfg.V // 3):
        xs = runner.CycleInputs(**vars(x0))
        xs.Z = torch.roll(x0.Z, shift, dims=-1).contiguous()
        xs.Zt = torch.roll(x0.Zt, shift, dims=-1).contiguous()
        sets.append(xs)
    o = runner.CycleOutputs(P, dev)
    torch.cuda.synchronize()
    log("inputs resident on the GPU (3 rotating sets)")

    for i in range(args.warmup):
        runner.run_cycle(P, sets[i % 3], o)
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")

    # timed region: exactly `steps` whole steps, back to back; an event between
    # consecutive steps also gives each step's own duration (for the median)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    start.record()
    marks[0].record()
    for i in range(args.steps):
        runner.run_cycle(P, sets[i % 3], o)
        marks[i + 1].record()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    ms_median = float(np.median(per_step))
    log(f"{args.steps} timed steps: {ms_step:.3f} ms/step (median {ms_median:.3f}, "
        f"min {per_step.min():.3f}, max {per_step.max():.3f})")

    # per-call split (a separate pass over the same steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    split = np.zeros(3)
    for i in range(args.steps):
        xs = sets[i % 3]
        ev[0].record()
        runner.draft(P, xs, o)
        ev[1].record()
        runner.schedule(P, xs, o)
        ev[2].record()
        runner.verify(P, xs, o)
        ev[3].record()
        torch.cuda.synchronize()
        split += [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3])]
    split /= args.steps

    def secondary():
        """Graph replay, the asynchronous scheduler, STS fitting, the RNN head and the
        verification baselines on the same inputs (skipped with --main-only)."""
        # the same steps replayed from HIP graphs (one captured per input set, on the
        # same stable output buffers): what a serving loop that captures the cycle sees
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            runner.run_cycle(P, sets[0], o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for xs in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                runner.run_cycle(P, xs, o)
            graphs.append(gr)
        for i in range(args.warmup):
            graphs[i % 3].replay()
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            graphs[i % 3].replay()
        stop.record()
        torch.cuda.synchronize()
        ms_graph = start.elapsed_time(stop) / args.steps
        log(f"{args.steps} graph replays: {ms_graph:.3f} ms/step")
        del graphs
        # the asynchronous scheduler (budget from the survivals of two steps earlier):
        # the current step's survivals and those of a step on another input set
        runner.draft(P, sets[1], o)
        surv_lag = o.surv.clone()
        runner.draft(P, sets[0], o)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dspark.schedule_async(P, surv_lag, o.surv, sets[0].T, o.n_sched, o.n_total, o.workspace)
        e1.record()
        torch.cuda.synchronize()
        ms_async = e0.elapsed_time(e1) / args.steps

        # the verification baselines in place of the first-drop scheduler: whole
        # cycles (draft, baseline schedule, verify) on the same inputs
        def baseline_cycle(sched_fn):
            for i in range(args.warmup):
                xs = sets[i % 3]
                runner.draft(P, xs, o)
                sched_fn(xs)
                runner.verify(P, xs, o)
            torch.cuda.synchronize()
            e0.record()
            for i in range(args.steps):
                xs = sets[i % 3]
                runner.draft(P, xs, o)
                sched_fn(xs)
                runner.verify(P, xs, o)
            e1.record()
            torch.cuda.synchronize()
            h = o.host()
            return {"ms_per_step": e0.elapsed_time(e1) / args.steps, "scheduled_N": int(h["n_total"][0]),
                    "mean_accepted": float(h["n_acc"].mean())}

        # STS fitting on (raw confidence, accepted length, verified length) triples
        # produced by the verify path: 64 cycles at temperature 1 with every draft
        # verified, then one fit of the K temperatures over a 129-point grid
        n_cyc, G_sts, bins_sts = 64, 129, 15
        M_sts = n_cyc * cfg.B
        c_all = torch.empty((M_sts, cfg.K), dtype=torch.float32, device="cuda")
        acc_all = torch.empty((M_sts,), dtype=torch.int32, device="cuda")
        nv_all = torch.empty((M_sts,), dtype=torch.int32, device="cuda")
        ones = torch.ones_like(sets[0].tau)
        for i in range(n_cyc):
            xs = dataclasses.replace(sets[i % 3], tau=ones)
            runner.draft(P, xs, o)
            dspark.schedule_fixed(P, cfg.K, o.n_sched, o.n_total)
            runner.verify(P, xs, o)
            c_all[i * cfg.B:(i + 1) * cfg.B].copy_(o.conf)
            acc_all[i * cfg.B:(i + 1) * cfg.B].copy_(o.n_acc)
            nv_all[i * cfg.B:(i + 1) * cfg.B].copy_(o.n_sched)
        grid_sts = torch.from_numpy(synth.sts_grid(G_sts)).cuda()
        sts_out = [torch.empty(cfg.K, dtype=torch.float64, device="cuda"), torch.empty(cfg.K, dtype=torch.int32, device="cuda"),
                   torch.empty(cfg.K, dtype=torch.float64, device="cuda"), torch.empty(cfg.K, dtype=torch.float64, device="cuda")]
        ws_sts = torch.empty(dspark.sts_workspace_bytes(M_sts, cfg.K, G_sts, bins_sts), dtype=torch.uint8, device="cuda")
        for _ in range(2):
            dspark.sts_fit(c_all, acc_all, nv_all, grid_sts, *sts_out, ws_sts, n_bins=bins_sts)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dspark.sts_fit(c_all, acc_all, nv_all, grid_sts, *sts_out, ws_sts, n_bins=bins_sts)
        e1.record()
        torch.cuda.synchronize()
        ms_sts = e0.elapsed_time(e1) / args.steps
        sts_line = {"samples": M_sts, "positions": cfg.K, "grid": G_sts, "bins": bins_sts, "ms": ms_sts,
                    "candidate_evals_per_s": (G_sts + 1) * M_sts * cfg.K / (ms_sts / 1e3),
                    "source": f"verify path: {n_cyc} cycles x {cfg.B} requests, raw confidences, all {cfg.K} drafts verified",
                    "ece_raw_mean": float(np.nanmean(sts_out[3].cpu().numpy())),
                    "ece_fit_mean": float(np.nanmean(sts_out[2].cpu().numpy()))}

        # the RNN head as the sequential block: whole cycles (draft_rnn, schedule,
        # verify_rnn) on the same inputs, with seeded random GRU weights
        w_rnn = synth.make_rnn_weights(cfg)
        W_ih, W_hh = runner.to_device(w_rnn["W_ih"]), runner.to_device(w_rnn["W_hh"])
        b_ih, b_hh = runner.to_device(w_rnn["b_ih"]), runner.to_device(w_rnn["b_hh"])
        state = torch.empty((cfg.B, cfg.K, cfg.r), dtype=torch.float32, device="cuda")
        ws_rnn = torch.empty(dspark.rnn_workspace_bytes(P), dtype=torch.uint8, device="cuda")

        def rnn_cycle(xs):
            dspark.draft_rnn(P, xs.Z, xs.E, xs.Wt, xs.h, W_ih, b_ih, W_hh, b_hh, xs.w_c, xs.b_c, xs.tau, xs.anchor,
                             o.tok, o.logq, o.lse, o.conf, o.surv, state, ws_rnn)
            dspark.schedule(P, o.surv, xs.T, o.n_sched, o.n_total, ws_rnn)
            dspark.verify_rnn(P, xs.Zt, xs.Z, xs.E, xs.Wt, xs.anchor, o.tok, o.logq, o.lse, state, o.n_sched, o.out_tok,
                              o.n_acc, o.next_anchor, o.logp, o.resid_mass, ws_rnn)

        for i in range(args.warmup):
            rnn_cycle(sets[i % 3])
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            rnn_cycle(sets[i % 3])
        e1.record()
        torch.cuda.synchronize()
        ms_rnn = e0.elapsed_time(e1) / args.steps
        h_rnn = o.host()
        rnn_line = {"ms_per_step": ms_rnn, "positions_per_s": cfg.B * cfg.K / (ms_rnn / 1e3),
                    "scheduled_N": int(h_rnn["n_total"][0]), "mean_accepted": float(h_rnn["n_acc"].mean()),
                    "gate_gemm_gflop": 2.0 * cfg.B * cfg.K * 3 * cfg.r * cfg.d / 1e9}

        baselines = {
            f"fixed_gamma{cfg.K}": baseline_cycle(
                lambda xs: dspark.schedule_fixed(P, cfg.K, o.n_sched, o.n_total)),
            f"fixed_gamma{cfg.K // 4}": baseline_cycle(
                lambda xs: dspark.schedule_fixed(P, cfg.K // 4, o.n_sched, o.n_total)),
            "threshold_0.5": baseline_cycle(
                lambda xs: dspark.schedule_threshold(P, o.surv, 0.5, o.n_sched, o.n_total)),
        }
        return ms_graph, ms_async, baselines, sts_line, rnn_line

    ms_graph = ms_async = baselines = sts_line = rnn_line = None
    if not args.main_only:
        ms_graph, ms_async, baselines, sts_line, rnn_line = secondary()

    # the draft phase (every position: the persistent kernel, or the per-position
    # stream and selection kernels), timed by events the library records on its
    # own stream around the phase and around each launch of its stream kernel
    hip = Hip()
    K = cfg.K

    def draft_timing(path, n, per_launch):
        # per_launch: 2 + 2K events (the phase and each stream-kernel launch),
        # else 2 (the phase alone, without the launch events between its kernels)
        phase, launches = [], []
        for i in range(n):
            xs = sets[i % 3]
            evs = hip.events(2 + 2 * K if per_launch else 2)
            dspark.draft_timed(P, xs.Z, xs.E, xs.Wt, xs.h, xs.w_c, xs.b_c, xs.tau, xs.anchor,
                               o.tok, o.logq, o.lse, o.conf, o.surv, o.workspace, evs, path=path)
            torch.cuda.synchronize()
            phase.append(hip.elapsed_ms(evs[0], evs[1]))
            if per_launch:
                launches.append([hip.elapsed_ms(evs[2 + 2 * j], evs[3 + 2 * j]) for j in range(K)])
            hip.destroy(evs)
        return float(np.median(phase)), np.array(launches)

    def draft_phase_ms(path, n):
        return draft_timing(path, n, False)[0]

    launch_ms_all = draft_timing(dspark.DRAFT_AUTO, args.steps, True)[1]
    k_ms = draft_phase_ms(dspark.DRAFT_AUTO, args.steps)
    lib_path = dspark.draft_path(P)
    assert (lib_path == dspark.DRAFT_PERSISTENT) == draft_persistent(cfg), "bench's rule differs from the library's"
    # both schedules of the draft phase on the same inputs (the dispatch evidence)
    schedules = {"per_position": None, "persistent": None}
    if not args.no_schedule_compare or lib_path == dspark.DRAFT_PER_POSITION:
        schedules["per_position"] = draft_phase_ms(dspark.DRAFT_PER_POSITION, 20)
    if not args.no_schedule_compare or lib_path == dspark.DRAFT_PERSISTENT:
        try:
            schedules["persistent"] = draft_phase_ms(dspark.DRAFT_PERSISTENT, 20)
        except dspark.DsparkError:
            schedules["persistent"] = None  # not applicable to this workload
    log(f"draft phase: {schedules} ms (dspark_draft takes "
        f"{'persistent' if lib_path == dspark.DRAFT_PERSISTENT else 'per_position'})")

    # final outputs of one step on set 0 for the realised schedule
    runner.run_cycle(P, sets[0], o)
    torch.cuda.synchronize()
    g = o.host()
    N = int(g["n_total"][0])
    R = int((~np.isnan(g["resid_mass"])).sum())
    positions = cfg.B * cfg.K
    value = positions / (ms_step / 1e3)
    alg_bytes = cycle_bytes(cfg, N, R)
    nc = (cfg.V + 127) // 128                     # the library's stream grid: fewest workgroups
    G = -(-nc // -(-nc // 256))                    # with the busiest one's chunk count unchanged
    persistent = lib_path == dspark.DRAFT_PERSISTENT
    phase_bytes = cfg.K * stream_launch_bytes(cfg)            # Z once, Wt once, the E rows
    phase_bytes_full = cfg.K * stream_launch_bytes_full_wt(cfg, G)
    # the dominant kernel's average launch (events around each launch): the
    # persistent kernel's one launch per cycle, or k_draft at positions 2..K
    # (position 1 runs k_draft_first)
    if persistent or K == 1:
        launch_ms = float(np.mean(launch_ms_all[:, 0]))
    else:
        launch_ms = float(np.mean(launch_ms_all[:, 1:]))
    # bytes of one launch of the dominant kernel (the whole phase, or one position)
    launch_bytes = phase_bytes if persistent else stream_launch_bytes(cfg)
    achieved = launch_bytes / (launch_ms / 1e3) / 1e9
    traffic = traffic_from_profile(cfg.name)
    step_traffic = step_traffic_from_profile(cfg)
    mfma = mfma_from_profile(cfg.name)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_median,
        "positions_per_s_median_step": positions / (ms_median / 1e3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.logits_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "K": cfg.K, "V": cfg.V, "r": cfg.r, "d": cfg.d,
                   "logits": cfg.logits_dtype, "factors": cfg.weight_dtype, "T_s": cfg.T_s, "seed": cfg.seed},
        "hbm_gbs_algorithmic": alg_bytes / (ms_step / 1e3) / 1e9,
        "hbm_frac_algorithmic": alg_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "hbm_gbs_counters": None if step_traffic is None else step_traffic / (ms_step / 1e3) / 1e9,
        "hbm_frac_counters": None if step_traffic is None else step_traffic / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "counter_bytes_per_step": step_traffic,
        "algorithmic_bytes_per_step": alg_bytes,
        "traffic_over_algorithmic_step": None if step_traffic is None else step_traffic / alg_bytes,
        "logits_per_s": (positions + N) * cfg.V / (ms_step / 1e3),
        "ms_split": {"draft": split[0], "schedule": split[1], "verify": split[2]},
        "ms_per_step_graph_replay": ms_graph,
        "ms_schedule_async": ms_async,
        "baselines": baselines,
        "sts_fit": sts_line,
        "rnn_head": rnn_line,
        "scheduled_N": N,
        "mean_accepted": float(g["n_acc"].mean()),
        "mfma_bias": None if mfma is None else {
            "kernel": f"{dominant(cfg)} (bias contraction E[x]·Wt^T on v_mfma_f32_32x32x16_bf16)",
            "gflop_per_launch_counted": mfma["gflop"],
            "gflop_per_launch_algorithmic": 2.0 * cfg.B * cfg.r * cfg.V * (cfg.K if persistent else 1) / 1e9,
            "tflops": mfma["gflop"] / launch_ms,
            "frac_of_bf16_peak": mfma["gflop"] / launch_ms / 2500.0,
            "mfma_busy_pct": mfma["busy_pct"],
            "source": f"profiles/cycle_{cfg.name}_hbm_counters.md"},
        "roofline": {
            "kernel": (f"{DOMINANT}: the draft phase, all {cfg.K} positions in one launch" if persistent else
                       f"{DOMINANT_STEPWISE}: one draft position (vocabulary stream and bias contraction), "
                       f"average over positions 2..{cfg.K}"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_over_algorithmic": None if traffic is None else traffic / launch_bytes,
            "launch_ms": launch_ms,
            "launch_bytes": launch_bytes,
            "launch_bytes_note": ("K x (Z slab + E rows of the previous tokens) + Wt once per cycle" if persistent else
                                  "Z slab + Wt / K (Wt once per cycle) + E rows of the previous tokens"),
            "launch_bytes_full_wt": None if persistent else stream_launch_bytes_full_wt(cfg, G),
            "frac_full_wt": None if persistent else
            stream_launch_bytes_full_wt(cfg, G) / (launch_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "phase_ms": k_ms,
            "phase_bytes": phase_bytes,
            "phase_frac": phase_bytes / (k_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        },
        "draft_phase_ms_by_schedule": schedules,
    }
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_requests if args.cpu_requests > 0 else cfg.B
        log(f"timing the CPU oracle on {n_cpu} requests")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, n_cpu)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
