#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one spec_verify_sample call over the whole synthetic batch of the
Llama-class workload (B=64 requests, K=4 drafts each, V=128256, bf16 logits;
half the requests sampled at T=1, half greedy).  Inputs are resident in HBM
before timing starts; the step rotates over enough copies of the logits
(>= 1.25 GB) that every step streams from HBM rather than from the 256 MB
Infinity Cache.  Prints one JSON line.

Reported:
  value          verified draft positions per second (sum of K_b per step / time)
  roofline       the single verify kernel: algorithmic bytes per launch / its
                 mean duration, from HIP events on the launch stream around the
                 timed region (which holds nothing but back-to-back launches of
                 that kernel), against 8 TB/s; the library's own events around
                 each launch are reported beside it as a cross-check
  cpu_baseline   the float64 oracle on a bounded sample of the same batch
  copy_gbs       a plain 1 GiB device copy on the same stream (the achievable line)

--op draft times the draft-side sampler instead (spec_draft_sample over the
workload's draft rows at step 0, one row per request) against the VALU issue
rate, since its exponential race is arithmetic-bound; --op commit times the
commit step (spec_commit_tokens) on the workload's verify outputs; --op
early-exit times spec_verify_sample_early_exit on the same batch, whose
roofline counts only the rows a request needs up to its first rejection; --op
tree times greedy draft-tree verification (spec_verify_tree_greedy) on a
seeded tree workload (--tree); --op greedy times the all-greedy entry point
(spec_verify_greedy) on the workload with every request greedy.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "verified draft positions/sec + HBM GB/s (% peak), B=64 K=4 V=128256 bf16"
# the verify kernel's sources: committed traffic counters apply while these are unchanged
CSRC = os.path.join(ROOT, "rejection_sampling_verify_scaled_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, name) for name in ("spec_verify.hip", "device_common.h")]
EE_KERNEL_SOURCES = [os.path.join(CSRC, name) for name in ("early_exit.hip", "device_common.h")]


def kernel_source_sha256(sources=None) -> str:
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=int, default=2,
                    help="synthetic workload number (2: Llama-class, the metric's)")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tree", default="tree-eagle",
                    choices=("tree-small", "tree-eagle", "tree-ragged"),
                    help="tree workload for --op tree")
    ap.add_argument("--op", choices=("verify", "draft", "commit", "early-exit", "tree", "greedy"),
                    default="verify",
                    help="verify: the verify step (the metric); draft: the draft-side "
                         "sampler on the workload's draft rows at step 0; commit: the "
                         "commit step on the workload's verify outputs; early-exit: the "
                         "early-exit verify on the same batch; tree: greedy draft-tree "
                         "verification on --tree; greedy: spec_verify_greedy on the "
                         "workload with every request greedy")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs of --traffic-probe (FETCH_SIZE, "
                         "then WRITE_SIZE, -f csv) into the traffic record of --op on "
                         "--workload under profiles/, and print the summary")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="no GPU: per-kernel mean of every counter per dispatch in a "
                         "rocprofv3 --pmc -f csv run")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="no GPU: per-kernel dispatch durations (count, mean, median, "
                         "min, max) from a rocprofv3 --kernel-trace -f csv run")
    ap.add_argument("--valu-rates", action="store_true",
                    help="issue cycles per wave64 instruction of the VALU classes the "
                         "samplers use, from libspecverify_rates.so; prints a summary")
    ap.add_argument("--stage-trace", action="store_true",
                    help="per-stage timeline of the verify kernel on --workload, from its "
                         "stage-trace build (libspecverify_trace.so): --steps traced calls "
                         "after --warmup untraced ones; prints a summary, no JSON line")
    ap.add_argument("--crossover", action="store_true",
                    help="full verify against the early-exit verify on the first B requests "
                         "of workloads 2-5 (interleaved rounds, median); prints a table, no "
                         "JSON line")
    ap.add_argument("--traffic-probe", type=int, default=0, metavar="MIB",
                    help="for hardware-counter runs: after the warmup, run --steps verify "
                         "calls, then 5 device copies of MIB MiB (the counters' reference "
                         "kernel of known size), and exit without timing")
    return ap.parse_args()


def algorithmic_bytes(batch) -> int:
    """Each needed logit read once: (2K+1) rows per sampled request, K+1 per greedy."""
    esz = 2 if batch.dtype == 1 else 4
    tot = 0
    for b in range(batch.B):
        k = int(batch.offsets[b + 1] - batch.offsets[b])
        rows = (2 * k + 1) if batch.temperature[b] > 0 else (k + 1)
        tot += rows * batch.V * esz
    return tot


def early_exit_bytes(batch, accept_len) -> int:
    """The rows an early exit needs, each read once: a sampled request that
    rejects at position n reads target and draft rows 0..n, one that accepts
    all K_b reads all of them and the bonus row; a greedy request reads target
    rows 0..n."""
    esz = 2 if batch.dtype == 1 else 4
    tot = 0
    for b in range(batch.B):
        k = int(batch.offsets[b + 1] - batch.offsets[b])
        n = int(accept_len[b])
        if batch.temperature[b] > 0:
            rows = 2 * k + 1 if n == k else 2 * (n + 1)
        else:
            rows = n + 1
        tot += rows * batch.V * esz
    return tot


class Hip:
    """The few HIP runtime calls the per-kernel timing needs (events)."""

    def __init__(self):
        import torch  # noqa: F401  (binds libamdhip64 to torch's runtime first)
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)


def traffic_record(workload: int, kernel: str = "sv_verify", sources=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_workload{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_sha256(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


# VALU issue of the draft sampler.  A gfx950 SIMD issues a full-rate 32-bit
# wave64 instruction (fma, add, xor, compare, select) in 2 cycles: 32 lanes per
# cycle, the rate behind the published 157.3 TFLOP/s fp32.  `bench.py
# --valu-rates` measures (profiles/valu_issue_rates.txt) 2.34 cycles for such
# an instruction, 8.8 for a transcendental (v_exp_f32, v_log_f32) and 5.4 for
# v_mad_u64_u32 (Philox's 32 x 32 -> 64 product, counted in SQ_INSTS_VALU_INT64).
# Costs below are in full-rate lane slots: 1 for a full-rate instruction, 3.8
# for a transcendental and 2.3 for a 64-bit integer instruction.
VALU_SLOTS_TRANS = 3.8
VALU_SLOTS_INT64 = 2.3
# Per sampled token the kernel issues (counters SQ_INSTS_VALU,
# SQ_INSTS_VALU_TRANS_F32 and SQ_INSTS_VALU_INT64 per dispatch, over the
# tokens; profiles/sd_sample_*_valu.txt) 36.5 (bf16) or 31.7 (fp32) VALU
# instructions per lane, of which 2.2 are transcendental (the exp2 of the
# weight, the log2 of -log2 U, and a share of the finisher's) and 4.84 are
# 64-bit integer (a Philox4x32-10 call has 18.1 v_mad_u64_u32 for 4 tokens:
# the first round's product of a uniform counter word is scalar).  The rest
# are full rate: the uniform map, the weight's exponent, the sum, the
# cross-multiplied comparison, unpacking and the maximum, loop and reduction
# overhead.  A greedy token takes about 1.5 full-rate instructions (unpack,
# maximum and its share of the argmax search).
DRAFT_INSTS_SAMPLED = {True: 36.5, False: 31.7}  # keyed by "rows are bf16"
DRAFT_TRANS_PER_TOKEN = 2.2
DRAFT_INT64_PER_TOKEN = 4.84
DRAFT_SLOTS_SAMPLED = {
    bf: n - DRAFT_TRANS_PER_TOKEN - DRAFT_INT64_PER_TOKEN + DRAFT_TRANS_PER_TOKEN * VALU_SLOTS_TRANS
    + DRAFT_INT64_PER_TOKEN * VALU_SLOTS_INT64 for bf, n in DRAFT_INSTS_SAMPLED.items()}
DRAFT_SLOTS_GREEDY = 1.5
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz: full-rate 32-bit VALU lane slots / s
PEAK_VALU_SLOTS = 256 * 4 * 32 * 2.4e9


def host_description() -> dict:
    """CPU model and core counts of the host the CPU baseline ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


# ------------------------------------------------------------------ rocprofv3 summaries


def _csv_rows(directory: str, suffix: str):
    """Rows of every rocprofv3 CSV under `directory` whose name ends in `suffix`."""
    import csv
    found = []
    for dp, _, files in os.walk(directory):
        for fn in sorted(files):
            if fn.endswith(suffix):
                with open(os.path.join(dp, fn), newline="") as f:
                    found.extend(csv.DictReader(f))
    if not found:
        raise SystemExit(f"no *{suffix} under {directory}")
    return found


def kernel_base_name(name: str) -> str:
    """`sv_verify` from `void (anonymous namespace)::sv_verify<true, true>(...)`."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("<")[0].split("(")[0].split("::")[-1].strip()


def _per_dispatch(rows, counter: str):
    """{dispatch id: (kernel name, counter value summed over its rows)} in dispatch order."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = out.get(d, (r["Kernel_Name"], 0.0))
        out[d] = (name, v + float(r["Counter_Value"]))
    return dict(sorted(out.items()))


KERNEL_OF_OP = {"verify": "sv_verify", "early-exit": "sv_verify_ee", "greedy": "sv_verify"}
# file-name tags of the workloads' profile summaries
SLUG = {1: "tiny_b1_k4_f32", 2: "llama_b64_k4_bf16", 3: "large_batch_b256_k8_f32",
        4: "mtp_b512_k1_bf16", 5: "ragged_b1024_bf16"}


def summarize_counters(args):
    """Traffic record of one kernel from FETCH_SIZE and WRITE_SIZE runs of
    `bench.py --traffic-probe MIB` (KiB per dispatch).  Each counter is scaled by
    what it reads for the probe's device copies of MIB MiB (MIB MiB read and
    MIB MiB written per copy)."""
    import numpy as np
    kernel = KERNEL_OF_OP[args.op]
    sources = EE_KERNEL_SOURCES if args.op == "early-exit" else KERNEL_SOURCES
    lines = []
    vals = {}
    for counter, directory in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_counters):
        disp = _per_dispatch(_csv_rows(directory, "counter_collection.csv"), counter)
        copies = [v for n, v in disp.values() if "copyBuffer" in n]
        mine = [v for n, v in disp.values() if kernel_base_name(n) == kernel]
        if len(copies) < 3 or not mine:
            raise SystemExit(f"{counter}: {len(copies)} copy and {len(mine)} {kernel} dispatches")
        copy_kib = float(np.median(copies[-5:]))
        size_kib = float(args.traffic_probe << 10)
        scale = size_kib / copy_kib
        mean = float(np.mean(mine))
        vals[counter] = (mean, scale, len(mine), float(np.min(mine)), float(np.max(mine)))
        lines.append(f"  {counter} per copy (KiB): {[round(c, 1) for c in copies[-5:]]}"
                     f"  -> scale {scale:.4f}")
    fetch = vals["FETCH_SIZE"][0] * vals["FETCH_SIZE"][1] * 1024
    write = vals["WRITE_SIZE"][0] * vals["WRITE_SIZE"][1] * 1024
    from rejection_sampling_verify_scaled_amd import workloads as W
    batch = W.make_batch(args.workload, 0)
    alg = algorithmic_bytes(batch)
    rec = {"kernel": kernel, "workload": args.workload,
           "source_sha256": kernel_source_sha256(sources),
           "hbm_bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
           "fetch_scale": vals["FETCH_SIZE"][1], "write_scale": vals["WRITE_SIZE"][1],
           "summary": f"profiles/{kernel}_{SLUG[args.workload]}_traffic.txt"}
    with open(os.path.join(ROOT, "profiles", f"traffic_{kernel}_workload{args.workload}.json"),
              "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    m, sc, n, lo, hi = vals["FETCH_SIZE"]
    print(f"HBM traffic of {kernel}, workload {args.workload} ({W.WORKLOADS[args.workload].name})")
    print(f"kernel source sha256: {rec['source_sha256']}")
    print(f"reference: the probe's device copies of {args.traffic_probe} MiB")
    print("\n".join(lines))
    print(f"{kernel}, {n} dispatches: FETCH_SIZE mean {m:.1f} KiB (min {lo:.1f}, max {hi:.1f});"
          f" WRITE_SIZE mean {vals['WRITE_SIZE'][0]:.1f} KiB")
    print(f"  scaled: read {fetch / 1e6:.2f} MB + written {write / 1e6:.3f} MB = "
          f"{(fetch + write) / 1e6:.2f} MB per launch")
    if args.op != "early-exit":
        print(f"  algorithmic bytes per launch: {alg / 1e6:.2f} MB; measured / algorithmic = "
              f"{(fetch + write) / alg:.3f}")


def summarize_pmc(args):
    """Per-kernel mean of each counter per dispatch (values summed over the
    counter's dimensions within a dispatch)."""
    import numpy as np
    rows = _csv_rows(args.summarize_pmc, "counter_collection.csv")
    per = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), kernel_base_name(r["Kernel_Name"]), r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by = {}
    for (_, name, counter), v in per.items():
        by.setdefault((name, counter), []).append(v)
    print(f"{'kernel':32s} {'counter':28s} {'dispatches':>10s} {'mean':>16s} {'median':>16s}")
    for (name, counter), v in sorted(by.items()):
        a = np.array(v)
        print(f"{name[:32]:32s} {counter[:28]:28s} {a.size:10d} {a.mean():16.1f} {np.median(a):16.1f}")


def summarize_trace(args):
    """Per-kernel dispatch durations from a rocprofv3 --kernel-trace run."""
    import numpy as np
    rows = _csv_rows(args.summarize_trace, "kernel_trace.csv")
    by = {}
    for r in rows:
        name = kernel_base_name(r["Kernel_Name"])
        by.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'kernel':60s} {'calls':>6s} {'mean us':>9s} {'median':>9s} {'min':>9s} {'max':>9s}")
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(d)
        print(f"{name[:60]:60s} {a.size:6d} {a.mean():9.2f} {np.median(a):9.2f} {a.min():9.2f} "
              f"{a.max():9.2f}")


VALU_RATE_OPS = (  # (label, VALU instructions per loop body, the body)
    ("fma", 1, "v_fma_f32"),
    ("exp2", 1, "v_exp_f32"),
    ("log2", 1, "v_log_f32"),
    ("mad64", 2, "v_mad_u64_u32 + v_add_u32"),
    ("mul_lo", 2, "v_mul_lo_u32 + v_add_u32"),
    ("xor_add", 2, "v_xor_b32 + v_add_u32"),
)


def valu_rates():
    """Issue cycles per wave64 instruction on one SIMD for the VALU classes the
    samplers use (csrc/valu_rates.hip): each probe runs 16 independent chains
    of one operation per thread, 8 workgroups of 256 threads per CU; its rate
    is stated per SIMD and shader clock cycle, with the shader clock read by
    the probe itself.  The add that completes the two-instruction bodies is
    taken at the xor + add probe's cost per instruction."""
    import torch

    from rejection_sampling_verify_scaled_amd import build as hip_build
    if not torch.cuda.is_available():
        raise SystemExit("--valu-rates needs a HIP GPU")
    if not os.path.exists(hip_build.LIB_RATES):
        raise SystemExit(f"{hip_build.LIB_RATES} is missing: build it with "
                         "`python -m rejection_sampling_verify_scaled_amd.build --all`")
    lib = ctypes.CDLL(hip_build.LIB_RATES)
    lib.sv_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                 ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    lib.sv_valu_rate.restype = ctypes.c_int
    hip = Hip()
    khz = ctypes.c_int()
    hip.lib.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                              ctypes.c_int]
    HIP_ATTR_WALL_CLOCK_RATE = 10017  # hipDeviceAttributeWallClockRate (hip_runtime_api.h)
    if hip.lib.hipDeviceGetAttribute(ctypes.byref(khz), HIP_ATTR_WALL_CLOCK_RATE, 0) != 0:
        raise SystemExit("hipDeviceGetAttribute(wall clock rate) failed")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    simds = 4 * cus
    res = {}
    for op, (label, n_inst, body) in enumerate(VALU_RATE_OPS):
        ms, bodies, mhz = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
        if lib.sv_valu_rate(op, cus, khz.value / 1e3, ctypes.byref(ms), ctypes.byref(bodies),
                            ctypes.byref(mhz)) != 0:
            raise SystemExit(f"sv_valu_rate({op}) failed")
        rate = bodies.value / (ms.value * 1e-3)                  # loop bodies per second
        per_simd_cycle = rate / (simds * mhz.value * 1e6)       # lane bodies per SIMD cycle
        res[label] = (n_inst, body, ms.value, rate, mhz.value, 64.0 / per_simd_cycle)
    add_cycles = res["xor_add"][5] / 2
    print(f"VALU issue rates on {cus} CUs ({simds} SIMDs); cycles per wave64 instruction "
          f"on one SIMD at the shader clock the probe saw")
    print(f"  {'probe':8s} {'loop body':28s} {'ms':>7s} {'T bodies/s':>11s} {'MHz':>6s} "
          f"{'cycles/body':>11s} {'cycles/instr':>12s}")
    for label, (n_inst, body, ms, rate, mhz, cyc) in res.items():
        own = cyc if n_inst == 1 else (cyc / 2 if label == "xor_add" else cyc - add_cycles)
        print(f"  {label:8s} {body:28s} {ms:7.3f} {rate / 1e12:11.2f} {mhz:6.0f} {cyc:11.2f} "
              f"{own:12.2f}")


def stage_trace(args):
    """Per-stage timeline of sv_verify from the stage-trace build.

    Each workgroup of the trace build records its role and the wall clock at
    numbered stages (spec_verify.hip, SV_STAMP): statistics workgroups at
    start, scalars loaded, partials stored (and, for a greedy request's
    finisher, partials folded and outputs written); race workgroups at start,
    scalars loaded, last partial seen, partials folded, ratio tests done,
    chunks raced, winner stored, and the finisher at winners collected and
    outputs written.  Times are per call, from the first workgroup's start,
    averaged over the traced calls; a sampled request's chain is measured from
    the last store of its partials."""
    import numpy as np
    import torch

    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import build as hip_build
    from rejection_sampling_verify_scaled_amd import workloads as W

    if not os.path.exists(hip_build.LIB_TRACE):
        raise SystemExit(f"{hip_build.LIB_TRACE} is missing: build it with "
                         "`python -m rejection_sampling_verify_scaled_amd.build --all`")
    lib = binding.load_library(hip_build.LIB_TRACE)
    lib.spec_verify_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.spec_verify_trace_copy.restype = ctypes.c_int
    lib.spec_verify_trace_reset.restype = ctypes.c_int
    lib.spec_verify_trace_points.restype = ctypes.c_int
    npts = lib.spec_verify_trace_points()
    hip = Hip()
    khz = ctypes.c_int()
    hip.lib.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                              ctypes.c_int]
    HIP_ATTR_WALL_CLOCK_RATE = 10017  # hipDeviceAttributeWallClockRate (hip_runtime_api.h)
    if hip.lib.hipDeviceGetAttribute(ctypes.byref(khz), HIP_ATTR_WALL_CLOCK_RATE, 0) != 0:
        raise SystemExit("hipDeviceGetAttribute(wall clock rate) failed")
    us_per_tick = 1e3 / khz.value
    dev = torch.device("cuda:0")
    batch = W.make_batch(args.workload, 0)
    d = binding.to_device_batch(batch, dev)
    per_copy = d["target"].numel() * d["target"].element_size() + \
        d["draft"].numel() * d["draft"].element_size()
    copies = args.copies or max(1, math.ceil(1.25e9 / per_copy))
    targets = [d["target"]] + [d["target"].clone() for _ in range(copies - 1)]
    drafts = [d["draft"]] + [d["draft"].clone() for _ in range(copies - 1)]
    ws = binding.new_workspace(batch.B, batch.V, batch.max_k)

    def call(c):
        binding.spec_verify_sample(targets[c], drafts[c], d["offsets"], d["tokens"],
                                   d["temperature"], batch.seed, batch.max_k, workspace=ws,
                                   lib=lib)

    for i in range(args.warmup):
        call(i % copies)
    torch.cuda.synchronize()
    n_words = (1 << 16) * npts
    buf = np.zeros(n_words, dtype=np.uint64)
    rows, streams = [], []
    for i in range(args.steps):
        if lib.spec_verify_trace_reset() != 0:
            raise SystemExit("trace reset failed")
        call(i % copies)
        torch.cuda.synchronize()
        if lib.spec_verify_trace_copy(buf.ctypes.data_as(ctypes.c_void_p), n_words) != 0:
            raise SystemExit("trace copy failed")
        rec = buf.reshape(-1, npts).copy()
        rows.append(trace_summary(rec, batch, us_per_tick))
        streams.append(stream_profile(rec, batch, us_per_tick))
    keys = rows[0].keys()
    print(f"stage timeline of sv_verify, workload {args.workload} ({W.WORKLOADS[args.workload].name}),"
          f" {args.steps} traced calls after {args.warmup} untraced; trace build "
          f"(-DSV_TRACE); us, mean over calls")
    for k in keys:
        vals = [r[k] for r in rows if r.get(k) is not None]
        if vals:
            print(f"  {k:58s} {np.mean(vals):8.2f}   (min {np.min(vals):7.2f}, max {np.max(vals):7.2f})")
    if streams[0] is not None:
        prof = np.mean(np.stack(streams), axis=0)
        print("stream over time (flat grouping; mean over calls; t from the first workgroup's start):")
        print("  window (us)   blocks done (TB/s)   bytes in flight at t (MB)   "
              "race wgs resident at t   statistics wgs waiting for scalars at t")
        for i, (rate, infl, races, waiting) in enumerate(prof):
            if i > 0 and rate == 0 and infl == 0 and races < 0.5:
                break
            t = i * STREAM_WINDOW_US
            print(f"  [{t:4.0f},{t + STREAM_WINDOW_US:4.0f})   {rate:18.2f}   {infl:25.1f}   "
                  f"{races:22.0f}   {waiting:38.0f}")


STREAM_WINDOW_US = 2.0


def stream_profile(rec, batch, us_per_tick, n_windows=80):
    """One traced call's stream over time, for flat grouping (every request
    has max_k drafts; None otherwise): per window of STREAM_WINDOW_US from the
    first workgroup's start, the row bytes of the statistics blocks whose
    partial was stored in it (as TB/s), and at the window's start the bytes
    of blocks whose scalars had arrived but whose partial was not yet stored,
    the race workgroups started and not yet done, and the statistics
    workgroups started but still waiting for their request's scalars.  A
    block's bytes are its chunks of its row (8 KiB each, the row's last one
    shorter); a greedy request's groups past its K+1 rows hold none."""
    import numpy as np

    from rejection_sampling_verify_scaled_amd import workloads as W
    if batch.n_draft_rows != batch.B * batch.max_k:
        return None
    esz = 2 if batch.dtype == W.DTYPE_BF16 else 4
    chunk = 8192 // esz
    nc = -(-batch.V // chunk)
    bpr = -(-nc // 8)
    head = rec[:, 0]
    live = head != 0
    rec, head = rec[live].astype(np.int64), head[live]
    kind = (head & 0xFF).astype(int)
    req = ((head >> 8) & 0xFFFFFF).astype(int)
    grp = (head >> 32).astype(int)
    t0 = rec[:, 1][rec[:, 1] > 0].min()
    us = (rec - t0) * us_per_tick
    s_m = (kind == 1) & (rec[:, 3] > 0)
    nbytes = np.zeros(len(rec))
    for i in np.nonzero(s_m)[0]:
        b = req[i]
        nrows = batch.max_k + 1 if batch.temperature[b] == 0 else 2 * batch.max_k + 1
        row, blk = divmod(grp[i], bpr)
        if row >= nrows:
            continue
        c0, c1 = blk * 8, min(blk * 8 + 8, nc)
        tokens = min(c1 * chunk, batch.V) - c0 * chunk
        nbytes[i] = tokens * esz
    r_m = kind == 2
    r_end = us[:, 1:].max(axis=1)
    out = np.zeros((n_windows, 4))
    for w in range(n_windows):
        t = w * STREAM_WINDOW_US
        done = s_m & (us[:, 3] > t) & (us[:, 3] <= t + STREAM_WINDOW_US)
        out[w, 0] = nbytes[done].sum() / (STREAM_WINDOW_US * 1e6)
        infl = s_m & (us[:, 2] <= t) & (us[:, 3] > t)
        out[w, 1] = nbytes[infl].sum() / 1e6
        out[w, 2] = (r_m & (us[:, 1] <= t) & (r_end > t)).sum()
        out[w, 3] = ((kind == 1) & (us[:, 1] <= t) & (us[:, 2] > t)).sum()
    return out


CROSSOVER_CASES = {2: (16, 32, 64), 4: (64, 128, 256, 512), 3: (16, 32, 64, 128, 256),
                   5: (64, 128, 256, 512, 1024)}


def crossover(rounds: int = 7):
    """Full verify (spec_verify_sample) against the early-exit verify on the
    first B requests of each workload: both entry points in one process on
    the same inputs, rotated over enough input copies to leave the Infinity
    Cache, timed with HIP events over back-to-back calls in `rounds`
    interleaved rounds (median); the accept lengths of the two are compared."""
    import numpy as np
    import torch

    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import workloads as W

    lib = binding.load_library()
    dev = torch.device("cuda:0")
    vp = ctypes.c_void_p
    print(f"full verify against early exit, us per call (median of {rounds} interleaved rounds)")
    for wl, sizes in CROSSOVER_CASES.items():
        full = W.make_batch(wl, 0)
        for B in sizes:
            batch = W.subset_requests(full, range(B)) if B < full.B else full
            d = binding.to_device_batch(batch, dev)
            V, K, n_d = batch.V, batch.max_k, batch.n_draft_rows
            per_copy = d["target"].numel() * d["target"].element_size() + \
                d["draft"].numel() * d["draft"].element_size()
            copies = max(1, math.ceil(1.25e9 / per_copy))
            tg = [d["target"]] + [d["target"].clone() for _ in range(copies - 1)]
            dr = [d["draft"]] + [d["draft"].clone() for _ in range(copies - 1)]
            acc = torch.empty(B, dtype=torch.int32, device=dev)
            out = torch.empty(n_d + B, dtype=torch.int32, device=dev)
            st = torch.cuda.current_stream(dev)
            dt = binding.SV_BF16 if d["target"].dtype == torch.bfloat16 else binding.SV_F32
            fns = [(lib.spec_verify_sample, binding.workspace_bytes(B, V, K)),
                   (lib.spec_verify_sample_early_exit, binding.early_exit_workspace_bytes(B, V, K))]
            wss = [torch.zeros(n, dtype=torch.uint8, device=dev) for _, n in fns]

            def call(j, c):
                f, n = fns[j]
                rc = f(vp(tg[c].data_ptr()), vp(dr[c].data_ptr()), dt, B, V, K, n_d,
                       vp(d["offsets"].data_ptr()), vp(d["tokens"].data_ptr()),
                       vp(d["temperature"].data_ptr()), ctypes.c_uint64(batch.seed),
                       vp(acc.data_ptr()), vp(out.data_ptr()), None, None, vp(wss[j].data_ptr()),
                       n, vp(st.cuda_stream))
                if rc != 0:
                    raise SystemExit(f"call returned {rc}")
            accs = []
            for j in range(2):
                for i in range(5):
                    call(j, i % copies)
                call(j, 0)
                torch.cuda.synchronize()
                accs.append(acc.cpu().numpy().copy())
            steps = 50 if wl in (2, 4) else 10
            T = np.zeros((rounds, 2))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            for r in range(rounds):
                for j in ((0, 1) if r % 2 == 0 else (1, 0)):
                    for i in range(3):
                        call(j, i % copies)
                    e0.record(st)
                    for i in range(steps):
                        call(j, i % copies)
                    e1.record(st)
                    torch.cuda.synchronize()
                    T[r, j] = e0.elapsed_time(e1) * 1e3 / steps
            same = int((accs[0] == accs[1]).sum())
            print(f"  workload {wl} ({W.WORKLOADS[wl].name.split()[0]}) B={B:5d}  full {np.median(T[:, 0]):8.1f}"
                  f"  early exit {np.median(T[:, 1]):8.1f}  accept_len agree {same}/{B}", flush=True)


def trace_summary(rec, batch, us_per_tick) -> dict:
    """One traced call's stage figures (see stage_trace)."""
    import numpy as np
    head = rec[:, 0]
    live = head != 0
    rec, head = rec[live], head[live]
    kind = (head & 0xFF).astype(int)
    req = ((head >> 8) & 0xFFFFFF).astype(int)
    st = rec.astype(np.int64)
    t0 = st[:, 1][st[:, 1] > 0].min()

    def us(x):
        return (x - t0) * us_per_tick

    out = {}
    ends = st[:, 1:].max(axis=1)
    out["kernel span (first start to last stamp)"] = us(ends.max())
    s_m = kind == 1
    out["statistics workgroup: scalars loaded after start"] = float(
        np.mean((st[s_m, 2] - st[s_m, 1]) * us_per_tick)) if s_m.any() else None
    out["statistics workgroup: partials stored after start"] = float(
        np.mean((st[s_m & (st[:, 3] > 0), 3] - st[s_m & (st[:, 3] > 0), 1]) * us_per_tick))
    out["last partial stored (all requests)"] = us(st[s_m, 3].max())
    chain = {k: [] for k in ("seen", "fold", "ratio", "race", "winners", "collected", "outputs",
                             "race_start", "last_stats")}
    greedy_tail = []
    for b in range(batch.B):
        sb = s_m & (req == b)
        if not sb.any():
            continue
        last = st[sb, 3].max()
        rb = (kind == 2) & (req == b)
        if batch.temperature[b] > 0 and rb.any():
            r = st[rb]
            fin = r[r[:, 9] > 0]
            if len(fin) == 0:
                continue
            chain["last_stats"].append(us(last))
            chain["race_start"].append(float(np.median(r[:, 1]) - last) * us_per_tick)
            chain["seen"].append(float(np.median(r[:, 3]) - last) * us_per_tick)
            chain["fold"].append(float(np.median(r[:, 4]) - np.median(r[:, 3])) * us_per_tick)
            chain["ratio"].append(float(np.median(r[:, 5]) - np.median(r[:, 4])) * us_per_tick)
            chain["race"].append(float(r[:, 6].max() - np.median(r[:, 5])) * us_per_tick)
            chain["winners"].append(float(r[:, 7].max() - r[:, 6].max()) * us_per_tick)
            chain["collected"].append(float(fin[0, 8] - r[:, 7].max()) * us_per_tick)
            chain["outputs"].append(float(fin[0, 9] - fin[0, 8]) * us_per_tick)
        elif batch.temperature[b] == 0:
            f = st[sb & (st[:, 5] > 0)]
            if len(f):
                greedy_tail.append((f[0, 5] - last) * us_per_tick)
    # what ends the kernel: the latest sampled outputs against the latest greedy outputs
    s_out = st[(kind == 2) & (st[:, 9] > 0), 9]
    g_out = st[(kind == 1) & (st[:, 5] > 0), 5]
    if len(s_out):
        out["sampled: last request's outputs written"] = us(s_out.max())
        out["sampled: last request's statistics complete"] = float(np.max(chain["last_stats"])) \
            if chain["last_stats"] else None
    if len(g_out):
        out["greedy: last request's outputs written"] = us(g_out.max())
    if chain["seen"]:
        out["sampled: last partial stored (mean over requests)"] = float(np.mean(chain["last_stats"]))
        out["sampled: race workgroup start, from the last partial"] = float(np.mean(chain["race_start"]))
        out["sampled: last partial seen by the race workgroups"] = float(np.mean(chain["seen"]))
        out["sampled: partials folded"] = float(np.mean(chain["fold"]))
        out["sampled: ratio tests done (z(x_t) gathers)"] = float(np.mean(chain["ratio"]))
        out["sampled: row n loaded and raced (slowest workgroup)"] = float(np.mean(chain["race"]))
        out["sampled: winners stored"] = float(np.mean(chain["winners"]))
        out["sampled: finisher collected the winners"] = float(np.mean(chain["collected"]))
        out["sampled: outputs written"] = float(np.mean(chain["outputs"]))
        total = [sum(x) for x in zip(chain["seen"], chain["fold"], chain["ratio"], chain["race"],
                                     chain["winners"], chain["collected"], chain["outputs"])]
        out["sampled: chain, last partial to outputs"] = float(np.mean(total))
    if greedy_tail:
        out["greedy: last partial to outputs (finisher)"] = float(np.mean(greedy_tail))
    return out


def bench_draft(args):
    """Draft-side sampler: one spec_draft_sample call per step over the
    workload's draft rows at draft step 0 (one row per request)."""
    import numpy as np
    import torch

    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import workloads as W

    lib = binding.load_library()
    dev = torch.device("cuda:0")
    batch = W.make_batch(args.workload, 0)
    rows = W.draft_step_rows(batch, 0)
    B, V = rows.shape
    esz = 2 if batch.dtype == W.DTYPE_BF16 else 4
    if batch.dtype == W.DTYPE_BF16:
        x0 = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(
            torch.bfloat16)
    else:
        x0 = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).to(dev)
    per_copy = B * V * esz
    copies = args.copies or max(2, math.ceil(1.25e9 / per_copy))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    temp = torch.from_numpy(batch.temperature.astype(np.float32)).to(dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    q = torch.empty(B, dtype=torch.float32, device=dev)
    ws = torch.zeros(binding.draft_workspace_bytes(B, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    vp = ctypes.c_void_p
    dt = binding.SV_BF16 if batch.dtype == W.DTYPE_BF16 else binding.SV_F32

    def call(i):
        rc = lib.spec_draft_sample(vp(xs[i % copies].data_ptr()), dt, B, V, vp(temp.data_ptr()),
                                   ctypes.c_uint64(batch.seed), 0, vp(tok.data_ptr()),
                                   vp(q.data_ptr()), vp(ws.data_ptr()), ws.numel(), sh)
        if rc != 0:
            raise SystemExit(f"spec_draft_sample returned {rc}")

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    n_s = int((batch.temperature > 0).sum())
    slots = (n_s * DRAFT_SLOTS_SAMPLED[batch.dtype == W.DTYPE_BF16] +
             (B - n_s) * DRAFT_SLOTS_GREEDY) * V
    achieved = slots / (us * 1e-6)
    call(0)
    torch.cuda.synchronize()
    gpu_tok = tok.cpu().numpy()
    line = {
        "metric": "draft tokens drawn/sec (draft-side sampler, one token per request)",
        "value": B / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if batch.dtype == W.DTYPE_BF16 else "f32", "data": "synthetic",
        "config": {"workload": batch.label + ", draft rows at step 0", "B": B, "V": V,
                   "sampled_rows": n_s, "greedy_rows": B - n_s, "input_copies_rotated": copies},
        "kernel_us": {"sd_sample": us},
        "roofline": {"bound": "alu", "achieved": achieved / 1e12, "peak": PEAK_VALU_SLOTS / 1e12,
                     "unit": "T full-rate VALU lane-slots/s", "frac": achieved / PEAK_VALU_SLOTS,
                     "traffic": None, "kernel": "sd_sample"},
        "hbm_gbs": per_copy / (us * 1e-6) / 1e9,
        "hbm_frac": per_copy / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
    }
    if not args.no_cpu_baseline:
        import oracle
        olib = oracle.load()
        t0 = time.perf_counter()
        passes = 0
        while True:
            ref = oracle.draft_sample(batch.dtype, rows, batch.temperature, batch.seed, 0,
                                      lib=olib)
            passes += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        cpu_s = time.perf_counter() - t0
        flagged = (ref["flags"] & oracle.FLAG_RACE_NEAR_TIE) != 0
        line["cpu_baseline"] = {
            "value": B * passes / cpu_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes over the {B} draft rows (single-threaded float64 C "
                      f"oracle, {cpu_s:.1f} s)"}
        line["parity_check"] = {"rows": B, "unflagged_mismatches":
                                int(((gpu_tok != ref["tokens"]) & ~flagged).sum()),
                                "flagged": int(flagged.sum())}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def bench_commit(args):
    """Commit step: one spec_commit_tokens call per step, appending the
    workload's verify outputs (computed by the oracle before timing) to
    token histories of 4096 entries."""
    import numpy as np
    import torch

    import oracle
    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import workloads as W

    dev = torch.device("cuda:0")
    batch = W.make_batch(args.workload, 0)
    B = batch.B
    reqs = None if B <= 64 else list(range(0, B, 16))
    v = oracle.verify_batch(batch, reqs=reqs)
    acc = v["accept_len"].copy()
    acc[acc == -2] = -1
    cap = 4096
    rng = np.random.default_rng(args.workload)
    lens0 = rng.integers(0, 1024, size=B).astype(np.int32)
    seq = torch.zeros((B, cap), dtype=torch.int32, device=dev)
    lens = torch.from_numpy(lens0).to(dev)
    offs = torch.from_numpy(batch.offsets.astype(np.int32)).to(dev)
    acc_d = torch.from_numpy(acc).to(dev)
    out_d = torch.from_numpy(v["out_tokens"].astype(np.int32)).to(dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = min(args.steps, (cap - 1024) // (batch.max_k + 1))  # histories never fill

    lib = binding.load_library()
    vp = ctypes.c_void_p
    cargs = (B, batch.max_k, batch.n_draft_rows, vp(offs.data_ptr()), vp(acc_d.data_ptr()),
             vp(out_d.data_ptr()), vp(seq.data_ptr()), cap, vp(lens.data_ptr()), cap,
             vp(nxt.data_ptr()), vp(st.data_ptr()), vp(stream.cuda_stream))

    def call():
        rc = lib.spec_commit_tokens(*cargs)
        if rc != 0:
            raise SystemExit(f"spec_commit_tokens returned {rc}")

    for _ in range(min(args.warmup, 5)):
        call()
    torch.cuda.synchronize()
    lens.copy_(torch.from_numpy(lens0))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    # bytes each call must move: slices, accept_len, lengths (read and written),
    # the emitted tokens (read and written), next_tokens and status
    n_emit = int(np.where(acc >= 0, acc + 1, 0).sum())
    moved = 4 * (2 * (B + 1) + B + 2 * B + 2 * n_emit + 2 * B)
    line = {
        "metric": "requests committed/sec (commit step after verification)",
        "value": B / (us * 1e-6), "unit": "requests/s", "n_gpus": 1, "steps": steps,
        "warmup": min(args.warmup, 5), "ms_per_step": us * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": batch.label + ", its verify outputs", "B": B,
                   "emitted_tokens": n_emit, "history_capacity": cap},
        "kernel_us": {"commit_kernel": us},
        "roofline": {"bound": "hbm", "achieved": moved / (us * 1e-6) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": moved / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "kernel": "commit_kernel",
                     "note": "a few KB per call: launch- and latency-bound"},
    }
    if not args.no_cpu_baseline:
        seq0 = np.zeros((B, cap), np.int32)
        t0 = time.perf_counter()
        passes = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 3.0):
            oracle.commit_tokens(batch.offsets, acc, v["out_tokens"], seq0, lens0, batch.max_k,
                                 n_draft_rows=batch.n_draft_rows)
            passes += 1
        cpu_s = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": B * passes / cpu_s, "unit": "requests/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes over the {B} requests (C oracle, {cpu_s:.1f} s, "
                      "including its copy of the histories)"}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def bench_tree(args):
    """Greedy draft-tree verification: one spec_verify_tree_greedy call per step
    over a seeded tree workload; every node's row is read once."""
    import numpy as np
    import torch

    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import workloads as W

    dev = torch.device("cuda:0")
    print(f"[bench] generating {args.tree}", file=sys.stderr, flush=True)
    tb = W.make_tree_batch(args.tree)
    d = binding.to_device_tree_batch(tb, dev)
    B, V, n = tb.B, tb.V, int(tb.offsets[-1])
    nodes = n - B  # draft nodes verified per step
    alg = n * V * (2 if tb.dtype == W.DTYPE_BF16 else 4)
    copies = args.copies or max(1, math.ceil(1.25e9 / alg))
    targets = [d["target"]] + [d["target"].clone() for _ in range(copies - 1)]
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    acc_nodes = torch.empty(n, dtype=torch.int32, device=dev)
    lib = binding.load_library()
    ws_n = binding.tree_workspace_bytes(B, V, tb.max_nodes)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p
    dtype = binding.SV_BF16 if tb.dtype == W.DTYPE_BF16 else binding.SV_F32
    argsets = [(vp(t.data_ptr()), dtype, B, V, tb.max_nodes, n, vp(d["offsets"].data_ptr()),
                vp(d["parents"].data_ptr()), vp(d["tokens"].data_ptr()), vp(acc.data_ptr()),
                vp(out.data_ptr()), vp(acc_nodes.data_ptr()), vp(ws.data_ptr()), ws_n,
                vp(stream.cuda_stream)) for t in targets]

    def call(i):
        rc = lib.spec_verify_tree_greedy(*argsets[i % copies])
        if rc != 0:
            raise SystemExit(f"spec_verify_tree_greedy returned {rc}")

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    us = ms * 1e3
    print(f"[bench] tv_verify {us:.2f} us per launch over the timed region", file=sys.stderr,
          flush=True)
    call(0)
    torch.cuda.synchronize()
    g_acc, g_out, g_nodes = acc.cpu().numpy(), out.cpu().numpy(), acc_nodes.cpu().numpy()
    achieved = alg / (us * 1e-6) / 1e9
    line = {
        "metric": "verified draft-tree nodes/sec (greedy tree verification) + HBM GB/s",
        "value": nodes / (us * 1e-6), "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dtype == binding.SV_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": tb.label, "B": B, "V": V, "nodes": n, "max_nodes": tb.max_nodes,
                   "input_copies_rotated": copies, "entry_point": "spec_verify_tree_greedy"},
        "algorithmic_bytes_per_step": alg,
        "kernel_us": {"tv_verify": us},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": "tv_verify"},
    }
    if not args.no_cpu_baseline:
        import oracle
        olib = oracle.load()
        t0 = time.perf_counter()
        passes = 0
        while True:
            res = oracle.tree_verify(tb.dtype, tb.target, tb.offsets, tb.parents, tb.tokens, V,
                                     tb.max_nodes, lib=olib)
            passes += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        cpu_s = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": nodes * passes / cpu_s, "unit": "nodes/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes over the full {B}-tree batch (single-threaded float64 C "
                      f"oracle, {cpu_s:.1f} s)"}
        line["parity_check"] = {
            "requests": B,
            "mismatches": int((g_acc != res["accept_len"]).sum()
                              + (g_out != res["out_tokens"]).any()
                              + (g_nodes != res["accept_nodes"]).any())}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.valu_rates:
        valu_rates()
        return
    if args.stage_trace:
        if args.gpus != 1:
            raise SystemExit("bench.py measures one GPU")
        stage_trace(args)
        return
    if args.crossover:
        if args.gpus != 1:
            raise SystemExit("bench.py measures one GPU")
        crossover()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the verify step is per request, so several GPUs would each run it on "
              "their own requests; no multi-GPU layer is part of this library)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a HIP GPU")
    if args.op == "draft":
        bench_draft(args)
        return
    if args.op == "commit":
        bench_commit(args)
        return
    if args.op == "tree":
        bench_tree(args)
        return
    from rejection_sampling_verify_scaled_amd import binding
    from rejection_sampling_verify_scaled_amd import workloads as W

    lib = binding.load_library()
    hip = Hip()
    dev = torch.device("cuda:0")
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    greedy = args.op == "greedy"
    batch = W.make_batch(args.workload, 0, temperature_override=0.0 if greedy else None)
    d = binding.to_device_batch(batch, dev)
    B, V, K = batch.B, batch.V, batch.max_k
    n_d = batch.n_draft_rows
    positions = int(batch.k.sum())
    alg = algorithmic_bytes(batch)
    per_copy = d["target"].numel() * d["target"].element_size() + \
        d["draft"].numel() * d["draft"].element_size()
    copies = args.copies or max(1, math.ceil(1.25e9 / per_copy))
    targets = [d["target"]] + [d["target"].clone() for _ in range(copies - 1)]
    drafts = [d["draft"]] + [d["draft"].clone() for _ in range(copies - 1)]
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(n_d + B, dtype=torch.int32, device=dev)
    pa = torch.empty(n_d, dtype=torch.float32, device=dev)
    qa = torch.empty(n_d, dtype=torch.float32, device=dev)
    ee = args.op == "early-exit"
    ws_n = binding.early_exit_workspace_bytes(B, V, K) if ee else binding.workspace_bytes(B, V, K)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    dtype = binding.SV_BF16 if d["target"].dtype == torch.bfloat16 else binding.SV_F32
    vp = ctypes.c_void_p
    argsets = []
    for c in range(copies):
        if greedy:  # the all-greedy entry point: no draft logits, temperatures or seed
            argsets.append((vp(targets[c].data_ptr()), dtype, B, V, K, n_d,
                            vp(d["offsets"].data_ptr()), vp(d["tokens"].data_ptr()),
                            vp(acc.data_ptr()), vp(out.data_ptr()), vp(ws.data_ptr()), ws_n, sh))
            continue
        argsets.append((vp(targets[c].data_ptr()), vp(drafts[c].data_ptr()), dtype, B, V, K, n_d,
                        vp(d["offsets"].data_ptr()), vp(d["tokens"].data_ptr()),
                        vp(d["temperature"].data_ptr()), ctypes.c_uint64(batch.seed),
                        vp(acc.data_ptr()), vp(out.data_ptr()), vp(pa.data_ptr()),
                        vp(qa.data_ptr()), vp(ws.data_ptr()), ws_n, sh))
    call = (lib.spec_verify_sample_early_exit if ee else
            lib.spec_verify_greedy if greedy else lib.spec_verify_sample)
    name = ("spec_verify_sample_early_exit" if ee else
            "spec_verify_greedy" if greedy else "spec_verify_sample")
    torch.cuda.synchronize()
    print(f"[bench] B={B} K={K} V={V} copies={copies} ({copies * per_copy / 1e9:.2f} GB); "
          f"warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        rc = call(*argsets[i % copies])
        if rc != 0:
            raise SystemExit(f"{name} returned {rc}")
    torch.cuda.synchronize()

    if args.traffic_probe:
        for i in range(args.steps):
            call(*argsets[i % copies])
        src = torch.ones(args.traffic_probe << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] traffic probe: {args.steps} verify calls, 5 copies of "
              f"{args.traffic_probe} MiB", file=sys.stderr, flush=True)
        return

    # ---- timed region: exactly `steps` steps, synchronised on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        call(*argsets[i % copies])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = positions / (ms_per_step * 1e-3)
    print(f"[bench] {ms_per_step * 1e3:.2f} us/step (wall {wall / args.steps * 1e6:.2f} us/step)",
          file=sys.stderr, flush=True)

    # ---- cross-check: events the library records around each single launch
    # (each pair of event records adds its own small overhead to the figure)
    k_us = ms_per_step * 1e3
    if ee or greedy:
        # the timed region is `steps` back-to-back calls of two launches each:
        # sv_verify_ee, then the small kernel that clears its decision records
        ev_us = None
        what = "sv_verify_ee + ee_clear_records" if ee else "sv_verify (all greedy)"
        print(f"[bench] {what} {k_us:.2f} us per call over the timed region", file=sys.stderr,
              flush=True)
    else:
        n_t = min(args.steps, 200)
        evs = [(hip.event(), hip.event()) for _ in range(n_t)]
        timed = lib.spec_verify_sample_timed
        for i in range(n_t):
            rc = timed(*argsets[i % copies], evs[i][0], evs[i][1])
            if rc != 0:
                raise SystemExit(f"spec_verify_sample_timed returned {rc}")
        torch.cuda.synchronize()
        ev_us = 1e3 * sum(hip.elapsed_ms(a, b) for a, b in evs) / n_t
        # the timed region is `steps` back-to-back launches of the one kernel
        print(f"[bench] sv_verify kernel {k_us:.2f} us per launch over the timed region, "
              f"{ev_us:.2f} us with events around each launch", file=sys.stderr, flush=True)

    # ---- the achievable line: a plain 1 GiB device-to-device copy (torch's copy
    # kernel) on the same stream, counted as bytes read plus bytes written
    cp_src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        cp_dst.copy_(cp_src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    n_cp = 10
    c0.record(stream)
    for _ in range(n_cp):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * cp_src.numel() * n_cp / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cp_src, cp_dst

    # ---- correctness spot check of this exact launch configuration
    call(*argsets[0])
    torch.cuda.synchronize()
    gpu_acc = acc.cpu().numpy()
    gpu_out = out.cpu().numpy()
    if ee:
        # the rows this outcome needs (the accept lengths are checked against
        # the oracle below)
        alg = early_exit_bytes(batch, gpu_acc)
    achieved = alg / (k_us * 1e-6) / 1e9

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dtype == binding.SV_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": batch.label, "B": B, "K": K, "V": V,
                   "sampled_requests": int((batch.temperature > 0).sum()),
                   "greedy_requests": int((batch.temperature == 0).sum()),
                   "input_copies_rotated": copies,
                   "entry_point": name},
        "hbm_gbs_step": alg / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_step": alg / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": alg,
        "bytes_per_verified_position": alg / positions,
        "kernel_us": ({"sv_verify_ee_and_clear": k_us} if ee else {"sv_verify": k_us} if greedy
                      else {"sv_verify": k_us, "sv_verify_single_launch_events": ev_us}),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": (traffic_record(args.workload, "sv_verify_ee", EE_KERNEL_SOURCES)
                                 if ee else None if greedy else traffic_record(args.workload)),
                     "kernel": "sv_verify_ee" if ee else "sv_verify"},
        "copy_gbs": {"value": copy_gbs, "frac": copy_gbs / PEAK_HBM_GBS,
                     "what": "1 GiB device-to-device copy on the same stream, read + written bytes"},
    }
    # tokens emitted per step: the accepted drafts and one stop or bonus token
    # per request that did not fail (every timed step runs the same inputs)
    emitted = int(sum(int(a) + 1 for a in gpu_acc if a >= 0))
    line["emitted_tokens_per_s"] = emitted / (ms_per_step * 1e-3)
    if line["roofline"]["traffic"] is not None:
        # counter bytes per launch over the kernel's duration in the timed region
        line["traffic_gbs"] = line["roofline"]["traffic"] / (k_us * 1e-6) / 1e9

    if not args.no_cpu_baseline:
        import oracle
        print(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        olib = oracle.load()
        threads = oracle.default_threads()
        legs = {}
        res = None
        # the same oracle single-threaded, then with its requests split over
        # `threads` worker threads; half the CPU time each
        for n_thr in (1, threads):
            t0 = time.perf_counter()
            passes = 0
            while True:
                res = oracle.verify_batch(batch, lib=olib, threads=n_thr)
                passes += 1
                if time.perf_counter() - t0 >= args.cpu_seconds / 2:
                    break
            legs[n_thr] = (passes, time.perf_counter() - t0)
        greedy = batch.temperature == 0
        mism = 0
        for b in range(B):
            base = int(batch.offsets[b]) + b
            k = int(batch.offsets[b + 1] - batch.offsets[b])
            same = gpu_acc[b] == res["accept_len"][b] and \
                (gpu_out[base:base + k + 1] == res["out_tokens"][base:base + k + 1]).all()
            flagged = (not greedy[b]) and res["flags"][b] != 0
            if not same and not flagged:
                mism += 1
        (p1, s1), (pn, sn) = legs[1], legs[threads]
        line["cpu_baseline"] = {
            "value": positions * pn / sn, "unit": "positions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{pn} passes over the full {B}-request batch of the same workload "
                      f"(float64 C oracle, requests split over {threads} threads, {sn:.1f} s)",
            "single_core": {"value": positions * p1 / s1, "cores": 1,
                            "sample": f"{p1} passes, one thread, {s1:.1f} s"},
            "host": host_description()}
        line["parity_check"] = {"requests": B, "unflagged_mismatches": int(mism),
                                "flagged": int((res["flags"] != 0).sum())}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
