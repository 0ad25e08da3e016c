#!/usr/bin/env python3
"""Throughput of the fused K-quant dequant-GEMV on one MI355X.

Default workload: one decode step of a Llama-3-70B-shaped model at batch 1 --
80 distinct layers, each wq/wo 8192x8192, wk 1024x8192, w1/w3 28672x8192 in
Q4_K and wv 1024x8192, w2 8192x28672 in Q6_K (the Q4_K_M mix), all resident
in HBM (43.5 GB of packed weights).  One step = one product over every one of
the 560 matrices; matrices that read the same activations (k, q and v; w1
and w3) go through one grouped call -- 320 launches per step, k+q+v as one
launch with the Q4_K and Q6_K rows side by side (--no-group: one launch per
matrix).  The metric is packed-weight bytes moved per second
(algorithmic bytes: every weight byte read once), reported in GB/s, as a
fraction of the 8 TB/s HBM3E peak and of the read ceiling measured on the
same GPU, and as equivalent tokens/s.

Before anything is timed, sampled rows of every matrix of the step's last
layer are checked against the CPU oracle (|dy| <= 1e-4 * sum|w*x| + 1e-6); a
mismatch ends the run with a non-zero status and no value.  The roofline
object covers the launch class (wv+wk+wq, wo, w1+w3, w2, ...) that takes the
most time; every class's rate is reported beside it.

Other workloads (--workload) measure the remaining shapes the same way:
  8b      Llama-3-8B-shaped layers x32
  single  one Q4_K 4096x4096 matrix, rotated over 1 GB of copies
  verify  70B shapes, M activation rows (--m), all-Q4_K_M / all-Q2_K / all-Q8_0
  moe     Qwen3-30B-A3B-shaped MoE FFN x48, T tokens (--m) routed top-8
          (gate and up in one grouped launch; --no-group: separately)
  stream  8B-shaped layers x32 held in page-locked HOST memory, copied
          through a ring of --slots device slots ahead of each grouped GEMV
          (host-to-device link bound; value includes the copies)
  dequant the standalone dequantizer over a 70B layer's matrices to fp32
          (value counts packed bytes read plus fp32 bytes written)
and the measurement kernels of libkqprobe.so:
  ceiling HBM read stream of 4 GiB with the GEMV kernels' load forms,
          12 to 144 KB in flight per compute unit
  floor   back-to-back launches of an empty kernel
  barrier dependent weight-stream phases: a launch per phase vs one
          persistent launch with grid barriers
  stamps  per-work-group timestamps of the 70B wo, w1+w3 and w2 launches (the
          library's batch-1 kernels with stamps at their phase boundaries)

Inputs are seeded synthetic data drawn directly in device memory.  Only one
GPU is supported: the path has no collectives.
"""
import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved weight GB/s (% of 8 TB/s HBM) + equiv tok/s, 70B-layer Q4_K_M GEMV M=1"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_LIB = os.path.join(ROOT, "dequant_gemv_gguf_amd", "libkqgemv.so")
PROBE_LIB = os.path.join(ROOT, "dequant_gemv_gguf_amd", "libkqprobe.so")
PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction
TOL_REL, TOL_ABS = 1e-4, 1e-6
PROBES = ("ceiling", "floor", "barrier", "stamps")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="70b",
                    choices=["70b", "8b", "single", "verify", "moe", "stream", "dequant"] + list(PROBES))
    ap.add_argument("--slots", type=int, default=3, help="stream: device slots in the ring")
    ap.add_argument("--m", type=int, default=1, help="activation rows (verify) or tokens (moe)")
    ap.add_argument("--quant", default="mix", choices=["mix", "q2_k", "q8_0"], help="verify: re-encoding")
    ap.add_argument("--mc", action="store_true",
                    help="verify / 70b (Q4_K_M mix): every call on the matrix-core GEMV (kq_qgemv_mc_multi)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the model's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling and launch-floor measurement")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip sampling the clocks under load (for profiled runs: it repeats the step for ~2 s)")
    ap.add_argument("--no-group", action="store_true",
                    help="one launch per matrix (no grouped calls for matrices sharing an input)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bounded CPU oracle sample length")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy before the warmup (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter_collection.csv files of a FETCH_SIZE pass and a "
                         "WRITE_SIZE pass (both run with --copy-calibration) into profiles/traffic_<workload>.json")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="no GPU: turn a rocprofv3 kernel_stats.csv into profiles/<--profile-name>.txt")
    ap.add_argument("--profile-name", default="", help="with --summarize-trace: file name (no extension)")
    ap.add_argument("--dominant", default="", help="with --summarize-*: the dominant kernel's name (its start)")
    ap.add_argument("--bench-line", help="with --summarize-trace: the JSON line the profiled bench run printed")
    ap.add_argument("--launch-class", default="", help="with --summarize-pmc: the launch class it serves")
    ap.add_argument("--pmc-command", default="", help="with --summarize-*: the command the passes ran")
    ap.add_argument("--phase-mb", type=float, default=136.0,
                    help="barrier: weight MB per phase (136 = a 70B layer's 544 MB over its 4 launches)")
    ap.add_argument("--phases", type=int, default=320, help="barrier: phases per step")
    ap.add_argument("--x-kb", type=int, default=32, help="barrier: activation KB staged per phase")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def check(status):
    if status != 0:
        raise RuntimeError("kq_qgemv_multi failed with status %d" % status)


def library_hash():
    """Hash of the built library (its kernels and launch logic): traffic
    counters taken with another build are not reported.  The build is
    reproducible (fixed compilation-unit ids), so the same sources give the
    same hash wherever they are built."""
    h = hashlib.sha256()
    with open(KERNEL_LIB, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def clocks():
    """Best-effort GPU clocks from amd-smi (None when unavailable)."""
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        g = d[0] if isinstance(d, list) else d.get("gpu_data", [d])[0]
        c = g.get("clock", g)
        out = {}
        for key, val in c.items():
            if isinstance(val, dict) and "clk" in val:
                v = val["clk"]
                out[key] = v.get("value", v) if isinstance(v, dict) else v
        return out or None
    except Exception:
        return None


def clocks_under_load(torch, run_step, seconds=2.0):
    """GPU clocks sampled (amd-smi) while the timed step runs again, untimed,
    for about `seconds`: the graphics clocks while the kernels stream, not
    at idle.  None when amd-smi gives nothing."""
    import threading
    stop = threading.Event()

    def spin():
        while not stop.is_set():
            run_step()
            torch.cuda.synchronize()

    th = threading.Thread(target=spin, daemon=True)
    th.start()
    t0 = time.perf_counter()
    time.sleep(0.3)
    samples = []
    while time.perf_counter() - t0 < seconds:
        c = clocks()
        if c:
            samples.append(c)
    stop.set()
    th.join()
    if not samples:
        return None
    keys = sorted({k for c in samples for k in c if k.startswith("gfx") or k.startswith("mem")})
    out = {}
    for k in keys:
        vals = [c[k] for c in samples if isinstance(c.get(k), (int, float))]
        if vals:
            out[k] = sorted(vals)[len(vals) // 2]
    return out or None


CALIB_BYTES = 1 << 30


def pmc_per_dispatch(path, counter):
    """{dispatch id: (kernel name, value)} for one counter of a counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def squash(name):
    return name.replace(" ", "").replace("void", "").replace("kq::", "")


def summarize_pmc(args):
    """Traffic of the dominant kernel from a FETCH_SIZE and a WRITE_SIZE pass.
    Each counter is calibrated on the 1 GiB copy the passes ran first: the
    factor is 1 GiB over what the counter read for it."""
    if not args.dominant or not args.launch_class:
        raise SystemExit("--summarize-pmc needs --dominant KERNEL_NAME_START and --launch-class CLASS")
    result = {"kernel": args.dominant, "launch": args.launch_class, "library_sha256_16": library_hash(),
              "workload": args.workload, "m": args.m, "mc": bool(getattr(args, "mc", False)),
              "command": args.pmc_command}
    per = {}
    for key, path, counter in (("fetch", args.summarize_pmc[0], "FETCH_SIZE"),
                               ("write", args.summarize_pmc[1], "WRITE_SIZE")):
        d = pmc_per_dispatch(path, counter)
        copies = [v for (n, v) in d.values() if "copy" in n]
        if not copies:
            raise SystemExit("no copy kernel in %s: run the pass with --copy-calibration" % path)
        ref = max(copies)                              # the 1 GiB copy is the largest one
        factor = CALIB_BYTES / (ref * 1024.0)
        dom = [v for (n, v) in d.values() if squash(n).startswith(squash(args.dominant))]
        if not dom:
            raise SystemExit("no dispatch of %s in %s" % (args.dominant, path))
        per[key] = sum(dom) / len(dom) * 1024.0 * factor
        result["%s_kib_copy_1gib" % key] = round(ref, 1)
        result["%s_factor" % key] = round(factor, 4)
        result["%s_bytes_per_launch" % key] = int(per[key])
        result["%s_dispatches" % key] = len(dom)
    result["bytes_per_launch"] = int(per["fetch"] + per["write"])
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "traffic_%s.json" % args.workload)
    with open(out, "w") as f:
        json.dump(result, f, indent=1)
        f.write("\n")
    print(json.dumps(result))
    return 0


def summarize_trace(args):
    """A rocprofv3 kernel_stats.csv as a short text summary in profiles/."""
    import csv
    if not args.profile_name:
        raise SystemExit("--summarize-trace needs --profile-name")
    with open(args.summarize_trace) as f:
        rows = list(csv.DictReader(f))
    lines = ["# rocprofv3 kernel summary", "", "command (from the repository root, one MI355X):",
             "  " + args.pmc_command, "",
             "%-80s %7s %11s %10s %10s %6s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns", "pct")]
    for r in rows[:14]:
        lines.append("%-80s %7s %11.0f %10s %10s %6.2f" % (
            r["Name"][:80], r["Calls"], float(r["AverageNs"]), r["MinNs"], r["MaxNs"], float(r["Percentage"])))
    if args.dominant:
        dom = [r for r in rows if squash(r["Name"]).startswith(squash(args.dominant))]
        calls = sum(int(r["Calls"]) for r in dom)
        total = sum(float(r["TotalDurationNs"]) for r in dom)
        lines += ["", "dominant kernel %s: %d calls, average %.0f ns" % (args.dominant, calls, total / max(1, calls))]
    if args.bench_line:
        # the bench line the profiled run printed: its per-class HIP-event averages
        with open(args.bench_line) as f:
            b = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
        lines += ["", "bench line of the same run (HIP-event averages per launch class; the profiler "
                  "lengthens launches a little):"]
        for c in b.get("launch_classes", []):
            lines.append("  %-10s %4d a step  %9.3f us  %8.1f GB/s  frac %.4f" % (
                c["launch"], c["per_step"], c["avg_us"], c["GBps"], c["frac"]))
        lines.append("  ms_per_step %.4f, value %.1f %s, parity %s" % (b["ms_per_step"], b["value"], b["unit"],
                                                                       b.get("parity")))
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, args.profile_name + ".txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def probe_lib():
    import dequant_gemv_gguf_amd  # noqa: F401  (fails loudly without the built libraries)
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("%s is missing: build it first (python __graft_entry__.py build)" % PROBE_LIB)
    L = ctypes.CDLL(PROBE_LIB)
    P, I, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    L.kqp_read_stream.argtypes = [P, U64, I, I, I, I, P, P]
    L.kqp_empty.argtypes = [I, I, P]
    L.kqp_phased_stream.argtypes = [P, U64, U64, I, P, I, I, I, P, P, P]
    L.kqp_stamped_qgemv1.argtypes = [I, I, P, P, ctypes.c_int64, P, P, P, I, P, P]
    return L


def stamp_stats(st, groups):
    """Phases of one stamped launch (µs; the stamps count a 100 MHz clock)."""
    import numpy as np
    t = st[:groups, :4].astype(np.int64)
    base = t[:, 0].min()
    rel = (t - base) * 0.01
    end = rel[:, 3]
    xcd = st[:groups, 4].astype(np.int64)
    per_xcd = {int(x): float(np.median(end[xcd == x])) for x in np.unique(xcd)}
    return {"span": float(end.max()), "start_spread": float(rel[:, 0].max()),
            "staging": float(np.median(rel[:, 1] - rel[:, 0])), "to_registers": float(np.median(rel[:, 2] - rel[:, 1])),
            "weight_stream": float(np.median(rel[:, 3] - rel[:, 2])), "end_median": float(np.median(end)),
            "end_first": float(end.min()), "xcd_end_median": per_xcd}


def timed(torch, stream, fn, reps, warmup):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def chk(r, what):
    if r != 0:
        raise RuntimeError("%s failed with status %d" % (what, r))


def read_ceiling(torch, stream, P, cus, reps=5):
    """HBM read ceiling: 4 GiB streamed once through a per-wave LDS ring
    (8 waves x 4 slots of 3 KB a compute unit, non-temporal), in GB/s."""
    nbytes = (1 << 32) - 4096
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 16 * 64, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    ms = timed(torch, stream, lambda: chk(P.kqp_read_stream(buf.data_ptr(), nbytes, 1, cus, 8, 4, sink.data_ptr(), sp),
                                          "kqp_read_stream"), reps, 1)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def stream_twins(torch, stream, P, cus, sizes, xbytes=32 * 1024, reps=4):
    """For each launch size: microseconds of one launch of the plain read
    stream (kqp_phased_stream, one launch per phase: 16 waves x 2 slots of
    3 KB a compute unit, buffer-to-LDS, after staging xbytes of activations)
    moving the same bytes -- what one launch of that size can reach on this
    GPU with no arithmetic.  Launches rotate over 4 GiB, so no phase finds
    its bytes in a cache."""
    nbytes = 1 << 32
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 16 * 64, dtype=torch.int32, device="cuda")
    x = torch.randn(xbytes // 4, device="cuda")
    ctr = torch.zeros(2, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = []
    for size in sizes:
        pbytes = max(3072, int(size) // 3072 * 3072)
        nph = max(1, min(320, nbytes // pbytes))
        ms = timed(torch, stream, lambda: chk(P.kqp_phased_stream(buf.data_ptr(), pbytes, pbytes, nph, x.data_ptr(),
                                                                  xbytes, 0, 0, ctr.data_ptr(), sink.data_ptr(), sp),
                                              "kqp_phased_stream"), reps, 1)
        out.append(1e3 * ms / nph * size / pbytes)
    del buf
    return out


def launch_floor(torch, stream, P, cus, reps=500):
    sp = ctypes.c_void_p(stream.cuda_stream)
    return 1e3 * timed(torch, stream, lambda: chk(P.kqp_empty(cus, 1024, sp), "kqp_empty"), reps, 20)


def run_probe(args):
    """Ceilings and fixed costs the GEMV kernels are judged against:
    ceiling  HBM read stream (4 GiB) with the kernels' load forms
    floor    back-to-back launches of an empty kernel
    barrier  dependent phases of a weight stream: one launch per phase vs one
             persistent launch with a grid barrier between phases (with and
             without issuing the next phase's first loads before the wait)
    stamps   per-work-group timestamps of the library's persistent batch-1 launches"""
    import torch
    P = probe_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(65535 * 16 * 64, dtype=torch.int32, device=dev)

    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "vs_baseline": None,
           "data": "synthetic (uninitialised device memory; only the read rate matters)", "compute_units": cus,
           "clocks_idle_mhz": clocks()}
    if args.workload == "ceiling":
        nbytes = (1 << 32) - 4096
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        rows = []
        # bytes in flight per compute unit = waves x depth x 3 KB, from 12 KB
        # to 144 KB, through registers and through LDS
        for (mode, waves, depth) in [(m, w, d) for m in (1, 0) for (w, d) in
                                     [(4, 1), (8, 1), (4, 2), (16, 1), (8, 2), (8, 3), (16, 2), (8, 4), (16, 3)]]:
            ms = timed(torch, stream, lambda: chk(P.kqp_read_stream(buf.data_ptr(), nbytes, mode, cus, waves, depth,
                                                                    sink.data_ptr(), sp), "kqp_read_stream"),
                       args.steps, args.warmup)
            rows.append({"loads": "buffer-to-LDS" if mode else "registers", "waves": waves, "depth": depth,
                         "kb_in_flight_per_cu": waves * depth * 3,
                         "us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        best = max(r["GBps"] for r in rows)
        out.update({"metric": "HBM read-stream ceiling (4 GiB, one persistent work-group per CU)", "value": best,
                    "unit": "GB/s", "pct_of_hbm_peak": round(100 * best / HBM_PEAK_GBS, 2), "variants": rows,
                    "config": {"workload": "read 4 GiB once, 3-KB spans, non-temporal", "bytes": nbytes}})
    elif args.workload == "floor":
        rows = []
        for (nwg, threads) in [(1, 64), (cus, 1024), (cus, 512)]:
            ms = timed(torch, stream, lambda: chk(P.kqp_empty(nwg, threads, sp), "kqp_empty"), 2000, args.warmup)
            rows.append({"workgroups": nwg, "threads": threads, "us_per_launch": round(ms * 1e3, 3)})
        out.update({"metric": "back-to-back launch floor of an empty kernel", "value": rows[1]["us_per_launch"],
                    "unit": "us", "higher_is_better": False, "variants": rows,
                    "config": {"workload": "2000 launches of an empty kernel on one stream"}})
    elif args.workload == "stamps":
        # where a launch's time goes: the library's batch-1 launches of a 70B
        # layer (wo and w1+w3 in one launch: the Q4_K LDS ring; w2: the Q6_K
        # register ring) with per-work-group timestamps
        import numpy as np
        import kqsynth
        rows_out = []
        for (name, qt, Ns, K) in [("wo", kqsynth.Q4_K, [8192], 8192), ("w1+w3", kqsynth.Q4_K, [28672, 28672], 8192),
                                  ("w2", kqsynth.Q6_K, [8192], 28672)]:
            nbytes = sum(Ns) * kqsynth.row_bytes(qt, K)
            copies = max(2, (2 << 30) // nbytes + 1)
            Ws = [[kqsynth.device_matrix(qt, n, K, seed=50 * c + i, device=dev) for i, n in enumerate(Ns)]
                  for c in range(copies)]
            x = torch.randn(1, K, device=dev)
            ys = [torch.empty(1, n, device=dev) for n in Ns]
            reps = max(4, args.steps)
            stamps = torch.zeros((reps, 4096, 8), dtype=torch.int64, device=dev)
            cnt = len(Ns)
            Na = (ctypes.c_int64 * cnt)(*Ns)
            Ya = (ctypes.c_void_p * cnt)(*[y.data_ptr() for y in ys])
            grid = ctypes.c_int(0)
            xp = ctypes.c_void_p(x.data_ptr())
            Wa = [(ctypes.c_void_p * cnt)(*[W.data_ptr() for W in Wc]) for Wc in Ws]

            def launch(r, c):
                chk(P.kqp_stamped_qgemv1(qt, cnt, Wa[c], Na, K, xp, Ya, ctypes.c_void_p(stamps[r].data_ptr()), 4096,
                                         ctypes.byref(grid), sp), "kqp_stamped_qgemv1")
            for c in range(copies):
                launch(0, c)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for r in range(reps):
                launch(r, r % copies)
            b.record(stream)
            torch.cuda.synchronize()
            launch_us = 1e3 * a.elapsed_time(b) / reps
            st = stamps.cpu().numpy()
            per = [stamp_stats(st[r], grid.value) for r in range(reps)]
            med = {k: round(float(np.median([p[k] for p in per])), 3) for k in per[0] if k != "xcd_end_median"}
            xcds = sorted(per[0]["xcd_end_median"])
            med["xcd_end_median"] = {str(k): round(float(np.median([p["xcd_end_median"].get(k, 0.0) for p in per])),
                                                    3) for k in xcds}
            rows_out.append({"launch": name, "bytes": nbytes, "work_groups": grid.value,
                             "back_to_back_us": round(launch_us, 3), "phases_us_median_of_launches": med})
            del Ws
            torch.cuda.empty_cache()
        out.update({"metric": "per-work-group timestamps of the persistent batch-1 GEMV launches of a 70B layer",
                    "value": rows_out[-1]["phases_us_median_of_launches"]["span"], "unit": "us",
                    "higher_is_better": False, "launches": rows_out,
                    "config": {"workload": "70B wo 8192x8192 and w1+w3 2x28672x8192 Q4_K, w2 8192x28672 Q6_K, "
                                           "M=1, weights rotated over > 2 GB"}})
    else:  # barrier
        pbytes = int(args.phase_mb * 1e6) // 3072 * 3072
        total = pbytes * args.phases
        buf = torch.empty(total, dtype=torch.uint8, device=dev)
        x = torch.randn(args.x_kb * 256, device=dev)
        ctr = torch.zeros(2, dtype=torch.int32, device=dev)
        rows = []
        for (pers, pref) in [(0, 0), (1, 0), (1, 1), (1, 2), (1, 3)]:
            def step(pers=pers, pref=pref):
                chk(P.kqp_phased_stream(buf.data_ptr(), pbytes, pbytes, args.phases, x.data_ptr(), args.x_kb * 1024,
                                        pers, pref, ctr.data_ptr(), sink.data_ptr(), sp), "kqp_phased_stream")
            ms = timed(torch, stream, step, args.steps, args.warmup)
            rows.append({"launch": "persistent, grid barrier" if pers else "one launch per phase",
                         "prefetch_next_phase": bool(pref & 1),
                         "barrier": ("device-scope data, no cache maintenance" if pref & 2 else
                                     "agent-scope release + acquire per work-group") if pers else None,
                         "ms_per_step": round(ms, 4),
                         "GBps": round(total / (ms * 1e-3) / 1e9, 1),
                         "us_per_phase": round(ms * 1e3 / args.phases, 3)})
        torch.cuda.synchronize()
        if int(ctr[1].item()) != 0:
            raise RuntimeError("a grid-barrier wait gave up (ctr[1] = %d)" % int(ctr[1].item()))
        best = max(r["GBps"] for r in rows)
        out.update({"metric": "dependent weight-stream phases: launch per phase vs persistent grid barrier",
                    "value": best, "unit": "GB/s", "pct_of_hbm_peak": round(100 * best / HBM_PEAK_GBS, 2),
                    "variants": rows,
                    "config": {"workload": "%d phases of %.1f MB, %d KB activations staged per phase" % (
                        args.phases, pbytes / 1e6, args.x_kb), "bytes_per_step": total}})
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------
# Parity gate: sampled outputs of the timed launches against the oracle

def sample_rows(N, seed, n=14):
    import numpy as np
    return np.unique(np.concatenate([[0, N - 1], np.random.default_rng(seed).integers(0, N, n)]))


def parity_gate(torch, checks):
    """Worst |dy| / (1e-4 * sum|w*x| + 1e-6) over sampled outputs of every
    check (dequant: 0 when bit-exact, inf otherwise) and the outputs checked."""
    import numpy as np
    import oracle
    worst, nrows = 0.0, 0
    for c in checks:
        kind = c["kind"]
        if kind == "gemv":
            qt, N, K, W, x, y = c["qtype"], c["N"], c["K"], c["W"], c["x"], c["y"]
            rows = sample_rows(N, N + K)
            Wr = W[torch.from_numpy(rows).to(W.device)].cpu().numpy()
            yo, S = oracle.gemv(qt, Wr, len(rows), K, x.cpu().numpy())
            yg = y[:, torch.from_numpy(rows).to(y.device)].cpu().numpy().astype(np.float64)
            worst = max(worst, float((np.abs(yg - yo) / (TOL_REL * S + TOL_ABS)).max()))
            nrows += yg.size
        elif kind == "dequant":
            qt, W, out, n = c["qtype"], c["W"], c["out"], c["n"]
            qk, nb = c["block"]
            nblk = n // qk
            pick = sample_rows(nblk, nblk, 30)
            ok = True
            Wf = W.view(-1)
            for b in pick:
                ref = oracle.dequant(qt, Wf[b * nb:(b + 1) * nb].cpu().numpy(), qk)
                got = out[b * qk:(b + 1) * qk].cpu().numpy()
                ok = ok and bool(np.array_equal(got.view(np.uint32), ref.view(np.uint32)))
            worst = max(worst, 0.0 if ok else float("inf"))
            nrows += len(pick) * qk
        else:  # moe: the same sampled rows of every expert
            qt, E, N, K, W, ids, p, x, xm, y = (c[k] for k in ("qtype", "E", "N", "K", "W", "ids", "p", "x",
                                                                 "x_mode", "y"))
            rows = sample_rows(N, N + K, 10)
            rb = W.shape[1]
            Wr = W.view(E, N, rb)[:, torch.from_numpy(rows).to(W.device)].contiguous().cpu().numpy()
            yo, S, _ = oracle.moe(qt, Wr, E, len(rows), K, ids.cpu().numpy(),
                                  None if p is None else p.cpu().numpy(), x.cpu().numpy(), xm)
            yg = y[..., torch.from_numpy(rows).to(y.device)].cpu().numpy().astype(np.float64)
            worst = max(worst, float((np.abs(yg - yo) / (TOL_REL * S + TOL_ABS)).max()))
            nrows += yg.size
    return worst, nrows


def main():
    args = parse()
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on exactly one GPU (no collectives, no sharding); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2
    if args.workload in PROBES:
        return run_probe(args)

    import numpy as np
    import torch
    import kqsynth
    import dequant_gemv_gguf_amd as kq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- the workload: launches (closure, weight bytes, class), the checks of
    # the parity gate (the last layer's matrices: a step leaves their outputs
    # in place) and the CPU baseline's sample
    launches = []
    checks = []
    host_sample = []
    M = 1
    if args.workload in ("70b", "8b", "verify"):
        spec = kqsynth.LLAMA3_70B if args.workload != "8b" else kqsynth.LLAMA3_8B
        layers = args.layers or spec["layers"]
        layer = kqsynth.dense_layer(spec["hidden"], spec["ffn"], spec["kv"])
        if args.workload == "verify":
            M = args.m
            if args.quant == "q2_k":
                layer = kqsynth.reencode(layer, kqsynth.Q2_K)
            elif args.quant == "q8_0":
                layer = kqsynth.reencode(layer, kqsynth.Q8_0)
        xs = {K: torch.randn(M, K, device=dev, generator=torch.Generator(device=dev).manual_seed(K))
              for K in {K for (_, _, _, K) in layer}}
        ys = {name: torch.empty(M, N, device=dev) for (name, _, N, _) in layer}
        # layer order as a decode step runs it: the three projections of the
        # attention input (any order: v, k, q), o after attention, the two FFN
        # inputs, the FFN output
        order = {"wv": 0, "wk": 1, "wq": 2, "wo": 3, "w1": 4, "w3": 5, "w2": 6}
        # matrices that read the same activations go through one grouped call
        # (k+q+v, w1+w3); the library runs two formats in one launch
        source = {"wq": "attn_in", "wk": "attn_in", "wv": "attn_in", "wo": "attn_out",
                  "w1": "ffn_in", "w3": "ffn_in", "w2": "ffn_hidden"}
        layer = sorted(layer, key=lambda t: order.get(t[0], 9))
        groups = []
        for t in layer:
            if (not args.no_group and groups
                    and source.get(groups[-1][0][0], groups[-1][0][0]) == source.get(t[0], t[0])):
                groups[-1].append(t)
            else:
                groups.append([t])
        L_ = kq.lib()
        if args.mc and args.quant != "mix":
            print("bench.py: --mc serves Q4_K and Q6_K matrices (the mix) only", file=sys.stderr)
            return 2
        weights = []
        n_mats = 0
        for L in range(layers):
            if L % 20 == 0:
                log("generating layer %d of %d" % (L, layers))
            for grp in groups:
                Ws = []
                for (name, qt, N, K) in grp:
                    W = kqsynth.device_matrix(qt, N, K, seed=1000 * L + order.get(name, 9), device=dev)
                    weights.append(W)
                    Ws.append(W)
                    if L == 0:
                        host_sample.append((qt, N, K, W))
                    if L == layers - 1:
                        checks.append({"kind": "gemv", "qtype": qt, "N": N, "K": K, "W": W, "x": xs[K],
                                       "y": ys[name]})
                qt, K = grp[0][1], grp[0][3]
                nbytes = sum(N * kq.kq_row_bytes(t, K) for (_, t, N, _) in grp)
                cls = "+".join(n for (n, _, _, _) in grp)
                x = xs[K]
                n_mats += len(grp)
                if args.mc:
                    n = len(grp)
                    Ta = (ctypes.c_int * n)(*[t for (_, t, _, _) in grp])
                    Wa = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws])
                    Na = (ctypes.c_int64 * n)(*[N for (_, _, N, _) in grp])
                    Ya = (ctypes.c_void_p * n)(*[ys[name].data_ptr() for (name, _, _, _) in grp])
                    sp = ctypes.c_void_p(stream.cuda_stream)
                    launches.append(((lambda n=n, Ta=Ta, Wa=Wa, Na=Na, K=K, x=x, Ya=Ya, sp=sp:
                                      check(L_.kq_qgemv_mc_multi(n, Ta, Wa, Na, K, ctypes.c_void_p(x.data_ptr()),
                                                                 M, Ya, sp))), nbytes, cls))
                elif len(grp) == 1:
                    N, y = grp[0][2], ys[grp[0][0]]
                    launches.append(((lambda qt=qt, W=Ws[0], N=N, K=K, x=x, y=y:
                                      kq.kq_qgemv(qt, W, N, K, x, M, y, stream)), nbytes, cls))
                else:
                    # host arrays marshalled once; the call is the C entry point itself
                    n = len(grp)
                    Ta = (ctypes.c_int * n)(*[t for (_, t, _, _) in grp])
                    Wa = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws])
                    Na = (ctypes.c_int64 * n)(*[N for (_, _, N, _) in grp])
                    Ya = (ctypes.c_void_p * n)(*[ys[name].data_ptr() for (name, _, _, _) in grp])
                    sp = ctypes.c_void_p(stream.cuda_stream)
                    launches.append(((lambda n=n, Ta=Ta, Wa=Wa, Na=Na, K=K, x=x, Ya=Ya, sp=sp:
                                      check(L_.kq_qgemv_multi(n, Ta, Wa, Na, K, ctypes.c_void_p(x.data_ptr()),
                                                              M, Ya, sp))), nbytes, cls))
        workload = {"70b": "llama3-70b decode layer x%d, Q4_K_M mix, M=1" % layers,
                    "8b": "llama3-8b decode layer x%d, Q4_K_M mix, M=1" % layers,
                    "verify": "llama3-70b layer shapes x%d, %s, M=%d" % (layers, args.quant, M)}[args.workload]
        if args.mc:
            workload += ", matrix-core GEMV"
        config = {"workload": workload, "layers": layers, "hidden": spec["hidden"], "ffn": spec["ffn"],
                  "kv_dim": spec["kv"], "M": M, "matrices_per_step": n_mats, "calls_per_step": len(launches),
                  "grouped": ", ".join("+".join(t[0] for t in g) for g in groups if len(g) > 1) or "none",
                  "gemv": "matrix-core (kq_qgemv_mc_multi)" if args.mc else "vector (kq_qgemv / kq_qgemv_multi)"}
    elif args.workload == "stream":
        spec = kqsynth.LLAMA3_8B
        layers = args.layers or spec["layers"]
        layer = kqsynth.dense_layer(spec["hidden"], spec["ffn"], spec["kv"])
        order = {"wv": 0, "wk": 1, "wq": 2, "wo": 3, "w1": 4, "w3": 5, "w2": 6}
        source = {"wq": "a", "wk": "a", "wv": "a", "wo": "o", "w1": "f", "w3": "f", "w2": "h"}
        layer = sorted(layer, key=lambda t: order[t[0]])
        groups = []
        for t in layer:
            if groups and source[groups[-1][0][0]] == source[t[0]]:
                groups[-1].append(t)
            else:
                groups.append([t])
        align = lambda b: (b + 255) // 256 * 256
        slot_bytes = max(sum(align(N * kq.kq_row_bytes(t, K)) for (_, t, N, K) in g) for g in groups)
        slots = torch.empty(args.slots * slot_bytes, dtype=torch.uint8, device=dev)
        streamer = kq.kq_streamer_create(slots, slot_bytes, args.slots, stream)
        xs = {K: torch.randn(1, K, device=dev, generator=torch.Generator(device=dev).manual_seed(K))
              for K in {K for (_, _, _, K) in layer}}
        ys = {name: torch.empty(1, N, device=dev) for (name, _, N, _) in layer}
        weights = []
        L_ = kq.lib()
        for L in range(layers):
            for grp in groups:
                Hs = []
                for (name, qt, N, K) in grp:
                    W = kqsynth.device_matrix(qt, N, K, seed=1000 * L + order[name], device=dev)
                    Wh = torch.empty(W.numel(), dtype=torch.uint8, pin_memory=True)
                    Wh.copy_(W.view(-1))
                    if L == 0:
                        host_sample.append((qt, N, K, W))
                    else:
                        del W
                    if L == layers - 1:
                        checks.append({"kind": "gemv", "qtype": qt, "N": N, "K": K,
                                       "W": Wh.view(N, kq.kq_row_bytes(qt, K)), "x": xs[K], "y": ys[name]})
                    Hs.append(Wh)
                weights += Hs
                n, K = len(grp), grp[0][3]
                Ta = (ctypes.c_int * n)(*[t for (_, t, _, _) in grp])
                Wa = (ctypes.c_void_p * n)(*[h.data_ptr() for h in Hs])
                Na = (ctypes.c_int64 * n)(*[N for (_, _, N, _) in grp])
                Ya = (ctypes.c_void_p * n)(*[ys[name].data_ptr() for (name, _, _, _) in grp])
                nbytes = sum(N * kq.kq_row_bytes(t, K) for (_, t, N, _) in grp)
                launches.append(((lambda n=n, Ta=Ta, Wa=Wa, Na=Na, K=K, x=xs[K], Ya=Ya:
                                  check(L_.kq_stream_qgemv_multi(ctypes.c_void_p(streamer), n, Ta, Wa, Na, K,
                                                                 ctypes.c_void_p(x.data_ptr()), 1, Ya))),
                                 nbytes, "+".join(t[0] for t in grp)))
        torch.cuda.synchronize()
        workload = "llama3-8b layers x%d streamed from pinned host memory, %d device slots, M=1" % (layers,
                                                                                                   args.slots)
        config = {"workload": workload, "layers": layers, "hidden": spec["hidden"], "ffn": spec["ffn"],
                  "kv_dim": spec["kv"], "M": 1, "slots": args.slots, "slot_bytes": slot_bytes,
                  "calls_per_step": len(launches)}
    elif args.workload == "single":
        N = K = 4096
        qt = kqsynth.Q4_K
        nbytes = N * kq.kq_row_bytes(qt, K)
        copies = max(1, (1 << 30) // nbytes + 1)          # > MALL: rotate over >= 1 GB
        x = torch.randn(1, K, device=dev)
        y = torch.empty(1, N, device=dev)
        weights = [kqsynth.device_matrix(qt, N, K, seed=c, device=dev) for c in range(copies)]
        for W in weights:
            launches.append(((lambda W=W: kq.kq_qgemv(qt, W, N, K, x, 1, y, stream)), nbytes, "q4_k 4096x4096"))
        host_sample.append((qt, N, K, weights[0]))
        checks.append({"kind": "gemv", "qtype": qt, "N": N, "K": K, "W": weights[-1], "x": x, "y": y})
        workload = "single Q4_K 4096x4096 M=1, rotated over %d copies" % copies
        config = {"workload": workload, "N": N, "K": K, "M": 1, "copies": copies}
    elif args.workload == "dequant":
        # the standalone dequantizer over a 70B layer's matrices (Q4_K_M mix):
        # packed bytes in, fp32 out; the bytes of a launch count both
        spec = kqsynth.LLAMA3_70B
        layer = kqsynth.dense_layer(spec["hidden"], spec["ffn"], spec["kv"])
        layers = args.layers or 1
        out = torch.empty(max(N * K for (_, _, N, K) in layer), dtype=torch.float32, device=dev)
        weights = []
        for L in range(layers):
            for i, (name, qt, N, K) in enumerate(layer):
                W = kqsynth.device_matrix(qt, N, K, seed=1000 * L + i, device=dev)
                weights.append(W)
                nbytes = N * kq.kq_row_bytes(qt, K) + 4 * N * K
                launches.append(((lambda qt=qt, W=W, n=N * K: kq.kq_dequant(qt, W, n, out, stream)), nbytes, name))
        qt, N, K = layer[-1][1], layer[-1][2], layer[-1][3]
        checks.append({"kind": "dequant", "qtype": qt, "W": weights[-1], "out": out, "n": N * K,
                       "block": kqsynth.BLOCK[qt][:2]})
        workload = "standalone dequant of llama3-70b layer matrices x%d to fp32" % layers
        config = {"workload": workload, "layers": layers, "matrices_per_step": len(launches),
                  "bytes": "packed in + fp32 out"}
    else:  # moe
        spec = kqsynth.QWEN3_30B_A3B_MOE
        layers = args.layers or spec["layers"]
        T, k, E, H, F = args.m, spec["top_k"], spec["experts"], spec["hidden"], spec["ffn"]
        M = T
        g = torch.Generator(device=dev).manual_seed(7)
        x = torch.randn(T, H, device=dev, generator=g)
        h = torch.randn(T * k, F, device=dev, generator=g)
        yg = torch.empty(T, k, F, device=dev)
        yu = torch.empty(T, k, F, device=dev)
        yd = torch.empty(T, H, device=dev)
        ws = torch.empty(kq.kq_qmoe_workspace_bytes(T, k, H) // 4, device=dev)
        weights = []
        for L in range(layers):
            rng = kqsynth.rng_for(0, 5, L)
            ids_np, p_np = kqsynth.routing(T, k, E, rng)
            ids = torch.from_numpy(ids_np).to(dev)
            p = torch.from_numpy(p_np).to(dev)
            distinct = len(set(ids_np.reshape(-1).tolist()))
            gate_up = []
            for (name, qt, EE, N, K) in kqsynth.moe_layer(H, E, F):
                W = kqsynth.device_matrix(qt, EE * N, K, seed=100 * L + len(weights), device=dev)
                weights.append(W)
                per_expert = N * kq.kq_row_bytes(qt, K)
                if L == layers - 1:
                    y_of = {"gate": yg, "up": yu, "down": yd}[name]
                    checks.append({"kind": "moe", "qtype": qt, "E": E, "N": N, "K": K, "W": W, "ids": ids,
                                   "p": p if name == "down" else None, "x": h if name == "down" else x,
                                   "x_mode": 1 if name == "down" else 0, "y": y_of})
                if name == "down":
                    fn = (lambda qt=qt, W=W, N=N, K=K, ids=ids, p=p:
                          kq.kq_qmoe_gemv(qt, W, E, N, K, ids, p, T, k, h, 1, yd, ws, None, stream))
                elif args.no_group:
                    out = yg if name == "gate" else yu
                    fn = (lambda qt=qt, W=W, N=N, K=K, ids=ids, out=out:
                          kq.kq_qmoe_gemv(qt, W, E, N, K, ids, None, T, k, x, 0, out, None, None, stream))
                else:
                    # gate and up share the routing and x: one grouped launch
                    gate_up.append((W, distinct * per_expert))
                    if len(gate_up) < 2:
                        continue
                    fn = (lambda qt=qt, Wg=gate_up[0][0], Wu=gate_up[1][0], N=N, K=K, ids=ids:
                          kq.kq_qmoe_gemv_multi(qt, [Wg, Wu], E, N, K, ids, T, k, x, 0, [yg, yu], None, stream))
                    launches.append((fn, gate_up[0][1] + gate_up[1][1], "gate+up"))
                    continue
                launches.append((fn, distinct * per_expert, name))
        workload = "qwen3-30b-a3b MoE FFN x%d, top-%d of %d experts, T=%d" % (layers, k, E, T)
        config = {"workload": workload, "layers": layers, "experts": E, "top_k": k, "hidden": H,
                  "expert_ffn": F, "tokens": T, "calls_per_step": len(launches),
                  "grouped": "none" if args.no_group else "gate+up"}
    torch.cuda.synchronize()
    step_bytes = sum(b for (_, b, _) in launches)

    def run_step():
        for (fn, _, _) in launches:
            fn()

    log("inputs resident: %.2f GB of packed weights per step, %d launches" % (step_bytes / 1e9, len(launches)))
    if args.copy_calibration:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(max(1, args.warmup)):
        run_step()
    torch.cuda.synchronize()
    log("warmup done")

    # ---- parity gate: the outputs the warmup left (the last layer's) against
    # the oracle, before anything is timed
    worst, nrows = parity_gate(torch, checks)
    parity = "pass" if worst <= 1.0 else "fail"
    log("parity %s: worst |dy|/bound %.3g over %d sampled outputs" % (parity, worst, nrows))
    if parity != "pass":
        print(json.dumps({"metric": METRIC if args.workload == "70b" else "achieved weight GB/s (%s)" % args.workload,
                          "parity": "fail", "max_dy_over_bound": worst, "parity_outputs_checked": nrows,
                          "config": config}), flush=True)
        return 3

    # ---- timed region: exactly `steps` steps
    # (one event at every step boundary, for the median / p10 / p90 of a step)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        run_step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    ms_total = marks[0].elapsed_time(marks[-1])
    ms_per_step = ms_total / args.steps
    gbs = step_bytes * args.steps / (ms_total * 1e-3) / 1e9
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))

    def pct(q):
        return step_ms[min(len(step_ms) - 1, int(round(q * (len(step_ms) - 1))))]

    # ---- per launch class: the same steps issuing only that class's launches,
    # back to back between two events (an event between two launches costs the
    # stream microseconds, so none is recorded inside the run)
    classes = []
    for (_, _, c) in launches:
        if c not in classes:
            classes.append(c)
    per_class = []
    for c in classes:
        idx = [i for i, (_, _, cc) in enumerate(launches) if cc == c]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            for i in idx:
                launches[i][0]()
        b.record(stream)
        torch.cuda.synchronize()
        avg_us = 1e3 * a.elapsed_time(b) / (len(idx) * args.steps)
        nb = sum(launches[i][1] for i in idx) / len(idx)
        per_class.append({"launch": c, "per_step": len(idx), "bytes_per_launch": int(nb),
                          "avg_us": round(avg_us, 3), "GBps": round(nb / (avg_us * 1e-6) / 1e9, 1),
                          "frac": round(nb / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    total_cls_us = sum(pc["avg_us"] * pc["per_step"] for pc in per_class)
    for pc in per_class:
        pc["share_of_step_time"] = round(pc["avg_us"] * pc["per_step"] / total_cls_us, 3)
    dom = max(per_class, key=lambda pc: pc["avg_us"] * pc["per_step"])

    # ---- ceilings on the same GPU
    ceiling = floor_us = None
    if not args.no_ceiling and args.workload != "stream":
        P = probe_lib()
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        ceiling = read_ceiling(torch, stream, P, cus)
        floor_us = launch_floor(torch, stream, P, cus)
        for pc, us in zip(per_class, stream_twins(torch, stream, P, cus, [pc["bytes_per_launch"] for pc in per_class])):
            pc["stream_twin_us"] = round(us, 3)
            pc["frac_of_stream_twin"] = round(us / pc["avg_us"], 4)
            log("class %s: %.2f us a launch, the plain read stream of its bytes %.2f us" % (
                pc["launch"], pc["avg_us"], us))

    traffic = None
    tfile = os.path.join(PROFILES, "traffic_%s.json" % args.workload)
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if (t.get("library_sha256_16") == library_hash() and t.get("launch") == dom["launch"]
                and t.get("m", 1) == args.m and bool(t.get("mc", False)) == bool(args.mc)):
            traffic = t.get("bytes_per_launch")

    out = {
        "metric": METRIC if args.workload == "70b" else "achieved weight GB/s (%s)" % args.workload,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, drawn in device memory)",
        "config": config,
        "parity": parity,
        "max_dy_over_bound": round(worst, 4),
        "parity_outputs_checked": nrows,
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s_equiv": round(1e3 / ms_per_step, 2),
        "step_ms_median_p10_p90": [round(pct(0.5), 4), round(pct(0.1), 4), round(pct(0.9), 4)],
        "weight_bytes_per_step": step_bytes,
        "wall_s_timed": round(wall1 - wall0, 3),
        "roofline": {
            "kernel": "%s launch (the launch class with the most step time)" % dom["launch"],
            "bound": "hbm",
            "achieved": dom["GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dom["frac"],
            "traffic": traffic,
            "avg_launch_us": dom["avg_us"],
            "algorithmic_bytes_per_launch": dom["bytes_per_launch"],
            "launches_timed": dom["per_step"] * args.steps,
            "timing": "HIP events around the class's launches of every step, issued back to back in a pass of "
                      "their own",
        },
        "launch_classes": per_class,
        "clocks_under_load_mhz": (clocks_under_load(torch, run_step)
                                  if args.workload != "stream" and not args.no_clocks else None),
    }
    if ceiling:
        out["read_ceiling_GBps"] = round(ceiling, 1)
        out["pct_of_read_ceiling"] = round(100.0 * gbs / ceiling, 2)
        out["roofline"]["frac_of_read_ceiling"] = round(dom["GBps"] / ceiling, 4)
        if "stream_twin_us" in dom:
            out["roofline"]["stream_twin_us"] = dom["stream_twin_us"]
            out["roofline"]["frac_of_stream_twin"] = dom["frac_of_stream_twin"]
        out["launch_floor_us"] = round(floor_us, 3)
    if args.workload == "stream":
        # every weight byte crosses the host link once per step: that link,
        # not HBM, bounds the streamed path
        out["roofline"] = {"kernel": "host-to-device copies through the slot ring, each overlapped with a grouped GEMV",
                           "bound": "pcie", "achieved": round(gbs, 1), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                           "timing": "whole step (copies and GEMVs), one event per step boundary"}

    if args.workload == "verify":
        out["positions_per_s"] = round(M * 1e3 / ms_per_step, 2)

    # ---- CPU baseline: the oracle on a bounded sample, host cores
    log("timed %d steps: %.3f ms/step, %.1f GB/s" % (args.steps, ms_per_step, gbs))
    if not args.no_cpu_baseline and host_sample:
        log("timing the CPU oracle on a bounded sample")
        import oracle
        threads = oracle.set_threads(0)
        hosts = []
        for (qt, N, K, W) in host_sample:
            rb = kq.kq_row_bytes(qt, K)
            xh = np.random.default_rng(0).standard_normal((M, K)).astype(np.float32)
            hosts.append((qt, N, K, rb, W.view(N, rb).cpu().numpy(), xh))

        # repeat the layer-0 matrices until the sample holds enough CPU time;
        # all host threads, then one thread on a quarter of that time
        def sample(seconds):
            done, t, n = 0, 0.0, 0
            while t < seconds:
                for (qt, N, K, rb, Wh, xh) in hosts:
                    s = time.perf_counter()
                    oracle.gemv(qt, Wh, N, K, xh)
                    t += time.perf_counter() - s
                    done += N * rb
                n += 1
            return done, t, n
        done_bytes, t_cpu, passes = sample(args.cpu_seconds)
        oracle.set_threads(1)
        done1, t1c, passes1 = sample(args.cpu_seconds / 4)
        oracle.set_threads(threads)
        used = ["%s %dx%d" % (kqsynth.TYPE_NAMES[qt], N, K) for (qt, N, K, _, _, _) in hosts]
        out["cpu_baseline"] = {
            "value": round(done_bytes / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "layer-0 matrices %s at M=%d, %d passes (%.1f s of CPU time, %.2f GB)" % (
                ", ".join(used), M, passes, t_cpu, done_bytes / 1e9),
            "value_1_thread": round(done1 / t1c / 1e9, 3),
            "sample_1_thread": "the same matrices, %d passes on one thread (%.1f s)" % (passes1, t1c),
            "host_cpu": cpu_model(),
        }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
