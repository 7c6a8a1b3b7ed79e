#!/usr/bin/env python3
"""Throughput of the binary g128 LM-head GEMV (and the rest of the hot path) on one MI355X.

Headline (one JSON line on stdout): packed-weight GB/s of the binary g128 GEMV on the largest
decode workload, the LM head: M = 1, N = 248320 vocabulary rows, K = 5120 (179 MB of sign bits
and scales per call).  A step is one such call on a distinct copy of the weights; the copies
rotate through more than 1 GiB so that no call finds its weights in the 256 MB Infinity Cache.
The K timed steps are replayed from a HIP graph, with inputs resident in HBM before the timed
region starts.

Beside it: the roofline of the kernel that runs the headline (per-launch algorithmic bytes over
the kernel's device duration, timed with HIP events recorded by hipExtLaunchKernel around each
launch, with median, p10 and p90), the read rate of a kernel that only reads (vector loads and
direct global->LDS copies over the same bytes), the shader clock under the workload and the
memory clock, the decode pair of projections (N = 13824 and 5120) with its launch floor, the
pp512 prefill GEMM for binary and ternary weights, the ternary, base-3, affine and small-M
paths, the embedding gather, and the CPU oracle timed on the host.

Progress lines go to stderr.  Only the CPU-baseline leg touches the oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_FP16_TFLOPS = 2500.0       # MI355X dense fp16 MFMA
ROTATE_BYTES = 1 << 30          # weight copies per shape span more than this
HOST_THREADS = 16               # host threads the GPU machine allots to one GPU
PREWARM_S = 0.4                 # untimed replays of the workload before the warmup steps, so the
PREWARM_STEPS = 400             #   timed steps do not run while the clocks are still ramping

# The headline workload: the LM-head projection at hidden size 5120 over the 248320-row
# vocabulary (the 1-bit article's technical details give both).
LM_N, LM_K = 248320, 5120
# Bytes per dispatch of the stream probes (a multiple of 1 KiB: the LM head's packed weights).
PROBE_BYTES = LM_N * LM_K // 8 + 2 * LM_N * (LM_K // 128)

# The kernel that runs the headline shape, and the source each profiled kernel is built from
# (the counter summaries are keyed to it).
HEADLINE_KERNEL = "q1_gemv_lut8_kernel"
KERNEL_SRC = {
    "q1_gemv_lut4_kernel": "ternary_weight_quantized_bonsai_amd/csrc/q1_gemv.hip",
    "q1_gemv_lutp_kernel": "ternary_weight_quantized_bonsai_amd/csrc/q1_gemv.hip",
    "q1_gemv_lut8_kernel": "ternary_weight_quantized_bonsai_amd/csrc/q1_lut8.hip",
    "q1_gemm_kernel": "ternary_weight_quantized_bonsai_amd/csrc/q1_gemm.hip",
    "gemv_mfma_kernel": "ternary_weight_quantized_bonsai_amd/csrc/gemv_mfma.hip",
    "skinny_gemm_kernel": "ternary_weight_quantized_bonsai_amd/csrc/gemm_skinny.hip",
}
# rocprofv3 names of the kernels behind the launchers the library's plan names.
KERNEL_OF_LAUNCHER = {
    "launch_lut4": "q1_gemv_lut4_kernel",
    "launch_lutp": "q1_gemv_lutp_kernel",
    "launch_lut8_t": "q1_gemv_lut8_kernel",
    "launch_rt": "gemv_mfma_kernel",
    "t5_launch_rt": "t5_gemv_kernel",
    "launch_skinny_t": "skinny_gemm_kernel",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---- HIP events through the process's one HIP runtime ------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev: int, stream: int) -> None:
        assert self.lib.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a: int, b: int) -> float:
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, ev: int) -> None:
        self.lib.hipEventDestroy(ev)

    def sync(self) -> None:
        assert self.lib.hipDeviceSynchronize() == 0


def q1_bytes(N: int, K: int) -> int:
    """Packed weight bytes: one sign bit per weight plus one binary16 scale per 128."""
    return N * K // 8 + 2 * N * (K // 128)


def q2t_bytes(N: int, K: int) -> int:
    return N * K // 4 + 2 * N * (K // 128)


def kernel_times(hip: Hip, bonsai, launches, prewarm_s: float = 0.1) -> list[float]:
    """Device durations (ms) of each launch, via hipExtLaunchKernel start/stop events.  The same
    launches first run untimed, in passes, for about prewarm_s seconds (at least one pass), so
    that the timed ones do not catch the clocks ramping after other work."""
    t0 = time.perf_counter()
    while True:
        for fn in launches:
            fn()
        hip.sync()
        if time.perf_counter() - t0 >= prewarm_s:
            break
    evs = [(hip.event(), hip.event()) for _ in launches]
    for (a, b), fn in zip(evs, launches):
        bonsai.time_next_launch(a, b)
        fn()
    out = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return out


def dist_us(ms: list[float]) -> dict:
    """Mean, median, p10 and p90 of launch durations given in ms, in microseconds."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean_us": round(float(a.mean()), 3), "median_us": round(float(np.median(a)), 3),
            "p10_us": round(float(np.percentile(a, 10)), 3), "p90_us": round(float(np.percentile(a, 90)), 3),
            "launches": int(a.size)}


def kernel_of(plan: str) -> str:
    """rocprofv3 kernel name behind a launch plan string of the library."""
    launcher = plan.split("[", 1)[0].split(" ", 1)[0]
    return KERNEL_OF_LAUNCHER.get(launcher, launcher.split("<", 1)[0])


def src_digest(path: Path) -> str:
    """Digest of a kernel source together with the library's build recipe (compiler flags), so
    that counters taken on one build are not reported for a kernel compiled differently."""
    h = hashlib.sha256(path.read_bytes())
    h.update((ROOT / "ternary_weight_quantized_bonsai_amd" / "build.py").read_bytes())
    return h.hexdigest()[:16]


def read_pmc(name: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the kernel source as it is now (else None)."""
    p = ROOT / "profiles" / name
    if not p.exists():
        return None
    kv = {}
    for line in p.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_build_sha256_16") != digest or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


# ---- clocks ----------------------------------------------------------------------------
def sysfs_clocks(pci_bus: str | None) -> dict:
    """Current SCLK / MCLK levels the driver reports (pp_dpm_sclk / pp_dpm_mclk, the line
    marked '*'), or None where the files cannot be read."""
    out = {"sclk_dpm_mhz": None, "mclk_dpm_mhz": None}
    if not pci_bus:
        return out
    base = Path("/sys/bus/pci/devices") / pci_bus
    for key, fname in (("sclk_dpm_mhz", "pp_dpm_sclk"), ("mclk_dpm_mhz", "pp_dpm_mclk")):
        try:
            for line in (base / fname).read_text().splitlines():
                if line.strip().endswith("*"):
                    tok = line.split(":", 1)[1].strip().split()[0].lower()
                    out[key] = float(tok.replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            pass
    return out


def pci_bus_id(torch) -> str | None:
    try:
        p = torch.cuda.get_device_properties(0)
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except Exception:      # older torch: no PCI fields
        return None


# ---- the oracle on the host (CPU baseline) -----------------------------------------------
def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, s, x, K, budget_s: float):
    """The oracle, as it stands, on a sample of the headline workload's rows: one thread, and
    HOST_THREADS threads (the box's allotment per GPU), each the median of three runs sized to
    about budget_s / 6 seconds.  Packed-weight bytes per second, as the GPU value."""
    import oracle
    orc = oracle.load()
    N = w.shape[0]
    row_bytes = q1_bytes(1, K)

    def run(rows: int, threads: int) -> float:
        step = (rows + threads - 1) // threads
        idx = [np.arange(r0, min(rows, r0 + step), dtype=np.int64) for r0 in range(0, rows, step)]
        t0 = time.perf_counter()
        if threads == 1:
            orc.q1_matmul(w, s, x, K, None, idx[0])
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(lambda i: orc.q1_matmul(w, s, x, K, None, i), idx))
        return time.perf_counter() - t0

    threads = max(1, min(os.cpu_count() or 1, HOST_THREADS))
    per_run = budget_s / 6.0
    out = {}
    for label, t in (("single", 1), ("multi", threads)):
        probe = min(N, 2048 * t)
        dt = run(probe, t)
        rows = int(min(N, max(probe, probe * per_run / max(dt, 1e-6))))
        times = sorted(run(rows, t) for _ in range(3))
        out[label] = (rows, times[1])
    rows_m, t_m = out["multi"]
    rows_1, t_1 = out["single"]
    return {"value": round(rows_m * row_bytes / t_m / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_GBps": round(rows_1 * row_bytes / t_1 / 1e9, 5),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"the first {rows_m} of the {N} LM-head rows (K={K}, M=1) on {threads} host threads "
                      f"(capped at the {HOST_THREADS} threads the GPU box allots per GPU; host has "
                      f"{os.cpu_count()} CPUs), median of 3 runs of {t_m:.2f} s; single thread: {rows_1} rows, "
                      f"median {t_1:.2f} s; packed-weight bytes per second as in the GPU value"}


# ---- rocprofv3 CSV summaries for profiles/ (host only, no GPU) ---------------------------
def short_name(name: str) -> str:
    name = name.replace("bonsai::(anonymous namespace)::", "").replace("bonsai::", "")
    if name.startswith("void "):          # the counter runs print the return type
        name = name[5:]
    return name.split("(", 1)[0]


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_trace(d: str, out: str, cmds: list[str]) -> None:
    """Per-kernel durations from a --kernel-trace --stats run: the stats table plus the mean
    per (kernel, grid), which separates the shapes one kernel runs on."""
    stats = _csv_rows(d, "_kernel_stats.csv")
    trace = _csv_rows(d, "_kernel_trace.csv")
    lines = [f"# rocprofv3 kernel trace: {out}", "# command:"] + [f"#   {c}" for c in cmds]
    lines += ["# summarised by: python bench.py --summarize-trace <output dir> --out " + out, "",
              "kernel | calls | average ns | min ns | max ns | share %", "---|---|---|---|---|---"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.1f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['Percentage']):.2f}")
    per = {}
    for r in trace:
        k = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]),
             r["LDS_Block_Size"], r["VGPR_Count"], r["Accum_VGPR_Count"], r["Scratch_Size"])
        per.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "kernel | grid (threads) | workgroup | LDS B | VGPR | AGPR | scratch | calls | average ns",
              "---|---|---|---|---|---|---|---|---"]
    for k, v in sorted(per.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        if k[0].startswith("__amd"):
            continue
        lines.append(" | ".join(str(x) for x in k) + f" | {len(v)} | {sum(v) / len(v):.1f}")
    (ROOT / "profiles").mkdir(exist_ok=True)
    (ROOT / "profiles" / out).write_text("\n".join(lines) + "\n")
    print((ROOT / "profiles" / out).read_text())


def summarize_pmc(fetch_dir: str, write_dir: str, out: str, cmds: list[str], kernel: str, src: str,
                  grid: int | None = None) -> None:
    """HBM bytes per launch of `kernel` (a prefix of the short kernel name; only dispatches of
    `grid` threads if given) from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch).
    Each counter is scaled by what it reads for the stream probes of the same runs, which move
    a known PROBE_BYTES per dispatch: the vector-load read probe calibrates FETCH_SIZE (the
    direct-to-LDS read probe is listed beside it as a check of that load path), the write probe
    calibrates WRITE_SIZE."""
    def per_dispatch(d, counter):
        acc = {}
        for r in _csv_rows(d, "_counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        return acc
    f, w = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")

    def probe_kib(acc, name):
        vals = sorted(v for (_, n, _), v in acc.items() if n.startswith(name))
        if not vals:
            raise SystemExit(f"no {name} dispatches in the counter run")
        return vals[len(vals) // 2], len(vals)
    probe_kib_bytes = PROBE_BYTES / 1024.0
    cf, ncf = probe_kib(f, "probe_read_kernel")
    cl, ncl = probe_kib(f, "probe_lds_kernel")
    cw, ncw = probe_kib(w, "probe_write_kernel")
    sf, sw = probe_kib_bytes / cf, probe_kib_bytes / cw

    def kern(acc):
        by = {}
        for (_, n, g), v in acc.items():
            if n.startswith(kernel) and (grid is None or g == grid):
                by.setdefault(g, []).append(v)
        return by
    kf, kw = kern(f), kern(w)
    if not kf:
        raise SystemExit(f"no dispatches of {kernel} in the fetch run")
    lines = [f"# HBM traffic per launch of {kernel} ({out})", "# commands:"] + [f"#   {c}" for c in cmds]
    lines += [f"# summarised by: python bench.py --summarize-pmc <fetch dir> <write dir> --out {out}",
              "# Counters are KiB per dispatch.  Each is scaled by the bytes a stream probe of the same run",
              f"# moves ({PROBE_BYTES} B per dispatch) over what the counter reads for it (median over its",
              "# dispatches): the vector-load read probe for FETCH_SIZE, the write probe for WRITE_SIZE.", "",
              f"kernel: {kernel}",
              f"kernel_build_sha256_16: {src_digest(ROOT / src)}",
              f"probe_bytes_per_dispatch: {PROBE_BYTES}",
              f"probe_read_fetch_kib: {cf:.1f} ({ncf} dispatches)",
              f"probe_lds_fetch_kib: {cl:.1f} ({ncl} dispatches; scaled {cl * sf * 1024:.0f} B)",
              f"probe_write_write_kib: {cw:.1f} ({ncw} dispatches)",
              f"fetch_scale: {sf:.4f}", f"write_scale: {sw:.4f}", ""]
    tot, n = 0.0, 0
    for g in sorted(kf):
        mf = sum(kf[g]) / len(kf[g])
        mw = sum(kw.get(g, [0.0])) / max(1, len(kw.get(g, [])))
        b = (mf * sf + mw * sw) * 1024.0
        lines.append(f"grid {g}: {len(kf[g])} dispatches, FETCH_SIZE {mf:.1f} KiB, WRITE_SIZE {mw:.1f} KiB, "
                     f"scaled {b:.0f} B")
        tot += b * len(kf[g])
        n += len(kf[g])
    lines += ["", f"hbm_bytes_per_launch: {tot / n:.0f}"]
    (ROOT / "profiles").mkdir(exist_ok=True)
    (ROOT / "profiles" / out).write_text("\n".join(lines) + "\n")
    print((ROOT / "profiles" / out).read_text())


def summarize_counters(d: str, out: str, cmds: list[str]) -> None:
    """Mean of every collected counter per (kernel, grid) from a --pmc run (values per dispatch,
    summed over the hardware instances by rocprofv3; derived metrics as rocprofv3 computes them)."""
    rows = _csv_rows(d, "_counter_collection.csv")
    per = {}
    names = []
    for r in rows:
        k = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        per.setdefault(k, {}).setdefault(c, {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
    lines = [f"# rocprofv3 counters: {out}", "# command:"] + [f"#   {c}" for c in cmds]
    lines += ["# summarised by: python bench.py --summarize-counters <output dir> --out " + out,
              "# mean per dispatch over the dispatches of each (kernel, grid)", "",
              "kernel | grid (threads) | dispatches | " + " | ".join(names),
              "---|---|---|" + "|".join("---" for _ in names)]
    for (kname, grid), cs in sorted(per.items()):
        if kname.startswith("__amd") or kname.startswith("at::"):
            continue
        n = max(len(v) for v in cs.values())
        vals = []
        for c in names:
            v = list(cs.get(c, {}).values())
            vals.append(f"{sum(v) / len(v):.4g}" if v else "")
        lines.append(f"{kname} | {grid} | {n} | " + " | ".join(vals))
    (ROOT / "profiles").mkdir(exist_ok=True)
    (ROOT / "profiles" / out).write_text("\n".join(lines) + "\n")
    print((ROOT / "profiles" / out).read_text())


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--summarize-trace", metavar="DIR", help="write a profiles/ summary of a kernel-trace run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ HBM-traffic summary of a kernel from two --pmc runs")
    ap.add_argument("--kernel", help="--summarize-pmc: kernel name prefix (default: the headline's)")
    ap.add_argument("--grid", type=int, help="--summarize-pmc: only dispatches of this many threads")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write a profiles/ summary of any rocprofv3 --pmc run (mean per kernel and grid)")
    ap.add_argument("--out", help="file name under profiles/ for --summarize-*")
    ap.add_argument("--cmd", action="append", default=[], help="profiler command recorded in the summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.cmd)
        return 0
    if args.summarize_pmc:
        kernel = args.kernel or HEADLINE_KERNEL
        summarize_pmc(*args.summarize_pmc, args.out, args.cmd, kernel, KERNEL_SRC[kernel.split("<")[0]], args.grid)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the GEMV shards by "
              "rows with no collective; see the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import synth
    import ternary_weight_quantized_bonsai_amd as bonsai

    dev = torch.device("cuda:0")
    hip = Hip()
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    bus = pci_bus_id(torch)

    def up(a):
        a = np.ascontiguousarray(a)
        view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.uint8}[a.dtype]
        return torch.from_numpy(a.view(view)).to(dev)

    def copies(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    # ---- headline: the LM-head GEMV ---------------------------------------------------
    N3, K = LM_N, LM_K
    host3 = synth.make_q1(1, N3, K)
    digests = {"wbits": synth.digest(host3[0]), "scales": synth.digest(host3[1]), "x": synth.digest(host3[2])}
    log(f"LM-head inputs: wbits {digests['wbits']} scales {digests['scales']} x {digests['x']}")
    pbytes3 = q1_bytes(N3, K)
    R3 = max(3, math.ceil(ROTATE_BYTES / pbytes3))
    w3, s3, x3 = (up(a) for a in host3)
    ws3, ss3 = copies(w3, R3), copies(s3, R3)
    y3 = torch.empty((1, N3), dtype=torch.float32, device=dev)
    plan3 = bonsai.plan("q1_gemv", 1, N3, K)
    kname3 = kernel_of(plan3)
    log(f"{R3} weight copies ({R3 * pbytes3 / 2**30:.2f} GiB); launch: {plan3}")

    def step(i):
        bonsai.q1_gemv(ws3[i % R3], ss3[i % R3], x3, out=y3)

    step(0)
    torch.cuda.synchronize()
    log("capturing graphs")
    g_pre, g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pre):
        for i in range(PREWARM_STEPS):
            step(i)
    with torch.cuda.graph(g_warm):
        for i in range(max(args.warmup, 1)):
            step(i)
    with torch.cuda.graph(g_main):
        for i in range(args.steps):
            step(i + args.warmup)
    # untimed: the same steps for PREWARM_S seconds, then the warmup steps
    torch.cuda.synchronize()
    t_pre, n_pre = time.perf_counter(), 0
    while time.perf_counter() - t_pre < PREWARM_S:
        g_pre.replay()
        n_pre += PREWARM_STEPS
        torch.cuda.synchronize()
    log(f"pre-warm: {n_pre} steps in {time.perf_counter() - t_pre:.2f} s")
    if args.warmup:
        g_warm.replay()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, stream())
    g_main.replay()
    hip.record(e1, stream())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = hip.elapsed_ms(e0, e1)
    value = args.steps * pbytes3 / (ms / 1e3) / 1e9
    log(f"{ms:.3f} ms for {args.steps} steps ({wall * 1e3:.3f} ms wall): {value:.1f} GB/s")

    # the kernel's own device durations, launch by launch (no graph)
    kt3 = kernel_times(hip, bonsai, [lambda j=j: step(j) for j in range(max(4 * R3, min(args.steps, 120)))])
    d3 = dist_us(kt3)
    alg3 = pbytes3 + 2 * K + 4 * N3                     # weights + x + y
    achieved = alg3 / (d3["mean_us"] / 1e6) / 1e9
    src3 = KERNEL_SRC.get(kname3)
    traffic = read_pmc(f"{kname3}_lm_head_hbm_traffic.txt", src_digest(ROOT / src3)) if src3 else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "kernel": kname3,
                "bytes_per_launch": alg3, **d3}
    log(f"{kname3}: mean {d3['mean_us']:.2f} us (p10 {d3['p10_us']:.2f}, p90 {d3['p90_us']:.2f}) -> "
        f"{achieved:.1f} GB/s")

    # ---- clocks under the workload: a one-wave stamp kernel on a second stream while the
    # timed graph replays again (an untimed pass), and the driver's current DPM levels
    side = torch.cuda.Stream()
    stamps = torch.zeros(4, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    g_main.replay()
    spin_ns = int(min(0.5 * ms * 1e6, 5e6))
    bonsai.probe_clock(stamps, spin_ns, side.cuda_stream)
    dpm = sysfs_clocks(bus)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().astype(np.int64)
    sclk_load = 100.0 * (st[2] - st[0]) / max(1, st[3] - st[1])
    bonsai.probe_clock(stamps, 200000, side.cuda_stream)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().astype(np.int64)
    sclk_idle = 100.0 * (st[2] - st[0]) / max(1, st[3] - st[1])
    clocks = {"sclk_under_load_mhz": round(sclk_load, 1), "sclk_idle_mhz": round(sclk_idle, 1), **dpm,
              "what": "sclk from s_memtime over s_memrealtime in a one-wave kernel on a second stream, during a "
                      "replay of the timed graph and alone; dpm: the driver's current level during the replay"}
    log(f"shader clock {sclk_load:.0f} MHz under the LM head, {sclk_idle:.0f} MHz alone; dpm {dpm}")

    # ---- read-only probe: the same bytes per launch, rotated over more than 1 GiB --------
    nreg = max(2, math.ceil(ROTATE_BYTES / PROBE_BYTES)) + 1
    pool = torch.empty(nreg * PROBE_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(16384, dtype=torch.int32, device=dev)
    pool.fill_(1)
    probe = {}
    for mode, label in ((0, "vector_loads"), (1, "lds_copies"), (2, "write")):
        def pcall(j, mode=mode):
            bonsai.probe_stream(pool[(j % nreg) * (PROBE_BYTES // 4):], PROBE_BYTES, mode, sink)
        pcall(0)
        kt = kernel_times(hip, bonsai, [lambda j=j: pcall(j) for j in range(4 * nreg)])
        d = dist_us(kt)
        probe[label] = {"GBps": round(PROBE_BYTES / (d["mean_us"] / 1e6) / 1e9, 1), **d}
        log(f"stream probe {label}: {probe[label]['GBps']:.1f} GB/s")
    best_read = max(probe["vector_loads"]["GBps"], probe["lds_copies"]["GBps"])
    probe = {"bytes_per_launch": PROBE_BYTES, "regions_rotated": nreg, **probe}
    roofline["frac_of_read_probe"] = round(achieved / best_read, 4)
    del pool

    torch.cuda.synchronize()
    del ws3, ss3, w3, s3, x3, y3, g_main, g_warm
    torch.cuda.empty_cache()

    extra = {}
    # ---- decode pair: one MLP-shaped and one attention-shaped projection per step ---------
    shapes = {"mlp": 13824, "attn": 5120}
    step_bytes = sum(q1_bytes(n, K) for n in shapes.values())
    R = max(3, math.ceil(ROTATE_BYTES / step_bytes))
    W = {}
    for k, n in shapes.items():
        w0, s0, x0 = (up(a) for a in synth.make_q1(1, n, K))
        W[k] = (copies(w0, R), copies(s0, R), x0, torch.empty((1, n), dtype=torch.float32, device=dev))

    def pair(i):
        for k in ("mlp", "attn"):
            ws, ss, x, y = W[k]
            bonsai.q1_gemv(ws[i % R], ss[i % R], x, out=y)

    pair(0)
    g_pair = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pair):
        for i in range(args.steps):
            pair(i)
    t_pre = time.perf_counter()
    while True:                                         # untimed, as for the headline
        g_pair.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_pre >= 0.1:
            break
    hip.record(e0, stream())
    g_pair.replay()
    hip.record(e1, stream())
    pms = hip.elapsed_ms(e0, e1)
    pair_gbps = args.steps * step_bytes / (pms / 1e3) / 1e9
    per_shape = {}
    for k, n in shapes.items():
        ws, ss, x, y = W[k]
        kt = kernel_times(hip, bonsai, [lambda j=j, ws=ws, ss=ss, x=x, y=y: bonsai.q1_gemv(ws[j % R], ss[j % R], x, out=y)
                                        for j in range(min(args.steps, 150))])
        d = dist_us(kt)
        per_shape[f"{k}_{n}x{K}"] = {"kernel": kernel_of(bonsai.plan("q1_gemv", 1, n, K)), **d,
                                     "GBps": round(q1_bytes(n, K) / (d["mean_us"] / 1e6) / 1e9, 1)}
    # launch floor: the same two calls with no work (K = 0 launches one kernel that zero-fills y)
    z_w = torch.empty((64, 0), dtype=torch.int32, device=dev)
    z_s = torch.empty((64, 0), dtype=torch.int16, device=dev)
    z_x = torch.empty((1, 0), dtype=torch.int16, device=dev)
    z_y = torch.empty((1, 64), dtype=torch.float32, device=dev)

    def zcall():
        bonsai.q1_gemv(z_w, z_s, z_x, out=z_y)

    kt0 = kernel_times(hip, bonsai, [zcall] * 150)
    g_zero = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_zero):
        for _ in range(args.steps):
            zcall()
            zcall()
    g_zero.replay()
    torch.cuda.synchronize()
    hip.record(e0, stream())
    g_zero.replay()
    hip.record(e1, stream())
    floor_step_us = hip.elapsed_ms(e0, e1) * 1e3 / args.steps
    extra["decode_pair_gemv"] = {
        "shape": "M=1 K=5120, N=13824 then N=5120 per step", "step_us": round(pms * 1e3 / args.steps, 3),
        "packed_weight_GBps": round(pair_gbps, 1), "frac_of_8TBps": round(pair_gbps / PEAK_HBM_GBPS, 4),
        "weight_copies_rotated": R, **per_shape,
        "launch_floor": {"empty_kernel": dist_us(kt0), "graph_step_us": round(floor_step_us, 3),
                         "what": "the two calls of a step with K = 0 (each launches one kernel that zero-fills y): "
                                 "per-launch events, and graph replay per step"}}
    log(f"decode pair: {pms * 1e3 / args.steps:.2f} us per step ({pair_gbps:.1f} GB/s); "
        + ", ".join(f"{k} {v['mean_us']:.2f} us" for k, v in per_shape.items())
        + f"; floor {floor_step_us:.2f} us per step")
    del W, g_pair, g_zero
    torch.cuda.empty_cache()

    if not args.headline_only:
        # Prefill GEMM pp512, binary and ternary
        M4, N4 = 512, 13824
        for key, make, fn in (("prefill_gemm", synth.make_q1, bonsai.q1_gemm),
                              ("ternary_prefill_gemm", synth.make_q2t, bonsai.q2t_gemm)):
            w, s, x = (up(a) for a in make(M4, N4, K))
            ws, ss = copies(w, 3), copies(s, 3)
            y = torch.empty((M4, N4), dtype=torch.float32, device=dev)
            fn(ws[0], ss[0], x, out=y)
            d = dist_us(kernel_times(hip, bonsai, [lambda j=j: fn(ws[j % 3], ss[j % 3], x, out=y) for j in range(30)]))
            tf = 2.0 * M4 * N4 * K / (d["mean_us"] / 1e6) / 1e12
            extra[key] = {"shape": "M=512 N=13824 K=5120", **d, "TFLOPs": round(tf, 2),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_FP16_TFLOPS, 4)}}
            log(f"{key}: {d['mean_us']:.1f} us, {tf:.1f} TFLOP/s")
            del ws, ss, w, s, x, y

        # The GEMM entry point at a few rows of x (draft tokens checked at once): the small-M path
        small = {}
        w, s, _ = (up(a) for a in synth.make_q1(1, N4, K))
        R6 = max(3, math.ceil(ROTATE_BYTES / q1_bytes(N4, K)))
        ws, ss = copies(w, R6), copies(s, R6)
        for M6 in (16, 32, 64, 128):
            x = up(synth.make_q1(M6, N4, K)[2])
            y = torch.empty((M6, N4), dtype=torch.float32, device=dev)
            bonsai.q1_gemm(ws[0], ss[0], x, out=y)
            d = dist_us(kernel_times(hip, bonsai, [lambda j=j: bonsai.q1_gemm(ws[j % R6], ss[j % R6], x, out=y)
                                                   for j in range(R6)]))
            small[f"M{M6}"] = {**d, "TFLOPs": round(2.0 * M6 * N4 * K / (d["mean_us"] / 1e6) / 1e12, 2),
                               "packed_weight_GBps": round(q1_bytes(N4, K) / (d["mean_us"] / 1e6) / 1e9, 1),
                               "kernel": kernel_of(bonsai.plan("q1_gemm", M6, N4, K))}
            log(f"small-M gemm M={M6}: {d['mean_us']:.2f} us")
        extra["small_m_gemm"] = {"shape": "N=13824 K=5120, binary", **small}
        del ws, ss, w, s, x, y

        # Ternary decode GEMV, M = 1 and 8, on the 2-bit codes and on the base-3 layout
        N5 = 5120
        tern, t5r = {}, {}
        for M5 in (1, 8):
            w, s, x = (up(a) for a in synth.make_q2t(M5, N5, K))
            R5 = max(3, math.ceil(ROTATE_BYTES / q2t_bytes(N5, K)))
            ws, ss = copies(w, R5), copies(s, R5)
            y = torch.empty((M5, N5), dtype=torch.float32, device=dev)
            bonsai.q2t_gemv(ws[0], ss[0], x, out=y)
            d = dist_us(kernel_times(hip, bonsai, [lambda j=j: bonsai.q2t_gemv(ws[j % R5], ss[j % R5], x, out=y)
                                                   for j in range(R5)]))
            gb = q2t_bytes(N5, K) / (d["mean_us"] / 1e6) / 1e9
            tern[f"M{M5}"] = {**d, "packed_weight_GBps": round(gb, 1), "frac_of_8TBps": round(gb / PEAK_HBM_GBPS, 4)}
            log(f"ternary M={M5}: {d['mean_us']:.2f} us, {gb:.1f} GB/s")
            del ws, ss, w, s, x, y
            c5, s5, x5 = (up(v) for v in synth.make_t5(M5, N5, K))
            nb5 = c5.numel() + 2 * s5.numel()
            R5 = max(3, math.ceil(ROTATE_BYTES / nb5))
            cs, ss = copies(c5, R5), copies(s5, R5)
            y = torch.empty((M5, N5), dtype=torch.float32, device=dev)
            bonsai.t5_matmul(cs[0], ss[0], x5, out=y)
            d = dist_us(kernel_times(hip, bonsai, [lambda j=j: bonsai.t5_matmul(cs[j % R5], ss[j % R5], x5, out=y)
                                                   for j in range(R5)]))
            gb = nb5 / (d["mean_us"] / 1e6) / 1e9
            t5r[f"M{M5}"] = {**d, "packed_weight_GBps": round(gb, 1), "frac_of_8TBps": round(gb / PEAK_HBM_GBPS, 4)}
            log(f"base-3 ternary M={M5}: {d['mean_us']:.2f} us, {gb:.1f} GB/s")
            del cs, ss, c5, s5, x5, y
        extra["ternary_gemv"] = {"shape": "N=5120 K=5120", **tern}
        extra["ternary_base3_gemv"] = {"shape": "N=5120 K=5120, 1.725 bits per weight", **t5r}

        # Affine 1-bit form (MLX's scale and bias per group): decode at the MLP shape, and one row
        # of x at the LM-head shape
        aff = {}
        for M7, N7 in ((1, N4), (8, N4), (1, N3)):
            w, a7, b7, x = (up(v) for v in synth.make_q1a(M7, N7, K))
            nb7 = q1_bytes(N7, K) + 2 * N7 * (K // 128)            # + the biases
            R7 = max(3, math.ceil(ROTATE_BYTES / nb7))
            ws, as_, bs = copies(w, R7), copies(a7, R7), copies(b7, R7)
            y = torch.empty((M7, N7), dtype=torch.float32, device=dev)
            bonsai.q1a_matmul(ws[0], as_[0], bs[0], x, out=y)
            d = dist_us(kernel_times(hip, bonsai, [lambda j=j: bonsai.q1a_matmul(ws[j % R7], as_[j % R7], bs[j % R7], x, out=y)
                                                   for j in range(R7 if N7 == N4 else 4 * R7)]))
            gb = nb7 / (d["mean_us"] / 1e6) / 1e9
            aff[(M7, N7)] = {**d, "packed_weight_GBps": round(gb, 1), "frac_of_8TBps": round(gb / PEAK_HBM_GBPS, 4),
                             "kernel": kernel_of(bonsai.plan("q1a_matmul", M7, N7, K))}
            log(f"affine M={M7} N={N7}: {d['mean_us']:.2f} us, {gb:.1f} GB/s")
            del ws, as_, bs, w, a7, b7, x, y
        extra["affine_gemv"] = {"shape": "N=13824 K=5120, 1-bit affine (scale + bias per group)",
                                "M1": aff[(1, N4)], "M8": aff[(8, N4)]}
        extra["affine_lm_head_gemv"] = {"shape": "M=1 N=248320 K=5120, 1-bit affine", **aff[(1, N3)]}

        # Embedding gather: 512 token ids from the binary vocabulary table (V = 248320, K = 5120)
        w, s, _ = (up(v) for v in synth.make_q1(1, N3, K))
        ids = torch.from_numpy(np.random.default_rng(7).integers(0, N3, 512).astype(np.int64)).to(dev)
        out = torch.empty((512, K), dtype=torch.float16, device=dev)
        bonsai.q1_embed(w, s, ids, out=out)
        d = dist_us(kernel_times(hip, bonsai, [lambda: bonsai.q1_embed(w, s, ids, out=out) for _ in range(20)]))
        nb8 = 512 * (2 * K + K // 8 + 2 * (K // 128) + 8)        # rows written + rows read + ids
        gb8 = nb8 / (d["mean_us"] / 1e6) / 1e9
        extra["embed_gather"] = {"shape": "512 ids, V=248320 K=5120", **d,
                                 "GBps": round(gb8, 1), "frac_of_8TBps": round(gb8 / PEAK_HBM_GBPS, 4)}
        log(f"embed gather: {d['mean_us']:.2f} us, {gb8:.1f} GB/s")
        del w, s, ids, out

    line = {
        "metric": "Binary g128 GEMV packed-weight GB/s (% HBM peak); PP512 GEMM TFLOP/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "binary g128 LM-head GEMV, M=1, N=248320 vocabulary rows, K=5120 (one call per step)",
                   "launch": plan3, "weight_copies_rotated": R3, "accumulate": "f32",
                   "frac_of_8TBps": round(value / PEAK_HBM_GBPS, 4),
                   "frac_of_read_probe": round(value / best_read, 4),
                   "timed_as": "HIP graph replay of the steps, HIP events on the launch stream",
                   "untimed_before": f"{n_pre} steps over {PREWARM_S} s, then the {args.warmup} warmup steps",
                   "input_digests": digests},
        "roofline": roofline,
        "hbm_read_probe": probe,
        "clocks": clocks,
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(host3[0], host3[1], host3[2], K, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
