#!/usr/bin/env python3
"""Throughput of the binary g128 decode GEMV (and the rest of the hot path) on one MI355X.

Headline (one JSON line on stdout): packed-weight GB/s of the decode GEMV on the workload
"binary g128 decode GEMV, M = 1, K = 5120, one MLP-shaped (N = 13824) and one attention-shaped
(N = 5120) projection per step".  A step is those two GEMV calls, each on a distinct copy of
the weights; the copies rotate through more than 1 GiB so no launch finds its weights in the
256 MB Infinity Cache.  The K timed steps are replayed from a HIP graph (the way a decode loop
is issued), with inputs resident in HBM before the timed region starts.

Beside it: the roofline of the dominant kernel (per-launch algorithmic bytes over the kernel's
device duration, timed with HIP events recorded by hipExtLaunchKernel around each launch), the
LM-head GEMV (N = 248320), the pp512 prefill GEMM (M = 512, N = 13824, K = 5120, TFLOP/s) for
binary and ternary weights, the ternary decode GEMV (M = 1 and 8), a device copy probe, the
launch floor of the decode step, and the CPU oracle timed on the host.

Progress lines go to stderr.  Only the CPU-baseline leg touches the oracle.
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
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_FP16_TFLOPS = 2500.0       # MI355X dense fp16 MFMA
ROTATE_BYTES = 1 << 30          # weight copies per shape span more than this


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


def q1_bytes(N: int, K: int) -> int:
    """Packed weight bytes: one sign bit per weight plus one binary16 scale per 128."""
    return N * K // 8 + 2 * N * (K // 128)


def q2t_bytes(N: int, K: int) -> int:
    return N * K // 4 + 2 * N * (K // 128)


def kernel_times(hip: Hip, bonsai, launches) -> list[float]:
    """Device durations (ms) of each launch, via hipExtLaunchKernel start/stop events."""
    evs = [(hip.event(), hip.event()) for _ in launches]
    for (a, b), fn in zip(evs, launches):
        bonsai.time_next_launch(a, b)
        fn()
    out = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return out


# The decode GEMV kernel both headline shapes run on (one 64-row tile per workgroup, 4-group
# K-slices per wave); its HBM-traffic summary under profiles/ carries this name.
HEADLINE_KERNEL = "q1_gemv_lut4_kernel"


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


# ---- the oracle on the host (CPU baseline) -----------------------------------------------
def cpu_baseline(wA, sA, xA, wB, sB, xB, K, budget_s: float):
    import oracle
    orc = oracle.load()
    threads = max(1, min(os.cpu_count() or 1, 16))
    jobs = []
    for (w, s, x) in ((wA, sA, xA), (wB, sB, xB)):
        N = w.shape[0]
        step = (N + threads - 1) // threads
        for n0 in range(0, N, step):
            idx = np.arange(n0, min(N, n0 + step), dtype=np.int64)
            jobs.append((w, s, x, idx))
    step_bytes = q1_bytes(wA.shape[0], K) + q1_bytes(wB.shape[0], K)
    t0 = time.perf_counter()
    passes = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(lambda j: orc.q1_matmul(j[0], j[1], j[2], K, None, j[3]), jobs))
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(passes * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} full step(s) of the workload (N=13824 and N=5120, K=5120, M=1), "
                      f"rows split over {threads} host threads, {dt:.1f} s wall; packed-weight bytes "
                      f"per second as in the GPU value"}


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


def summarize_pmc(fetch_dir: str, write_dir: str, out: str, cmds: list[str], kernel: str, src: str) -> None:
    """HBM bytes per launch of `kernel` from a FETCH_SIZE run and a WRITE_SIZE run (KiB per
    dispatch), each scaled by what the counter reads for the 1 GiB device copy of the copy
    probe (1 GiB read, 1 GiB written)."""
    def per_dispatch(d, counter):
        acc = {}
        for r in _csv_rows(d, "_counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        return acc
    f, w = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")

    def copy_kib(acc):
        # the copy probe's dispatches are the largest copies of the run (the weight clones
        # before them move a few MB each)
        cp = [v for (_, n, _), v in acc.items() if n.startswith("__amd_rocclr_copyBuffer")]
        top = max(cp)
        vals = sorted(v for v in cp if v >= 0.9 * top)
        return vals[len(vals) // 2], len(vals)
    cf, ncf = copy_kib(f)
    cw, ncw = copy_kib(w)
    gib_kib = float(1 << 20)
    sf, sw = gib_kib / cf, gib_kib / cw

    def kern(acc):
        by = {}
        for (_, n, g), v in acc.items():
            if n.split("<")[0] == kernel:
                by.setdefault(g, []).append(v)
        return by
    kf, kw = kern(f), kern(w)
    lines = [f"# HBM traffic per launch of {kernel} ({out})", "# commands:"] + [f"#   {c}" for c in cmds]
    lines += [f"# summarised by: python bench.py --summarize-pmc <fetch dir> <write dir> --out {out}",
              "# Counters are KiB per dispatch; each is scaled by 1 GiB over what it reads for the copy",
              "# probe's 1 GiB device-to-device copy (median over its dispatches).", "",
              f"kernel: {kernel}",
              f"kernel_build_sha256_16: {src_digest(ROOT / src)}",
              f"copy_kernel: __amd_rocclr_copyBuffer, the {ncf} (fetch run) / {ncw} (write run) 1 GiB copies",
              f"copy_fetch_kib: {cf:.1f}", f"copy_write_kib: {cw:.1f}",
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
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-trace", metavar="DIR", help="write a profiles/ summary of a kernel-trace run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ HBM-traffic summary of the decode GEMV from two --pmc runs")
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
        summarize_pmc(*args.summarize_pmc, args.out, args.cmd, HEADLINE_KERNEL,
                      "ternary_weight_quantized_bonsai_amd/csrc/q1_gemv.hip")
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

    def up(a):
        a = np.ascontiguousarray(a)
        view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.uint8}[a.dtype]
        return torch.from_numpy(a.view(view)).to(dev)

    # ---- headline workload: the two decode projections at hidden 5120 -------------------
    K = 5120
    shapes = {"mlp": 13824, "attn": 5120}
    host = {k: synth.make_q1(1, n, K) for k, n in shapes.items()}
    step_bytes = sum(q1_bytes(n, K) for n in shapes.values())
    R = max(3, math.ceil(ROTATE_BYTES / step_bytes))
    log(f"uploading {R} weight copies of each shape ({R * step_bytes / 2**30:.2f} GiB)")
    W = {}
    for k in shapes:
        w0, s0, x0 = (up(a) for a in host[k])
        W[k] = ([w0] + [w0.clone() for _ in range(R - 1)], [s0] + [s0.clone() for _ in range(R - 1)], x0,
                torch.empty((1, shapes[k]), dtype=torch.float32, device=dev))

    def step(i):
        j = i % R
        for k in ("mlp", "attn"):
            ws, ss, x, y = W[k]
            bonsai.q1_gemv(ws[j], ss[j], x, out=y)

    step(0)
    torch.cuda.synchronize()
    log("capturing graphs")
    g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for i in range(max(args.warmup, 1)):
            step(i)
    with torch.cuda.graph(g_main):
        for i in range(args.steps):
            step(i + args.warmup)
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
    value = args.steps * step_bytes / (ms / 1e3) / 1e9
    log(f"{ms:.3f} ms for {args.steps} steps ({wall * 1e3:.3f} ms wall): {value:.1f} GB/s")

    # ---- dominant kernel: device durations of the same launches, no graph ----------------
    n_t = min(args.steps, 300)
    launches = []
    for i in range(n_t):
        j = i % R
        for k in ("mlp", "attn"):
            ws, ss, x, y = W[k]
            launches.append(lambda ws=ws, ss=ss, x=x, y=y, j=j: bonsai.q1_gemv(ws[j], ss[j], x, out=y))
    kt = kernel_times(hip, bonsai, launches)
    t_mlp, t_attn = np.mean(kt[0::2]), np.mean(kt[1::2])
    alg = {k: q1_bytes(n, K) + 2 * K + 4 * n for k, n in shapes.items()}    # weights + x + y
    per_launch_bytes = (alg["mlp"] + alg["attn"]) / 2
    per_launch_ms = float(np.mean(kt))
    achieved = per_launch_bytes / (per_launch_ms / 1e3) / 1e9
    digest = src_digest(ROOT / "ternary_weight_quantized_bonsai_amd" / "csrc" / "q1_gemv.hip")
    traffic = read_pmc(f"{HEADLINE_KERNEL}_decode_pair_hbm_traffic.txt", digest)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": HEADLINE_KERNEL, "avg_launch_us": round(per_launch_ms * 1e3, 3),
                "bytes_per_launch": per_launch_bytes,
                "per_shape_us": {"mlp_13824x5120": round(t_mlp * 1e3, 3), "attn_5120x5120": round(t_attn * 1e3, 3)}}
    log(f"q1_gemv device time: mlp {t_mlp * 1e3:.2f} us, attn {t_attn * 1e3:.2f} us -> {achieved:.1f} GB/s")

    # ---- launch floor: the same two calls per step with no work (K = 0 launches one kernel
    # that zero-fills y), timed both ways the headline is ----------------------------------
    z_w = torch.empty((64, 0), dtype=torch.int32, device=dev)
    z_s = torch.empty((64, 0), dtype=torch.int16, device=dev)
    z_x = torch.empty((1, 0), dtype=torch.int16, device=dev)
    z_y = torch.empty((1, 64), dtype=torch.float32, device=dev)

    def zcall():
        bonsai.q1_gemv(z_w, z_s, z_x, out=z_y)

    kt0 = kernel_times(hip, bonsai, [zcall] * n_t)
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
    torch.cuda.synchronize()
    floor_step_us = hip.elapsed_ms(e0, e1) * 1e3 / args.steps
    launch_floor = {"kernel_us": round(float(np.mean(kt0)) * 1e3, 3), "graph_step_us": round(floor_step_us, 3),
                    "what": "the two decode calls of a step with K = 0 (each launches one kernel that zero-fills "
                            "y), timed like the headline: per-launch events, and graph replay per step"}
    roofline["launch_floor_us"] = launch_floor["kernel_us"]
    log(f"launch floor: {launch_floor['kernel_us']:.2f} us per call, {floor_step_us:.2f} us per graph step "
        f"(the headline step takes {ms * 1e3 / args.steps:.2f} us)")

    extra = {}
    if not args.headline_only:
        # LM head: N = 248320 vocabulary rows
        N3 = 248320
        w, s, x = (up(a) for a in synth.make_q1(1, N3, K))
        R3 = max(3, math.ceil(ROTATE_BYTES / q1_bytes(N3, K)))
        ws = [w] + [w.clone() for _ in range(R3 - 1)]
        ss = [s] + [s.clone() for _ in range(R3 - 1)]
        y = torch.empty((1, N3), dtype=torch.float32, device=dev)
        bonsai.q1_gemv(ws[0], ss[0], x, out=y)
        kt3 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q1_gemv(ws[j % R3], ss[j % R3], x, out=y)
                                         for j in range(4 * R3)])
        t3 = float(np.mean(kt3))
        gb3 = q1_bytes(N3, K) / (t3 / 1e3) / 1e9
        extra["lm_head_gemv"] = {"shape": "M=1 N=248320 K=5120", "avg_kernel_us": round(t3 * 1e3, 2),
                                 "packed_weight_GBps": round(gb3, 1), "frac_of_8TBps": round(gb3 / PEAK_HBM_GBPS, 4)}
        log(f"lm head: {t3 * 1e3:.1f} us, {gb3:.1f} GB/s")
        del ws, ss, w, s, x, y

        # Prefill GEMM pp512
        M4, N4 = 512, 13824
        w, s, x = (up(a) for a in synth.make_q1(M4, N4, K))
        ws = [w] + [w.clone() for _ in range(2)]
        ss = [s] + [s.clone() for _ in range(2)]
        y = torch.empty((M4, N4), dtype=torch.float32, device=dev)
        bonsai.q1_gemm(ws[0], ss[0], x, out=y)
        kt4 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q1_gemm(ws[j % 3], ss[j % 3], x, out=y)
                                         for j in range(30)])
        t4 = float(np.mean(kt4))
        tf = 2.0 * M4 * N4 * K / (t4 / 1e3) / 1e12
        extra["prefill_gemm"] = {"shape": "M=512 N=13824 K=5120", "avg_kernel_us": round(t4 * 1e3, 2),
                                 "TFLOPs": round(tf, 2),
                                 "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP16_TFLOPS,
                                              "unit": "TFLOP/s", "frac": round(tf / PEAK_FP16_TFLOPS, 4)}}
        log(f"prefill gemm: {t4 * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        del ws, ss, w, s, x, y

        # Ternary prefill GEMM at the same shape (2-bit codes)
        w, s, x = (up(a) for a in synth.make_q2t(M4, N4, K))
        ws = [w] + [w.clone() for _ in range(2)]
        ss = [s] + [s.clone() for _ in range(2)]
        y = torch.empty((M4, N4), dtype=torch.float32, device=dev)
        bonsai.q2t_gemm(ws[0], ss[0], x, out=y)
        kt6 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q2t_gemm(ws[j % 3], ss[j % 3], x, out=y)
                                         for j in range(30)])
        t6 = float(np.mean(kt6))
        tf6 = 2.0 * M4 * N4 * K / (t6 / 1e3) / 1e12
        extra["ternary_prefill_gemm"] = {"shape": "M=512 N=13824 K=5120", "avg_kernel_us": round(t6 * 1e3, 2),
                                         "TFLOPs": round(tf6, 2),
                                         "roofline": {"bound": "mfma", "achieved": round(tf6, 2),
                                                      "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                                                      "frac": round(tf6 / PEAK_FP16_TFLOPS, 4)}}
        log(f"ternary prefill gemm: {t6 * 1e3:.1f} us, {tf6:.1f} TFLOP/s")
        del ws, ss, w, s, x, y

        # The GEMM entry point at a few rows of x (several draft tokens checked at once): the
        # small-M kernel, 16 rows of x per pass over the weights
        small = {}
        w, s, _ = (up(a) for a in synth.make_q1(1, N4, K))
        R6 = max(3, math.ceil(ROTATE_BYTES / q1_bytes(N4, K)))
        ws = [w] + [w.clone() for _ in range(R6 - 1)]
        ss = [s] + [s.clone() for _ in range(R6 - 1)]
        for M6 in (16, 64):
            x = up(synth.make_q1(M6, N4, K)[2])
            y = torch.empty((M6, N4), dtype=torch.float32, device=dev)
            bonsai.q1_gemm(ws[0], ss[0], x, out=y)
            kt6 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q1_gemm(ws[j % R6], ss[j % R6], x, out=y)
                                             for j in range(R6)])
            t6 = float(np.mean(kt6))
            small[f"M{M6}"] = {"avg_kernel_us": round(t6 * 1e3, 2),
                               "TFLOPs": round(2.0 * M6 * N4 * K / (t6 / 1e3) / 1e12, 2),
                               "packed_weight_GBps": round(q1_bytes(N4, K) / (t6 / 1e3) / 1e9, 1)}
            log(f"small-M gemm M={M6}: {t6 * 1e3:.2f} us")
        extra["small_m_gemm"] = {"shape": "N=13824 K=5120, binary", **small}
        del ws, ss, w, s, x, y

        # Ternary decode GEMV, M = 1 and 8
        N5 = 5120
        tern = {}
        for M5 in (1, 8):
            w, s, x = (up(a) for a in synth.make_q2t(M5, N5, K))
            R5 = max(3, math.ceil(ROTATE_BYTES / q2t_bytes(N5, K)))
            ws = [w] + [w.clone() for _ in range(R5 - 1)]
            ss = [s] + [s.clone() for _ in range(R5 - 1)]
            y = torch.empty((M5, N5), dtype=torch.float32, device=dev)
            bonsai.q2t_gemv(ws[0], ss[0], x, out=y)
            kt5 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q2t_gemv(ws[j % R5], ss[j % R5], x, out=y)
                                             for j in range(R5)])
            t5 = float(np.mean(kt5))
            gb5 = q2t_bytes(N5, K) / (t5 / 1e3) / 1e9
            tern[f"M{M5}"] = {"avg_kernel_us": round(t5 * 1e3, 2), "packed_weight_GBps": round(gb5, 1),
                              "frac_of_8TBps": round(gb5 / PEAK_HBM_GBPS, 4)}
            log(f"ternary M={M5}: {t5 * 1e3:.2f} us, {gb5:.1f} GB/s")
            del ws, ss, w, s, x, y
        extra["ternary_gemv"] = {"shape": "N=5120 K=5120", **tern}

        # The same ternary decode on the base-3 layout (five trits per byte)
        t5r = {}
        for M5 in (1, 8):
            c5, s5, x5 = (up(v) for v in synth.make_t5(M5, N5, K))
            nb5 = c5.numel() + 2 * s5.numel()
            R5 = max(3, math.ceil(ROTATE_BYTES / nb5))
            cs = [c5] + [c5.clone() for _ in range(R5 - 1)]
            ss = [s5] + [s5.clone() for _ in range(R5 - 1)]
            y = torch.empty((M5, N5), dtype=torch.float32, device=dev)
            bonsai.t5_matmul(cs[0], ss[0], x5, out=y)
            kt5 = kernel_times(hip, bonsai, [lambda j=j: bonsai.t5_matmul(cs[j % R5], ss[j % R5], x5, out=y)
                                             for j in range(R5)])
            t5 = float(np.mean(kt5))
            gb5 = nb5 / (t5 / 1e3) / 1e9
            t5r[f"M{M5}"] = {"avg_kernel_us": round(t5 * 1e3, 2), "packed_weight_GBps": round(gb5, 1),
                             "frac_of_8TBps": round(gb5 / PEAK_HBM_GBPS, 4)}
            log(f"base-3 ternary M={M5}: {t5 * 1e3:.2f} us, {gb5:.1f} GB/s")
            del cs, ss, c5, s5, x5, y
        extra["ternary_base3_gemv"] = {"shape": "N=5120 K=5120, 1.725 bits per weight", **t5r}

        # Affine 1-bit form (MLX's scale and bias per group): decode at the MLP shape, and one row
        # of x at the LM-head shape
        aff = {}
        for M7, N7 in ((1, N4), (8, N4), (1, N3)):
            w, a7, b7, x = (up(v) for v in synth.make_q1a(M7, N7, K))
            nb7 = q1_bytes(N7, K) + 2 * N7 * (K // 128)            # + the biases
            R7 = max(3, math.ceil(ROTATE_BYTES / nb7))
            ws = [w] + [w.clone() for _ in range(R7 - 1)]
            as_ = [a7] + [a7.clone() for _ in range(R7 - 1)]
            bs = [b7] + [b7.clone() for _ in range(R7 - 1)]
            y = torch.empty((M7, N7), dtype=torch.float32, device=dev)
            bonsai.q1a_matmul(ws[0], as_[0], bs[0], x, out=y)
            kt7 = kernel_times(hip, bonsai, [lambda j=j: bonsai.q1a_matmul(ws[j % R7], as_[j % R7], bs[j % R7], x, out=y)
                                             for j in range(R7 if N7 == N4 else 4 * R7)])
            t7 = float(np.mean(kt7))
            gb7 = nb7 / (t7 / 1e3) / 1e9
            aff[(M7, N7)] = {"avg_kernel_us": round(t7 * 1e3, 2), "packed_weight_GBps": round(gb7, 1),
                             "frac_of_8TBps": round(gb7 / PEAK_HBM_GBPS, 4)}
            log(f"affine M={M7} N={N7}: {t7 * 1e3:.2f} us, {gb7:.1f} GB/s")
            del ws, as_, bs, w, a7, b7, x, y
        extra["affine_gemv"] = {"shape": "N=13824 K=5120, 1-bit affine (scale + bias per group)",
                                "M1": aff[(1, N4)], "M8": aff[(8, N4)]}
        extra["affine_lm_head_gemv"] = {"shape": "M=1 N=248320 K=5120, 1-bit affine", **aff[(1, N3)]}

        # Embedding gather: 512 token ids from the binary vocabulary table (V = 248320, K = 5120)
        w, s, _ = (up(v) for v in synth.make_q1(1, N3, K))
        ids = torch.from_numpy(np.random.default_rng(7).integers(0, N3, 512).astype(np.int64)).to(dev)
        out = torch.empty((512, K), dtype=torch.float16, device=dev)
        bonsai.q1_embed(w, s, ids, out=out)
        kt8 = kernel_times(hip, bonsai, [lambda: bonsai.q1_embed(w, s, ids, out=out) for _ in range(20)])
        t8 = float(np.mean(kt8))
        nb8 = 512 * (2 * K + K // 8 + 2 * (K // 128) + 8)        # rows written + rows read + ids
        gb8 = nb8 / (t8 / 1e3) / 1e9
        extra["embed_gather"] = {"shape": "512 ids, V=248320 K=5120", "avg_kernel_us": round(t8 * 1e3, 2),
                                 "GBps": round(gb8, 1), "frac_of_8TBps": round(gb8 / PEAK_HBM_GBPS, 4)}
        log(f"embed gather: {t8 * 1e3:.2f} us, {gb8:.1f} GB/s")
        del w, s, ids, out

    # Device copy probe: what a plain 1 GiB copy reaches on this machine (read + write bytes); its
    # dispatches also calibrate the HBM byte counters of the traffic summary
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = hip.event(), hip.event()
    hip.record(c0, stream())
    for _ in range(10):
        b.copy_(a)
    hip.record(c1, stream())
    tc = hip.elapsed_ms(c0, c1) / 10
    copy_probe = {"bytes_moved": 2 * nbytes, "GBps": round(2 * nbytes / (tc / 1e3) / 1e9, 1)}
    log(f"copy probe: {2 * nbytes / (tc / 1e3) / 1e9:.1f} GB/s")
    del a, b


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
        "config": {"workload": "binary g128 decode GEMV, M=1, K=5120: one MLP-shaped (N=13824) and one "
                               "attention-shaped (N=5120) projection per step",
                   "weight_copies_rotated": R, "accumulate": "f32", "frac_of_8TBps": round(value / PEAK_HBM_GBPS, 4),
                   "timed_as": "HIP graph replay of the steps, HIP events on the launch stream"},
        "roofline": roofline,
    }
    line["copy_probe"] = copy_probe
    line["launch_floor"] = launch_floor
    line.update(extra)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        hA, hB = host["mlp"], host["attn"]
        line["cpu_baseline"] = cpu_baseline(hA[0], hA[1], hA[2], hB[0], hB[1], hB[2], K, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
