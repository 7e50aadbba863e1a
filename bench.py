"""Benchmark of the fp16 GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the library's C-ABI (host validation and dispatch, then
the kernel or kernels the plan picks) on the MoE-derived dense GEMM
131072 x 2048 x 7168 (A [M,K] and B [K,N] row-major, U(-1,1) fp16 from the
seeded generator, fp32 accumulation, fp16 C), with inputs resident in HBM.
Prints one JSON line: throughput in TFLOPS of useful 2MNK work, the roofline
of the dominant kernel (MFMA-bound: fraction of the dense fp16 peak), the
CPU oracle timed on a bounded row sample, and the decode-shaped M = 1 case
(N = 2048, K = 7168) in GB/s of algorithmic bytes against HBM bandwidth.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS & %MFMA peak, fp16 GEMM 131072x2048x7168; GB/s at M=1"
PEAK_F16_TFLOPS = 2516.6      # MI355X dense fp16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_F8_TFLOPS = 5033.2       # MI355X dense FP8 MFMA (twice the fp16 rate)
PAGES_TFLOPS = 117.250897     # the pages' TileLang kernel on MetaX C500, same workload (context)
M, N, K = 131072, 2048, 7168


# Single workloads for profilers (bench.py --case NAME): M, N, K, B layout,
# seed.  Working sets under 1 GiB rotate over copies of A and B.
CASES = {
    "main": (131072, 2048, 7168, "row", 4001),
    "decode_m1": (1, 2048, 7168, "row", 3001),
    "decode_m16": (16, 2048, 7168, "row", 3016),
    "decode_m64": (64, 2048, 7168, "row", 3064),
    "splitk": (512, 512, 65536, "row", 3004),
    "square_4096": (4096, 4096, 4096, "row", 6096),
    "square_8192": (8192, 8192, 8192, "row", 10192),
    "stride": (262181, 1061, 8192, "col", 5001),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skinny-reps", type=int, default=400, help="decode calls timed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device copy (a known-size reference for HBM counters)")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload family (one JSON line each) instead of the headline")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="turn rocprofv3 --pmc counter_collection.csv files (pairs of FETCH_SIZE "
                         "and WRITE_SIZE passes of --copy-calibration runs, e.g. --case main and "
                         "--case decode_m1) into profiles/traffic.json")
    ap.add_argument("--summarize-profile", nargs="+", metavar="CSV",
                    help="markdown summary of one --case run under rocprofv3: a kernel_trace.csv "
                         "(durations) and counter_collection.csv files of --pmc passes")
    ap.add_argument("--operands", choices=["uniform", "int", "a_half", "b_half", "b_zero"],
                    default="uniform",
                    help="with --case: operand values (U(-1,1); integers in [-4,4]; or every "
                         "element of A or of B set to 0.5, or B to 0), to show how the clock "
                         "depends on the data the matrix cores multiply")
    ap.add_argument("--case", choices=sorted(CASES),
                    help="run only this workload's calls (--steps of them after --warmup), for "
                         "profilers; prints one JSON line with its per-call time")
    return ap.parse_args()


def library_hash():
    """Hash of the built libgemmf16.so, the code the counters describe (the
    build is reproducible: the same sources give the same bytes, whatever
    their comments), or None when it is not built."""
    path = os.path.join(ROOT, "dense_tiled_gemm_fp16_amd", "libgemmf16.so")
    try:
        with open(path, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None


def measured_traffic(kind):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the library as built now (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kind)
    if not e or e.get("library_hash") is None or e.get("library_hash") != library_hash():
        return None
    return e.get("bytes_per_launch")


COPY_KIB = float(1 << 20)      # the calibration copy reads and writes 1 GiB
# The fp16 main-kernel instantiation that the 131072x2048x7168 plan runs
# (N-contiguous B, one K range, not grouped).
MAIN_KERNEL = "void gemmf16::gemm_dma_a128_kernel<gemmf16::DmaA128Cfg<4, 2>, false, false, false, 0, false>"


def summarize_pmc(*paths):
    """Per-launch HBM bytes of the library's kernels from FETCH_SIZE / WRITE_SIZE.

    Each counter is scaled by bytes-moved / counter-reading of the 1 GiB
    device copy (the largest dispatches of the runtime's copy kernel in the
    same run), so the factor absorbs whatever fraction of the memory
    channels the counter samples."""
    import csv
    import statistics

    def load(counter):
        per, scales = {}, []
        for path in paths:
            mine = {}
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        mine.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            if not mine:
                continue
            copy = sorted(mine.get("__amd_rocclr_copyBuffer", []))[-3:]
            if not copy:
                raise SystemExit(f"{path}: no calibration copy found (run with --copy-calibration)")
            scales.append(COPY_KIB / statistics.median(copy))
            for k, v in mine.items():
                per.setdefault(k, []).extend(v)
        if not scales:
            raise SystemExit(f"no {counter} pass among the files")
        return per, statistics.median(scales)

    fetch, f_scale = load("FETCH_SIZE")
    write, w_scale = load("WRITE_SIZE")

    def kernel(prefix):
        # The instantiation itself: the grouped and bfloat16 launches of the
        # same kernel template run in the same process.
        names = [k for k in fetch if k.startswith(prefix)]
        if not names:
            return None
        name = max(names, key=lambda k: statistics.mean(fetch[k]))
        fb = statistics.mean(fetch[name]) * f_scale * 1024.0
        wb = statistics.mean(write.get(name, [0.0])) * w_scale * 1024.0
        return name, fb, wb

    out = {"calibration": {"copy_bytes": COPY_KIB * 1024, "fetch_scale": f_scale,
                           "write_scale": w_scale, "copy_kernel": "__amd_rocclr_copyBuffer"},
           "library_hash": library_hash()}
    alg = {"main_131072x2048x7168": (MAIN_KERNEL, 2.0 * (M * K + K * N), 2.0 * M * N),
           "skinny_m1_partials": ("void gemmf16::decode_kernel<16, 0, false>", 2.0 * (K + K * N), None),
           "skinny_m1_reduce": ("void gemmf16::splitk_reduce_elem<0>", None, 2.0 * N)}
    for key, (sub, alg_read, alg_write) in alg.items():
        k = kernel(sub)
        if k is None:
            continue
        name, fb, wb = k
        out[key] = {"kernel": name, "fetch_bytes": fb, "write_bytes": wb,
                    "bytes_per_launch": fb + wb, "algorithmic_read_bytes": alg_read,
                    "algorithmic_write_bytes": alg_write, "library_hash": out["library_hash"]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


SIMDS = 1024       # 256 CUs x 4 SIMDs
XCDS = 8


def summarize_profile(paths):
    """Markdown summary of a --case run under rocprofv3.

    From the kernel trace: per library kernel, the steady-state median,
    mean and minimum duration over its launches after the first fifth (the
    warm-up).  From counter passes: the per-dispatch mean of every counter
    over the same steady-state dispatches, and derived figures:
      clock       GRBM_GUI_ACTIVE / XCDs / median duration (GRBM_GUI_ACTIVE is
                  counted once per XCD), for launches of 100 us or more;
      MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles per XCD x 1024 SIMDs);
      LDS bank conflicts per active LDS cycle;
      L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS);
      FETCH/WRITE bytes, scaled by a 1 GiB device copy in the same pass
                  (--copy-calibration) when one is there."""
    import csv
    import statistics

    def steady(vals):
        return vals[len(vals) // 5:] if len(vals) >= 5 else vals

    dur, ctr = {}, {}
    for path in paths:
        with open(path) as f:
            rows = list(csv.DictReader(f))
        if rows and "Start_Timestamp" in rows[0] and "Counter_Name" not in rows[0]:
            for r in rows:
                dur.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        else:
            per = {}
            for r in rows:
                key = (r["Kernel_Name"], r["Counter_Name"])
                per.setdefault(key, {}).setdefault(r.get("Dispatch_Id", len(per)), 0.0)
                per[key][r.get("Dispatch_Id", len(per))] += float(r["Counter_Value"])
            for (k, c), d in per.items():
                ctr.setdefault(k, {})[c] = [d[i] for i in sorted(d, key=lambda x: int(x))]
    scale = {}
    for c, kib in (("FETCH_SIZE", COPY_KIB), ("WRITE_SIZE", COPY_KIB)):
        copy = sorted(ctr.get("__amd_rocclr_copyBuffer", {}).get(c, []))[-3:]
        if copy:
            scale[c] = kib * 1024.0 / statistics.median(copy)
    lines = ["| kernel | launches | median (us) | mean (us) | min (us) |", "|---|---|---|---|---|"]
    for k in sorted(dur, key=lambda k: -sum(dur[k])):
        if "gemmf16" not in k:
            continue
        v = steady(dur[k])
        lines.append(f"| `{k[:110]}` | {len(v)} | {statistics.median(v):.2f} | "
                     f"{statistics.mean(v):.2f} | {min(v):.2f} |")
    lines += ["", "| kernel | counter | per dispatch (steady mean) |", "|---|---|---|"]
    derived = ["", "| kernel | clock (GHz) | MFMA busy | LDS bank conflict / LDS active | "
               "L2 hit rate | fetched bytes | written bytes |", "|---|---|---|---|---|---|---|"]
    for k in sorted(ctr):
        if "gemmf16" not in k:
            continue
        m = {c: statistics.mean(steady(v)) for c, v in ctr[k].items()}
        for c in sorted(m):
            lines.append(f"| `{k[:70]}` | {c} | {m[c]:.6g} |")
        med = statistics.median(steady(dur[k])) if k in dur else None
        gui = m.get("GRBM_GUI_ACTIVE")
        cyc = gui / XCDS if gui else None
        # (over launches shorter than 100 us the GUI-active window, which
        # includes the dispatch's own set-up and cache actions, overstates it)
        clock = f"{cyc / (med * 1e3):.3f}" if cyc and med and med >= 100.0 else "-"
        mfma = (f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * SIMDS):.1f}%"
                if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m else "-")
        lds = (f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.4f}"
               if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m else "-")
        hit = (f"{m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.3f}"
               if "TCC_HIT_sum" in m and m.get("TCC_HIT_sum", 0) + m.get("TCC_MISS_sum", 0) > 0 else "-")
        fb = f"{m['FETCH_SIZE'] * scale['FETCH_SIZE']:.4g}" if "FETCH_SIZE" in m and "FETCH_SIZE" in scale else "-"
        wb = f"{m['WRITE_SIZE'] * scale['WRITE_SIZE']:.4g}" if "WRITE_SIZE" in m and "WRITE_SIZE" in scale else "-"
        derived.append(f"| `{k[:70]}` | {clock} | {mfma} | {lds} | {hit} | {fb} | {wb} |")
    if scale:
        derived.append("")
        derived.append("Byte scale factors from the 1 GiB copy: " +
                       ", ".join(f"{c} x{v / 1024.0:.4f} per KiB" for c, v in scale.items()))
    print("\n".join(lines + derived))


def timed_launches(fn, stream, steps, warmup):
    """Per-launch durations (ms) from HIP events recorded on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def timed_pair(fn1, fn2, stream, steps, warmup):
    """Per-launch durations (ms) of fn1 and fn2 called in alternation."""
    import torch
    for _ in range(warmup):
        fn1()
        fn2()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fn1()
        e[1].record(stream)
        e[2].record(stream)
        fn2()
        e[3].record(stream)
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev], [e[2].elapsed_time(e[3]) for e in ev]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=15.0):
    """The CPU oracle (as is) on whole output rows of the same product, with
    the time of the whole product projected from the sample's row rate."""
    import numpy as np
    import oracle
    import synth
    threads = oracle.threads()
    B = synth.matrix(K, N, 4001, synth.TENSOR_B)

    def rows_time(r):
        A = synth.rows_of(np.arange(r), K, 4001, synth.TENSOR_A)
        t = time.perf_counter()
        oracle.gemm(A, (K, 1), B, (N, 1), r, N, K, nthreads=threads)
        return time.perf_counter() - t

    pilot = rows_time(threads)
    rows = int(max(threads, min(4096, threads * round(budget_s / max(pilot, 1e-3)))))
    dt = rows_time(rows)
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {M}x{N}x{K} product ({rows}x{N} outputs, "
                      f"full K), {dt:.1f} s",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "threads_note": "one oracle thread per core of this process's affinity, at most 16 "
                            "(the host share of one GPU)",
            "projected_full_product_s": round(dt * M / rows, 1)}


# The workload families (the pages' shapes and the MoE product), as (name,
# M, N, K, B layout[, forced plans: a variant name or a dict of options]);
# the configurations sweep times each one (not the headline line).
CONFIGS = [
    ("edge_130x70x65", 130, 70, 65, "row"), ("edge_130x70x65_bt", 130, 70, 65, "col"),
    ("square_256", 256, 256, 256, "row"),
    ("square_1024", 1024, 1024, 1024, "row", ({"variant": "main", "tile": 1},)),
    ("square_4096", 4096, 4096, 4096, "row"), ("square_8192", 8192, 8192, 8192, "row"),
    ("skinny_m1", 1, 2048, 7168, "row"), ("skinny_m16", 16, 2048, 7168, "row"),
    ("skinny_m64", 64, 2048, 7168, "row"),
    # B as [N, K] rows (the usual storage of weights): not one of the pages' workloads
    ("skinny_m1_bt", 1, 2048, 7168, "col"), ("skinny_m16_bt", 16, 2048, 7168, "col"),
    ("splitk_512x512x65536", 512, 512, 65536, "row"),
    ("moe_131072x2048x7168", 131072, 2048, 7168, "row"),
    ("stride_262181x1061x8192_bt", 262181, 1061, 8192, "col", ("main", "streamk")),
    # not one of the pages' workloads: 17 x 16 tiles, a final wave of 16 tiles on 256 CUs
    ("tail_4352x4096x8192", 4352, 4096, 8192, "row", ("main",)),
    # not one of the pages' workloads: mid-size products under a wave of 256 x 256 tiles
    ("mid_2048", 2048, 2048, 2048, "row", ({"variant": "main", "tile": 1}, {"variant": "main", "tile": 14})),
    ("splitk_1024x1024x4096", 1024, 1024, 4096, "row", ({"variant": "splitk", "tile": 14},)),
]


def configs_sweep():
    """One JSON line per configuration: GPU time per call and the rate
    against the roofline its arithmetic intensity selects.  Working sets
    under 1 GiB rotate over copies (up to 64) so calls do not run from the
    previous call's caches; calls are captured in a graph so per-call host
    cost is not timed."""
    import numpy as np
    import torch

    import dense_tiled_gemm_fp16_amd as g
    import synth

    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)

    for i, cfg in enumerate(CONFIGS):
        name, m, n, k, bl = cfg[:5]
        for forced in ("auto",) + (cfg[5] if len(cfg) > 5 else ()):
            sweep_one(g, synth, dev, to_dev, i, name, m, n, k, bl, forced)


def sweep_one(g, synth, dev, to_dev, i, name, m, n, k, bl, forced):
    """Time one configuration under one plan (see configs_sweep)."""
    import torch
    opts = {"variant": forced} if isinstance(forced, str) else dict(forced)
    label = forced if isinstance(forced, str) else " ".join(f"{q}={v}" for q, v in forced.items())
    a0 = to_dev(synth.matrix(m, k, 7000 + i, synth.TENSOR_A))
    bt = synth.matrix(k, n, 7000 + i, synth.TENSOR_B, order="col" if bl == "col" else "row")
    b0 = to_dev(bt).t() if bl == "col" else to_dev(bt)
    byts = 2.0 * (m * k + k * n + m * n)
    copies = int(min(64, max(1, -(-(1 << 30) // int(byts)))))
    As = [a0] + [a0.clone() for _ in range(copies - 1)]
    Bs = [b0] + [(b0.t().clone().t() if bl == "col" else b0.clone()) for _ in range(copies - 1)]
    c = torch.empty((m, n), dtype=torch.float16, device=dev)
    p = g.plan(a0, b0, c, **opts)
    ws = (torch.empty(p["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)
          if p["workspace_bytes"] else None)
    cap = torch.cuda.Stream(dev)
    with torch.cuda.stream(cap):
        g.gemm(a0, b0, out=c, workspace=ws, stream=cap, **opts)
    torch.cuda.synchronize()
    # Enough calls per replay that a replay holds about 1.5e13 FLOP (some
    # 11 ms at the main kernel's rate; at most 1024 calls, at least 4): a
    # replay of a few milliseconds runs partly after the idle gap that the
    # wait between replays leaves, and read 10-15% under the steady rate
    # (4096^3: 135 us per call against 119 back to back).
    reps = max(copies, 4) if byts * copies >= (1 << 28) else max(copies, 64)
    reps = int(min(1024, max(reps, -(-1.5e13 // (2.0 * m * n * k)))))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for r in range(reps):
            g.gemm(As[r % copies], Bs[r % copies], out=c, workspace=ws, stream=cap, **opts)
    times = []
    for r in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        e1.synchronize()
        if r >= 1:
            times.append(e0.elapsed_time(e1) / reps)
    ms = sorted(times)[len(times) // 2]
    flops = 2.0 * m * n * k
    ai = flops / byts
    tf, gbs = flops / (ms * 1e-3) / 1e12, byts / (ms * 1e-3) / 1e9
    bound = "mfma" if ai >= PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    print(json.dumps({"config": name, "M": m, "N": n, "K": k, "b_layout": bl,
                      "forced": label,
                      "plan": {q: p[q] for q in ("variant", "tile_id", "split_k", "grid",
                                                 "sk_tiles", "b_path")},
                      "us_per_call": ms * 1e3, "TFLOPS": tf, "GBps": gbs, "AI": ai,
                      "bound": bound,
                      "frac": tf / PEAK_F16_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS,
                      "copies": copies}), flush=True)
    del As, Bs, a0, b0, c, ws, graph
    torch.cuda.empty_cache()


def copy_calibration():
    """Three device copies of 1 GiB: a known-size reference for the HBM
    byte counters of a profiling pass."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_case(name, steps, warmup, operands="uniform"):
    """--steps calls of one workload's automatic plan after --warmup, on the
    current stream; one JSON line with the mean time per call (HIP events
    around the whole loop)."""
    import numpy as np
    import torch

    import dense_tiled_gemm_fp16_amd as g
    import synth

    m, n, k, bl, seed = CASES[name]
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)

    mode = "int" if operands == "int" else "uniform"
    a0 = to_dev(synth.matrix(m, k, seed, synth.TENSOR_A, mode))
    bt = synth.matrix(k, n, seed, synth.TENSOR_B, mode, order="col" if bl == "col" else "row")
    b0 = to_dev(bt).t() if bl == "col" else to_dev(bt)
    if operands == "a_half":
        a0.fill_(0.5)
    elif operands == "b_half":
        b0.fill_(0.5)
    elif operands == "b_zero":
        b0.zero_()
    byts = 2.0 * (m * k + k * n + m * n)
    copies = int(min(64, max(1, -(-(1 << 30) // int(byts)))))
    As = [a0] + [a0.clone() for _ in range(copies - 1)]
    Bs = [b0] + [(b0.t().clone().t() if bl == "col" else b0.clone()) for _ in range(copies - 1)]
    c = torch.empty((m, n), dtype=torch.float16, device=dev)
    p = g.plan(a0, b0, c)
    ws = (torch.empty(p["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)
          if p["workspace_bytes"] else None)
    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        g.gemm(As[i % copies], Bs[i % copies], out=c, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        g.gemm(As[i % copies], Bs[i % copies], out=c, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"case": name, "operands": operands, "M": m, "N": n, "K": k, "b_layout": bl,
                      "copies": copies,
                      "steps": steps, "warmup": warmup, "us_per_call": us,
                      "TFLOPS": 2.0 * m * n * k / us / 1e6, "GBps": byts / us / 1e3,
                      "plan": {q: p[q] for q in ("variant", "tile_id", "tile_m", "tile_n",
                                                 "split_k", "grid", "grid2", "b_path")}}),
          flush=True)


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.case:
        if args.copy_calibration:
            copy_calibration()
        run_case(args.case, args.steps, args.warmup, args.operands)
        return
    if args.configs:
        configs_sweep()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dense_tiled_gemm_fp16_amd as g
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)

    if args.copy_calibration:
        copy_calibration()

    # ---- headline workload
    a = to_dev(synth.matrix(M, K, 4001, synth.TENSOR_A))
    b = to_dev(synth.matrix(K, N, 4001, synth.TENSOR_B))
    c = torch.empty((M, N), dtype=torch.float16, device=dev)
    plan = g.plan(a, b, c)
    ws = None
    if plan["workspace_bytes"]:
        ws = torch.empty(plan["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        g.gemm(a, b, out=c, workspace=ws, stream=stream)

    durs, wall = timed_launches(step, stream, args.steps, args.warmup)
    flops = 2.0 * M * N * K
    ms = sum(durs) / len(durs)
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic("main_131072x2048x7168")

    # ---- decode-shaped M = 1, B N-contiguous (the workload) and as [N, K]
    # rows; in fp16, and with E4M3 operands (fp16 out)
    def decode_line(b_layout, fmt="f16"):
        m1 = 1
        esz = 1 if fmt == "e4m3" else 2
        copies = 40 * (2 // esz)                      # 40 x 28 MiB (80 x 14 MiB) of B > 1 GiB

        def dev_bits(bits):
            if fmt == "e4m3":
                return torch.from_numpy(bits).to(dev).view(torch.float8_e4m3fn)
            return to_dev(bits)
        kw = {} if fmt == "f16" else {"fmt": fmt}
        a1 = dev_bits(synth.matrix(m1, K, 3001, synth.TENSOR_A, **kw))
        if b_layout == "col":
            b1 = dev_bits(synth.matrix(K, N, 3001, synth.TENSOR_B, order="col", **kw)).t()
            bs = [b1.t().clone().t() for _ in range(copies)]
        else:
            b1 = dev_bits(synth.matrix(K, N, 3001, synth.TENSOR_B, **kw))
            bs = [b1.clone() for _ in range(copies)]
        c1 = torch.empty((m1, N), dtype=torch.float16, device=dev)
        p1 = g.plan(a1, b1, c1)
        ws1 = None
        if p1["workspace_bytes"]:
            ws1 = torch.empty(p1["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)
        # One CUDA/HIP graph holds 25 passes of one call per copy of B (about
        # 10 ms of calls), so the timing is GPU time per call (both launches
        # and the gap between them) at the steady rate, free of the Python
        # wrapper's per-call host cost and of the idle gap between replays.
        cap = torch.cuda.Stream(dev)
        with torch.cuda.stream(cap):
            g.gemm(a1, bs[0], out=c1, workspace=ws1, stream=cap)
        torch.cuda.synchronize()
        eager = c1.clone()
        graph = torch.cuda.CUDAGraph()
        rounds = 25
        with torch.cuda.graph(graph, stream=cap):
            for rnd in range(rounds):
                for i in range(copies):
                    g.gemm(a1, bs[i], out=c1, workspace=ws1, stream=cap)
        calls = rounds * copies
        reps = max(3, args.skinny_reps // calls)
        per_call = []
        graph_ok = True
        for r in range(reps + 2):
            c1.fill_(float("nan"))
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            e1.synchronize()
            graph_ok = graph_ok and torch.equal(c1.view(torch.int16), eager.view(torch.int16))
            if r >= 2:
                per_call.append(e0.elapsed_time(e1) / calls)
        per_call.sort()
        med1 = per_call[len(per_call) // 2]
        bytes1 = esz * (m1 * K + K * N) + 2.0 * m1 * N
        del graph, bs
        what = "B [K, N]" if b_layout == "row" else "B as [N, K] rows"
        what += ", E4M3 operands, fp16 out" if fmt == "e4m3" else ""
        return {"workload": f"M={m1} N={N} K={K}, {what}, B rotated over {copies} copies",
                "plan": {k: p1[k] for k in ("variant", "tile_m", "tile_n", "split_k", "grid",
                                             "grid2", "b_path")},
                "median_us": med1 * 1e3, "GBps": bytes1 / (med1 * 1e-3) / 1e9,
                "frac_hbm": bytes1 / (med1 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "replays_match_eager": graph_ok,
                "timing": f"HIP events around replays of a graph of {calls} calls ({rounds} passes over the copies) "
                          f"({reps} replays, median per call)"}

    skinny = decode_line("row")
    skinny_nk = decode_line("col")
    skinny_f8 = decode_line("row", "e4m3")
    skinny_f8_nk = decode_line("col", "e4m3")

    # ---- grouped product: the same tokens routed to 32 experts
    G = 32
    sizes = synth.group_sizes(G, M, 11)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)).to(dev)
    bg = torch.empty((G, K, N), dtype=torch.float16, device=dev)
    for e in range(G):
        bg[e] = to_dev(synth.matrix(K, N, 4101, 16 + e))
    wsg = torch.empty(g.lib.gemm_f16_grouped_workspace_bytes(G) // 4 + 64, dtype=torch.float32,
                      device=dev)

    def step_g():
        g.gemm_grouped(a, bg, offs, out=c, workspace=wsg, stream=stream)

    # In alternation with the dense product on the same rows, so both run
    # under the same clocks.
    dg, dd = timed_pair(step_g, step, stream, max(10, args.steps // 2), 4)
    msg, msd = sum(dg) / len(dg), sum(dd) / len(dd)
    grouped = {"workload": f"{M} routed tokens over {G} experts (seeded skewed counts "
                           f"{int(sizes.min())}..{int(sizes.max())}), K={K}, N={N}, one B per expert",
               "ms": msg, "TFLOPS": flops / (msg * 1e-3) / 1e12,
               "frac": flops / (msg * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
               "dense_TFLOPS_same_loop": flops / (msd * 1e-3) / 1e12,
               "timing": "HIP events around each call (set-up and product launches), alternating "
                         "with the dense product's call"}
    del bg

    # ---- bfloat16: the same product in the other 16-bit format
    del a
    ab = to_dev(synth.matrix(M, K, 4001, synth.TENSOR_A, fmt="bf16")).view(torch.bfloat16)
    bb = to_dev(synth.matrix(K, N, 4001, synth.TENSOR_B, fmt="bf16")).view(torch.bfloat16)
    cb = c.view(torch.bfloat16)

    def step_b():
        g.gemm(ab, bb, out=cb, stream=stream)

    db, _ = timed_launches(step_b, stream, max(5, args.steps // 5), 2)
    msb = sum(db) / len(db)
    bf16 = {"workload": f"{M}x{N}x{K}, bfloat16 inputs and output, fp32 accumulation",
            "plan": {k: g.plan(ab, bb, cb)[k] for k in ("variant", "tile_id", "split_k")},
            "ms": msb, "TFLOPS": flops / (msb * 1e-3) / 1e12,
            "frac": flops / (msb * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
            "timing": "HIP events around each call"}
    del ab, bb

    # ---- pre-packed B: the same product with B packed once (not timed)
    a = to_dev(synth.matrix(M, K, 4001, synth.TENSOR_A))
    packed = g.pack_b(b)
    torch.cuda.synchronize()

    def step_p():
        g.gemm_packed(a, packed, out=c, stream=stream)

    # Alternating with the general call on the same operands, so that both
    # run under the same clocks (the chip's clock drifts over a run).
    dp, dgen = timed_pair(step_p, step, stream, max(10, args.steps // 2), 4)
    msp, msgen = sum(dp) / len(dp), sum(dgen) / len(dgen)
    packed_b = {"workload": f"{M}x{N}x{K} fp16, B packed once by gemm_f16_pack_b (not timed)",
                "ms": msp, "TFLOPS": flops / (msp * 1e-3) / 1e12,
                "frac": flops / (msp * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                "general_TFLOPS_same_loop": flops / (msgen * 1e-3) / 1e12,
                "timing": "HIP events around each call, alternating with the general path's call"}
    del packed

    # ---- K-contiguous B (B as [N, K] weights): the automatic plan packs B
    # into the workspace, then runs the packed-B product; timed with the
    # packing launch, in alternation with the direct K-major plan.
    bk = b.t().contiguous().t()
    pk = g.plan(a, bk, c)
    wsk = torch.empty(pk["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)

    def step_k():
        g.gemm(a, bk, out=c, workspace=wsk, stream=stream)

    def step_kd():
        g.gemm(a, bk, out=c, variant="main", tile=14, stream=stream)

    dk, dkd = timed_pair(step_k, step_kd, stream, max(10, args.steps // 2), 4)
    msk, mskd = sum(dk) / len(dk), sum(dkd) / len(dkd)
    b_kmajor = {"workload": f"{M}x{N}x{K} fp16, B as [N, K] weights (K-contiguous)",
                "plan": {k: pk[k] for k in ("variant", "tile_id", "b_path", "workspace_bytes")},
                "ms": msk, "TFLOPS": flops / (msk * 1e-3) / 1e12,
                "frac": flops / (msk * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                "direct_TFLOPS_same_loop": flops / (mskd * 1e-3) / 1e12,
                "timing": "HIP events around each call (packing and product launches), "
                          "alternating with the direct K-major plan's call"}
    del a, bk, wsk

    # ---- FP8: the same product with E4M3 operands (B as [N, K] weights), fp16 out
    af = torch.from_numpy(synth.matrix(M, K, 4001, synth.TENSOR_A, fmt="e4m3")).to(dev).view(
        torch.float8_e4m3fn)
    bf = torch.from_numpy(synth.matrix(K, N, 4001, synth.TENSOR_B, fmt="e4m3", order="col")).to(
        dev).view(torch.float8_e4m3fn).t()

    pf = g.plan(af, bf, c)
    wsf = (torch.empty(pf["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=dev)
           if pf["workspace_bytes"] else None)

    def step_f():
        g.gemm(af, bf, out=c, workspace=wsf, stream=stream)

    def step_fd():
        g.gemm(af, bf, out=c, variant="main", stream=stream)

    # The automatic plan packs B ([N, K] rows) first; timed with the packing
    # launch, in alternation with the direct plan.
    df, dfd = timed_pair(step_f, step_fd, stream, max(10, args.steps // 2), 4)
    msf, msfd = sum(df) / len(df), sum(dfd) / len(dfd)
    f8 = {"workload": f"{M}x{N}x{K}, E4M3 inputs (B as [N, K] weights), fp32 accumulation, fp16 out",
          "plan": {k: pf[k] for k in ("variant", "tile_id", "split_k", "b_path", "workspace_bytes")},
          "ms": msf, "TFLOPS": flops / (msf * 1e-3) / 1e12,
          "frac": flops / (msf * 1e-3) / 1e12 / PEAK_F8_TFLOPS, "peak": PEAK_F8_TFLOPS,
          "direct_TFLOPS_same_loop": flops / (msfd * 1e-3) / 1e12,
          "timing": "HIP events around each call (packing and product launches), "
                    "alternating with the direct plan's call"}

    # ---- FP8 with B [K, N] row-major, the fp16 workload's own layout
    bfn = torch.from_numpy(synth.matrix(K, N, 4001, synth.TENSOR_B, fmt="e4m3")).to(dev).view(
        torch.float8_e4m3fn)

    pfn = g.plan(af, bfn, c)

    def step_fn():
        g.gemm(af, bfn, out=c, stream=stream)

    # In alternation with the [N, K]-weights call above (its packing plan),
    # so the two B layouts are compared under the same clocks.
    dfn, dfk = timed_pair(step_fn, step_f, stream, max(10, args.steps // 2), 4)
    msfn, msfk = sum(dfn) / len(dfn), sum(dfk) / len(dfk)
    f8_bn = {"workload": f"{M}x{N}x{K}, E4M3 inputs, B [K, N] row-major, fp32 accumulation, fp16 out",
             "plan": {k: pfn[k] for k in ("variant", "tile_id", "split_k", "b_path", "workspace_bytes")},
             "ms": msfn, "TFLOPS": flops / (msfn * 1e-3) / 1e12,
             "frac": flops / (msfn * 1e-3) / 1e12 / PEAK_F8_TFLOPS, "peak": PEAK_F8_TFLOPS,
             "nk_weights_TFLOPS_same_loop": flops / (msfk * 1e-3) / 1e12,
             "timing": "HIP events around each call, alternating with the [N, K]-weights call"}
    del af, bf, wsf, bfn

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded U(-1,1) fp16, counter-based generator)",
        "config": {"workload": "MoE-derived dense GEMM 131072x2048x7168 fp16, fp32 accumulate",
                   "M": M, "N": N, "K": K, "a_layout": "row-major", "b_layout": "row-major",
                   "plan": {k: plan[k] for k in ("variant", "tile_m", "tile_n", "tile_k",
                                                 "split_k", "panel", "a_path", "b_path",
                                                 "grid")}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic},
        "timing": {"method": "HIP events around each launch on its stream",
                   "median_ms": sorted(durs)[len(durs) // 2], "min_ms": min(durs),
                   "wall_s": wall},
        "skinny_m1": skinny,
        "skinny_m1_nk": skinny_nk,
        "skinny_m1_f8": skinny_f8,
        "skinny_m1_f8_nk": skinny_f8_nk,
        "grouped_moe": grouped,
        "bf16": bf16,
        "f8": f8,
        "f8_bn": f8_bn,
        "packed_b": packed_b,
        "b_kmajor": b_kmajor,
        "context": {"pages_tilelang_metax_c500_tflops": PAGES_TFLOPS,
                    "note": "another machine's figure for the same workload; not a target"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
        # the stated baseline is the CPU oracle on this host (vs_baseline stays
        # null: the pages' figure is another machine's, context only)
        out["cpu_baseline"]["gpu_over_cpu"] = round(tflops / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
