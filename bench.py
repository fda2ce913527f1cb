"""Benchmark of the W4A4 block-scaled FP4 linear on one MI355X.

Default workload (one step): one square NVFP4 W4A4 linear, M = N = K = 16384
(fp4_linear: activation quantization + GEMM), the largest single-GPU
configuration of the metric's compute-bound half. Operands are bf16 ~N(0, 1);
the weight is quantized once before timing, the activations inside every call.
The same run times the GEMM alone on pre-quantized activations (fp4_gemm).

Other workloads (--workload): square4096, square8192 (the rest of the square
sweep), decode (M in {1, 8, 32} x (K, N) in {(5120, 5120), (5120, 17408),
(17408, 5120)}: nine calls per step, each weight in enough copies that every
shape's copies exceed 768 MB and consecutive calls never reuse one, so the
weight stream comes from HBM rather than the 256 MB Infinity Cache), mid (M in
{64, 128} on the two large decode weights, the mid-size GEMM's regime, weights
rotated like decode's), prefill (a Llama-style 3B block at M = 4096), single
(A[16,256] x W[256,256]) and forward (a synthetic 24-layer forward at M = 1,
8, 32, 128).

Prints one JSON line: throughput incl. activation quantization (TFLOP/s), a
roofline entry for the dominant kernel (square/prefill: the tile GEMM against
the FP4 matrix peak, NVFP4 also against the f16 ceiling its exact products run
at; decode and mid: the skinny or mid-size GEMM against HBM bandwidth;
algorithmic work per launch
over its average duration, timed with HIP events on the launch stream) and the
CPU oracle timed on a bounded sample of the same work on every host core.

    python bench.py [--steps K] [--warmup W] [--fmt nvfp4|mxfp4]
                    [--workload square16384|square8192|square4096|decode|mid|prefill|single|forward]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0          # dense FP4 MFMA, published
F16_PEAK_TFLOPS = 2500.0           # dense f16/bf16 MFMA, published
METRIC = "W4A4 NVFP4 GEMM TFLOPS incl. act-quant; % FP4 MFMA peak / % HBM BW"
ROTATE_BYTES = 768 << 20           # bytes of one shape's weight copies (decode rotation)
WORKLOADS = ["square16384", "square8192", "square4096", "decode", "mid", "prefill", "single", "forward"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--fmt", default="nvfp4", choices=["nvfp4", "mxfp4"])
    p.add_argument("--recipe", default="", choices=["", "rotate", "oas", "rotate+oas", "mbs"],
                   help="quantization recipe flags for weights and activations: block "
                        "Hadamard rotation, MXFP4 overflow-aware exponent, MXFP4 macro-block scales")
    p.add_argument("--w4a16", action="store_true",
                   help="time the weight-only linear (bf16 activations x FP4 weights) instead")
    p.add_argument("--workload", default="square16384", choices=WORKLOADS)
    p.add_argument("--api", default="linear", choices=["linear", "canonical"],
                   help="linear: fp4_linear per call; canonical: fp4_quantize_act into the canonical "
                        "layout, then fp4_gemm (the two public calls)")
    p.add_argument("--nv-tile", default="", choices=["", "registers", "lds"],
                   help="NVFP4 256 x 256 tiles: convert codes to f16 in each wave's registers "
                        "or once per workgroup in LDS (default: the library's)")
    p.add_argument("--fuse-large", action="store_true",
                   help="large M: quantize the activations inside the GEMM launch (static NVFP4 "
                        "scale or MXFP4) instead of in a launch of their own")
    p.add_argument("--fuse-decode", action="store_true",
                   help="1-32 rows: quantize the activations inside the skinny GEMM's launch "
                        "instead of in a launch of their own")
    p.add_argument("--no-mid", action="store_true",
                   help="17-128 rows on large weights: run the GEMM on the skinny kernel instead of "
                        "the mid-size kernel")
    p.add_argument("--static-scale", type=float, default=0.0,
                   help="NVFP4: quantize the activations with this static tensor scale instead of "
                        "their dynamic one")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    p.add_argument("--kernel-reps", type=int, default=50)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target wall time of the oracle's GEMM sample in the CPU baseline")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="oracle threads (default: the host cores this process may use, at most 16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (a reference for "
                        "hardware byte counters)")
    p.add_argument("--pmc-step", action="store_true",
                   help="run the copy (--copy-mib) and one eager step only, for hardware "
                        "counter passes (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)")
    p.add_argument("--summarize-util", metavar="CSV",
                   help="no GPU: turn a rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LDSBankConflict "
                        "pass of --pmc-step into the utilization summary under profiles/")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn the two counter passes of --pmc-step into the traffic "
                        "summary under profiles/")
    return p.parse_args()


# 33-128 activation rows on the decode shapes whose weights are large enough
# for the mid-size GEMM (K x N = 5120 x 17408 and 17408 x 5120)
MID_SHAPES = [(5120, 17408), (17408, 5120)]
MID_M = [64, 128]


def workload_configs(name):
    import synth
    if name == "decode":
        return [(m, k, n) for (k, n) in synth.DECODE_SHAPES for m in synth.DECODE_M], \
            "decode-shaped W4A4 linear, M in {1,8,32} x (K,N) in {(5120,5120),(5120,17408),(17408,5120)}"
    if name == "mid":
        return [(m, k, n) for (k, n) in MID_SHAPES for m in MID_M], \
            "mid-size W4A4 linear, M in {64,128} x (K,N) in {(5120,17408),(17408,5120)}"
    if name == "prefill":
        return [(synth.PREFILL_M, k, n) for (k, n) in synth.PREFILL_LAYERS.values()], \
            "prefill-shaped W4A4 GEMMs of a Llama-style 3B block, M=4096"
    if name.startswith("square"):
        n = int(name[len("square"):])
        return [(n, n, n)], f"square W4A4 linear M=N=K={n}"
    return [(16, 256, 256)], "single W4A4 GEMM A[16,256] x W[256,256]"


def gemm_bytes(m, k, n, fmt):
    """Algorithmic HBM bytes of one GEMM launch: W codes + W scales + A codes +
    A scales + C (bf16). Padding is not counted."""
    bs = 16 if fmt == 0 else 32
    q = k // 2 + k // bs
    return n * q + m * q + 2 * m * n


DOMINANT = ("k_gemm_decode", "k_linear_decode", "k_gemm_mid", "k_gemm_tile", "k_gemm_prefill",
            "k_w4a16_decode", "k_w4a16_tile")


SPEC_SCLK_MHZ = 2400.0             # MI355X peak engine clock, at which the peaks are quoted


def sample_clocks(busy, seconds=1.5):
    """Graphics and memory clocks (MHz) while `busy()` keeps the GPU working:
    `amd-smi metric -c` polled from a child process for about `seconds`
    (after every timing, so the polls perturb none). The graphics clock is
    averaged over the XCDs of each sample. None when amd-smi is missing or
    prints no clock."""
    import re
    import shutil
    import subprocess
    import threading
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run([exe, "metric", "-c"], capture_output=True, text=True,
                                     timeout=20).stdout
            except Exception:
                return
            sec, gfx, mem = None, [], []
            for line in out.splitlines():
                t = line.strip()
                m = re.match(r"(GFX|MEM)_\d+:", t)
                if m:
                    sec = m.group(1)
                    continue
                m = re.match(r"CLK:\s*(\d+)\s*MHz", t)
                if m and sec:
                    (gfx if sec == "GFX" else mem).append(int(m.group(1)))
                    sec = None
            if gfx:
                samples.append((sum(gfx) / len(gfx), max(mem) if mem else None))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or (not samples and time.perf_counter() < t_end + 20):
        busy()
    stop.set()
    th.join(timeout=30)
    if not samples:
        return None
    g = sorted(x[0] for x in samples)
    mem = [x[1] for x in samples if x[1] is not None]
    return {"sclk_median": round(g[len(g) // 2]), "sclk_min": round(g[0]), "sclk_max": round(g[-1]),
            "mclk": max(mem) if mem else None, "samples": len(samples),
            "how": "amd-smi polled while the same steps replay for ~%.1f s after the timed region"
                   % seconds}


def kernel_source_hash():
    """Hash of the HIP sources: stored counter figures apply only to the build
    they were taken from."""
    import hashlib
    d = os.path.join(ROOT, "block_scaled_fp4_quantize_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def variant_tag(args):
    """Profile-file suffix of a run: the weight-only linear, the recipe flags and
    the two-call canonical API have summaries of their own ("" for plain W4A4)."""
    parts = (["w4a16"] if args.w4a16 else []) + ([args.recipe.replace("+", "_")] if args.recipe else []) + \
        (["canonical"] if getattr(args, "api", "linear") == "canonical" else [])
    return "".join("_" + x for x in parts)


def variant_flags(args):
    """The bench.py flags that select the same variant (for the commands quoted
    in the summaries)."""
    return (" --w4a16" if args.w4a16 else "") + (f" --recipe {args.recipe}" if args.recipe else "") + \
        (" --api canonical" if getattr(args, "api", "linear") == "canonical" else "")


def traffic_path(workload, fmt, tag=""):
    return os.path.join(ROOT, "profiles", f"{workload}_{fmt}{tag}_hbm_traffic.md")


def stored_traffic(workload, fmt, tag=""):
    """HBM bytes per launch of the dominant kernels from the committed counter
    summary, or None when there is none or the kernels changed since."""
    try:
        with open(traffic_path(workload, fmt, tag)) as fh:
            for line in fh:
                if line.startswith("<!-- traffic-json: "):
                    rec = json.loads(line[len("<!-- traffic-json: "):].rsplit(" -->", 1)[0])
                    if rec.get("src_hash") == kernel_source_hash():
                        return rec["bytes_per_launch"]
    except OSError:
        pass
    return None


UTIL_COUNTERS = ("MfmaUtil", "VALUBusy", "LdsUtil", "LDSBankConflict")


def summarize_util(args):
    """Per-dispatch utilization of the dominant kernels (rocprofv3's derived
    counters, percent of the kernel's active cycles) from one counter pass over
    an eager step, written under profiles/."""
    import csv
    import re
    vals = {}
    with open(args.summarize_util) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") in UTIL_COUNTERS and any(d in r["Kernel_Name"] for d in DOMINANT):
                vals.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})[r["Counter_Name"]] = \
                    float(r["Counter_Value"])
    configs, desc = workload_configs(args.workload)
    disp = [vals[d] for d in sorted(vals)]
    if len(disp) != len(configs):
        raise SystemExit(f"expected {len(configs)} dominant-kernel dispatches, found {len(disp)}")
    tag, flags = variant_tag(args), variant_flags(args)
    lines = [f"# Utilization of the dominant kernels: {args.workload}, {args.fmt}{tag.replace('_', ' ')}", "",
             "rocprofv3 derived counters per dispatch over one eager step, in percent of the",
             "kernel's active GPU cycles: MfmaUtil (matrix-unit busy cycles per SIMD), VALUBusy",
             "(vector-ALU instruction cycles per CU), LdsUtil (LDS busy), LDSBankConflict.", "",
             "```", "cd /tmp && export TMPDIR=/tmp",
             f"rocprofv3 --pmc {' '.join(UTIL_COUNTERS)} --output-format csv -d <out>/util -o util -- "
             f"python3 bench.py --workload {args.workload} --fmt {args.fmt}{flags} --pmc-step",
             f"python3 bench.py --workload {args.workload} --fmt {args.fmt}{flags} --summarize-util <util csv>",
             "```", "", f"Workload: {desc}.", "",
             "| M | K | N | kernel | " + " | ".join(UTIL_COUNTERS) + " |",
             "|---:|---:|---:|---|" + "---:|" * len(UTIL_COUNTERS)]
    for (m, k, n), d in zip(configs, disp):
        short = re.search(r"(k_[a-z_]+<[^>]*>)", d["name"])
        lines.append(f"| {m} | {k} | {n} | `{short.group(1) if short else d['name']}` | " +
                     " | ".join(f"{d.get(c, float('nan')):.1f}" for c in UTIL_COUNTERS) + " |")
    mean = {c: round(sum(d.get(c, 0.0) for d in disp) / len(disp), 2) for c in UTIL_COUNTERS}
    lines += ["", "Mean over the dispatches: " + ", ".join(f"{c} {v}" for c, v in mean.items()) + ".", "",
              "<!-- util-json: " + json.dumps({"workload": args.workload, "fmt": args.fmt, "variant": tag,
                                                "src_hash": kernel_source_hash(), "mean": mean}) + " -->"]
    out = util_path(args.workload, args.fmt, tag)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def util_path(workload, fmt, tag=""):
    return os.path.join(ROOT, "profiles", f"{workload}_{fmt}{tag}_utilization.md")


def stored_util(workload, fmt, tag=""):
    """Mean utilization counters of the dominant kernels from the committed
    summary, or None when there is none or the kernels changed since."""
    try:
        with open(util_path(workload, fmt, tag)) as fh:
            for line in fh:
                if line.startswith("<!-- util-json: "):
                    rec = json.loads(line[len("<!-- util-json: "):].rsplit(" -->", 1)[0])
                    if rec.get("src_hash") == kernel_source_hash():
                        return rec["mean"]
    except OSError:
        pass
    return None


def summarize_pmc(args):
    """Scale the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of one eager step by
    what the same counters read for the calibration copy (N MiB read, N MiB
    written) and write the summary the benchmark reads its traffic from."""
    import csv
    import re
    fetch_csv, write_csv = args.summarize_pmc

    def load(path, counter):
        rows = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return rows

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    calib_kib = args.copy_mib * 1024.0

    def scale(rows, what):
        cal = [v for (_, name, v) in rows if "neg" in name.lower()]
        if len(cal) != 1:
            raise SystemExit(f"expected one calibration copy in the {what} pass, found {len(cal)}")
        return calib_kib / cal[0], cal[0], [(name, v) for (_, name, v) in rows
                                             if any(d in name for d in DOMINANT)]

    f_fac, f_cal, f_dom = scale(fetch, "FETCH_SIZE")
    w_fac, w_cal, w_dom = scale(write, "WRITE_SIZE")
    configs, _ = workload_configs(args.workload)
    if len(f_dom) != len(configs) or len(w_dom) != len(configs):
        raise SystemExit(f"expected {len(configs)} dominant-kernel dispatches, found "
                         f"{len(f_dom)} / {len(w_dom)}")
    fmt = 0 if args.fmt == "nvfp4" else 1
    bs = 16 if fmt == 0 else 32
    per, tot_meas, tot_alg = [], 0.0, 0.0
    for (m, k, n), (fname, fv), (_, wv) in zip(configs, f_dom, w_dom):
        meas = (fv * f_fac + wv * w_fac) * 1024.0
        w_bytes = n * (k // 2 + k // bs)
        bf16_act = "linear" in fname or "w4a16" in fname   # the kernel reads bf16 activations
        alg = w_bytes + (2 * m * k if bf16_act else m * (k // 2 + k // bs)) + 2 * m * n
        short = re.search(r"(k_[a-z_]+<[^>]*>)", fname)
        per.append({"m": m, "k": k, "n": n, "kernel": short.group(1) if short else fname, "fetch_kib": round(fv, 1),
                    "write_kib": round(wv, 1), "hbm_bytes": round(meas), "algorithmic_bytes": alg,
                    "ratio": round(meas / alg, 3)})
        tot_meas += meas
        tot_alg += alg
    tag, flags = variant_tag(args), variant_flags(args)
    rec = {"workload": args.workload, "fmt": args.fmt, "variant": tag, "src_hash": kernel_source_hash(),
           "bytes_per_launch": round(tot_meas / len(configs)),
           "algorithmic_bytes_per_launch": round(tot_alg / len(configs)),
           "calibration": {"copy_mib": args.copy_mib, "fetch_kib": f_cal, "write_kib": w_cal,
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "per_config": per}
    out = traffic_path(args.workload, args.fmt, tag)
    lines = [f"# HBM traffic of the dominant kernels: {args.workload}, {args.fmt}{tag.replace('_', ' ')}", "",
             "Per-dispatch hardware counters from two rocprofv3 passes over one eager step,",
             "scaled by what the same counters read for a plain copy kernel of known size.", "",
             "```",
             "cd /tmp && export TMPDIR=/tmp",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o fetch -- python3 bench.py "
             f"--workload {args.workload} --fmt {args.fmt}{flags} --pmc-step --copy-mib {args.copy_mib}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o write -- python3 bench.py "
             f"--workload {args.workload} --fmt {args.fmt}{flags} --pmc-step --copy-mib {args.copy_mib}",
             f"python3 bench.py --workload {args.workload} --fmt {args.fmt}{flags} --copy-mib {args.copy_mib} "
             "--summarize-pmc <fetch csv> <write csv>",
             "```", "",
             f"Calibration: a {args.copy_mib} MiB float32 negate read {f_cal:.0f} KiB (FETCH_SIZE) and "
             f"wrote {w_cal:.0f} KiB (WRITE_SIZE) for {calib_kib:.0f} KiB each way: factors "
             f"{f_fac:.4f} and {w_fac:.4f}.", "",
             "| M | K | N | kernel | FETCH KiB | WRITE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
             "|---:|---:|---:|---|---:|---:|---:|---:|---:|"]
    for p in per:
        lines.append(f"| {p['m']} | {p['k']} | {p['n']} | `{p['kernel']}` | {p['fetch_kib']} | "
                     f"{p['write_kib']} | {p['hbm_bytes']} | {p['algorithmic_bytes']} | {p['ratio']} |")
    lines += ["", f"Average per launch: {rec['bytes_per_launch']} HBM bytes for "
              f"{rec['algorithmic_bytes_per_launch']} algorithmic bytes.", "",
              "<!-- traffic-json: " + json.dumps(rec) + " -->", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(out)


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_util:
        summarize_util(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_scaled_fp4_quantize_amd as fp4
    import synth

    if not os.path.exists(fp4.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.nv_tile:
        fp4.fp4_set_nvfp4_tile_mode(fp4.NV_TILE_LDS if args.nv_tile == "lds" else fp4.NV_TILE_REGISTERS)
    if args.fuse_large:
        fp4.fp4_set_large_linear_fusion(True)
    if args.fuse_decode:
        fp4.fp4_set_decode_linear_fusion(True)
    if args.no_mid:
        fp4.fp4_set_mid_gemm(False)
    fmt = fp4.FORMATS[args.fmt]
    # qfmt: the format value with the recipe flags, given to every library call
    qfmt = fp4._fmt(args.fmt + ("+" + args.recipe if args.recipe else ""))
    st_dev = (torch.tensor([args.static_scale], dtype=torch.float32, device=dev)
              if args.static_scale and fmt == 0 else None)
    if args.workload == "forward":
        bench_forward(args, fmt, qfmt)
        return
    configs, desc = workload_configs(args.workload)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs: weights quantized once (several copies), activations per config
    shapes = sorted({(k, n) for (_, k, n) in configs})
    bs = 16 if fmt == 0 else 32
    shape_bytes = {(k, n): n * (k // 2 + k // bs) for (k, n) in shapes}
    uses = {kn: sum(1 for (_, k, n) in configs if (k, n) == kn) for kn in shapes}
    # Decode: each shape's copies total >= ROTATE_BYTES and a step's calls of
    # one shape take consecutive copies, so a copy is reused only after all of
    # that shape's copies (>= 768 MB) have been read. Every shape cycles
    # through its copies in the same number of steps (`cycle`), so a graph of
    # `cycle` steps (or a multiple) leaves each copy's reuse distance intact
    # across replays.
    if args.workload in ("decode", "mid"):
        cycle = max(-(-ROTATE_BYTES // (shape_bytes[kn] * uses[kn])) for kn in shapes)
        copies = {kn: cycle * uses[kn] for kn in shapes}
    else:
        cycle, copies = 1, {kn: 1 for kn in shapes}
    weights, w_host, a_host = {}, {}, {}
    layer_of = {kn: name for name, kn in synth.PREFILL_LAYERS.items()}
    for (k, n) in shapes:
        if args.workload in ("decode", "mid"):
            w_bits = synth.decode_inputs(1, k, n, seed=0)[1]
        elif args.workload == "prefill":
            w_bits = synth.prefill_inputs(layer_of[(k, n)], seed=0, m=16)[1]
        elif args.workload.startswith("square"):
            w_bits = synth.square_inputs(k, seed=0)[1]
        else:
            w_bits = synth.single_gemm_inputs(0)[1]
        w_host[(k, n)] = w_bits
        w_dev = to_dev(w_bits)
        weights[(k, n)] = [fp4.fp4_quantize_weight(w_dev, qfmt) for _ in range(copies[(k, n)])]
        del w_dev
    xs, outs, wss = {}, {}, {}
    for (m, k, n) in configs:
        if args.workload in ("decode", "mid"):
            a_bits = synth.normal((m, k), 1.0, 0, 2 * k + 1)   # the activation decode_inputs draws
        elif args.workload == "prefill":
            a_bits = synth.prefill_inputs(layer_of[(k, n)], seed=0, m=m)[0]
        elif args.workload.startswith("square"):
            a_bits = synth.square_inputs(k, seed=0)[0]
        else:
            a_bits = synth.single_gemm_inputs(0)[0]
        a_host[(m, k, n)] = a_bits
        xs[(m, k, n)] = to_dev(a_bits)
        outs[(m, k, n)] = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        wss[(m, k, n)] = torch.zeros(max(1, fp4.fp4_linear_workspace_bytes(qfmt, m, n, k)),
                                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    if args.copy_mib:
        # one elementwise kernel that reads N MiB and writes N MiB (float32 negate)
        src = torch.ones((args.copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    qcanon, qws, gws = {}, {}, {}
    if args.api == "canonical":
        for cfg in configs:
            m, k, n = cfg
            qcanon[cfg] = fp4.Fp4Tensor(qfmt, fp4.CANONICAL, m, k, dev)
            qws[cfg] = torch.zeros(max(1, fp4.lib().fp4_quantize_workspace_bytes(qfmt, m, k)),
                                   dtype=torch.uint8, device=dev)
            gws[cfg] = torch.empty(max(16, fp4.lib().fp4_gemm_workspace_bytes(qfmt, m, n, k)),
                                   dtype=torch.uint8, device=dev)

    def linear(cfg, w):
        if args.w4a16:
            fp4.fp4_linear_w4a16(xs[cfg], w, out=outs[cfg])
        elif args.api == "canonical":
            fp4.fp4_quantize_act(xs[cfg], qfmt, workspace=qws[cfg], out=qcanon[cfg])
            fp4.fp4_gemm(qcanon[cfg], w, out=outs[cfg], workspace=gws[cfg])
        else:
            fp4.fp4_linear(xs[cfg], w, static_scale=st_dev, out=outs[cfg], workspace=wss[cfg])

    # the j-th call of a shape in step i takes copy (i * uses + j) mod copies
    slot = {}
    for cfg in configs:
        kn = cfg[1:]
        slot[cfg] = sum(1 for c in configs[:configs.index(cfg)] if c[1:] == kn)

    def step(i):
        for cfg in configs:
            kn = cfg[1:]
            linear(cfg, weights[kn][(i * uses[kn] + slot[cfg]) % copies[kn]])

    if args.pmc_step:
        step(0)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_step": desc, "configs": configs}), flush=True)
        return

    # ---- graphs: a long graph replays G consecutive steps, so a graph launch
    # is paid once per G steps, as in a serving loop that captures many layers
    # in one graph; one-step graphs run any remainder, so that exactly the
    # requested steps run (G is a multiple of the copy cycle).
    use_graph = not args.no_graph
    G = cycle * max(1, -(-16 // cycle))
    one, long_graph = [], None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(cycle):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(cycle):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            one.append(g)
        long_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(long_graph):
            for i in range(G):
                step(i)
        torch.cuda.synchronize()

    def run_steps(count):
        if not use_graph:
            for i in range(count):
                step(i)
            return
        q, r = divmod(count, G)
        for _ in range(q):
            long_graph.replay()
        for i in range(r):
            one[i % cycle].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    run_steps(args.steps)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    flops = sum(2.0 * m * n * k for (m, k, n) in configs)
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # ---- dominant kernel: the GEMM (fused with the activation quantization
    # when fp4_linear runs as one launch), timed alone: R back-to-back launches
    # captured in a graph, HIP events on the launch stream; the launches rotate
    # over the shape's weight copies as the steps do.
    def graph_time(fn, reps):
        fn(0)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for r in range(reps):
                    fn(r)
            g.replay()
            s.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    kern, per_cfg = {}, []
    for cfg in configs:
        m, k, n = cfg
        wl, nc = weights[(k, n)], copies[(k, n)]
        reps = max(nc, args.kernel_reps) if m * n * k < (1 << 36) else max(nc, 5)
        w_bytes = shape_bytes[(k, n)]
        lin_us = graph_time(lambda r: linear(cfg, wl[r % nc]), reps)
        if args.w4a16:
            name = ("k_w4a16_decode<%s,MG=%d>" % (args.fmt, 1 if m <= 16 else 2) if m <= 32
                    else "k_w4a16_tile<%s>" % args.fmt)
            us = lin_us
            nbytes = w_bytes + 2 * m * k + 2 * m * n          # W + bf16 A + bf16 C
        elif m <= 128 and fp4.fp4_linear_launches(qfmt, m, n, k, st_dev is not None) == 1:
            # one launch: quantization inside the skinny GEMM, by every
            # workgroup (k_linear_decode, small activations) or by producer
            # workgroups ahead of the GEMM workgroups
            prev = fp4.fp4_set_decode_linear_fusion(False)
            try:
                every_wg = fp4.fp4_linear_launches(qfmt, m, n, k, st_dev is not None) == 1
            finally:
                fp4.fp4_set_decode_linear_fusion(prev)
            if every_wg:
                name = "k_linear_decode<%s>" % args.fmt
            else:
                name = "%s<%s,MG=%d,producers>" % (
                    "k_gemm_decode_ring" if fmt == 0 else "k_gemm_decode", args.fmt,
                    1 if m <= 16 else 2)
            us = lin_us
            nbytes = w_bytes + 2 * m * k + 2 * m * n          # W + bf16 A + bf16 C
        else:
            # the activation layout fp4_linear uses internally (fragment-tiled)
            qa = fp4.fp4_quantize_act(xs[cfg], qfmt, layout=fp4.TILED)
            mg = 1 if m <= 16 else 2 if m <= 32 else 4 if m <= 64 else 8
            splits = fp4.fp4_linear_mid_splits(qfmt, m, n, k) if m <= 128 else 0
            if splits:   # the mid-size GEMM (and its slice-combining launch)
                name = "k_gemm_mid<%s,MG=%d>%s" % (args.fmt, mg, "+k_mid_sum" if splits > 1 else "")
            elif m <= 128:
                name = "%s<%s,MG=%d>" % ("k_gemm_decode_ring" if fmt == 0 else "k_gemm_decode",
                                         args.fmt, mg)
            elif "mbs" in args.recipe:   # macro-block scales: direct-load tiles
                name = "k_gemm_prefill<%s,MB>" % args.fmt
            else:   # LDS-staged tiles; 256 x 256 when that fills the 256 CUs
                big = -(-m // 256) * -(-n // 256) >= 256
                name = "k_gemm_tile<%s,%s>" % (args.fmt, "256x256" if big else "128x128")
            part_ws = torch.empty(max(16, fp4.lib().fp4_gemm_workspace_bytes(qfmt, m, n, k)),
                                  dtype=torch.uint8, device=dev)
            us = graph_time(lambda r: fp4.fp4_gemm(qa, wl[r % nc], out=outs[cfg], workspace=part_ws), reps)
            nbytes = w_bytes + m * (k // 2 + k // bs) + 2 * m * n  # W + FP4 A + bf16 C
            del qa, part_ws
        d = kern.setdefault(name, {"launches": 0, "us": 0.0, "bytes": 0.0, "flops": 0.0})
        d["launches"] += 1
        d["us"] += us
        d["bytes"] += nbytes
        d["flops"] += 2.0 * m * n * k
        per_cfg.append({"m": m, "k": k, "n": n, "kernel": name, "kernel_us": round(us, 3),
                        "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "TFLOPs": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1),
                        "linear_us": round(lin_us, 3), "weight_copies": nc})
    tot_us = sum(d["us"] for d in kern.values())
    tot_launch = sum(d["launches"] for d in kern.values())
    if args.workload in ("decode", "mid"):
        achieved = sum(d["bytes"] for d in kern.values()) / (tot_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = sum(d["flops"] for d in kern.values()) / (tot_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": None}
        if fmt == 0 and not args.w4a16:
            # exact NVFP4 products (q * s_b: up to 6 significant bits) run on the
            # f16 matrix instructions, whose dense peak bounds this kernel
            roof["f16_ceiling"] = {"peak": F16_PEAK_TFLOPS, "frac": round(achieved / F16_PEAK_TFLOPS, 4)}
    # the clocks the steps run at (a separate pass after every timing): the
    # matrix peaks are quoted at 2.4 GHz, and sustained matrix work runs lower
    def busy():
        run_steps(G if use_graph else 1)
        torch.cuda.synchronize()
    clocks = sample_clocks(busy)
    if clocks and roof["bound"] == "mfma":
        roof["frac_at_measured_sclk"] = round(
            roof["achieved"] / (roof["peak"] * clocks["sclk_median"] / SPEC_SCLK_MHZ), 4)
    # HBM bytes per launch from the committed counter summary of this variant
    roof["traffic"] = stored_traffic(args.workload, args.fmt, variant_tag(args))
    # rocprofv3 MfmaUtil / VALUBusy / LdsUtil (percent) of the same kernels
    roof["counters_pct"] = stored_util(args.workload, args.fmt, variant_tag(args))
    roof.update({"kernel": " + ".join(sorted(kern)), "avg_launch_us": round(tot_us / tot_launch, 3),
                 "launches_per_step": tot_launch,
                 "per_kernel": {nm: {"launches": d["launches"], "avg_us": round(d["us"] / d["launches"], 3),
                                     "GBps": round(d["bytes"] / (d["us"] * 1e-6) / 1e9, 1),
                                     "TFLOPs": round(d["flops"] / (d["us"] * 1e-6) / 1e12, 1)}
                                for nm, d in kern.items()},
                 "per_config": per_cfg})
    config = {"workload": desc + (" (weight-only: bf16 activations)" if args.w4a16 else "") +
              (f" (static activation scale {args.static_scale})" if st_dev is not None else "") +
              (" (fp4_quantize_act canonical + fp4_gemm)" if args.api == "canonical" else ""),
              "format": args.fmt, "recipe": args.recipe or "none",
              "launch": ("hip-graph replay, %d steps per graph" % G) if use_graph else "eager",
              "weight_copies": {f"{k}x{n}": copies[(k, n)] for (k, n) in shapes},
              "calls_per_step": len(configs),
              "fraction_of_fp4_peak": round(tflops / FP4_PEAK_TFLOPS, 6),
              "clocks_mhz": clocks}
    if args.workload.startswith("square") or args.workload == "prefill":
        # the sweep's two timings: GEMM alone on pre-quantized activations, and
        # quantization + GEMM (the value)
        gemm_us = sum(c["kernel_us"] for c in per_cfg)
        config["gemm_only"] = {"us_per_step": round(gemm_us, 3),
                               "TFLOPs": round(flops / (gemm_us * 1e-6) / 1e12, 1)}
        config["quant_plus_gemm"] = {"us_per_step": round(ms_per_step * 1e3, 3), "TFLOPs": round(tflops, 1)}

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.w4a16 else ("f16" if fmt == 0 else "fp4"),
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(configs, fmt, args, a_host, w_host)
    print(json.dumps(result), flush=True)


def bench_forward(args, fmt, qfmt):
    """Synthetic 24-layer forward: per layer Q, K, V, O and four (up, down)
    pairs, 288 W4A4 linear calls per forward, at M = 1, 8, 32 and 128. The
    weights (3.82 G values, ~N(0, 0.02)) are drawn on the GPU from a seeded
    generator and quantized once; every call gets its own pre-drawn
    activation ~N(0, 1) (calls are not chained). One step = one forward at each
    of the four M (HIP-graph replays); value = Σ 2·M·N·K / step time."""
    import numpy as np
    import torch

    import block_scaled_fp4_quantize_amd as fp4
    import synth
    dev = torch.device("cuda:0")
    layer, nl, ms = synth.FORWARD_LAYER, synth.FORWARD_LAYERS, synth.FORWARD_M
    def note(msg):
        print(f"[forward] {msg}", file=sys.stderr, flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    note("quantizing 288 weights")
    weights = []
    for _ in range(nl):
        for (_, k, n) in layer:
            w = (torch.randn(n, k, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            weights.append(fp4.fp4_quantize_weight(w, qfmt))
            del w
    calls = [(k, n) for _ in range(nl) for (_, k, n) in layer]
    note("drawing activations, capturing graphs")
    acts, outs, wss, graphs = {}, {}, {}, {}
    for m in ms:
        acts[m] = [torch.randn(m, k, generator=gen, device=dev).to(torch.bfloat16) for (k, n) in calls]
        outs[m] = {n: torch.empty(m, n, dtype=torch.bfloat16, device=dev) for (_, n) in calls}
        wsz = max(fp4.fp4_linear_workspace_bytes(qfmt, m, n, k) for (k, n) in calls)
        wss[m] = torch.zeros(max(1, wsz), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def forward(m):
        for i, (k, n) in enumerate(calls):
            fp4.fp4_linear(acts[m][i], weights[i], out=outs[m][n], workspace=wss[m])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for m in ms:
            forward(m)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for m in ms:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            forward(m)
        graphs[m] = g
    torch.cuda.synchronize()
    note("timing")
    for _ in range(args.warmup):
        for m in ms:
            graphs[m].replay()
    torch.cuda.synchronize()
    steps = max(1, args.steps // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        for m in ms:
            graphs[m].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / steps
    per_m = {}
    for m in ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            graphs[m].replay()
        b.record()
        torch.cuda.synchronize()
        per_m[m] = a.elapsed_time(b) / steps
    sum_nk = sum(n * k for (k, n) in calls)
    flops = sum(2.0 * m * sum_nk for m in ms)
    bs = 16 if fmt == 0 else 32
    w_bytes = sum(n * (k // 2 + k // bs) for (k, n) in calls)
    def call_bytes(m):   # weights + bf16 activations + bf16 outputs of one forward
        return w_bytes + sum(2 * m * k + 2 * m * n for (k, n) in calls)
    achieved = sum(call_bytes(m) for m in ms) / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if fmt == 0 else "fp4",
        "data": "synthetic",
        "config": {"workload": "synthetic 24-layer forward, 288 W4A4 linear calls per forward "
                               "(Q 2880->4096, K/V 2880->512, O 4096->2880, 4 x (up 2880->5760, "
                               "down 5760->2880)), one forward at each M in {1,8,32,128}",
                   "format": args.fmt, "recipe": args.recipe or "none",
                   "launch": "hip-graph replay (one graph per M)",
                   "weight_bytes": w_bytes,
                   "per_forward_ms": {str(m): round(per_m[m], 4) for m in ms},
                   "per_forward_tflops": {str(m): round(2.0 * m * sum_nk / (per_m[m] * 1e-3) / 1e12, 2)
                                          for m in ms}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole fp4_linear calls (activation quantization included)",
                     "note": "algorithmic bytes of all calls of the step over the step time"},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        note("cpu baseline")
        cfgs = [(8, k, n) for (_, k, n) in layer]
        a_host = {(8, k, n): synth.forward_act(0, j, 8) for j, (_, k, n) in enumerate(layer)}
        w_host = {(k, n): synth.forward_weight(0, j) for j, (_, k, n) in enumerate(layer)}
        result["cpu_baseline"] = cpu_baseline(cfgs, fmt, args, a_host, w_host)
    print(json.dumps(result), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(configs, fmt, args, a_host, w_host):
    """The CPU oracle (plain C, binary64) on the same linear calls, on every
    host core this process may use (threads over row or column slices; the
    oracle's C calls release the interpreter lock). Per call: the activation
    quantization of the whole tensor (NVFP4 dynamic: the tensor's maximum, then
    row slices quantized with that scale, which the pins show equals the
    one-piece dynamic quantization), then the k-ordered binary64 GEMM on a
    sample: every output when it fits the time budget, else the first R <= 64
    activation rows (M > 128) or the first output columns (M <= 128), with the
    full call's time extrapolated linearly from the sample. Weights are
    quantized beforehand, untimed, as on the GPU. Reported in the metric's
    unit: the calls' flops over their (extrapolated) oracle time."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
    rk = {"rotate": "rotate" in args.recipe, "oas": "oas" in args.recipe, "mbs": "mbs" in args.recipe}
    pool = cf.ThreadPoolExecutor(max_workers=threads)

    def chunks(n, parts):
        step = -(-n // parts)
        return [(i, min(n, i + step)) for i in range(0, n, step)]

    def quantize_par(bits):
        """The oracle's quantization of a whole tensor, split over row slices."""
        if fmt == oracle.NVFP4 and not rk["rotate"]:
            st = float(oracle.tensor_scale(bits))
            parts = list(pool.map(lambda rr: oracle.quantize(fmt, bits[rr[0]:rr[1]], mode=oracle.STATIC,
                                                             static_scale=st),
                                  chunks(bits.shape[0], threads)))
            return oracle.Quantized(fmt, np.concatenate([q.codes for q in parts]),
                                    np.concatenate([q.scales for q in parts]), st, bits.shape[1])
        if fmt == oracle.NVFP4:   # rotated dynamic: the maximum is over the rotated tensor
            rot = np.concatenate(list(pool.map(lambda rr: oracle.hadamard(bits[rr[0]:rr[1]], 16),
                                               chunks(bits.shape[0], threads))))
            st = float(oracle.tensor_scale(rot))
            parts = list(pool.map(lambda rr: oracle.quantize(fmt, rot[rr[0]:rr[1]], mode=oracle.STATIC,
                                                             static_scale=st),
                                  chunks(bits.shape[0], threads)))
            return oracle.Quantized(fmt, np.concatenate([q.codes for q in parts]),
                                    np.concatenate([q.scales for q in parts]), st, bits.shape[1])
        parts = list(pool.map(lambda rr: oracle.quantize(fmt, bits[rr[0]:rr[1]], **rk),
                              chunks(bits.shape[0], threads)))
        return oracle.Quantized(fmt, np.concatenate([q.codes for q in parts]),
                                np.concatenate([q.scales for q in parts]), 1.0, bits.shape[1],
                                np.concatenate([q.macro for q in parts]) if rk["mbs"] else None)

    def gemm_par(qa, qw):
        """k-ordered binary64 GEMM, the weight's rows (output columns) split over threads."""
        def run(cc):
            sub = qw.row_slice(cc[0], cc[1])
            if args.w4a16:
                return oracle.gemm_w4a16(qa, sub)
            return oracle.gemm_loop(qa, sub)
        list(pool.map(run, chunks(qw.rows, threads)))

    def w_rows(q, r0, r1):
        return q.row_slice(r0, r1)

    budget = args.cpu_seconds / len(configs)
    tot_flops, tot_s, parts, wq_cache = 0.0, 0.0, [], {}
    for (m, k, n) in configs:
        a_bits, w_bits = a_host[(m, k, n)], w_host[(k, n)]
        if (k, n) not in wq_cache:
            wq_cache[(k, n)] = quantize_par(w_bits)
        qw = wq_cache[(k, n)]
        t = time.perf_counter()
        qa = a_bits if args.w4a16 else quantize_par(a_bits)

        def a_rows(r0, r1):
            return a_bits[r0:r1] if args.w4a16 else w_rows(qa, r0, r1)
        t_q = time.perf_counter() - t

        def timed(a_part, w_part):
            t0 = time.perf_counter()
            gemm_par(a_part, w_part)
            return time.perf_counter() - t0
        # The sample grows until it fills the budget: large M takes whole
        # activation rows (every output column; at most 64 rows), small M takes
        # every row and the first output columns.
        if m > 128:
            t_g = timed(a_rows(0, 1), qw)
            rows, cols = min(m, 64, max(1, int(budget / max(t_g, 1e-6)))), n
            if rows > 1:
                t_g += timed(a_rows(1, rows), qw)
        else:
            c1 = min(n, 16 * threads)
            t_g = timed(a_rows(0, m), w_rows(qw, 0, c1))
            rows, cols = m, min(n, max(c1, int(c1 * budget / max(t_g, 1e-6))))
            if cols > c1:
                t_g += timed(a_rows(0, m), w_rows(qw, c1, cols))
        est = t_q + t_g * (m / rows) * (n / cols)
        tot_flops += 2.0 * m * n * k
        tot_s += est
        what = "all outputs" if (rows, cols) == (m, n) else \
            (f"{rows}/{m} rows" if rows < m else f"{cols}/{n} columns")
        parts.append(f"{m}x{k}x{n}: quantize {t_q:.2f} s, GEMM on {what} {t_g:.2f} s")
    pool.shutdown()
    return {"value": tot_flops / tot_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": ("per call: " + ("" if args.w4a16 else "activation quantization of the whole tensor + ")
                       + "k-ordered binary64 GEMM on a sample, the call's time extrapolated from it ("
                       + "; ".join(parts) + f"); total {tot_s:.1f} s estimated for the full calls")}


if __name__ == "__main__":
    main()
