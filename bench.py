"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the layer's training pass over one batch of synthetic input: for
the default workload (one LLaMA-65B-shaped decoder layer: q, k, v, o, gate, up,
down; 4096 tokens; LoRA r = 64, alpha = 16 on every projection) the seven
forwards in layer order, then the seven backwards in reverse order.  The
frozen weights are quantized once beforehand (as in training); that codec
path, and the few-token dequant-GEMV, are measured in the same run and
reported under "paths", with the adapter optimizer step (AdamW, device-resident
and paged) and the page's codebook comparison (NF4, integer grids, Lloyd).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `roofline` covers the dominant kernel (the fused
dequant GEMM of the forward), timed with HIP events that the library records
around each fused product on the launch stream (the kernel, plus the small
kernel that sums the contraction pieces of split tail tiles where a launch
has them); `cpu_baseline` times the CPU oracle on a bounded sample of the
same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QLoRA NF4 linear fwd+bwd TFLOP/s (% MFMA peak); NF4 dequant/quant GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
NF4_BYTES_PER_PARAM = 0.5 + 1.0 / 64 + 4.0 / (64 * 256)


def rocminfo_peaks():
    """The GPU agent's compute-unit count and maximum engine clock as rocminfo reports them,
    and the dense bf16 MFMA peak they give (4096 flops per clock per CU: four matrix cores
    of 1024); None where rocminfo is missing or reports no GPU agent."""
    import re
    import subprocess

    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in out.split("*******")[1:]:
        kind = re.search(r"Device Type:\s+(\w+)", agent)
        if not kind or kind.group(1) != "GPU":
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        name = re.search(r"Name:\s+(gfx\w+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"agent": name.group(1) if name else None, "cus": cus, "max_sclk_mhz": clk,
                    "bf16_tflops_at_max_sclk": round(cus * clk * 1e6 * 4096 / 1e12, 1)}
    return None


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama65b_layer",
                   choices=["llama65b_layer", "llama7b_layer", "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-paths", action="store_true", help="skip the codec and GEMV path figures")
    p.add_argument("--cpu-tokens", type=int, default=256, help="tokens in the CPU-oracle sample")
    p.add_argument("--pmc-workload", action="store_true",
                   help="one step of the workload, then a plain 512 MiB device copy (for counter runs)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) into the traffic summary")
    p.add_argument("--summarize-mfma", nargs=3, metavar=("COUNTER_CSV", "TRACE_CSV", "COMMAND"),
                   help="matrix-core utilisation and clock of the fused products from a GRBM_COUNT / "
                        "SQ_VALU_MFMA_BUSY_CYCLES counter pass with its kernel trace")
    p.add_argument("--pmc-codec-workload", action="store_true",
                   help="one pass of each codec and few-token kernel over the 65B layer, then a plain "
                        "512 MiB device copy (for counter runs)")
    p.add_argument("--summarize-pmc-codec", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="per-kernel traffic table of two counter runs over --pmc-codec-workload")
    p.add_argument("--hbm-ceiling", action="store_true",
                   help="read / write / copy streaming probes over 4 GiB, as a markdown table")
    p.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "COMMAND"),
                   help="turn a rocprofv3 kernel-stats CSV into a short summary naming its command")
    p.add_argument("--gemv-sweep", action="store_true",
                   help="few-token forward only: 10 queued calls for each LLaMA-65B shape and M in "
                        "{1, 4, 16} (for a kernel trace; see --summarize-gemv-trace)")
    p.add_argument("--summarize-gemv-pmc", nargs=2, metavar=("COUNTER_CSV", "COMMAND"),
                   help="per-shape counters of k_gemv_part from a --gemv-sweep counter run, as a markdown table")
    p.add_argument("--summarize-gemv-trace", metavar="KERNEL_TRACE_CSV",
                   help="per-shape kernel durations of a --gemv-sweep kernel trace, as a markdown table")
    p.add_argument("--codebooks-only", action="store_true",
                   help="the codebook comparison only (the 'codebooks' path figures), as a JSON line")
    p.add_argument("--gemv-only", action="store_true",
                   help="the few-token forward only (the 'gemv' path figures over the 65B layer), as a JSON line")
    p.add_argument("--loftq-only", action="store_true",
                   help="the LoftQ initialisation only (the 'loftq' path figures), as a JSON line")
    p.add_argument("--bulk-codec-only", action="store_true",
                   help="the bulk codec round trip over 32 LLaMA-7B-shaped layers only, as a JSON line")
    p.add_argument("--adamw-only", action="store_true",
                   help="the adapter optimizer step only (the 'adamw' path figures), as a JSON line "
                        "(for kernel traces and counter runs)")
    p.add_argument("--plain-gemm", action="store_true",
                   help="time the vendor library's plain bf16 GEMM (torch.matmul) at the layer shapes, "
                        "for context, and print a markdown table")
    return p.parse_args()


GEMV_SWEEP_SHAPES = ((8192, 8192), (22016, 8192), (8192, 22016))
GEMV_SWEEP_M = (1, 4, 16)
GEMV_SWEEP_CALLS = 10


def gemv_sweep():
    """The few-token forward alone: for each shape and token count, GEMV_SWEEP_CALLS calls
    queued behind a sleeping kernel, so that they run back to back.  The calls rotate
    through copies of the packed weight at different addresses, together more than twice
    the 256 MB Infinity Cache, so that every call streams its weight from HBM."""
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import linear_inputs, seed_of

    for (N, K) in GEMV_SWEEP_SHAPES:
        W, X, A, B, _ = linear_inputs(N, K, 16, 64, seed=seed_of(3, N, K), device="cuda", with_dy=False)
        copies = []
        while sum(c.nbytes() for c in copies) < (512 << 20):
            copies.append(nf4.quantize_weight(W))
        del W
        for M in GEMV_SWEEP_M:
            x = X[:M].contiguous()
            torch.cuda.synchronize()
            torch.cuda._sleep(int(2e7))
            for i in range(GEMV_SWEEP_CALLS):
                nf4.qlora_linear_fwd(copies[i % len(copies)], x, A, B, 16.0)
            torch.cuda.synchronize()
            print("gemv sweep N=%d K=%d M=%d done (%d weight copies)" % (N, K, M, len(copies)),
                  file=sys.stderr, flush=True)
        del copies
        torch.cuda.empty_cache()


def summarize_gemv_pmc(counter_csv, command):
    """Per-dispatch counters of k_gemv_part in a --gemv-sweep counter run, medians per
    (shape, tokens), as a markdown table."""
    import csv

    per = {}
    for row in csv.DictReader(open(counter_csv)):
        k = row.get("Kernel_Name") or ""
        if "k_gemv_part" not in k:
            continue
        d = int(row["Dispatch_Id"])
        per.setdefault(d, {})
        per[d][row["Counter_Name"]] = per[d].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    disp = [per[d] for d in sorted(per)]
    names = sorted({c for v in disp for c in v})
    out = ["# k_gemv_part counters per launch, LLaMA-65B shapes", "", "Command (GPU, repository root):", "",
           "    " + command, "",
           "Medians over the %d calls of each (shape, tokens) row of `bench.py --gemv-sweep` (each call "
           "streams its weight from HBM: the calls rotate through copies of it)." % GEMV_SWEEP_CALLS, "",
           "| N x K | M | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    i = 0
    for (N, K) in GEMV_SWEEP_SHAPES:
        for M in GEMV_SWEEP_M:
            grp = disp[i:i + GEMV_SWEEP_CALLS]
            i += GEMV_SWEEP_CALLS
            med = lambda c: sorted(v.get(c, 0.0) for v in grp)[len(grp) // 2] if grp else float("nan")
            out.append("| %d x %d | %d | " % (N, K, M) + " | ".join("%.4g" % med(c) for c in names) + " |")
    print("\n".join(out))


def summarize_gemv_trace(trace_csv):
    import csv

    rows = [r for r in csv.DictReader(open(trace_csv)) if "k_gemv_" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = ["| N x K | M | k_gemv_part us | k_gemv_reduce us | call us | codes+constants GB/s (part) | "
           "algorithmic GB/s (call) |", "|---|---|---|---|---|---|---|"]
    i = 0
    for (N, K) in GEMV_SWEEP_SHAPES:
        for M in GEMV_SWEEP_M:
            grp = rows[i:i + 2 * GEMV_SWEEP_CALLS]
            i += 2 * GEMV_SWEEP_CALLS
            dur = lambda key: sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                                     for r in grp if key in r["Kernel_Name"])
            part, red = dur("k_gemv_part"), dur("k_gemv_reduce")
            pm, rm = part[len(part) // 2], red[len(red) // 2]
            wbytes = NF4_BYTES_PER_PARAM * N * K
            cbytes = wbytes + 2 * 64 * (N + K) + 2 * M * K + 2 * M * N + 2 * M * 64
            out.append("| %d x %d | %d | %.2f | %.2f | %.2f | %.0f | %.0f |" % (
                N, K, M, pm, rm, pm + rm, wbytes / pm / 1e3, cbytes / (pm + rm) / 1e3))
    print("\n".join(out))


def plain_gemm_table():
    """torch.matmul (hipBLASLt) bf16 products of the forward's (NT) and the dX product's (NN)
    layouts at the LLaMA shapes: a library GEMM with no dequantization, for context."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(0)
    rows = ["| M x N x K | NT (Y = X W^T, the forward's layout) | NN (the dX product's layout) |",
            "|---|---|---|"]
    for (M, N, K) in ((4096, 8192, 8192), (4096, 22016, 8192), (4096, 8192, 22016), (2048, 4096, 4096),
                      (2048, 11008, 4096), (2048, 4096, 11008)):
        X = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=gen)
        W = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=gen) * 0.02
        cells = []
        for op in (W.t(), W.t().contiguous()):
            for _ in range(3):
                X @ op
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                X @ op
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 20 * 1e3
            cells.append("%.1f us, %.0f TFLOP/s" % (us, 2.0 * M * N * K / us / 1e6))
        rows.append("| %d x %d x %d | %s | %s |" % (M, N, K, cells[0], cells[1]))
        print(rows[-1], file=sys.stderr, flush=True)
        del X, W
    print("\n".join(rows))


# ---- HBM traffic of the dominant kernel, from hardware counters -------------------
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are read in two rocprofv3 --pmc runs
# of `bench.py --pmc-workload`; each counter is scaled by the factor that makes it
# match the known bytes of a plain device copy measured in the same run.  The
# summary records the hash of the kernel sources it was measured on; the traffic is
# reported only while the sources still hash to that value.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_fused_fwd_llama65b_layer_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_nf4_quantized_09_amd", "csrc", f)
                  for f in ("fused.hip", "nf4_common.h", "tile_map.h", "bufio.h")]
COPY_BYTES = 512 << 20


def kernel_source_hash(names=None):
    import hashlib
    h = hashlib.sha256()
    files = KERNEL_SOURCES if names is None else [os.path.join(ROOT, "bit_nf4_quantized_09_amd", "csrc", f)
                                                  for f in names]
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _read_counters(path, counter):
    import csv
    per = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            key = (row.get("Dispatch_Id"), row.get("Kernel_Name"))
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    return per


def summarize_pmc(fetch_csv, write_csv):
    fetch = _read_counters(fetch_csv, "FETCH_SIZE")
    write = _read_counters(write_csv, "WRITE_SIZE")

    def pick(table, pred):
        return [v for (d, k), v in sorted(table.items()) if pred(k or "")]

    is_fused = lambda k: "k_fused<false" in k or "k_fusedILb0E" in k
    is_copy = lambda k: "copy" in k.lower()
    fc, wc = pick(fetch, is_copy), pick(write, is_copy)
    ff, wf = pick(fetch, is_fused), pick(write, is_fused)
    if not (fc and wc and ff and wf):
        raise SystemExit("counter files lack the copy or the fused kernel")
    # the copy of COPY_BYTES: largest dispatch of each kind; the pure read and pure write
    # of the same size, where the run has them, calibrate each counter on its own
    kf_copy = (COPY_BYTES / 1024.0) / max(fc)
    kw_copy = (COPY_BYTES / 1024.0) / max(wc)
    pr = [v for (d, k), v in fetch.items() if "k_probe_read" in (k or "")]
    pw = [v for (d, k), v in write.items() if "k_probe_write" in (k or "")]
    kf = (COPY_BYTES / 1024.0) / pr[0] if pr else kf_copy
    kw = (COPY_BYTES / 1024.0) / pw[0] if pw else kw_copy
    fetch_b = sum(ff) / len(ff) * 1024.0 * kf
    write_b = sum(wf) / len(wf) * 1024.0 * kw
    lines = [
        "# k_fused<false> (forward fused dequant GEMM): HBM traffic per launch, LLaMA-65B layer",
        "",
        "Commands (GPU, from the repository root; one counter per run):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE -d pmc_fetch -o run --output-format csv -- python bench.py --pmc-workload",
        "    rocprofv3 --pmc WRITE_SIZE -d pmc_write -o run --output-format csv -- python bench.py --pmc-workload",
        "    python bench.py --summarize-pmc <pmc_fetch>/run_counter_collection.csv <pmc_write>/run_counter_collection.csv",
        "",
        "Calibration: a plain device copy of %d MiB in the same run reads %.1f KiB by FETCH_SIZE and writes "
        "%.1f KiB by WRITE_SIZE (factors %.4f and %.4f to %d KiB); a pure read of the same size fetches %s KiB "
        "and a pure write writes %s KiB. The table uses %.4f (fetch) and %.4f (write)%s."
        % (COPY_BYTES >> 20, max(fc), max(wc), kf_copy, kw_copy, COPY_BYTES >> 10,
           "%.1f" % pr[0] if pr else "-", "%.1f" % pw[0] if pw else "-", kf, kw,
           ", from the pure read and write" if pr and pw else ", from the copy"),
        "",
        "| launches | FETCH_SIZE KiB (avg) | WRITE_SIZE KiB (avg) | fetch bytes | write bytes |",
        "|---|---|---|---|---|",
        "| %d | %.1f | %.1f | %.4g | %.4g |" % (len(ff), sum(ff) / len(ff), sum(wf) / len(wf), fetch_b, write_b),
        "",
        "traffic_bytes_per_launch = %.6g" % (fetch_b + write_b),
        "kernel_source_sha256 = %s" % kernel_source_hash(),
    ]
    print("\n".join(lines))


def summarize_trace(stats_csv, command):
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = ["# Kernel trace: rocprofv3 --kernel-trace --stats", "", "Command (GPU, repository root):", "",
           "    " + command, "",
           "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            100.0 * float(r["TotalDurationNs"]) / total))
    print("\n".join(out))


def summarize_mfma(counter_csv, trace_csv, command):
    """Clock and matrix-core utilisation of the fused products from one counter pass
    (GRBM_COUNT, SQ_VALU_MFMA_BUSY_CYCLES, summed over the 8 XCDs) with a kernel trace of the
    same run (durations): clock = (GRBM_COUNT / 8) / duration; MFMA work = algorithmic flops /
    1024 SIMD-cycles (a v_mfma_f32_32x32x16_bf16, 32768 flops, occupies a SIMD's matrix core
    for 32 cycles); utilisation = MFMA work / (1024 SIMDs x cycles of the launch).  The shape
    of each launch is read back from the workload's launch order (7 forwards q..down, then 7
    backwards down..q)."""
    import csv
    from workloads import LLAMA65B, layer_projections

    dur = {}
    for r in csv.DictReader(open(trace_csv)):
        if "k_fused" in r["Kernel_Name"]:
            dur[r["Dispatch_Id"]] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    cnt = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Dispatch_Id"] in dur:
            cnt.setdefault(r["Dispatch_Id"], {}).setdefault(r["Counter_Name"], 0.0)
            cnt[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    projs = layer_projections(LLAMA65B["d"], LLAMA65B["ffn"])
    M, rr = 4096, 64
    order = [("forward", N, K) for _, N, K in projs] + [("dX", N, K) for _, N, K in reversed(projs)]
    ids = sorted(dur, key=int)
    out = ["# MFMA utilisation and clock of the fused products (LLaMA-65B layer, 4096 tokens)", "",
           "Command (GPU, repository root; one counter pass with the kernel trace for the durations):", "",
           "    " + command, "",
           "    python bench.py --summarize-mfma <dir>/run_counter_collection.csv <dir>/run_kernel_trace.csv '<command>'", "",
           "`--pmc-workload` runs one step of the layer (7 forwards, then 7 backwards) and a plain copy.",
           "Counter values are summed over the 8 XCDs; per launch: clock = (`GRBM_COUNT` / 8) / duration;",
           "MFMA work = algorithmic flops / 1024 SIMD-cycles; `SQ_VALU_MFMA_BUSY_CYCLES` / MFMA work",
           "checks that the kernel issues exactly the algorithmic MFMA work; utilisation = MFMA work /",
           "(1024 SIMDs x clock cycles of the launch).", "",
           "| product | N x K | duration | clock | MFMA busy / work | MFMA utilisation at that clock | TFLOP/s |",
           "|---|---|---|---|---|---|---|"]
    for i, d in enumerate(ids[:len(order)]):
        kind, N, K = order[i]
        name, t = dur[d]
        c = cnt.get(d, {})
        flops = 2 * M * N * K + (2 * M * N * rr if kind == "forward" else 2 * M * K * rr)
        work = flops / 1024.0
        clock = c.get("GRBM_COUNT", 0.0) / 8.0 / t
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = work / (1024.0 * clock * t) if clock > 0 else 0.0
        out.append("| %s | %d x %d | %.1f us | %.2f GHz | %.3f | %.3f | %.0f |" % (
            kind, N, K, t * 1e6, clock / 1e9, busy / work if work else 0.0, util, flops / t / 1e12))
    print("\n".join(out))


def traffic_per_launch(workload):
    """HBM bytes per fused forward launch from the committed counter summary, or None
    when there is none, it covers another workload, or the kernel sources changed
    since it was measured."""
    if workload != "llama65b_layer":
        return None
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = dict(l.split(" = ", 1) for l in text.splitlines() if " = " in l and not l.startswith(" "))
    if vals.get("kernel_source_sha256", "").strip() != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def layer_flops(M, projs, r):
    """Algorithmic flops of one fwd+bwd pass (no dW; T saved from the forward)."""
    fwd = bwd = 0
    for _, N, K in projs:
        fwd += 2 * M * N * K + 2 * M * K * r + 2 * M * r * N
        bwd += 2 * M * N * K + 2 * M * N * r + 2 * M * r * K + 2 * r * M * K + 2 * N * M * r
    return fwd, bwd


def build_layer(workload, dev):
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import (LLAMA7B, LLAMA65B, Draw, layer_projections, linear_inputs, seed_of)

    if workload == "tiny":
        projs = [("w", 256, 256)]
        M, r, alpha = 16, 8, 16.0
    elif workload == "llama7b_layer":
        projs = layer_projections(LLAMA7B["d"], LLAMA7B["ffn"])
        M, r, alpha = 2048, 64, 16.0
    else:
        projs = layer_projections(LLAMA65B["d"], LLAMA65B["ffn"])
        M, r, alpha = 4096, 64, 16.0
    layer = []
    for i, (name, N, K) in enumerate(projs):
        W, X, A, B, dY = linear_inputs(N, K, M, r, seed=seed_of(5, i, N, K), device=dev)
        Wq = nf4.quantize_weight(W)
        layer.append(dict(name=name, N=N, K=K, W=W, Wq=Wq, X=X, A=A, B=B, dY=dY))
    torch.cuda.synchronize()
    return layer, projs, M, r, alpha


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    releases at device scope instead of system scope, so it does not write the L2 back
    to memory between the kernels it brackets (after a kernel that leaves megabytes of
    output in L2, that write-back idles the GPU for microseconds).  Same record /
    elapsed_time interface as torch.cuda.Event, and `cuda_event` is the raw hipEvent_t;
    recorded on torch's current stream."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7")     # the runtime torch has loaded
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
        self.cuda_event = h.value

    def record(self):
        import torch
        rc = self.hip().hipEventRecord(self.cuda_event, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.cuda_event:
            self._hip.hipEventDestroy(self.cuda_event)


def event_pool(n):
    """n pairs of timing-only events (TimingEvent), each recorded once here, outside
    any timed region."""
    import torch

    pool = [(TimingEvent(), TimingEvent()) for _ in range(n)]
    for a, b in pool:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return iter(pool)


def run_step(layer, alpha, events=None, pool=None, weight="Wq", recompute=False):
    """The layer's seven forwards, then its seven backwards.  `weight` picks the weight
    tuple (double-quantized "Wq", or "Wq_plain" with the constants kept as fp32);
    recompute=True keeps nothing of the forward but its output and recomputes T = X A^T
    in the backward (gradient checkpointing of the adapter activations)."""
    import bit_nf4_quantized_09_amd as nf4

    saved = []
    for p in layer:
        if events is not None:
            ev = next(pool)
            events["fwd"].append((ev, p))
            nf4.nf4_profile_next_fused(*ev)
        Y, T = nf4.qlora_linear_fwd(p[weight], p["X"], p["A"], p["B"], alpha, save_t=not recompute)
        saved.append((Y, T))
    grads = []
    for p, (Y, T) in zip(reversed(layer), reversed(saved)):
        if events is not None:
            ev = next(pool)
            events["bwd"].append((ev, p))
            nf4.nf4_profile_next_fused(*ev)
        grads.append(nf4.qlora_linear_bwd(p[weight], p["X"], p["dY"], p["A"], p["B"], alpha, T=T))
    return saved, grads


def variant_paths(layer, alpha, flops, steps=5):
    """The step with double quantization off (plain fp32 constants, "Double
    quantization") and with T recomputed in the backward (gradient checkpointing of the
    adapter activations): TFLOP/s over `steps` timed steps each, and the weight storage
    of the layer with and without double quantization."""
    import torch
    import bit_nf4_quantized_09_amd as nf4

    for p in layer:
        p["Wq_plain"] = nf4.quantize_weight(p["W"], double_quant=False)
    torch.cuda.synchronize()
    out = {}
    for name, kw in (("dq_off", dict(weight="Wq_plain")), ("recompute_t", dict(recompute=True))):
        run_step(layer, alpha, **kw)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step(layer, alpha, **kw)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        out[name] = dict(tflops=flops / dt / 1e12, ms_per_step=dt * 1e3)
    n = sum(p["N"] * p["K"] for p in layer)
    dq = sum(p["Wq"].nbytes() for p in layer)
    plain = sum(p["Wq_plain"].nbytes() for p in layer)
    out["weight_bits_per_param"] = dict(dq_on=8 * dq / n, dq_off=8 * plain / n)
    for p in layer:
        del p["Wq_plain"]
    return out


def kernel_roofline(events, M, r, kind):
    """Average duration of the fused kernel launches and its achieved TFLOP/s."""
    tot_ms = 0.0
    tot_flops = 0
    for (start, stop), p in events[kind]:
        tot_ms += start.elapsed_time(stop)
        N, K = p["N"], p["K"]
        tot_flops += 2 * M * N * K + (2 * M * N * r if kind == "fwd" else 2 * M * K * r)
    n = len(events[kind])
    avg_ms = tot_ms / n
    achieved = tot_flops / (tot_ms / 1e3) / 1e12
    return dict(kernel="k_fused_fwd" if kind == "fwd" else "k_fused_bwd_dx", launches=n,
                avg_us=avg_ms * 1e3, flops_per_launch=tot_flops / n, achieved=achieved)


def codec_paths(layer, dev, reps=3):
    """GB/s of quantize, double-quantize and dequantize over the layer's fp32 weights."""
    import torch
    import bit_nf4_quantized_09_amd as nf4

    n_total = sum(p["N"] * p["K"] for p in layer)
    res = {}
    for _ in range(1):   # warm-up pass
        for p in layer:
            c, a = nf4.nf4_quantize(p["W"])
            nf4.nf4_double_quantize(a)
    torch.cuda.synchronize()

    def timed(fn):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / 1e3 / reps

    absmax = {}

    def quant():
        for p in layer:
            absmax[p["name"]] = nf4.nf4_quantize(p["W"])[1]

    tq = timed(quant)
    bq = n_total * (4 + 0.5 + 4 / 64)
    res["quantize_fp32"] = dict(GBps=bq / tq / 1e9, ms=tq * 1e3, bytes=bq)

    def dq():
        for p in layer:
            nf4.nf4_double_quantize(absmax[p["name"]])

    tdq = timed(dq)
    bdq = n_total * (4 / 64 + 1 / 64 + 4 / (64 * 256))
    res["double_quantize"] = dict(GBps=bdq / tdq / 1e9, ms=tdq * 1e3, bytes=bdq)

    # the layer's seven constant vectors in one batched call (two launches), as a layer
    # is quantized: the per-tensor figure above is bound by the host's seven calls
    def dq_batch():
        nf4.nf4_double_quantize_batch([absmax[p["name"]] for p in layer])

    dq_batch()
    tdqb = timed(dq_batch)
    res["double_quantize_layer_batched"] = dict(GBps=bdq / tdqb / 1e9, ms=tdqb * 1e3, bytes=bdq)

    def deq():
        for p in layer:
            nf4.nf4_dequantize(p["Wq"], torch.float32)

    tdeq = timed(deq)
    bdeq = n_total * (NF4_BYTES_PER_PARAM + 4)
    res["dequantize_fp32"] = dict(GBps=bdeq / tdeq / 1e9, ms=tdeq * 1e3, bytes=bdeq)
    for v in res.values():
        v["frac_hbm"] = v["GBps"] / PEAK_HBM_GBS
    res["params"] = n_total
    return res


def bulk_codec_paths(dev):
    """The bulk round trip over every weight of 32 LLaMA-7B-shaped decoder layers
    (6,476,005,376 values, N(0, 0.02) with 1% of the entries scaled by 10), in fp32
    and in bf16: NF4 quantize of every tensor, double quantization of every absmax
    vector (batched: two launches per 32 tensors), then dequantize back to the input's
    dtype.  Inputs, codes and outputs stay
    resident (6.5e9 values at fresh addresses, far beyond the Infinity Cache).  One
    untimed pass first fills the allocator's cache, so that the timed pass allocates
    nothing; the timed pass is queued behind a sleeping kernel and timed with events
    between its phases, so the figures are GPU time (host_bound says whether the host
    still had calls to submit when the sleep ended)."""
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import LLAMA7B, Draw, layer_projections, seed_of

    projs = layer_projections(LLAMA7B["d"], LLAMA7B["ffn"])
    out = {}

    def round_trip(ws, dtype, ev=None):
        if ev is not None:
            ev[0].record()
        qs = [nf4.nf4_quantize(w) for w in ws]
        if ev is not None:
            ev[1].record()
        dqs = nf4.nf4_double_quantize_batch([a for _, a in qs])
        if ev is not None:
            ev[2].record()
        wts = [nf4.NF4Weight(c, q, c2, m, (int(w.shape[0]), int(w.shape[1])))
               for w, (c, _), (q, c2, m) in zip(ws, qs, dqs)]
        outs = [nf4.nf4_dequantize(wt, dtype) for wt in wts]
        if ev is not None:
            ev[3].record()
        return qs, dqs, outs

    for dtype, tag, nbytes in ((torch.float32, "fp32", 4), (torch.bfloat16, "bf16", 2)):
        ws = []
        for layer in range(LLAMA7B["layers"]):
            for pi, (name, N, K) in enumerate(projs):
                ws.append(Draw(seed_of(20, layer, pi), dev).normal((N, K), 0.02, outlier_frac=0.01).to(dtype))
        n = sum(w.numel() for w in ws)
        res = round_trip(ws, dtype)                 # untimed: fills the allocator's cache
        torch.cuda.synchronize()
        del res
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        gate = torch.cuda.Event()
        torch.cuda._sleep(int(2e8))               # holds the queue while the calls are submitted
        gate.record()
        res = round_trip(ws, dtype, ev)
        host_bound = gate.query()
        torch.cuda.synchronize()
        del res
        t = [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(3)]
        b = [n * (nbytes + 0.5 + 4 / 64), n * (4 / 64 + 1 / 64 + 4 / (64 * 256)),
             n * (NF4_BYTES_PER_PARAM + nbytes)]
        rec = {}
        for key, ti, bi in zip(("quantize", "double_quantize", "dequantize"), t, b):
            rec[key] = dict(GBps=bi / ti / 1e9, ms=ti * 1e3, bytes=bi, frac_hbm=bi / ti / 1e9 / PEAK_HBM_GBS)
        rec["round_trip"] = dict(GBps=sum(b) / sum(t) / 1e9, ms=sum(t) * 1e3, bytes=sum(b),
                                 frac_hbm=sum(b) / sum(t) / 1e9 / PEAK_HBM_GBS)
        rec["params"] = n
        rec["tensors"] = len(ws)
        rec["host_bound"] = bool(host_bound)
        out[tag] = rec
        del ws
        torch.cuda.empty_cache()
    return out


def gemv_paths(layer, dev, r, alpha, reps=5):
    """Few-token forward (dequant-GEMV): GB/s over the layer's weights, M in {1, 4, 16}.

    The calls are queued behind a sleeping kernel and timed with one event pair
    around the whole batch, so the figure is GPU time per call (both launches of the
    path included) and neither host overhead nor event overhead enters it.  The
    seven projections rotate through > 256 MB, more than the Infinity Cache holds."""
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import Draw, seed_of

    out = {}
    for M in (1, 4, 16):
        d = Draw(seed_of(6, M), dev)
        xs = {p["name"]: d.bf16((M, p["K"]), 1.0) for p in layer}
        for p in layer:
            nf4.qlora_linear_fwd(p["Wq"], xs[p["name"]], p["A"], p["B"], alpha)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(5e7))           # holds the queue while the calls are submitted
        t0.record()
        h0 = time.perf_counter()
        for _ in range(reps):
            for p in layer:
                nf4.qlora_linear_fwd(p["Wq"], xs[p["name"]], p["A"], p["B"], alpha)
        h1 = time.perf_counter()
        t1.record()
        torch.cuda.synchronize()
        n = reps * len(layer)
        gpu_s = t0.elapsed_time(t1) / 1e3 / n
        # algorithmic bytes of one call: packed weight + A + B + X + Y (+ T)
        nbytes = sum(NF4_BYTES_PER_PARAM * p["N"] * p["K"] + 2 * r * (p["N"] + p["K"]) + 2 * M * p["K"]
                     + 2 * M * p["N"] + 2 * M * r for p in layer) / len(layer)
        out["M%d" % M] = dict(GBps=nbytes / gpu_s / 1e9, frac_hbm=nbytes / gpu_s / 1e9 / PEAK_HBM_GBS,
                              gpu_us_per_call=gpu_s * 1e6, host_us_per_call=(h1 - h0) * 1e6 / n,
                              bytes_per_call=nbytes, calls=n)
    return out


def adamw_paths(layer, dev, r, layers=80, reps=10):
    """The adapter optimizer step ("Paged optimizers, and QLoRA end to end"): AdamW over
    the LoRA parameters of `layers` decoder layers shaped like this one (A r x K and B
    N x r on every projection), held as one flat fp32 state (master p, m, v) with an fp32
    gradient and a bf16 copy of p: 30 bytes per parameter.  Device-resident state is
    timed over `reps` steps; state paged out to page-locked host memory (one layer's
    adapters through a 64 MiB staging buffer) is timed over one step and reported as
    host-link traffic (24 bytes per parameter: p, m, v in and out)."""
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import Draw, seed_of

    per_layer = sum(r * (p["N"] + p["K"]) for p in layer)
    n = per_layer * layers
    d = Draw(seed_of(8, layers), dev)
    pp = d.normal((n,), 0.02)
    g = d.normal((n,), 1e-3)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    pbf = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for t in range(1, 3):
        nf4.adamw_step(pp, g, m, v, 1e-4, t, p_bf16=pbf)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for t in range(3, 3 + reps):
        nf4.adamw_step(pp, g, m, v, 1e-4, t, p_bf16=pbf)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) / 1e3 / reps
    dev_rate = 30 * n / sec / 1e9
    del pp, m, v, pbf
    # one layer's adapters paged out to host memory
    k = per_layer
    ph, mh, vh = (torch.empty(k, dtype=torch.float32, pin_memory=True) for _ in range(3))
    ph.copy_(g[:k].cpu())
    mh.zero_()
    vh.zero_()
    stage = nf4._workspace(64 << 20, torch.device(dev))
    nf4.adamw_step_paged(ph, g[:k], mh, vh, 1e-4, 1, stage=stage)
    torch.cuda.synchronize()
    t0.record()
    nf4.adamw_step_paged(ph, g[:k], mh, vh, 1e-4, 2, stage=stage)
    t1.record()
    torch.cuda.synchronize()
    psec = t0.elapsed_time(t1) / 1e3
    del g, stage
    return dict(params=n, layers=layers,
                device=dict(GBps=dev_rate, frac_hbm=dev_rate / PEAK_HBM_GBS, us_per_step=sec * 1e6,
                            bytes_per_param=30),
                paged=dict(params=k, host_link_GBps=24 * k / psec / 1e9, us_per_step=psec * 1e6,
                           stage_bytes=64 << 20))


def codebook_paths(dev, n=1 << 28, reps=5):
    """The page's codebook comparison ("NF4, derived from normal quantiles") at GPU scale:
    n N(0,1) fp32 values in blocks of 64, quantized with NF4, the symmetric int4 grid
    {-7..7}/7, the grid {-8..7}/8 and a Lloyd codebook (30 GPU Lloyd steps from NF4);
    code entropy and RMS error of each, and the rates of the quantize and statistics
    kernels (the statistics pass reads 4 + 0.5 + 4/64 bytes per value)."""
    import numpy as np
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import Draw, seed_of

    w = Draw(seed_of(9), dev).normal((n,), 1.0)
    tables = {"nf4": [float(x) for x in nf4.nf4_codebook()], "int4_sym": nf4.codebook_int4_symmetric(),
              "uniform16": nf4.codebook_uniform16()}
    tables["lloyd"] = nf4.lloyd_codebook(w, tables["nf4"], iters=30)
    out = {"values": n}
    for name, lv in tables.items():
        codes, absmax = nf4.nf4_quantize_codebook(w, lv)
        count, _, sse = nf4.nf4_codebook_stats(w, codes, absmax, lv)
        p = count[count > 0] / count.sum()
        out[name] = dict(entropy_bits=float(-(p * np.log2(p)).sum()), rms=float(np.sqrt(sse / n)))
    out["rms_gain_nf4_vs_int4_sym"] = 1 - out["nf4"]["rms"] / out["int4_sym"]["rms"]
    out["rms_gain_lloyd_vs_nf4"] = 1 - out["lloyd"]["rms"] / out["nf4"]["rms"]
    lv = tables["nf4"]
    codes, absmax = nf4.nf4_quantize_codebook(w, lv)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        nf4.nf4_quantize_codebook(w, lv)
    t1.record()
    torch.cuda.synchronize()
    tq = t0.elapsed_time(t1) / 1e3 / reps
    t0.record()
    for _ in range(reps):
        nf4.nf4_codebook_stats(w, codes, absmax, lv)
    t1.record()
    torch.cuda.synchronize()
    ts = t0.elapsed_time(t1) / 1e3 / reps
    qb, sb = n * (4 + 0.5 + 4 / 64), n * (4 + 0.5 + 4 / 64)
    out["quantize"] = dict(GBps=qb / tq / 1e9, frac_hbm=qb / tq / 1e9 / PEAK_HBM_GBS)
    out["stats"] = dict(GBps=sb / ts / 1e9, frac_hbm=sb / ts / 1e9 / PEAK_HBM_GBS,
                        note="includes the host copy of the 33 results")
    return out


def loftq_paths(dev, r=64, alpha=16.0, l=80, power=2, iters=5):
    """LoftQ-style initialisation ("Paged optimizers, and QLoRA end to end", closing remark):
    `iters` alternations of NF4 + double quantization of the residual and a rank-r randomized
    SVD of the quantization error, on the LLaMA-65B q (8192 x 8192) and gate (22016 x 8192)
    shapes (W ~ N(0, 0.02^2), seeded; sketch width l, `power` subspace iterations).  Reports
    the time per alternation, the residual norm after the first and the last alternation
    relative to plain NF4's ||W - dequant(Q)||_F, and the rate of the tall fp32 products
    (2 N K l flops per pass, 2 + 2 power passes per alternation, over the whole alternation
    time: a lower bound on the kernels' own rate)."""
    import torch
    import bit_nf4_quantized_09_amd as nf4
    from workloads import Draw, seed_of

    out = {"r": r, "alpha": alpha, "sketch_l": l, "power_iters": power, "alternations": iters}
    for (name, N, K) in (("q65b", 8192, 8192), ("gate65b", 22016, 8192)):
        W = Draw(seed_of(10, N, K), dev).normal((N, K), 0.02)
        om = Draw(seed_of(11, K, l), dev).normal((K, l), 1.0)
        nf4.loftq_init(W, r, alpha, om, iters=1, power_iters=power)
        Wq0 = nf4.quantize_weight(W)
        plain = float(torch.linalg.vector_norm(W - nf4.nf4_dequantize(Wq0, torch.float32)).item())
        del Wq0
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        _, _, _, err = nf4.loftq_init(W, r, alpha, om, iters=iters, power_iters=power)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / iters
        err = err.cpu().tolist()
        tall_flops = (2 + 2 * power) * 2.0 * N * K * l
        out[name] = dict(N=N, K=K, ms_per_alternation=ms, err_plain_nf4=plain,
                         err_rel_first=err[0] / plain, err_rel_last=err[-1] / plain,
                         tall_tflops_lower_bound=tall_flops / (ms / 1e3) / 1e12)
        del W, om
        torch.cuda.empty_cache()
    return out


def cpu_baseline(layer, alpha, r, tokens):
    """The CPU oracle (float64, OpenMP) on `tokens` tokens through every projection."""
    import numpy as np
    import oracle
    from workloads import host_f32

    t_total = 0.0
    flops = 0
    for p in layer:
        codes, absmax = oracle.nf4_quantize(host_f32(p["W"]).reshape(-1))
        q, c2, mean = oracle.double_quantize(absmax)
        Wd = oracle.nf4_dequantize(codes, q, c2, mean, (p["N"], p["K"]))
        X = host_f32(p["X"][:tokens])
        dY = host_f32(p["dY"][:tokens])
        A, B = host_f32(p["A"]), host_f32(p["B"])
        t0 = time.perf_counter()
        oracle.qlora_linear_fwd(Wd, X, A, B, alpha)
        oracle.qlora_linear_bwd(Wd, X, dY, A, B, alpha)
        t_total += time.perf_counter() - t0
        f, b = layer_flops(tokens, [(p["name"], p["N"], p["K"])], r)
        flops += f + b
        del Wd
    return dict(value=flops / t_total / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                kind="oracle", seconds=t_total,
                sample="fwd+bwd of %d tokens through all %d projections (same weights, "
                       "float64 oracle)" % (tokens, len(layer)))


def hbm_ceiling(reps=10):
    """The streaming ceilings of this GPU's HBM, for context: a linear read, a linear
    write and a copy over 4 GiB buffers (16-byte accesses, grid-stride, plain and
    nontemporal, several grid sizes), each timed over `reps` back-to-back launches
    with one event pair on the current stream.  Prints a markdown table."""
    import ctypes
    import torch
    from bit_nf4_quantized_09_amd.build import PROBE_LIB

    if not os.path.exists(PROBE_LIB):
        raise SystemExit("the probe library is not built (python bit_nf4_quantized_09_amd/build.py)")
    L = ctypes.CDLL(PROBE_LIB)
    L.nf4probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.nf4probe_stream.restype = ctypes.c_int
    nbytes = 4 << 30
    src = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    names = {0: "read", 1: "write", 2: "copy"}
    rows = ["| pattern | nontemporal | workgroups | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
    best = {}
    for kind in (0, 1, 2):
        for nt in (0, 1):
            for grid in (1024, 2048, 4096, 8192, 16384):
                args = (kind, src.data_ptr(), sink.data_ptr() if kind == 0 else dst.data_ptr(), nbytes, grid, nt,
                        stream)
                if L.nf4probe_stream(*args) != 0:
                    raise SystemExit("probe launch failed")
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                t0.record()
                for _ in range(reps):
                    L.nf4probe_stream(*args)
                t1.record()
                torch.cuda.synchronize()
                moved = nbytes * (2 if kind == 2 else 1)
                gbs = moved / (t0.elapsed_time(t1) / 1e3 / reps) / 1e9
                best[names[kind]] = max(best.get(names[kind], 0.0), gbs)
                rows.append("| %s | %s | %d | %.0f | %.1f%% |" % (names[kind], "yes" if nt else "no", grid, gbs,
                                                                   100.0 * gbs / PEAK_HBM_GBS))
            print("hbm ceiling: %s nontemporal=%d done" % (names[kind], nt), file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes / (t0.elapsed_time(t1) / 1e3 / reps) / 1e9
    rows.append("| copy (torch copy_) | - | - | %.0f | %.1f%% |" % (gbs, 100.0 * gbs / PEAK_HBM_GBS))
    rows += ["", "best: " + ", ".join("%s %.0f GB/s" % kv for kv in best.items())]
    del src, dst
    rows += ["", "One launch over a buffer of the few-token forward's size (the packed 8192 x 8192 and",
             "22016 x 8192 weights): GPU time per launch over launches queued behind a sleeping",
             "kernel, rotating through copies of more than 1 GB, so each reads from HBM.", "",
             "| MB read | nontemporal | workgroups | us per launch | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|"]
    for mb in (34.6, 92.9):
        size = int(mb * 1e6) // 16 * 16
        copies = max(2, (1 << 30) // size + 1)
        bufs = [torch.empty(size // 4, dtype=torch.int32, device="cuda:0").fill_(i) for i in range(copies)]
        for nt in (0, 1):
            for grid in (1024, 2048, 4096, 8192):
                for b in bufs:
                    L.nf4probe_stream(0, b.data_ptr(), sink.data_ptr(), size, grid, nt, stream)
                torch.cuda.synchronize()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(int(5e7))
                t0.record()
                for b in bufs:
                    L.nf4probe_stream(0, b.data_ptr(), sink.data_ptr(), size, grid, nt, stream)
                t1.record()
                torch.cuda.synchronize()
                us = t0.elapsed_time(t1) * 1e3 / copies
                gbs = size / (us * 1e-6) / 1e9
                rows.append("| %.1f | %s | %d | %.2f | %.0f | %.1f%% |" % (size / 1e6, "yes" if nt else "no", grid, us,
                                                                           gbs, 100.0 * gbs / PEAK_HBM_GBS))
        del bufs
        print("hbm ceiling: %.1f MB reads done" % mb, file=sys.stderr, flush=True)
    print("\n".join(rows), flush=True)


def pmc_codec_workload():
    """For counter runs: one pass of each HBM-bound kernel over the LLaMA-65B layer's
    seven weights (fp32 and bf16 quantize, double quantization, fp32- and bf16-out
    dequantize, the few-token forward at M = 1, 4, 16), then a plain copy of COPY_BYTES."""
    import torch
    import bit_nf4_quantized_09_amd as nf4

    layer, projs, M, r, alpha = build_layer("llama65b_layer", "cuda:0")
    absmax = [nf4.nf4_quantize(p["W"])[1] for p in layer]
    wb = [p["W"].to(torch.bfloat16) for p in layer]
    torch.cuda.synchronize()
    for w in wb:
        nf4.nf4_quantize(w)
    del wb
    for a in absmax:
        nf4.nf4_double_quantize(a)
    for dt in (torch.float32, torch.bfloat16):
        for p in layer:
            nf4.nf4_dequantize(p["Wq"], dt)
    for m in (1, 4, 16):
        for p in layer:
            nf4.qlora_linear_fwd(p["Wq"], p["X"][:m].contiguous(), p["A"], p["B"], alpha)
    torch.cuda.synchronize()
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    calibration_probes()
    print("pmc codec workload done", flush=True)


def calibration_probes():
    """A pure read and a pure write of COPY_BYTES (the ceiling probes), each touching a
    buffer no kernel has touched before, for calibrating FETCH_SIZE and WRITE_SIZE."""
    import ctypes
    import torch
    from bit_nf4_quantized_09_amd.build import PROBE_LIB

    L = ctypes.CDLL(PROBE_LIB)
    L.nf4probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.nf4probe_stream.restype = ctypes.c_int
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    if (L.nf4probe_stream(0, src.data_ptr(), sink.data_ptr(), COPY_BYTES, 8192, 0, stream) != 0 or
            L.nf4probe_stream(1, None, dst.data_ptr(), COPY_BYTES, 8192, 0, stream) != 0):
        raise SystemExit("probe launch failed")
    torch.cuda.synchronize()


def summarize_pmc_codec(fetch_csv, write_csv):
    """Per-kernel HBM traffic of the counter runs over --pmc-codec-workload, next to the
    algorithmic bytes of the same dispatches."""
    from workloads import LLAMA65B, layer_projections

    fetch = _read_counters(fetch_csv, "FETCH_SIZE")
    write = _read_counters(write_csv, "WRITE_SIZE")
    is_copy = lambda k: "copy" in k.lower()
    fc = [v for (d, k), v in fetch.items() if is_copy(k or "")]
    wc = [v for (d, k), v in write.items() if is_copy(k or "")]
    if not (fc and wc):
        raise SystemExit("counter files lack the copy kernel")
    kf_copy = (COPY_BYTES / 1024.0) / max(fc)
    kw_copy = (COPY_BYTES / 1024.0) / max(wc)
    pr = [v for (d, k), v in fetch.items() if "k_probe_read" in (k or "")]
    pw = [v for (d, k), v in write.items() if "k_probe_write" in (k or "")]
    # the pure read and pure write of the same size calibrate each counter on its own
    kf = (COPY_BYTES / 1024.0) / pr[0] if pr else kf_copy
    kw = (COPY_BYTES / 1024.0) / pw[0] if pw else kw_copy
    projs = layer_projections(LLAMA65B["d"], LLAMA65B["ffn"])
    n = sum(N * K for _, N, K in projs)
    nk = [(N, K) for _, N, K in projs]
    n1 = n / 64
    # algorithmic bytes over the workload's dispatches of each kernel (all 7 weights)
    fams = [
        ("quantize, fp32 in", lambda k: "k_quantize<unsigned int>" in k, 7, n * (4 + 0.5 + 4 / 64)),
        ("quantize, bf16 in", lambda k: "k_quantize<unsigned short>" in k, 7, n * (2 + 0.5 + 4 / 64)),
        ("double quantization: chunk sums", lambda k: "k_dqb_chunks" in k, 7, n1 * 4),
        ("double quantization: mean + 8-bit encode", lambda k: "k_dqb_encode" in k or "k_dq_encode" in k, 7,
         n1 * (4 + 1) + n1 / 256 * 4),
        ("dequantize, fp32 out", lambda k: "k_dequantize<false, false>" in k, 7, n * (NF4_BYTES_PER_PARAM + 4)),
        ("dequantize, bf16 out", lambda k: "k_dequantize<true, false>" in k, 7, n * (NF4_BYTES_PER_PARAM + 2)),
        ("few-token forward: part (M = 1, 4, 16)", lambda k: "k_gemv_part" in k, 21,
         sum(NF4_BYTES_PER_PARAM * N * K + 2 * 64 * (N + K) + 2 * m * K for (N, K) in nk for m in (1, 4, 16))),
    ]
    lines = [
        "# HBM traffic of the codec and few-token kernels, LLaMA-65B layer weights",
        "",
        "Commands (GPU, from the repository root; one counter per run):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE -d pmc_fetch -o run --output-format csv -- python bench.py --pmc-codec-workload",
        "    rocprofv3 --pmc WRITE_SIZE -d pmc_write -o run --output-format csv -- python bench.py --pmc-codec-workload",
        "    python bench.py --summarize-pmc-codec <pmc_fetch>/run_counter_collection.csv "
        "<pmc_write>/run_counter_collection.csv",
        "",
        "The workload makes one pass of each kernel over the seven weights (%.4g values); the "
        "few-token forward runs once per weight at M = 1, 4 and 16. Calibration: a plain device "
        "copy of %d MiB in the same run reads %.1f KiB by FETCH_SIZE and writes %.1f KiB by "
        "WRITE_SIZE (factors %.4f and %.4f); a pure read of the same size (the read probe) "
        "fetches %s KiB and a pure write writes %s KiB. The table uses the factors %.4f (fetch) "
        "and %.4f (write)%s." % (n, COPY_BYTES >> 20, max(fc), max(wc), kf_copy, kw_copy,
                                 "%.1f" % pr[0] if pr else "-", "%.1f" % pw[0] if pw else "-", kf, kw,
                                 ", from the pure read and write" if pr and pw else ", from the copy"),
        "",
        "| kernel | dispatches | fetched bytes | written bytes | traffic | algorithmic bytes | traffic / algorithmic |",
        "|---|---|---|---|---|---|---|",
    ]
    def last(table, pred, count):
        # the workload's own dispatches are the last `count` of each kernel (the layer's
        # set-up quantizes the weights first)
        v = sorted((int(d), x) for (d, k), x in table.items() if pred(k or ""))
        return [x for _, x in v[-count:]]

    for label, pred, expect, alg in fams:
        fv = last(fetch, pred, expect)
        wv = last(write, pred, expect)
        if not fv or not wv:
            lines.append("| %s | 0 | - | - | - | %.4g | - |" % (label, alg))
            continue
        fb = sum(fv) * 1024.0 * kf
        wb_ = sum(wv) * 1024.0 * kw
        lines.append("| %s | %d | %.4g | %.4g | %.4g | %.4g | %.3f |" % (
            label, len(fv), fb, wb_, fb + wb_, alg, (fb + wb_) / alg))
        if len(fv) != expect:
            lines.append("| (%s: %d dispatches found, %d expected) | | | | | | |" % (label, len(fv), expect))
    red_f = last(fetch, lambda k: "k_gemv_reduce" in k, 21)
    red_w = last(write, lambda k: "k_gemv_reduce" in k, 21)
    if red_f and red_w:
        lines.append("| few-token forward: slice reduce | %d | %.4g | %.4g | %.4g | - | - |" % (
            len(red_f), sum(red_f) * 1024.0 * kf, sum(red_w) * 1024.0 * kw,
            sum(red_f) * 1024.0 * kf + sum(red_w) * 1024.0 * kw))
    lines += ["", "kernel_source_sha256 (codec.hip, gemv.hip, nf4_common.h, bufio.h) = %s"
              % kernel_source_hash(["codec.hip", "gemv.hip", "nf4_common.h", "bufio.h"])]
    print("\n".join(lines))


def pmc_workload(args):
    """One untimed step of the workload, then a plain device copy of COPY_BYTES."""
    import torch

    layer, projs, M, r, alpha = build_layer(args.workload, "cuda:0")
    run_step(layer, alpha)
    torch.cuda.synchronize()
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    calibration_probes()
    print("pmc workload done", flush=True)


def main():
    args = _args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_pmc_codec:
        summarize_pmc_codec(*args.summarize_pmc_codec)
        return
    if args.summarize_gemv_pmc:
        summarize_gemv_pmc(*args.summarize_gemv_pmc)
        return
    if args.summarize_gemv_trace:
        summarize_gemv_trace(args.summarize_gemv_trace)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.plain_gemm:
        plain_gemm_table()
        return
    if args.gemv_sweep:
        gemv_sweep()
        return
    if args.pmc_workload:
        pmc_workload(args)
        return
    if args.pmc_codec_workload:
        pmc_codec_workload()
        return
    if args.hbm_ceiling:
        hbm_ceiling()
        return
    if args.codebooks_only:
        print(json.dumps({"codebooks": codebook_paths(dev)}), flush=True)
        return
    if args.gemv_only:
        layer, projs, M, r, alpha = build_layer(args.workload, dev)
        print(json.dumps({"gemv": gemv_paths(layer, dev, r, alpha)}), flush=True)
        return
    if args.loftq_only:
        print(json.dumps({"loftq": loftq_paths(dev)}), flush=True)
        return
    if args.bulk_codec_only:
        print(json.dumps({"codec_llama7b_32_layers": bulk_codec_paths(dev)}), flush=True)
        return
    if args.adamw_only:
        from workloads import LLAMA65B, layer_projections
        shapes = [dict(N=N, K=K) for _, N, K in layer_projections(LLAMA65B["d"], LLAMA65B["ffn"])]
        print(json.dumps({"adamw": adamw_paths(shapes, dev, 64)}), flush=True)
        return
    layer, projs, M, r, alpha = build_layer(args.workload, dev)
    fwd_flops, bwd_flops = layer_flops(M, projs, r)

    for _ in range(args.warmup):
        run_step(layer, alpha)
    torch.cuda.synchronize()

    events = {"fwd": [], "bwd": []}
    # The fused launches of every 5th timed step (the last one when there are fewer than
    # 5) are bracketed by timing events for their average duration: each event is a
    # marker packet that idles the GPU for ~5 us, which on every launch of every step
    # would take ~1% off the step rate measured around them.
    sampled = [i for i in range(args.steps) if i % 5 == 4] or [args.steps - 1]
    pool = event_pool(len(sampled) * 2 * len(layer))
    # step boundaries on the stream the kernels run on: per-step GPU times (median, min)
    marks = [ev for pair in event_pool((args.steps + 2) // 2) for ev in pair][:args.steps + 1]
    t0 = time.perf_counter()
    for i in range(args.steps):
        marks[i].record()
        if i in sampled:
            run_step(layer, alpha, events, pool)
        else:
            run_step(layer, alpha)
    marks[args.steps].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = (fwd_flops + bwd_flops) / (ms / 1e3) / 1e12
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    step_median = (step_ms[(args.steps - 1) // 2] + step_ms[args.steps // 2]) / 2

    kf = kernel_roofline(events, M, r, "fwd")
    kb = kernel_roofline(events, M, r, "bwd")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "ms_per_step_gpu": {"median": round(step_median, 3), "min": round(step_ms[0], 3),
                            "tflops_at_median": round((fwd_flops + bwd_flops) / (step_median / 1e3) / 1e12, 2)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian weights/activations at LLaMA shapes)",
        "config": {"workload": args.workload, "tokens": M, "projections": [p[0] for p in projs],
                   "shapes_NxK": [[p[1], p[2]] for p in projs], "r": r, "alpha": alpha,
                   "nf4_blocksize": 64, "dq_blocksize": 256, "parallelism": "single-gpu",
                   "fwd_tflop": fwd_flops / 1e12, "bwd_tflop": bwd_flops / 1e12,
                   "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "kernel": kf["kernel"], "achieved": round(kf["achieved"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kf["achieved"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic_per_launch(args.workload),
                     "avg_us": round(kf["avg_us"], 2), "launches": kf["launches"],
                     "bwd_dx_kernel": {"kernel": kb["kernel"], "achieved": round(kb["achieved"], 2),
                                       "frac": round(kb["achieved"] / PEAK_BF16_TFLOPS, 4),
                                       "avg_us": round(kb["avg_us"], 2)}},
    }
    line["peaks"] = {"bf16_tflops_used": PEAK_BF16_TFLOPS, "hbm_gbps_used": PEAK_HBM_GBS,
                     "source": "MI355X published dense figures", "rocminfo": rocminfo_peaks()}
    if not args.no_paths and args.workload != "tiny":
        line["paths"] = {"codec": codec_paths(layer, dev), "codec_llama7b_32_layers": bulk_codec_paths(dev),
                         "gemv": gemv_paths(layer, dev, r, alpha),
                         "adamw": adamw_paths(layer, dev, r), "codebooks": codebook_paths(dev),
                         "variants": variant_paths(layer, alpha, fwd_flops + bwd_flops),
                         "loftq": loftq_paths(dev)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layer, alpha, r, min(args.cpu_tokens, M))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
