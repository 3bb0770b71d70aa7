#!/usr/bin/env python3
"""Benchmark of the fused-epilogue GEMM on one MI355X.

One step = one launch of D = ReLU(op(A) op(B) + bias[N]) on the headline workload, fp16 8192^3
NN with fp32 accumulation and fp16 output (inputs resident in HBM before the timed region).
Prints one JSON line with TFLOP/s, the roofline position of the kernel (its average duration
from HIP events recorded on the launch stream) and the CPU oracle timed on a bounded row sample
of the same workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME[:IDX]] [--no-cpu]
                  [--no-graph]
  python bench.py --calibrate-copy     (plain 1 GiB device copies, for scaling HBM counters)
  python bench.py --calibrate-read     (read-only 1 GiB reductions, the same for FETCH_SIZE)

The K timed launches are captured once into a HIP graph and replayed, so that a short kernel
is timed without the host's per-call overhead (every launch still runs the full product);
--no-graph times K eager calls instead.  For a memory-bound workload the launches cycle through
copies of the operands (> 512 MB together), so that every launch reads from HBM rather than from
the 256 MB infinity cache; the cache-hot figure of one reused set is reported beside it.

roofline.traffic is the measured HBM traffic per launch (FETCH_SIZE + WRITE_SIZE from rocprofv3,
each scaled by what the same counter reads for a plain copy of known size), taken from the
summary profiles/traffic_<workload>.json when that summary was measured on the current kernel
sources (it records their hash); otherwise null.  clocks holds the driver's current core and
memory clock levels (sysfs) just before the warm-up and right after the timed launches.

Timing protocol: W untimed warm-up launches, then blocks of exactly K launches (one HIP graph of
K launches, replayed), each bracketed by device synchronisations and timed with HIP events on
the launch stream; blocks repeat until the last five agree within a coefficient of variation of
2 % (at most 30 blocks), and the reported time per launch is the median of those five blocks
("Flexible Performant GEMM Kernels on GPUs", section 5: samples are taken until the spread of
the timings is small).  Every block runs the full product on the same resident inputs.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (and % of MFMA peak) fp16->fp32 GEMM 8192^3 with bias+ReLU epilogue"
# MI355X published dense peaks (TFLOP/s, TOP/s for int8) and HBM bandwidth (GB/s)
PEAK = {"f16": 2516.6, "bf16": 2516.6, "i8": 5033.2, "f32": 157.3,
        "cf16": 2516.6, "df16": 2516.6}   # complex / dual: fp16 parts on the fp16 MFMA
HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit():
        n = min(n, int(cap))
    return max(1, n)


def _code_only(text):
    """C++ source without comments and blank space: edits to comments keep the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the code (comments and spacing left out) of the HIP sources the timed kernels are
    built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_gemm_epilogues_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from a committed counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def calibrate_copy():
    """Plain device-to-device copies of 1 GiB (the reference for scaling FETCH/WRITE_SIZE)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


def calibrate_read():
    """Read-only reductions of a 1 GiB buffer (each byte read once, a few bytes written): a second
    reference for FETCH_SIZE, made of full-line reads like the GEMM kernels' loads."""
    import torch
    n = 1 << 29
    x = torch.ones(n, dtype=torch.float16, device="cuda:0")
    for _ in range(5):
        x.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "read", "bytes_read": 2 * n, "launches": 5}))


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_clocks():
    """Current GPU core (sclk) and memory (mclk) clocks in MHz, read in-process from the amdgpu
    driver's sysfs tables (the level marked '*' in pp_dpm_sclk / pp_dpm_mclk); None where the
    files are absent.  No child process: this runs after the GPU has been initialised."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        clk = {}
        for name in ("sclk", "mclk"):
            try:
                with open(os.path.join(dev, f"pp_dpm_{name}")) as fh:
                    lines = fh.read().splitlines()
            except OSError:
                continue
            for line in lines:
                if line.rstrip().endswith("*"):
                    digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                    clk[name + "_MHz"] = int(digits) if digits else None
        if clk:
            out[os.path.basename(os.path.dirname(dev))] = clk
    return out or None


def pick_workload(spec):
    import synth
    name, _, idx = spec.partition(":")
    probs = synth.WORKLOADS[name]()
    return probs[int(idx) if idx else 0]


def vendor_context(p, A, B, bias, stream, args):
    """torch.matmul (hipBLASLt on ROCm) on the same operands, for context: the product alone, and
    the product with the bias add and ReLU as the separate kernels an unfused framework runs.
    Same block timing as the library's launches (graphs of --steps launches).  Only for one
    fp16/bf16 -> same-type product of tight row-major operands, not transposed."""
    import torch
    if not (p.batch == 1 and p.batch2 == 1 and p.op_a == "N" and p.op_b == "N" and p.ab == p.cd
            and p.ab in ("f16", "bf16") and p.beta == 0 and p.lda == p.K and p.ldb == p.N
            and p.ldc == p.N and p.kind_a == p.kind_b == "dense"
            and (p.transform_a, p.transform_b, p.transform_c) == ("none", "none", "none")):
        return {"note": "not timed: torch comparison only for dense NN fp16/bf16 products"}
    tA = A[: p.M * p.K].view(p.M, p.K)
    tB = B[: p.K * p.N].view(p.K, p.N)
    out = torch.empty(p.M, p.N, dtype=tA.dtype, device=tA.device)
    bias_t = bias.to(tA.dtype) if bias is not None else None
    alpha = p.alpha

    def plain():
        torch.matmul(tA, tB, out=out)

    def unfused():
        if bias_t is not None:
            torch.addmm(bias_t, tA, tB, alpha=alpha, out=out)
        else:
            torch.matmul(tA, tB, out=out)
        if p.relu:
            torch.relu_(out)

    res = {}
    for name, fn in (("matmul_ms", plain), ("matmul_bias_relu_ms", unfused)):
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(args.steps):
                fn()
        torch.cuda.synchronize()
        times = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        while True:
            with torch.cuda.stream(stream):
                e0.record(stream)
                graph.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / args.steps)
            last = np.array(times[-5:])
            if (len(last) == 5 and last.std() / last.mean() < 0.02) or len(times) >= args.max_blocks:
                break
        res[name] = round(float(np.median(last)), 5)
        del graph
    res["note"] = ("torch " + torch.__version__ + " on the same operands (hipBLASLt); bias and ReLU "
                   "as separate kernels in the second figure; context only, not a parity reference")
    log(f"[bench] vendor context: {res}")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="fp16_8192_bias_relu")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--no-graph", action="store_true",
                    help="time K eager launches instead of one graph of K launches")
    ap.add_argument("--max-blocks", type=int, default=30,
                    help="most timed blocks of --steps launches (fewer once they agree)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--vendor-context", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the same operands, plain and with "
                         "bias and ReLU as separate kernels (context only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB copies (reference for the HBM byte counters)")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only run read-only reductions of 1 GiB (reference for FETCH_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this GEMM runs on one GPU; multi-GPU runs are not part of this "
              "build (the path shards by output rows or columns with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import tiled_gemm_epilogues_amd as tge
    from tiled_gemm_epilogues_amd import Plan

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_read:
        calibrate_read()
        return

    p = pick_workload(args.workload)
    log(f"[bench] workload {p.label()}")
    t0 = time.time()
    x = synth.make_inputs(p)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    def dev(dtype, raw):
        flat = np.ascontiguousarray(raw).reshape(-1)
        if flat.dtype == np.uint16 and dtype not in ("f16", "bf16"):
            return torch.from_numpy(flat.view(np.int16)).to("cuda:0")   # fp16 parts of pairs
        if dtype in ("f16", "bf16"):
            t = torch.from_numpy(flat.view(np.int16)).view(
                {"f16": torch.float16, "bf16": torch.bfloat16}[dtype])
        else:
            t = torch.from_numpy(flat)
        return t.to("cuda:0")

    A = dev(p.a_store, x["A"])
    B = dev(p.b_store, x["B"])
    C = dev(p.cd, x["C"]) if x["C"] is not None else None
    bias = dev(p.bias_dt, x["bias"]) if x["bias"] is not None else None
    pair = p.cd in synth.PART          # complex / dual output: interleaved parts
    D = torch.empty((max(p.batch - 1, 0) * p.stride_c + max(p.batch2 - 1, 0) * p.stride2_c +
                     p.M * p.ldc) * (2 if pair else 1),
                    dtype={"f16": torch.float16, "bf16": torch.bfloat16,
                           "f32": torch.float32, "i32": torch.int32}[synth.PART.get(p.cd, p.cd)],
                    device="cuda:0")
    plan = Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c,
                stride_bias=p.stride_bias, transform_a=p.transform_a, transform_b=p.transform_b,
                transform_c=p.transform_c, kind_a=p.kind_a, kind_b=p.kind_b, batch2=p.batch2,
                stride2_a=p.stride2_a, stride2_b=p.stride2_b, stride2_c=p.stride2_c,
                stride2_bias=p.stride2_bias)
    log(f"[bench] kernel: {plan.describe()}")

    flops = p.flops
    peak = PEAK[p.ab]
    bytes_alg = p.algorithmic_bytes()
    # the skinny and diagonal shapes are bound by HBM; the rest by MFMA
    hbm_bound = flops / bytes_alg < peak * 1e12 / (HBM_GBS * 1e9)

    # every launch goes to one non-default stream (the graph is captured and replayed there)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def time_launches(sets):
        """(median ms per launch, wall ms per launch, blocks) over blocks of args.steps launches
        cycling through the operand sets."""
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                plan.run(*sets[i % len(sets)], p.alpha, p.beta)
        torch.cuda.synchronize()
        graph = None
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(args.steps):
                    plan.run(*sets[i % len(sets)], p.alpha, p.beta)
            torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        times, walls = [], []
        window = 5
        while True:
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            with torch.cuda.stream(stream):
                ev0.record(stream)
                if graph is not None:
                    graph.replay()
                else:
                    for i in range(args.steps):
                        plan.run(*sets[i % len(sets)], p.alpha, p.beta)
                ev1.record(stream)
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - w0) * 1e3 / max(1, args.steps))
            times.append(ev0.elapsed_time(ev1) / max(1, args.steps))
            last = np.array(times[-window:])
            cv = float(last.std() / last.mean()) if len(last) >= 2 else 1.0
            if (len(last) == window and cv < 0.02) or len(times) >= args.max_blocks:
                break
        log(f"[bench] blocks of {args.steps} launches (ms/launch): "
            + " ".join(f"{t:.4f}" for t in times) + f"; last {len(last)}: CV {cv:.4f}")
        blocks = {"launches_per_block": args.steps, "blocks": len(times),
                  "window": len(last), "cv": round(cv, 5),
                  "median_of_window_ms": round(float(np.median(last)), 5),
                  "first_block_ms": round(times[0], 5)}
        return float(np.median(last)), float(np.median(walls[-window:])), blocks

    base = (A, B, C, D, bias)
    clocks = {"before": gpu_clocks()}
    ms_hot, ms_wall, blocks = time_launches([base])
    # right after the timed launches (the clock reading comes from sysfs a moment later)
    clocks["after"] = gpu_clocks()
    log(f"[bench] clocks before / after the timed launches: {clocks}")
    log(f"[bench] {args.steps} steps per block: {ms_hot:.4f} ms/launch (events, median), "
        f"{ms_wall:.4f} ms/step (wall)")
    ms_events, hot = ms_hot, None
    if hbm_bound:
        # a working set this small stays in the 256 MB infinity cache when one set of operands
        # is reused: the launches also cycle through enough copies (> 512 MB) that every launch
        # reads its operands from HBM; that is the reported figure, the cache-hot one beside it
        nsets = max(16 if bytes_alg < 64e6 else 2, int(np.ceil(512e6 / bytes_alg)))
        clone = lambda t: None if t is None else t.clone()
        sets = [base] + [tuple(clone(t) for t in base) for _ in range(nsets - 1)]
        ms_events, ms_wall, blocks = time_launches(sets)
        log(f"[bench] {nsets} rotating operand sets: {ms_events:.4f} ms/launch (events)")
        hot = {"ms_per_step": round(ms_hot, 5), "operand_sets": 1,
               "achieved_GBps": round(bytes_alg / (ms_hot * 1e-3) / 1e9, 1)}
        del sets
    graph = None if args.no_graph else True

    vendor = vendor_context(p, A, B, bias, stream, args) if args.vendor_context else None

    tflops = flops / (ms_events * 1e-3) / 1e12
    if hbm_bound:
        gbs = bytes_alg / (ms_events * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_GBS, 4), "traffic": None,
                "operand_sets": nsets, "cache_hot": hot}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": None}
    roof["traffic"] = measured_traffic(args.workload.replace(":", "_"))

    cpu = None
    parity = None
    if not args.no_cpu:
        # the CPU-baseline leg: the oracle timed on a row sample, which also checks those rows
        # of the timed output (not timed)
        import oracle
        # product 0 of a batch (the sample is taken from it)
        part = synth.PART.get(p.cd, p.cd)
        D0 = D[: p.M * p.ldc * (2 if pair else 1)]
        Dh = D0.view(torch.int16).cpu().numpy().view(np.uint16) if part in ("f16", "bf16") \
            else D0.cpu().numpy()
        Dh = Dh.reshape((p.M, p.ldc, 2) if pair else (p.M, p.ldc))
        threads = host_threads()
        # two pilots separate the fixed cost (decoding B) from the per-row cost; the sample is
        # then sized for about --cpu-seconds of oracle work
        def oracle_rows(r):
            t0 = time.perf_counter()
            if pair:
                out = oracle.gemm_pair(p.M, p.N, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb,
                                       p.ab, C=x["C"], ldc=p.ldc, cd=p.cd, alpha=p.alpha,
                                       beta=p.beta, rows=(0, r), threads=threads)
                return time.perf_counter() - t0, out
            out = oracle.gemm(p.M, p.N, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, p.ab,
                              C=x["C"], ldc=p.ldc, cd=p.cd, bias=x["bias"], alpha=p.alpha,
                              beta=p.beta, relu=p.relu, rows=(0, r), threads=threads,
                              transform_a=p.transform_a, transform_b=p.transform_b,
                              transform_c=p.transform_c, kind_a=p.kind_a, kind_b=p.kind_b)
            return time.perf_counter() - t0, out
        r1, r2 = min(32, p.M), min(96, p.M)
        t1, _ = oracle_rows(r1)
        t2, _ = oracle_rows(r2) if r2 > r1 else (t1, None)
        per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
        fixed = max(t1 - r1 * per_row, 0.0)
        rows = int((args.cpu_seconds - fixed) / per_row) // 32 * 32
        rows = max(r1, min(p.M, rows))
        t_cpu, ref = oracle_rows(rows)
        sample_flops = p.flops * rows / p.M / max(p.batch * p.batch2, 1)
        cpu = {"value": round(sample_flops / t_cpu / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"output rows 0..{rows - 1} of {p.M}"
                         f"{' of product 0' if p.batch * p.batch2 != 1 else ''} "
                         f"(all {p.N} columns, full K={p.K}): "
                         f"{sample_flops:.3e} flop in {t_cpu:.1f}s, fp64/int64 accumulation"}
        log(f"[bench] cpu oracle: {cpu['sample']}")
        got = oracle.decode(part, Dh[:rows, : p.N]) if p.cd != "i32" else Dh[:rows, : p.N].astype(np.int64)
        if pair:   # the parts of every stored number (ld padding included) bound |op(X)|
            maxa = float(np.abs(oracle.decode(synth.PART[p.ab], x["A"])).max())
            maxb = float(np.abs(oracle.decode(synth.PART[p.ab], x["B"])).max())
        else:
            maxa = (float(np.abs(oracle.decode(p.ab, x["A"])).max()) if p.kind_a == "diagonal"
                    else oracle.max_abs_op(p.ab, x["A"], p.op_a, p.M, p.K, p.lda, p.transform_a))
            maxb = (float(np.abs(oracle.decode(p.ab, x["B"])).max()) if p.kind_b == "diagonal"
                    else oracle.max_abs_op(p.ab, x["B"], p.op_b, p.K, p.N, p.ldb, p.transform_b))
        den = p.K * maxa * maxb
        err = float(np.max(np.abs(got - ref)) / den) if den else float(np.max(np.abs(got - ref)))
        parity = {"rows_checked": rows, "max_normalised_error": err, "tolerance": 2e-3,
                  "ok": bool(err <= 2e-3) if p.cd != "i32" else bool(err == 0)}
        log(f"[bench] parity on rows 0..{rows - 1}: {parity}")

    out = {
        "metric": METRIC if args.workload == "fp16_8192_bias_relu" else
        f"TFLOP/s {p.label()}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s" if p.ab != "i8" else "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_events, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.ab,
        "data": "synthetic",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
                   "batch2": p.batch2,
                   "transforms": [p.transform_a, p.transform_b, p.transform_c],
                   "kinds": [p.kind_a, p.kind_b],
                   "layout": p.op_a + p.op_b,
                   "ab": p.ab, "cd": p.cd, "epilogue": p.epi, "alpha": p.alpha, "beta": p.beta,
                   "kernel": plan.describe(), "frac_of_peak": round(tflops / peak, 4),
                   "launch": "eager" if graph is None else
                   f"blocks of one HIP graph of {args.steps} launches, median of the last "
                   f"{blocks['window']}"},
        "roofline": roof,
        "timing": blocks,
        "clocks": clocks,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if vendor is not None:
        out["vendor_context"] = vendor
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
