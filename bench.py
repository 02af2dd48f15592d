"""Benchmark of the MXFP8 MoE routed-expert hot path on one MI355X.

One step = one training pass of the routed-expert grouped GEMMs over one
batch of routed tokens, Llama4-Scout-shaped (E=16 experts, 16384 tokens
routed top-1 by a uniform multinomial, K=5120, N=8192, groups padded with
zero rows to multiples of 32):
    weights  W -> both MX orientations in one pass (mx_quantize_weights)
    forward  out = A @ W[e]^T      (A -> both orientations in one pass, grouped
                                    GEMM on the rowwise one)
    dgrad    dA  = dOut @ W[e]     (dOut -> both orientations in one pass,
                                    GEMM on W's colwise orientation)
    wgrad    dW  = dOut^T @ A      (GEMM on the token-blocked orientations of
                                    dOut and A quantized above)
as the differentiable primitive composes it, so the quantize kernels, the
tile scheduler, the GEMM main loop and the bf16 epilogue all run in the step.
The tokens arrive grouped by expert (the grouping is outside this step).

Printed: one JSON line.  `value` = algorithmic GEMM TFLOP/s of the whole
step, 3 GEMMs x 2*T*N*K on the T real tokens (quantization included).
Also measured in the same run and reported beside it:
  - the same step with the weights' MX codes cached (the weights change once
    per optimizer step), amortized over 4 micro-batches, routed from token
    order on the device (mx_route + gathered quantization + row-mapped
    epilogue), and through the three all-bf16 entry points;
  - GEMM-only TFLOP/s per op on prequantized operands, on the real tokens
    and on the padded rows, for the Llama4, debug-shard and DeepSeek-style
    workloads (each timed launch preceded by an untimed 1 GiB write that
    evicts the caches);
  - quantize GB/s per kernel on the [65600, 5120] sweep tensor and on the
    Llama4 weights;
  - the roofline of the dominant kernel (the forward GEMM launch inside the
    timed steps, HIP events on the stream it runs on) and the CPU oracle on a
    bounded sample;
  - the SHA-256 of every input, the host CPU model and core count.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
       python bench.py --summarize-trace <rocprofv3 kernel_trace.csv>
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MXFP8_TFLOPS = 5000.0      # MI355X dense MXFP8 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
GEMM_KERNEL = "mxk::grouped_gemm_kernel<0, false>"
GEMM_SOURCE = os.path.join(ROOT, "mxfp8_block_scaled_06_amd", "csrc", "mx_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fwd_llama4_traffic.json")
WARMUP_LAUNCHES = 5          # untimed launches before each per-kernel figure
FLUSH_BYTES = 1 << 30
MICRO_BATCHES = 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--reps", type=int, default=20, help="timed launches per GEMM-only / quantize figure")
    p.add_argument("--quick", action="store_true",
                   help="only the timed Llama4 step and the roofline of its forward GEMM launches (no GEMM-only "
                        "figures, step variants, quantize sweep, other workloads or CPU leg): the launches a "
                        "rocprofv3 trace of this mode sees are exactly the step's")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--vendor", action="store_true",
                   help="also time hipBLASLt's GEMMs (through torch) and this library's GEMM on one dense "
                        "GEMM of the forward's FLOPs (M=16384, N=8192, K=5120): a same-run vendor reference")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration for rocprofv3 --pmc)")
    p.add_argument("--summarize-trace", metavar="CSV",
                   help="print a per-kernel, per-grid table of a rocprofv3 kernel_trace.csv and exit")
    return p.parse_args()


# ---------------------------------------------------------------------------
# rocprofv3 kernel-trace summary (no GPU needed)
# ---------------------------------------------------------------------------
def _short_kernel(name: str) -> str:
    """Kernel name without its return type and argument list (templates kept)."""
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            name = name[:i]
            break
    return name if len(name) <= 90 else name[:87] + "..."


def summarize_trace(path):
    """Markdown table of a rocprofv3 CSV, one row per kernel and grid size
    (one launch shape per row).  A --kernel-trace CSV gives calls and
    average / min / max duration in microseconds; a --pmc counter_collection
    CSV gives dispatches and the average per-dispatch value of each counter."""
    import csv
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    if rows and "Counter_Name" in rows[0]:
        groups, counters = {}, []
        for r in rows:
            key = (_short_kernel(r["Kernel_Name"]), r["Grid_Size"], r["Workgroup_Size"])
            g = groups.setdefault(key, {})
            c = r["Counter_Name"]
            if c not in counters:
                counters.append(c)
            g.setdefault(c, {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
        print("| kernel | grid (work-items) | workgroup | dispatches | " +
              " | ".join(f"avg {c}" for c in counters) + " |")
        print("|---|---|---|---|" + "---|" * len(counters))
        for (name, grid, wg), g in sorted(groups.items(), key=lambda kv: kv[0]):
            n = max(len(v) for v in g.values())
            vals = " | ".join(f"{sum(g[c].values()) / len(g[c]):.6g}" if c in g else "" for c in counters)
            print(f"| `{name}` | {grid} | {wg} | {n} | {vals} |")
        return
    groups = {}
    for r in rows:
        grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
        wg = "x".join(r.get(k, "?") for k in ("Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        groups.setdefault((_short_kernel(r["Kernel_Name"]), grid, wg), []).append(dur)
    print("| kernel | grid (work-items) | workgroup | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid, wg), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {grid} | {wg} | {len(ds)} | {sum(ds) / len(ds):.1f} | {min(ds):.1f} | "
              f"{max(ds):.1f} |")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def dev_bf16(torch, bits, dev):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def sha256(a) -> str:
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def host_info():
    model = platform.processor() or "?"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"cpu_model": model, "cores_available": cores, "python": platform.python_version()}


class Timer:
    """Per-launch durations with HIP events on the current stream.  With
    flush=True every timed launch is preceded by an untimed 1 GiB write that
    evicts the L2s and the Infinity Cache, so each launch starts from HBM;
    step-level figures run back to back like the timed step."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def flush(self):
        self.flush_buf.fill_(1)

    def time(self, fn, reps, flush=True):
        torch = self.torch
        ts = []
        for _ in range(reps):
            if flush:
                self.flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return self._stats(ts)

    def time_pair(self, fa, fb, reps, flush=False):
        """Two functions timed in alternating reps, so both see the same clock
        and cache state (a variant against its baseline)."""
        ta = self.time(fa, 1, flush)["all_ms"]
        tb = self.time(fb, 1, flush)["all_ms"]
        for _ in range(reps - 1):
            ta += self.time(fa, 1, flush)["all_ms"]
            tb += self.time(fb, 1, flush)["all_ms"]
        return self._stats(ta), self._stats(tb)

    @staticmethod
    def _stats(ts):
        ts = sorted(ts)
        return {"mean_ms": sum(ts) / len(ts), "median_ms": ts[len(ts) // 2], "min_ms": ts[0], "max_ms": ts[-1],
                "all_ms": ts}


def traffic_for_current_kernel():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    if the GEMM source changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
        if rec.get("gemm_source_sha256") != src:
            return None
        return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def gemm_entry(t, flops_real, flops_rows):
    return {"ms": t["median_ms"], "mean_ms": t["mean_ms"], "min_ms": t["min_ms"], "max_ms": t["max_ms"],
            "tflops_real_tokens": flops_real / (t["median_ms"] * 1e-3) / 1e12,
            "tflops_rows": flops_rows / (t["median_ms"] * 1e-3) / 1e12,
            "frac_of_peak_real_tokens": flops_real / (t["median_ms"] * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS,
            "frac_of_peak_rows": flops_rows / (t["median_ms"] * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS,
            "flops_per_launch_real_tokens": flops_real, "flops_per_launch_rows": flops_rows}


def gemm_only(torch, mx, timer, x, dev, reps, ops, tag):
    """GEMM-only timings on prequantized operands of one workload: weights in
    both orientations, activations and grads both ways (token axis padded to
    a multiple of 128 for the wgrad contraction)."""
    E, N, K = x.W.shape
    M = x.M_rows
    T = int(x.counts.sum())
    Mq = (M + 127) // 128 * 128
    W = dev_bf16(torch, x.W, dev)
    qW, sW, qWt, sWt = mx.mx_quantize_weights(W)
    del W
    A = dev_bf16(torch, x.A, dev)
    qA, sA, qAt, sAt = mx.mx_quantize_dual(A, Mq)
    del A
    qG = sG = qGt = sGt = None
    if x.dOut is not None:
        G = dev_bf16(torch, x.dOut, dev)
        qG, sG, qGt, sGt = mx.mx_quantize_dual(G, Mq)
        del G
    offs = torch.from_numpy(x.offs).to(dev)
    fns = {"fwd": lambda: mx.mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0),
           "dgrad": lambda: mx.mx_grouped_gemm_mx(qG, sG, qWt, sWt, offs, 0),
           "wgrad": lambda: mx.mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, offs, 1)}
    res = {"E": E, "rows": M, "tokens": T, "K": K, "N": N,
           "counts_min_max": [int(x.counts.min()), int(x.counts.max())]}
    for op in ops:
        for _ in range(WARMUP_LAUNCHES):
            fns[op]()
        torch.cuda.synchronize()
        t = timer.time(fns[op], reps)
        res[op] = gemm_entry(t, 2.0 * T * N * K, 2.0 * M * N * K)
        log(f"{tag} gemm-only {op}: {t['median_ms']:.3f} ms  "
            f"{res[op]['tflops_real_tokens']:.0f} TFLOP/s real tokens "
            f"({100 * res[op]['frac_of_peak_real_tokens']:.1f}% of peak; rows {res[op]['tflops_rows']:.0f})")
    del fns, qA, sA, qAt, sAt, qW, sW, qWt, sWt, qG, sG, qGt, sGt, offs
    torch.cuda.empty_cache()
    return res


def quant_sweep(torch, mx, timer, inp, dev, reps, W, wq):
    """Quantize GB/s per kernel: the [65600, 5120] sweep tensor in each mode and
    the one-pass dual, and the Llama4 weights in both orientations.  Bytes are
    algorithmic: 2 B read + 1 B written per element, plus the scale bytes."""
    X_bits = inp.make_sweep()
    X = dev_bf16(torch, X_bits, dev)
    R, C = X.shape
    E, N, K = W.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=dev)
    s_row = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
    qt = torch.empty((C, R), dtype=torch.uint8, device=dev)
    s_col = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
    s_sq = torch.empty((R // 32, C // 32), dtype=torch.uint8, device=dev)
    Rq = (R + 127) // 128 * 128
    dq = (q, torch.empty((C // 128, R, 4), dtype=torch.uint8, device=dev),
          torch.empty((C, Rq), dtype=torch.uint8, device=dev),
          torch.empty((Rq // 128, C, 4), dtype=torch.uint8, device=dev))
    res = {}
    for name, kernel, fn, nbytes in (
            ("weights_both_orientations_16x8192x5120", "mxk::quant_dual256_kernel<true>",
             lambda: mx.mx_quantize_weights(W, *wq), E * N * K * 4 + 2 * E * N * K // 32),
            ("rowwise_65600x5120", "mxk::quant_rowwise_kernel",
             lambda: mx.mx_quantize_rowwise(X, q, s_row), 3 * R * C + R * C // 32),
            ("colwise_65600x5120", "mxk::quant_dual256_kernel<false>",
             lambda: mx.mx_quantize_colwise(X, qt, s_col), 3 * R * C + R * C // 32),
            ("32x32_65600x5120", "mxk::quant_32x32_kernel",
             lambda: mx.mx_quantize_32x32(X, q, s_sq), 3 * R * C + R * C // 1024),
            ("dual_rowwise_and_colwise_65600x5120", "mxk::quant_dual256_kernel<true>",
             lambda: mx.mx_quantize_dual(X, Rq, *dq), 4 * R * C + 2 * R * C // 32)):
        for _ in range(WARMUP_LAUNCHES):
            fn()
        torch.cuda.synchronize()
        t = timer.time(fn, reps)
        gbs = nbytes / (t["median_ms"] * 1e-3) / 1e9
        res[name] = {"kernel": kernel, "ms": t["median_ms"], "min_ms": t["min_ms"], "max_ms": t["max_ms"],
                     "GB_s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "bytes": nbytes}
        log(f"quant {name}: {t['median_ms']:.3f} ms  {gbs:.0f} GB/s  {100 * gbs / PEAK_HBM_GBS:.1f}%")
    digest = sha256(X_bits)
    del X, X_bits, q, s_row, qt, s_col, s_sq, dq
    torch.cuda.empty_cache()
    return res, digest


def vendor_reference(torch, mx, timer, dev, reps):
    """hipBLASLt (bf16 matmul, per-tensor-scaled FP8 and MXFP8 `torch._scaled_mm`)
    and this library's MX GEMM (one expert, unit scales) on the same dense
    GEMM: 16384 x 8192 x 5120, the forward's FLOPs as one matrix product.
    Context for the roofline fraction; nothing here is on the library's path."""
    M, N, K = 16384, 8192, 5120
    flops = 2.0 * M * N * K
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    a16 = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
    w16 = torch.randn((N, K), device=dev, generator=gen).to(torch.bfloat16)
    a8, w8 = a16.to(torch.float8_e4m3fn), w16.to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    unit = lambda r: torch.full((r, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
    sa, sb = unit(M), unit(N)
    X, Y = a8.view(torch.uint8), w8.view(torch.uint8).view(1, N, K)
    sX = torch.full((K // 128, M, 4), 127, dtype=torch.uint8, device=dev)
    sY = torch.full((1, K // 128, N, 4), 127, dtype=torch.uint8, device=dev)
    offs = torch.tensor([M], dtype=torch.int32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    cases = (
        ("hipblaslt_bf16", lambda: torch.matmul(a16, w16.t()), 2500.0),
        ("hipblaslt_fp8_per_tensor_scale",
         lambda: torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 5000.0),
        ("hipblaslt_mxfp8", lambda: torch._scaled_mm(a8, w8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16),
         5000.0),
        ("mxmoe_mxfp8_one_expert", lambda: mx.mx_grouped_gemm_mx(X, sX, Y, sY, offs, 0, out=c), 5000.0),
    )
    res = {"shape_MNK": [M, N, K]}
    for name, fn, peak in cases:
        try:
            fn()
            torch.cuda.synchronize()
            t = timer.time(fn, reps)
            tf = flops / (t["median_ms"] * 1e-3) / 1e12
            res[name] = {"ms": t["median_ms"], "tflops": tf, "frac_of_peak": tf / peak, "peak_tflops": peak}
            log(f"vendor reference {name}: {t['median_ms']:.3f} ms  {tf:.0f} TFLOP/s  {100 * tf / peak:.1f}%")
        except Exception as ex:   # an op this torch build lacks is reported, not fatal
            res[name] = {"error": f"{type(ex).__name__}: {str(ex)[:200]}"}
            log(f"vendor reference {name}: {res[name]['error']}")
    return res


def cpu_baseline(x, experts=8, rows_per_expert=128):
    """The oracle, as it stands, on a bounded sample of the forward: for
    `experts` experts, quantize the expert's weights and multiply
    `rows_per_expert` of its tokens in fp64 (numpy BLAS on every core)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    bounds = oracle.group_bounds(x.offs, x.M_rows)
    order = np.argsort([-(b - a) for a, b in bounds])[:experts]
    flops = 0.0
    t0 = time.perf_counter()
    for e in order:
        a, b = bounds[int(e)]
        rows = np.arange(a, min(b, a + rows_per_expert))
        qW, sW = oracle.quantize_rowwise(x.W[int(e)])
        qA, sA = oracle.quantize_rowwise(x.A[rows])
        out = oracle.dequant_rowwise(qA, sA) @ oracle.dequant_rowwise(qW, sW).T
        flops += 2.0 * len(rows) * x.W.shape[1] * x.W.shape[2]
        assert out.shape == (len(rows), x.W.shape[1])
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"forward of {rows_per_expert} tokens for each of {len(order)} experts, including "
                      f"quantizing those experts' [{x.W.shape[1]}, {x.W.shape[2]}] weights (fp64 numpy); "
                      f"{dt:.1f} s",
            "seconds": dt}


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path runs on a single MI355X "
              f"and multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp8_block_scaled_06_amd as mx
    from mxfp8_block_scaled_06_amd import inputs as inp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mx.load_library()
    dev = torch.device("cuda:0")
    timer = Timer(torch, dev)

    # ---------------- inputs (resident in HBM before timing) ----------------
    t0 = time.perf_counter()
    x = inp.make_inputs("llama4_bwd", with_grad=True)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s: M_pad={x.M_rows} real={int(x.counts.sum())}")
    digests = {"llama4_A": sha256(x.A), "llama4_W": sha256(x.W), "llama4_dOut": sha256(x.dOut),
               "llama4_offs": sha256(x.offs)}
    E, N, K = x.W.shape
    M = x.M_rows
    T = int(x.counts.sum())
    A = dev_bf16(torch, x.A, dev)
    W = dev_bf16(torch, x.W, dev)
    G = dev_bf16(torch, x.dOut, dev)
    offs = torch.from_numpy(x.offs).to(dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    wq = (torch.empty((E, N, K), dtype=torch.uint8, device=dev),
          torch.empty((E, K // 128, N, 4), dtype=torch.uint8, device=dev),
          torch.empty((E, K, N), dtype=torch.uint8, device=dev),
          torch.empty((E, N // 128, K, 4), dtype=torch.uint8, device=dev))
    # activations in both orientations; the token axis of the transposed
    # orientation is padded to a multiple of 128 (the wgrad contraction)
    Mq = (M + 127) // 128 * 128

    def dual_bufs(rows, cols, ldq):
        return (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=dev),
                torch.empty((cols, ldq), dtype=torch.uint8, device=dev),
                torch.empty((ldq // 128, cols, 4), dtype=torch.uint8, device=dev))
    aq, gq = dual_bufs(M, K, Mq), dual_bufs(M, N, Mq)

    def mark(ev, i):
        if ev is not None:
            ev[i].record()

    def activations_and_gemms(ev=None):
        qW, sW, qWt, sWt = wq
        qA, sA, qAt, sAt = mx.mx_quantize_dual(A, Mq, *aq)
        mark(ev, 2)
        mx.mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0, out=out)
        mark(ev, 3)
        qG, sG, qGt, sGt = mx.mx_quantize_dual(G, Mq, *gq)
        mark(ev, 4)
        mx.mx_grouped_gemm_mx(qG, sG, qWt, sWt, offs, 0, out=dA)
        mark(ev, 5)
        mx.mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, offs, 1, out=dW)
        mark(ev, 6)

    def step(ev=None):
        mark(ev, 0)
        mx.mx_quantize_weights(W, *wq)
        mark(ev, 1)
        activations_and_gemms(ev)

    # ---------------- the timed step ----------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    names = ("quantize_weights", "quantize_A", "gemm_fwd", "quantize_dOut", "gemm_dgrad", "gemm_wgrad")
    step_breakdown = {}
    for i, n in enumerate(names):
        v = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        step_breakdown[n] = {"median_ms": v[len(v) // 2], "mean_ms": sum(v) / len(v)}
    flops_step_real = 3 * 2.0 * T * N * K
    flops_step_rows = 3 * 2.0 * M * N * K
    value = flops_step_real / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms  {value:.0f} TFLOP/s on real tokens; wall {wall:.2f}s for {args.steps} steps")

    # roofline of the dominant kernel: the forward GEMM launch of the timed
    # steps (HIP events recorded on the stream the library launches on)
    fwd_launch = [e[2].elapsed_time(e[3]) for e in evs]
    fwd_ms = sum(fwd_launch) / len(fwd_launch)
    flops_fwd_real, flops_fwd_rows = 2.0 * T * N * K, 2.0 * M * N * K
    achieved = flops_fwd_real / (fwd_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MXFP8_TFLOPS, "traffic": traffic_for_current_kernel(),
                "kernel": GEMM_KERNEL + " (forward launch of the timed steps)",
                "flops_per_launch": flops_fwd_real, "flops_per_launch_padded_rows": flops_fwd_rows,
                "achieved_on_padded_rows": flops_fwd_rows / (fwd_ms * 1e-3) / 1e12,
                "avg_launch_ms": fwd_ms, "launches": len(fwd_launch)}
    log(f"roofline: forward GEMM {fwd_ms:.3f} ms avg over {len(fwd_launch)} launches, {achieved:.0f} TFLOP/s "
        f"({100 * roofline['frac']:.1f}% of peak)")

    gemm = others = variants = quant = None
    if not args.quick:
        # ---------------- GEMM only, prequantized operands ----------------
        del out, dA, dW
        torch.cuda.empty_cache()
        gemm = gemm_only(torch, mx, timer, x, dev, args.reps, ("fwd", "dgrad", "wgrad"), "llama4_bwd")
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dW = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
        variants = {}
        mx.mx_quantize_weights(W, *wq)

        # weights cached: one step without the weight quantization
        def cached():
            activations_and_gemms()
        cached()
        torch.cuda.synchronize()
        t = timer.time(cached, max(3, args.steps // 2), flush=False)
        variants["weights_cached"] = {"ms": t["median_ms"],
                                      "tflops_real_tokens": flops_step_real / (t["median_ms"] * 1e-3) / 1e12}

        # micro-batches of one optimizer step: one weight quantization, then
        # MICRO_BATCHES x (fwd, dgrad, wgrad)
        def microbatches():
            mx.mx_quantize_weights(W, *wq)
            for _ in range(MICRO_BATCHES):
                activations_and_gemms()
        microbatches()
        torch.cuda.synchronize()
        t = timer.time(microbatches, max(3, args.steps // 3), flush=False)
        per = t["median_ms"] / MICRO_BATCHES
        variants["micro_batch_amortized"] = {"micro_batches": MICRO_BATCHES, "ms_per_micro_batch": per,
                                             "tflops_real_tokens": flops_step_real / (per * 1e-3) / 1e12}

        # the same tokens in token order, routed on the device: mx_route,
        # gathered dual quantization, row-mapped epilogue (output, dx in
        # token order), wgrad over the routed grouping
        rng = np.random.default_rng(17)
        ids = inp.expert_ids(rng, x.counts)
        order = np.argsort(ids, kind="stable")          # token of each grouped real row, expert by expert
        starts = np.concatenate([[0], x.offs[:-1]]).astype(np.int64)
        grouped_row = np.empty(T, dtype=np.int64)
        k = 0
        for e in range(E):
            c = int(x.counts[e])
            grouped_row[order[k:k + c]] = starts[e] + np.arange(c)
            k += c
        x_tok = A[torch.from_numpy(grouped_row).to(dev)]
        g_tok = G[torch.from_numpy(grouped_row).to(dev)]
        ids_d = torch.from_numpy(ids).to(dev)
        cap = mx.route_capacity(T, E)
        r_offs = torch.empty(E, dtype=torch.int32, device=dev)
        r_rows = torch.empty(cap, dtype=torch.int32, device=dev)
        r_pos = torch.empty(T, dtype=torch.int32, device=dev)
        r_status = torch.empty(1, dtype=torch.int32, device=dev)
        r_ws = torch.empty(max(mx.mx_route_workspace_bytes(T, E), 4), dtype=torch.uint8, device=dev)
        ra, rg = dual_bufs(cap, K, cap), dual_bufs(cap, N, cap)
        out_t = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        dx_t = torch.empty((T, K), dtype=torch.bfloat16, device=dev)

        def routed():
            mx.mx_route(ids_d, E, cap, r_offs, r_rows, r_pos, r_status, r_ws)
            qW, sW, qWt, sWt = mx.mx_quantize_weights(W, *wq)
            qA, sA, qAt, sAt = mx.mx_quantize_dual_gather(x_tok, r_rows, 1, cap, *ra)
            mx.mx_grouped_gemm_mx_rows(qA, sA, qW, sW, r_offs, r_rows, out=out_t)
            qG, sG, qGt, sGt = mx.mx_quantize_dual_gather(g_tok, r_rows, 1, cap, *rg)
            mx.mx_grouped_gemm_mx_rows(qG, sG, qWt, sWt, r_offs, r_rows, out=dx_t)
            mx.mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, r_offs, 1, out=dW)
        routed()
        step()
        torch.cuda.synchronize()
        same = (torch.equal(out_t.view(torch.int16), out[torch.from_numpy(grouped_row).to(dev)].view(torch.int16))
                and torch.equal(dx_t.view(torch.int16), dA[torch.from_numpy(grouped_row).to(dev)].view(torch.int16)))
        assert int(r_status.item()) == 0
        # reps alternate with the grouped step, so the two see the same clock
        t, tg = timer.time_pair(routed, step, max(4, args.steps // 2), flush=False)
        variants["routed_from_token_order"] = {
            "ms": t["median_ms"], "tflops_real_tokens": flops_step_real / (t["median_ms"] * 1e-3) / 1e12,
            "grouped_step_ms_alternating": tg["median_ms"],
            "rows_capacity": cap, "outputs_bit_identical_to_grouped_step": bool(same)}
        log(f"routed step {t['median_ms']:.3f} ms against {tg['median_ms']:.3f} ms for the grouped step in "
            f"alternating reps (outputs identical to the grouped step: {same})")
        del x_tok, g_tok, ra, rg, out_t, dx_t

        # the same step through the three all-bf16 entry points (W quantized twice)
        ws_bf = {op: torch.empty(mx.mx_grouped_mm_workspace_bytes(op, M, N, K, E), dtype=torch.uint8, device=dev)
                 for op in (mx.OP_FWD, mx.OP_DGRAD, mx.OP_WGRAD)}

        def step_bf16():
            mx.mx_grouped_mm_fwd(A, W, offs, out=out, ws=ws_bf[mx.OP_FWD])
            mx.mx_grouped_mm_dgrad(G, W, offs, out=dA, ws=ws_bf[mx.OP_DGRAD])
            mx.mx_grouped_mm_wgrad(G, A, offs, out=dW, ws=ws_bf[mx.OP_WGRAD])
        step_bf16()
        torch.cuda.synchronize()
        t = timer.time(step_bf16, max(3, args.steps // 2), flush=False)
        variants["bf16_entry_points"] = {"ms": t["median_ms"],
                                         "tflops_real_tokens": flops_step_real / (t["median_ms"] * 1e-3) / 1e12}
        log(f"step variants: {json.dumps(variants)}")
        del ws_bf, out, dA, dW
        torch.cuda.empty_cache()

        # ---------------- quantize sweep ----------------
        quant, digests["sweep_65600x5120"] = quant_sweep(torch, mx, timer, inp, dev, args.reps, W, wq)
        del W, wq

        # ---------------- the other workloads, GEMM only ----------------
        import dataclasses
        others = {}
        del A, G
        torch.cuda.empty_cache()
        for name, w, ops in (
                ("debug_shard", inp.WORKLOADS["debug_shard"], ("fwd", "dgrad", "wgrad")),
                ("deepseek_share", inp.WORKLOADS["deepseek_share"], ("fwd",)),
                ("deepseek_share_pad32", dataclasses.replace(inp.WORKLOADS["deepseek_share"], pad32=True),
                 ("dgrad", "wgrad"))):
            t0 = time.perf_counter()
            xo = inp.make_inputs(w, with_grad=any(o != "fwd" for o in ops))
            log(f"{name}: inputs in {time.perf_counter() - t0:.1f}s")
            digests[f"{name}_A"] = sha256(xo.A)
            digests[f"{name}_W"] = sha256(xo.W)
            if xo.dOut is not None:
                digests[f"{name}_dOut"] = sha256(xo.dOut)
            others[name] = gemm_only(torch, mx, timer, xo, dev, args.reps, ops, name)
            del xo

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    vendor = None
    if args.vendor:
        vendor = vendor_reference(torch, mx, timer, dev, args.reps)
        torch.cuda.empty_cache()

    # ---------------- CPU oracle leg ----------------
    cpu = None
    if not (args.no_cpu or args.quick):
        cpu = cpu_baseline(x)
        log(f"cpu oracle: {cpu['value']:.5f} TFLOP/s on {cpu['cores']} threads ({cpu['sample']})")
        cpu.pop("seconds", None)

    rec = {
        "metric": "MXFP8 grouped-GEMM TFLOP/s (fwd/dgrad/wgrad) and % of MX-FP8 peak; quant GB/s",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3/e8m0 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded N(0,1) activations with 0.1% x50 outliers, N(0,0.02) weights, "
                "N(0,1e-3) grads)",
        "config": {"workload": "Llama4-Scout-shaped routed experts, fwd + dgrad + wgrad: E=16, "
                               f"{T} tokens (uniform top-1 routing, groups padded to 32 -> {M} rows), "
                               "K=5120, N=8192",
                   "E": E, "tokens": T, "rows_padded": M, "K": K, "N": N},
        "frac_of_peak": value / PEAK_MXFP8_TFLOPS,
        "step_tflops_on_padded_rows": flops_step_rows / (ms_per_step * 1e-3) / 1e12,
        "step_breakdown": step_breakdown,
        "step_variants": variants,
        "gemm_only": gemm,
        "gemm_only_other_workloads": others,
        "quant": quant,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "vendor_reference": vendor,
        "timing": "step and step variants: HIP events around back-to-back steps (caches as the previous step "
                  f"leaves them); GEMM-only and quantize figures: {WARMUP_LAUNCHES} untimed launches, then the median "
                  f"of {args.reps} per-launch HIP events, each launch after an untimed 1 GiB write",
        "inputs_sha256": digests,
        "host": host_info(),
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "library": mx.version(),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
