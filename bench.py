"""Benchmark of the fused pairwise-score consumers on one MI355X.

A step is one full pass of the hot path over one synthetic workload: the
consumer call(s) of that workload (epilogue pre-pass, tile kernel, split
merge), with inputs, outputs and workspace already resident in HBM.

Headline (the JSON line's value): k-NN retrieval, 65536 queries against
2^20 references, D = 32, float32, top-10 smallest squared distances (the
k-NN row of the torchpairwise guide's Task Map), the largest configuration
that fits one GPU. The same run times every other fused consumer at its
full size -- softmax attention, the InfoNCE log-sum-exp, the SVGD kernel
product and displacement (float64) and the narrow rbf kernel product -- and
reports each in roofline.kernels with its own oracle sample and parity.

Prints ONE JSON line: pair evaluations per second (Gpairs/s), the roofline
of the dominant kernel, the CPU oracle timed on bounded row samples on the
host cores, and the parity of the timed outputs on those samples.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--also NAME,NAME,...] [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import workloads  # noqa: E402

# Algorithmic flops per pair (FMA = 2; add, mul, max, compare = 1; exp = 1;
# row norms precomputed; distances through |x|^2 + |y|^2 - 2 x.y).
PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6}
# Kernels with no contraction run on the vector ALU. On gfx950 a plain
# (unpacked) v_fma_f32 issues every 2 cycles per wave64 (measured), so the
# fp32 vector FMA peak is 256 CUs x 4 SIMDs x 32 lanes x 2 flop x 2.4 GHz =
# 157.3 TFLOP/s; fp64 vector FMA runs 16 lanes per cycle: 78.6 TFLOP/s.
ALU_PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_digest():
    """Digest of the HIP/C++ sources of libpw and of its build script (the
    compiler flags); a counter reading taken on other sources or flags no
    longer describes the kernel."""
    h = hashlib.sha1()
    files = glob.glob(os.path.join(ROOT, "lazy_score_matrix_amd", "csrc", "*"))
    files.append(os.path.join(ROOT, "lazy_score_matrix_amd", "build.py"))
    for f in sorted(files):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summary, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(workload)
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def flops_per_pair(case, D, C):
    body = 0
    if case.metric == "linear":
        body = 2 * D
    else:
        body = 2 * D + 2
        if case.metric == "rbf":
            body += 2  # scale and exp
    body += sum(1 for _ in case.ops)
    if case.consumer == "matmul":
        return body + 2 * C
    if case.consumer == "displacement":
        return body + 2 * (D + 1)
    if case.consumer == "logsumexp":
        return body + 4
    if case.consumer == "softmax_matmul":
        return body + 4 + 2 * C
    if case.consumer == "topk":
        return body + 1
    if case.consumer == "mean":
        return body + 1 + 2  # the 1/M scale, then a product with a ones column
    if case.consumer == "cg_solve":
        return body + 2 * C  # one kernel product per iteration
    if case.consumer == "mmd":
        return body + 2  # each of its products sums the scores against a ones column
    if case.consumer == "backward_softmax_matmul":
        # Both sides replay the pair: metric and ops, the upstream dot
        # product (2C) and exp, the gradient sums (2D); the column side
        # also sums dV (2C).
        return 2 * (body + 2 * C + 4) + 4 * D + 2 * C
    raise ValueError(case.consumer)


SWAP = {"add_rows": "add_columns", "add_columns": "add_rows", "weight_rows": "weight_columns",
        "weight_columns": "weight_rows"}


def lib_consumer(c):
    """The tile-kernel consumer behind a case (a mean is a product with
    ones; a CG solve runs one product per iteration; a backward is planned
    as its forward consumer)."""
    if c.consumer.startswith("backward_"):
        return c.consumer[len("backward_"):]
    return "matmul" if c.consumer in ("mean", "cg_solve", "mmd") else c.consumer


def case_operands(c, arrays):
    """(X, Y, ops) of a case; a transposed case reduces over the rows, so it
    binds (Y, X) with row and column ops swapped."""
    X, Y = arrays[c.x], arrays[c.y]
    ops = [(n, workloads.resolve(a, arrays)) for n, a in c.ops]
    if c.transpose:
        X, Y = Y, X
        ops = [(SWAP.get(n, n), a) for n, a in ops]
    if c.consumer == "mean":
        ops = ops + [("mul", 1.0 / Y.shape[0])]
    return X, Y, ops


# Workloads timed beside the headline by default: every fused consumer at
# its full size (attention softmax@V, InfoNCE log-sum-exp, the SVGD product
# and displacement in float64, the narrow rbf kernel product).
DEFAULT_ALSO = ("attention", "infonce", "svgd", "rbf_large")


def build_calls(name, dev):
    """Bind every call of a workload on the device, with its outputs and
    workspace allocated. Returns (arrays, calls, pairs_per_step,
    solve_infos); calls are (case, expr, fn, outputs, C)."""
    import torch
    import lazy_score_matrix_amd as pw

    arrays, cases = workloads.make(name)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in arrays.items()}
    calls = []
    pairs_per_step = 0
    solve_infos = []
    for c in cases:
        X, Y, ops = case_operands(c, t)
        e = pw.lazy(X, Y, c.metric, gamma=c.gamma, ops=ops)
        N, D = X.shape
        M = Y.shape[0]
        C = t[c.v].shape[1] if c.v else (1 if c.consumer in ("mean", "mmd") else 0)
        if c.consumer == "backward_softmax_matmul":
            # One step is the backward given dO and the forward output (the
            # forward itself runs once, before the timed region).
            V = t[c.v]
            C = V.shape[1]
            lse = torch.empty(N, dtype=X.dtype, device=dev)
            O = e.softmax_matmul(V, lse=lse)  # the forward keeps its row statistics
            G = t[c.params["G"]]
            grads = {"X": torch.empty(N, D, dtype=X.dtype, device=dev), "Y": torch.empty(M, D, dtype=X.dtype, device=dev),
                     "V": torch.empty(M, C, dtype=X.dtype, device=dev)}
            ws = e.backward_workspace("softmax_matmul", C)
            fn = (lambda e=e, G=G, V=V, O=O, grads=grads, ws=ws, lse=lse:
                  e.backward("softmax_matmul", G, V=V, out=O, grads=grads, workspace=ws, lse=lse))
            outs = (grads["X"], grads["Y"], grads["V"])
        elif c.consumer == "cg_solve":
            # One step is one whole solve; its pairs are iterations * N * M,
            # counted from the solver's own iteration count.
            B = t[c.v]
            C = B.shape[1]
            A = torch.empty(N, C, dtype=X.dtype, device=dev)
            n = ctypes.c_size_t()
            pw.check(e._lib.pw_cg_workspace_size(e._h, C, ctypes.byref(n)))
            ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
            solve_infos.append([])
            fn = (lambda e=e, B=B, A=A, ws=ws, p=c.params, log=solve_infos[-1]:
                  log.append(e.solve(B, p["shift"], rtol=p["rtol"], max_iter=p["max_iter"], out=A,
                                     workspace=ws)[1]))
            outs = (A,)
        elif c.consumer == "mmd":
            # One step is the whole statistic (pw_mmd2: three products with
            # ones and the finishing kernel). Its tile events keep the last
            # product's launch: the cross-cloud one, N * M pairs.
            lib = pw.load_library()
            dt, mt = pw.DTYPES[X.dtype], pw.METRICS[c.metric]
            n_ws = ctypes.c_size_t()
            pw.check(lib.pw_mmd2_workspace_size(dt, mt, c.gamma, N, M, D, 1, ctypes.byref(n_ws)))
            ws = torch.empty(n_ws.value, dtype=torch.uint8, device=dev)
            out = torch.empty(1, dtype=X.dtype, device=dev)
            unb = int(c.params.get("unbiased", True))
            fn = (lambda X=X, Y=Y, out=out, ws=ws, dt=dt, mt=mt, g=c.gamma, unb=unb, N=N, M=M, D=D, lib=lib:
                  pw.check(lib.pw_mmd2(dt, mt, g, X.data_ptr(), N, D, 0, Y.data_ptr(), M, D, 0, D, 1, unb,
                                       out.data_ptr(), ws.data_ptr(), ws.numel(), pw._stream(X.device)), "pw_mmd2"))
            outs = (out,)
        elif c.consumer == "mean":
            # The row mean: the scores scaled by 1/M (an extra op bound
            # above) times a ones column, as LazyScores.mean computes it.
            ones = torch.ones(M, 1, dtype=X.dtype, device=dev)
            out = torch.empty(N, 1, dtype=X.dtype, device=dev)
            ws = e.workspace("matmul", 1)
            fn = (lambda e=e, V=ones, out=out, ws=ws: e.matmul(V, out=out, workspace=ws))
            outs = (out,)
        elif c.consumer in ("matmul", "softmax_matmul"):
            out = torch.empty(N, C, dtype=X.dtype, device=dev)
            ws = e.workspace(c.consumer, C)
            V = t[c.v]
            fn = (lambda e=e, V=V, out=out, ws=ws, m=c.consumer: getattr(e, m)(V, out=out, workspace=ws))
            outs = (out,)
        elif c.consumer == "displacement":
            out = torch.empty(N, D, dtype=X.dtype, device=dev)
            ws = e.workspace("displacement")
            fn = (lambda e=e, out=out, ws=ws: e.displacement(out=out, workspace=ws))
            outs = (out,)
        elif c.consumer == "logsumexp":
            out = torch.empty(N, dtype=X.dtype, device=dev)
            ws = e.workspace("logsumexp")
            fn = (lambda e=e, out=out, ws=ws, x=c.exclude_self: e.logsumexp(x, out=out, workspace=ws))
            outs = (out,)
        else:
            vals = torch.empty(N, c.k, dtype=X.dtype, device=dev)
            idx = torch.empty(N, c.k, dtype=torch.int64, device=dev)
            ws = e.workspace("topk", 0, c.k)
            fn = (lambda e=e, vals=vals, idx=idx, ws=ws, k=c.k, lg=c.largest:
                  e.topk(k, lg, values=vals, indices=idx, workspace=ws))
            outs = (vals, idx)
        calls.append((c, e, fn, outs, C))
        if c.consumer != "cg_solve":
            pairs_per_step += c.pairs if c.pairs is not None else N * M
    return arrays, calls, pairs_per_step, solve_infos


class _Hip:
    """HIP events through the runtime's C API: the library records them on
    the stream it launches on."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed(self, a, b):
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def time_calls(calls, steps, warmup, hip, min_warmup_s=0.0):
    """W untimed steps (more, until min_warmup_s has passed, if given), then
    exactly K steps between two events on the launch stream, each bracketed
    by synchronisation. Per step and call, the library records a pair of HIP
    events around its tile-kernel launch on the same stream
    (pw_set_tile_events). Returns (ms per step, average tile-kernel ms per
    call, warm-up steps run)."""
    import torch
    import lazy_score_matrix_amd as pw

    lib = pw.load_library()
    stream = torch.cuda.current_stream()
    done = 0
    t0 = time.perf_counter()
    while done < warmup or (time.perf_counter() - t0 < min_warmup_s and done < 100000):
        for _, _, fn, _, _ in calls:
            fn()
        done += 1
        if done >= warmup and min_warmup_s > 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    kev = [[(hip.event(), hip.event()) for _ in calls] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for st in range(steps):
        for ci, (_, _, fn, _, _) in enumerate(calls):
            lib.pw_set_tile_events(kev[st][ci][0], kev[st][ci][1])
            fn()
    lib.pw_set_tile_events(None, None)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    kernel_ms = [sum(hip.elapsed(*kev[st][ci]) for st in range(steps)) / steps for ci in range(len(calls))]
    for row in kev:
        for a_, b_ in row:
            hip.destroy(a_)
            hip.destroy(b_)
    return ms, kernel_ms, done


def dtype_name(e):
    import torch
    return "f32" if e.dtype == torch.float32 else "f64"


def is_contraction(c, e, C):
    """Whether a call's tile kernel runs on the matrix cores."""
    if c.consumer.startswith("backward_"):
        return e.backward_plan(lib_consumer(c), C).startswith("family=mfma")
    return e.plan(lib_consumer(c), C, c.k).startswith("family=mfma")


def kernel_entries(name, calls, kernel_ms):
    """One roofline entry per call: its tile kernel's average duration,
    algorithmic flops and fraction of the peak of the unit it runs on."""
    out = []
    for (c, e, _, _, C), kms in zip(calls, kernel_ms):
        dtype = dtype_name(e)
        mfma = is_contraction(c, e, C)
        peak = PEAK_TFLOPS[dtype] if mfma else ALU_PEAK_TFLOPS[dtype]
        fpp = flops_per_pair(c, e.D, C)
        # An MMD step's timed tile kernel is its cross-cloud product.
        pairs = float(e.N * e.M if c.consumer == "mmd" or c.pairs is None else c.pairs)
        tf = pairs * fpp / (kms * 1e-3) / 1e12
        plan = (e.backward_plan(lib_consumer(c), C) if c.consumer.startswith("backward_")
                else e.plan(lib_consumer(c), C, c.k))
        out.append({"workload": name, "call": c.name, "dtype": dtype, "bound": "mfma" if mfma else "alu",
                    "plan": plan, "pairs": int(pairs), "avg_ms": round(kms, 4),
                    "gpairs_per_s": round(pairs / (kms * 1e-3) / 1e9, 3), "flops_per_pair": fpp,
                    "tflops": round(tf, 3), "peak": peak, "frac": round(tf / peak, 4)})
    return out


# The workloads timed beside the headline warm up for at least this long
# (the headline takes exactly --warmup steps): the clock settles over a few
# hundred milliseconds after a change of load (measured on the narrow rbf
# product: 0.96 ms per launch after 3 warm-up steps, 0.86 ms after 300).
ALSO_MIN_WARMUP_S = 0.3


def run_workload(name, args, dev, hip, min_warmup_s=0.0):
    """Time one workload; returns its summary, kernel entries and the state
    the oracle leg needs."""
    arrays, calls, pairs_per_step, solve_infos = build_calls(name, dev)
    ms, kernel_ms, warm = time_calls(calls, args.steps, args.warmup, hip, min_warmup_s)
    solve_summary = None
    if solve_infos:
        # Timed solves: the last args.steps entries of each solve's log.
        timed = [log[-args.steps:] for log in solve_infos]
        its = [sum(i["iterations"] for i in log) / len(log) for log in timed]
        cg_calls = [(c, e) for c, e, *_ in calls if c.consumer == "cg_solve"]
        pairs_per_step += sum(it * e.N * e.M for it, (c, e) in zip(its, cg_calls))
        solve_summary = [{"call": c.name, "iterations_per_solve": it, "info": log[-1]}
                         for it, (c, e), log in zip(its, cg_calls, timed)]
    e0 = calls[0][1]
    summary = {
        "workload": name,
        "consumers": [c.consumer for c, *_ in calls],
        "N": int(e0.N), "M": int(e0.M), "D": int(e0.D),
        "C": [C for *_, C in calls],
        "dtype": dtype_name(e0),
        "pairs_per_step": pairs_per_step,
        "warmup_steps": warm,
        "ms_per_step": round(ms, 4),
        "gpairs_per_s": round(pairs_per_step / (ms * 1e-3) / 1e9, 3),
    }
    if solve_summary:
        summary["solves"] = solve_summary
    return summary, kernel_entries(name, calls, kernel_ms), (arrays, calls)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="knn", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed beside the headline (default: every other fused "
                         "consumer at full size when the headline is knn; 'none' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="target oracle wall time per call for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.also is None:
        also = list(DEFAULT_ALSO) if args.workload == "knn" else []
    else:
        also = [w for w in args.also.split(",") if w and w != "none"]
    for w in also:
        if w not in workloads.WORKLOADS:
            ap.error("unknown workload %r in --also" % w)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = _Hip()

    names = [args.workload] + [w for w in also if w != args.workload]
    summaries, kernels, cpu_parts, parity = [], [], [], []
    for wi, name in enumerate(names):
        summary, kern, (arrays, calls) = run_workload(name, args, dev, hip, ALSO_MIN_WARMUP_S if wi else 0.0)
        summaries.append(summary)
        kernels.extend(kern)
        if not args.no_cpu:
            cpu, par = cpu_leg(name, calls, arrays, args.cpu_seconds)
            cpu_parts.append(cpu)
            parity.extend(par)
        del calls, arrays
        torch.cuda.empty_cache()

    head = summaries[0]
    head_k = [k for k in kernels if k["workload"] == head["workload"]]
    dom = max(head_k, key=lambda k: k["avg_ms"])
    roofline = {
        "bound": dom["bound"],
        "achieved": dom["tflops"],
        "peak": dom["peak"],
        "unit": "TFLOP/s",
        "frac": dom["frac"],
        "traffic": recorded_traffic(head["workload"]),
        "peak_basis": ("dense %s MFMA (equal to the vector FMA rate on gfx950)" % dom["dtype"] if dom["bound"] == "mfma"
                       else "%s vector FMA: 256 CU x 4 SIMD x %d lanes x 2 flop x 2.4 GHz"
                       % (dom["dtype"], 32 if dom["dtype"] == "f32" else 16)),
        "kernel": dom["call"],
        "kernel_avg_ms": dom["avg_ms"],
        "kernels": kernels,
    }
    config = {k: head[k] for k in ("workload", "consumers", "N", "M", "D", "C", "pairs_per_step")}
    if "solves" in head:
        config["solves"] = head["solves"]
    config["also"] = [{k: s_[k] for k in ("workload", "consumers", "N", "M", "D", "dtype", "pairs_per_step",
                                          "warmup_steps", "ms_per_step", "gpairs_per_s")} for s_ in summaries[1:]]
    result = {
        "metric": "pair evaluations/sec (Gpairs/s) per consumer + % of gfx950 FP32/FP64 peak",
        "value": head["gpairs_per_s"],
        "unit": "Gpairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
    }
    if cpu_parts:
        cb = dict(cpu_parts[0])
        cb["workloads"] = cpu_parts
        result["cpu_baseline"] = cb
        result["parity"] = parity
    print(json.dumps(result), flush=True)


def backward_cpu_leg(c, oe, arrays, outs, budget, threads):
    """The oracle's backward on sampled rows (dX) and the same number of
    sampled columns (dY, dV). Its pair count is the
    rows' and columns' pairs plus, for the softmax backward, the full pass
    over all pairs that its per-row log-sum-exp and delta take."""
    import oracle
    from gpu_cases import grad_report
    base = c.consumer[len("backward_"):]
    G = arrays[c.params["G"]]
    V = arrays[c.v] if c.v else None

    def run(rows):
        return oracle.backward(oe, base, G, V, rows=rows, cols=rows)

    # One call (its full row-statistics pass is a fixed cost): a sample of
    # 4 rows and columns per host thread.
    rows = np.unique(np.linspace(0, oe.N - 1, min(oe.N, 4 * threads)).astype(np.int64))
    t0 = time.perf_counter()
    ref = run(rows)
    dt = time.perf_counter() - t0
    kept = c.pairs if c.pairs is not None else oe.N * oe.M  # masked workloads count kept pairs
    pairs = 2 * len(rows) * kept / oe.N + (kept if base in ("softmax_matmul", "logsumexp") else 0)
    import torch
    sel = torch.as_tensor(rows, device=outs[0].device)
    dtype = np.dtype(oe.np_dtype)
    worst, ok = 0.0, True
    for g, r, terms in ((outs[0][sel], ref["dX"], oe.M), (outs[1][sel], ref["dY"], oe.N),
                        (outs[2][sel], ref["dV"], oe.N)):
        good, ratio = grad_report(g, r, dtype, terms)
        ok &= good
        worst = max(worst, ratio)
    desc = ("%s: oracle backward on %d evenly spaced rows (dX) and the same %d columns (dY, dV), plus its full "
            "per-row log-sum-exp and delta pass" % (c.name, len(rows), len(rows)))
    return pairs, dt, desc, {"call": c.name, "rows": len(rows), "pass": bool(ok), "worst_err_over_tol": worst}


def mmd_cpu_leg(c, X, Y, seconds, threads):
    """The oracle's statistic on the first s points of each cloud, s sized
    to the time budget (the statistic has no row sample), and the GPU's
    pw_mmd2 on the same sub-clouds against it."""
    import torch
    import oracle
    import lazy_score_matrix_amd as pw
    from parity import value_report

    unb = c.params.get("unbiased", True)
    s = 256
    t0 = time.perf_counter()
    oracle.mmd2(X[:s], Y[:s], c.metric, c.gamma, unb)
    tp = max(time.perf_counter() - t0, 1e-6)
    s = int(min(X.shape[0], Y.shape[0], 4096, s * max(1.0, (seconds / tp) ** 0.5)))
    t0 = time.perf_counter()
    o, mag = oracle.mmd2(X[:s], Y[:s], c.metric, c.gamma, unb)
    dt = time.perf_counter() - t0
    pairs = s * (s - 1) + s * s  # the within-cloud sums (distinct pairs) and the cross sum
    dev = torch.device("cuda:0")
    g = pw.mmd_statistics(torch.from_numpy(np.ascontiguousarray(X[:s])).to(dev),
                          torch.from_numpy(np.ascontiguousarray(Y[:s])).to(dev), c.metric, c.gamma, unb)
    ok, ratio, rel = value_report(np.atleast_1d(g.cpu().numpy()), np.atleast_1d(o), np.atleast_1d(mag),
                                  np.dtype(X.dtype), n_terms=s * s)
    desc = ("%s: the oracle's statistic on the first %d points of each cloud (its dense scores), and pw_mmd2 "
            "on the same sub-clouds checked against it" % (c.name, s))
    return pairs, dt, desc, {"call": c.name, "points": s, "pass": bool(ok), "worst_err_over_tol": ratio,
                             "max_plain_rel_err": rel}


def cpu_leg(name, calls, arrays, seconds):
    """Time the oracle on a bounded row sample of one workload on the host
    cores (about `seconds` per call), and check the timed GPU outputs
    against it on the same rows. Returns (cpu_baseline entry, parity
    entries)."""
    import oracle
    from parity import topk_report, value_report

    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    total_pairs, total_s, rows_desc, parity = 0, 0.0, [], []
    budget = seconds
    for c, e, _, outs, C in calls:
        X, Y, ops = case_operands(c, arrays)
        oe = oracle.Expr(X, Y, c.metric, gamma=c.gamma, ops=ops)
        V = arrays[c.v] if c.v else (np.ones((Y.shape[0], 1), dtype=Y.dtype) if c.consumer == "mean" else None)
        if c.consumer == "cg_solve":
            # The oracle's unit of work is the product inside every
            # iteration: timed as S @ A on the sampled rows, which is also
            # the true residual's product for the parity check.
            A_gpu = outs[0].cpu().numpy()
        if c.consumer == "mmd":
            total_pairs_m, dt_m, desc_m, par_m = mmd_cpu_leg(c, X, Y, budget, threads)
            total_pairs += total_pairs_m
            total_s += dt_m
            rows_desc.append(desc_m)
            parity.append(par_m)
            continue
        if c.consumer.startswith("backward_"):
            total_pairs_b, dt_b, desc_b, par_b = backward_cpu_leg(c, oe, arrays, outs, budget, threads)
            total_pairs += total_pairs_b
            total_s += dt_b
            rows_desc.append(desc_b)
            parity.append(par_b)
            continue

        def run(rows):
            if c.consumer in ("matmul", "mean"):
                return oracle.matmul(oe, V, rows)
            if c.consumer == "cg_solve":
                return oracle.matmul(oe, A_gpu, rows)
            if c.consumer == "softmax_matmul":
                return oracle.softmax_matmul(oe, V, rows)
            if c.consumer == "displacement":
                return oracle.displacement(oe, rows)
            if c.consumer == "logsumexp":
                return oracle.logsumexp(oe, c.exclude_self, rows)
            return oracle.topk(oe, c.k, c.largest, extra=16, rows=rows)

        # Probe on a few rows, then size the sample to the time budget.
        probe = np.arange(0, oe.N, max(1, oe.N // (4 * threads)))[: 4 * threads]
        t0 = time.perf_counter()
        run(probe)
        tp = max(time.perf_counter() - t0, 1e-6)
        n_rows = int(min(oe.N, max(len(probe), len(probe) * budget / tp)))
        rows = np.unique(np.linspace(0, oe.N - 1, n_rows).astype(np.int64))
        t0 = time.perf_counter()
        res = run(rows)
        dt = time.perf_counter() - t0
        # Masked workloads count the kept pairs (the rows' average share).
        per_row = (c.pairs / oe.N) if c.pairs is not None else oe.M
        total_pairs += len(rows) * per_row
        total_s += dt
        rows_desc.append("%s: %d of %d rows evenly spaced (incl. first and last), %s"
                         % (c.name, len(rows), oe.N, "all %d columns" % oe.M if c.pairs is None
                            else "their kept pairs (%.0f per row on average)" % per_row))
        dtype = np.dtype(oe.np_dtype)
        if c.consumer == "cg_solve":
            from gpu_cases import solve_report
            ok, ratio = solve_report(oe, A_gpu, V, c.params["shift"], c.params["rtol"], rows)
            parity.append({"call": c.name, "rows": len(rows), "pass": ok, "residual_over_bound": ratio})
        elif c.consumer == "topk":
            gv = outs[0].cpu().numpy()[rows]
            gi = outs[1].cpu().numpy()[rows]
            fails = topk_report(gv, gi, res[0], res[1], res[2], c.k, c.largest, dtype)
            parity.append({"call": c.name, "rows": len(rows), "pass": not fails, "failing_rows": len(fails)})
        else:
            g = outs[0].cpu().numpy()[rows]
            vmax = float(np.max(np.abs(V))) if V is not None else float(np.max(np.abs(oe.Y)) + np.max(np.abs(oe.X)))
            ok, ratio, rel = value_report(g, res[0], res[1], dtype, n_terms=oe.M, vmax=vmax)
            parity.append({"call": c.name, "rows": len(rows), "pass": bool(ok), "worst_err_over_tol": ratio,
                           "max_plain_rel_err": rel})
    for p_ in parity:
        p_["workload"] = name
    return {
        "workload": name,
        "value": round(total_pairs / total_s / 1e9, 6),
        "unit": "Gpairs/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "; ".join(rows_desc),
    }, parity


if __name__ == "__main__":
    main()
