"""Benchmark: RMSNorm forward + backward on one MI355X.

A step is one pass of the whole path over one batch: the forward (rmsnorm_fwd)
and both backward stages (rmsnorm_bwd_rows, rmsnorm_bwd_reduce), called
through the C ABI on torch's current stream with inputs already in HBM.

Workload: bf16, M = 32768 rows (8 sequences x 4096 tokens) x N = 4096 hidden,
eps = 1e-6; x ~ N(0,1), gamma ~ U(0.5,1.5), dy ~ N(0,1e-2), seed 0.

Printed: one JSON line.  ``value`` = algorithmic bytes of forward + backward
per step / measured step time, in GB/s.  Algorithmic bytes (s = 2 bytes):
forward 2*M*N*s + N*s + 4*M, backward 3*M*N*s + N*s + 4*M + 4*N (the dgamma
partial-sum workspace is not counted).  ``roofline`` describes the dominant
kernel, backward stage 1, timed with events on its launch stream inside the
timed steps.  A cold-cache figure (each call preceded by a 1 GiB read that
evicts L2 and the 256 MB Infinity Cache) is reported beside it, a 1 GiB
device copy as an achievable-bandwidth reference, and the CPU oracle's
throughput on the same workload as ``cpu_baseline`` (the float64 golden on
one thread, with the float32 torch CPU reference timed beside it).

Three timing scopes are reported.  ``value`` comes from the K timed steps,
back to back on one set of buffers (W untimed steps first).  ``cold_cache``
is the per-call protocol: 50 samples per pass, each call preceded by an
untimed 1 GiB read that evicts L2 and the Infinity Cache, median reported
(with p10/p90).  ``rotating_warm`` times back-to-back steps that cycle over
three independent buffer sets, so no step finds its inputs in the 256 MB
Infinity Cache from the step before.  The cold-cache and rotating legs run
before the warmup, so the timed steps start on a GPU that is already busy.

``--op layernorm`` measures the LayerNorm path of the same library instead
(layernorm_fwd, layernorm_bwd_rows, layernorm_bwd_reduce) on the LayerNorm
inputs of the workload (the same x, gamma and dy draws plus a bias and
per-row mean shifts).  Algorithmic bytes: forward 2*M*N*s + 2*N*s + 8*M
(x, gamma, beta read; y, mean, rstd written), backward stage 1
3*M*N*s + N*s + 8*M, stage 2 8*N (dgamma and dbeta).

``--op add_rmsnorm`` measures the residual add fused with RMSNorm
(rmsnorm_add_fwd, rmsnorm_add_bwd_rows, rmsnorm_add_bwd_reduce): forward
4*M*N*s + N*s + 4*M (x and res read, y and h written), backward stage 1
4*M*N*s + N*s + 4*M (dy, dh and h read, dx written), stage 2 4*N.  The
same step unfused (torch's add, rmsnorm_fwd, rmsnorm_bwd, torch's add of
dh) is timed beside it as ``unfused_step_us``.

``--op rmsnorm_cast`` measures RMSNorm with its output cast to a narrower
dtype (rmsnorm_cast_fwd, rmsnorm_cast_bwd_rows, rmsnorm_cast_bwd_reduce) on
the workload's draws with float32 x and gamma and y, dy in the workload's
16-bit dtype: forward 6*M*N + 4*N + 4*M (x read, y written), backward
stage 1 10*M*N + 4*N + 4*M (dy and x read, dx written in float32), stage 2
4*N.  The unfused step (float32 rmsnorm_fwd, torch's cast of y, torch's
widening of dy, float32 rmsnorm_bwd) is timed beside it.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0
TRAFFIC_NOTE = os.path.join(ROOT, "profiles", "bwd_rows_c2_bf16_32768x4096_hbm_traffic.md")


def kernel_source_hash():
    """sha256 over the library's kernel and host sources (sorted by name)."""
    csrc = os.path.join(ROOT, "backward_rmsnorm_fwd_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per backward-stage-1 launch from the committed counter
    summary, or None when it covers another workload or the kernels changed
    since the counters were taken."""
    if workload != "c2" or not os.path.exists(TRAFFIC_NOTE):
        return None
    fields = {}
    with open(TRAFFIC_NOTE) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("|", "#", " ")):
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def alg_bytes(M, N, s, op="rmsnorm"):
    if op == "rmsnorm_cast":  # float32 x, gamma, dx; 16-bit y and dy
        return 6 * M * N + 4 * N + 4 * M, 10 * M * N + 4 * N + 4 * M, 4 * N
    if op == "add_rmsnorm":
        return 4 * M * N * s + N * s + 4 * M, 4 * M * N * s + N * s + 4 * M, 4 * N
    if op == "layernorm":
        return 2 * M * N * s + 2 * N * s + 8 * M, 3 * M * N * s + N * s + 8 * M, 8 * N
    fwd = 2 * M * N * s + N * s + 4 * M
    bwd_rows = 3 * M * N * s + N * s + 4 * M
    bwd_reduce = 4 * N
    return fwd, bwd_rows, bwd_reduce


OP_NAMES = {"rmsnorm": "RMSNorm", "layernorm": "LayerNorm",
            "add_rmsnorm": "residual add + RMSNorm", "rmsnorm_cast": "RMSNorm + output cast"}
DTYPE_NAMES = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


def metric_label(op, dtype, M, N):
    """The metric named after the op and the workload's own dtype and shape."""
    return (f"{OP_NAMES[op]} fwd/bwd achieved HBM GB/s and % of peak, "
            f"{DTYPE_NAMES[dtype]} M={M} N={N}")


def metric_for(op, workload):
    """The metric line of ``--op op --workload workload``: the cast path reads
    float32 x, the others the workload's own dtype."""
    from backward_rmsnorm_fwd_amd import workloads
    wl = workloads.WORKLOADS[workload]
    dtype = torch.float32 if op == "rmsnorm_cast" else wl.dtype
    return metric_label(op, dtype, wl.M, wl.N)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: about 0.1 s of timed GPU work at the headline workload, after
    # a warmup long enough for clocks and caches to settle.
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c2", help="workload name (c2..c5)")
    ap.add_argument("--op", choices=("rmsnorm", "layernorm", "add_rmsnorm", "rmsnorm_cast"),
                    default="rmsnorm")
    ap.add_argument("--cold-samples", type=int, default=50)
    ap.add_argument("--rotating-sets", type=int, default=3,
                    help="independent buffer sets the rotating-warm leg cycles over")
    ap.add_argument("--rotating-steps", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1 << 62,
                    help="rows of the workload the CPU oracle is timed on")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not "
              "supported (the row-sharded multi-GPU path is designed, not implemented).",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import backward_rmsnorm_fwd_amd as rn
    from backward_rmsnorm_fwd_amd import workloads

    if args.workload not in workloads.WORKLOADS:
        print(f"bench.py: unknown workload {args.workload!r} "
              f"(known: {', '.join(sorted(workloads.WORKLOADS))})", file=sys.stderr, flush=True)
        sys.exit(2)
    row_cap = {"layernorm": rn.LAYERNORM_MAX_N, "add_rmsnorm": rn.RMSNORM_ADD_MAX_N,
               "rmsnorm_cast": rn.RMSNORM_CAST_MAX_N}.get(args.op)
    if row_cap is not None and workloads.WORKLOADS[args.workload].N > row_cap:
        print(f"bench.py: --op {args.op} takes rows of N <= {row_cap}; workload "
              f"{args.workload} has N = {workloads.WORKLOADS[args.workload].N}",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    rn.load_library()
    wl = workloads.WORKLOADS[args.workload]
    t0 = time.time()
    ln = args.op == "layernorm"
    fused = args.op == "add_rmsnorm"
    cast = args.op == "rmsnorm_cast"
    cast_to = wl.dtype if wl.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
    make = {"layernorm": workloads.make_layernorm_inputs,
            "add_rmsnorm": workloads.make_add_inputs,
            "rmsnorm_cast": lambda name: workloads.make_cast_inputs(name, out_dtype=cast_to),
            }.get(args.op, workloads.make_inputs)
    inp = make(args.workload)
    M, N, T, off, eps = inp["M"], inp["N"], inp["dtype"], inp["offset"], inp["eps"]
    s = torch.tensor([], dtype=T).element_size()
    if ln:
        nbytes = rn.layernorm_bwd_workspace_bytes(M, N, T)
    elif fused:
        nbytes = rn.rmsnorm_add_bwd_workspace_bytes(M, N, T, off)
    elif cast:
        nbytes = rn.rmsnorm_cast_bwd_workspace_bytes(M, N, cast_to, off)
    else:
        nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, T, off)

    def alloc_set(src=None):
        """Device buffers of one step: inputs copied from `src` (another set)
        or from the host draws, outputs and workspace fresh."""
        b = {}
        for k in ("x", "w", "dy") + (("b",) if ln else ()) + (("res", "dh") if fused else ()):
            b[k] = src[k].clone() if src is not None else inp[k].to(dev)
        x = b["x"]
        b["y"] = torch.empty_like(x, dtype=cast_to) if cast else torch.empty_like(x)
        b["rstd"] = torch.empty(M, device=dev, dtype=torch.float32)
        b["dx"] = torch.empty_like(x)
        b["dgamma"] = torch.empty(N, device=dev, dtype=torch.float32)
        if ln:
            b["mean"] = torch.empty(M, device=dev, dtype=torch.float32)
            b["dbeta"] = torch.empty(N, device=dev, dtype=torch.float32)
        if fused:
            b["h"] = torch.empty_like(x)
        b["ws"] = torch.empty(max(4, nbytes) // 4, device=dev, dtype=torch.float32)
        return b

    def stages_for(b):
        x, w, dy, y, rstd, dx, dgamma, ws = (b[k] for k in ("x", "w", "dy", "y", "rstd", "dx",
                                                             "dgamma", "ws"))
        if fused:
            res, dh, h = b["res"], b["dh"], b["h"]

            def fwd():
                rn.rmsnorm_add_fwd(x, res, w, eps, y, h, rstd, off)

            def bwd_rows():
                rn.rmsnorm_add_bwd_rows(dy, dh, h, w, rstd, dx, ws, off)

            def bwd_reduce():
                rn.rmsnorm_add_bwd_reduce(ws, M, N, T, dgamma, off)
        elif cast:
            def fwd():
                rn.rmsnorm_cast_fwd(x, w, eps, y, rstd, off)

            def bwd_rows():
                rn.rmsnorm_cast_bwd_rows(dy, x, w, rstd, dx, ws, off)

            def bwd_reduce():
                rn.rmsnorm_cast_bwd_reduce(ws, M, N, cast_to, dgamma, off)
        elif ln:
            bias, mean, dbeta = b["b"], b["mean"], b["dbeta"]

            def fwd():
                rn.layernorm_fwd(x, w, bias, eps, y, mean, rstd)

            def bwd_rows():
                rn.layernorm_bwd_rows(dy, x, w, mean, rstd, dx, ws)

            def bwd_reduce():
                rn.layernorm_bwd_reduce(ws, M, N, T, dgamma, dbeta)
        else:
            def fwd():
                rn.rmsnorm_fwd(x, w, eps, y, rstd, off)

            def bwd_rows():
                rn.rmsnorm_bwd_rows(dy, x, w, rstd, dx, ws, off)

            def bwd_reduce():
                rn.rmsnorm_bwd_reduce(ws, M, N, T, dgamma, off)
        return fwd, bwd_rows, bwd_reduce

    main_set = alloc_set()
    x, w, dy = main_set["x"], main_set["w"], main_set["dy"]
    if fused:
        res, dh = main_set["res"], main_set["dh"]
    fwd, bwd_rows, bwd_reduce = stages_for(main_set)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    fb, rb, db = alg_bytes(M, N, s, args.op)
    step_bytes = fb + rb + db

    # ---- cold-cache per-call samples (the primary per-call protocol) ----
    # Before each sample a 1 GiB buffer is read (not written), so L2 and the
    # 256 MB Infinity Cache hold only clean, unrelated lines.
    flush = torch.ones(1 << 28, device=dev, dtype=torch.float32)  # 1 GiB
    for _ in range(3):
        for f in (fwd, bwd_rows, bwd_reduce):
            f()
    cold = {}
    for name, calls in (("fwd", [fwd]), ("bwd", [bwd_rows, bwd_reduce])):
        if args.cold_samples <= 0:
            break
        samples = []
        for _ in range(args.cold_samples):
            flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for f in calls:
                f()
            b.record()
            b.synchronize()
            samples.append(a.elapsed_time(b) * 1e3)
        samples.sort()
        med = statistics.median(samples)
        nb = fb if name == "fwd" else rb + db
        cold[name] = {"median_us": round(med, 2),
                      "p10_us": round(samples[len(samples) // 10], 2),
                      "p90_us": round(samples[(9 * len(samples)) // 10], 2),
                      "GBps": round(nb / (med * 1e-6) / 1e9, 1),
                      "pct_of_8TBps": round(100 * nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    if cold:
        step_cold = cold["fwd"]["median_us"] + cold["bwd"]["median_us"]
        cold["samples_per_pass"] = args.cold_samples
        cold["flush_bytes"] = flush.numel() * 4
        cold["step_us"] = round(step_cold, 2)
        cold["GBps"] = round(step_bytes / (step_cold * 1e-6) / 1e9, 1)
        cold["pct_of_8TBps"] = round(100 * cold["GBps"] / HBM_PEAK_GBS, 1)
    del flush

    # ---- rotating warm: back-to-back steps over independent buffer sets ----
    rotating = None
    if args.rotating_sets > 1 and args.rotating_steps > 0:
        sets = [main_set] + [alloc_set(main_set) for _ in range(args.rotating_sets - 1)]
        rot_stages = [stages_for(b) for b in sets]
        for i in range(2 * len(sets)):
            for f in rot_stages[i % len(sets)]:
                f()
        torch.cuda.synchronize()
        t_rot = time.perf_counter()
        for i in range(args.rotating_steps):
            for f in rot_stages[i % len(sets)]:
                f()
        torch.cuda.synchronize()
        rot_us = (time.perf_counter() - t_rot) * 1e6 / args.rotating_steps
        per_set = sum(t.numel() * t.element_size() for t in sets[1].values())
        rotating = {"sets": len(sets), "steps": args.rotating_steps,
                    "bytes_per_set": per_set, "step_us": round(rot_us, 2),
                    "GBps": round(step_bytes / (rot_us * 1e-6) / 1e9, 1),
                    "pct_of_8TBps": round(100 * step_bytes / (rot_us * 1e-6) / 1e9
                                          / HBM_PEAK_GBS, 1)}
        del sets, rot_stages
        torch.cuda.synchronize()

    stages = [("fwd", fwd), ("bwd_rows", bwd_rows), ("bwd_reduce", bwd_reduce)]
    for _ in range(args.warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()

    # ---- timed steps ----
    # Events bracket only the dominant kernel (backward stage 1) on the stream
    # it is launched on; the step time comes from the host clock around K
    # steps bracketed by device synchronization.
    # An event pair costs a few microseconds of queue time, so only a few
    # steps carry one: one pair per ten steps, between 2 and 10 pairs.
    n_ev = max(2, min(10, args.steps // 10))
    every = max(1, args.steps // n_ev)
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in list(range(0, args.steps, every))[:n_ev]}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        fwd()
        if i in ev:
            ev[i][0].record()
        bwd_rows()
        if i in ev:
            ev[i][1].record()
        bwd_reduce()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    dominant_us = statistics.mean(a.elapsed_time(b) for a, b in ev.values()) * 1e3

    # ---- per-kernel averages, in the same order, outside the timed region ----
    per_kernel_us = {}
    for k in ("fwd", "bwd_rows", "bwd_reduce"):
        evs = []
        for _ in range(max(5, min(100, args.steps // 2))):
            for name, f in stages:
                if name == k:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    f()
                    b.record()
                    evs.append((a, b))
                else:
                    f()
        torch.cuda.synchronize()
        per_kernel_us[k] = statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = rb / (dominant_us * 1e-6) / 1e9

    # ---- the same step unfused (add kernels around the plain norm) ----
    unfused_us = None
    if fused:
        h2, y2, dx2 = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
        r2 = torch.empty(M, device=dev, dtype=torch.float32)
        dg2 = torch.empty(N, device=dev, dtype=torch.float32)
        ws2 = torch.empty(max(4, rn.rmsnorm_bwd_workspace_bytes(M, N, T, off)) // 4, device=dev)

        def unfused_step():
            torch.add(x, res, out=h2)
            rn.rmsnorm_fwd(h2, w, eps, y2, r2, off)
            rn.rmsnorm_bwd(dy, h2, w, r2, dx2, dg2, ws2, off)
            dx2.add_(dh)

        for _ in range(max(10, args.warmup // 4)):
            unfused_step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        n_unf = max(10, args.steps // 2)
        for _ in range(n_unf):
            unfused_step()
        torch.cuda.synchronize()
        unfused_us = (time.perf_counter() - t) * 1e6 / n_unf
        del h2, y2, dx2, ws2
    elif cast:
        y32, dx2 = torch.empty_like(x), torch.empty_like(x)
        y2 = torch.empty_like(x, dtype=cast_to)
        dy32 = torch.empty_like(x)
        r2 = torch.empty(M, device=dev, dtype=torch.float32)
        dg2 = torch.empty(N, device=dev, dtype=torch.float32)
        ws2 = torch.empty(max(4, rn.rmsnorm_bwd_workspace_bytes(M, N, T, off)) // 4, device=dev)

        def unfused_step():
            rn.rmsnorm_fwd(x, w, eps, y32, r2, off)
            y2.copy_(y32)
            dy32.copy_(dy)
            rn.rmsnorm_bwd(dy32, x, w, r2, dx2, dg2, ws2, off)

        for _ in range(max(10, args.warmup // 4)):
            unfused_step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        n_unf = max(10, args.steps // 2)
        for _ in range(n_unf):
            unfused_step()
        torch.cuda.synchronize()
        unfused_us = (time.perf_counter() - t) * 1e6 / n_unf
        del y32, y2, dy32, dx2, ws2

    # ---- plain device copy of 1 GiB, for an achievable-bandwidth reference ----
    src = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    b.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    # ---- CPU oracle on the same workload ----
    cpu_baseline = None
    if not args.no_cpu_baseline:
        from oracle import fused as fused_oracle
        from oracle import golden
        from oracle import layernorm as ln_oracle
        from oracle import reference as ref_oracle
        R = min(args.cpu_rows, M)
        xs, dys = inp["x"][:R], inp["dy"][:R]
        nthreads = torch.get_num_threads()
        torch.set_num_threads(1)
        times = []
        for _ in range(3):
            t = time.perf_counter()
            if fused:
                hs, _, _ = fused_oracle.golden_add_forward(xs, inp["res"][:R], inp["w"], eps, off)
                fused_oracle.golden_add_backward(dys, inp["dh"][:R], hs, inp["w"], eps, off)
            elif cast:
                fused_oracle.golden_cast_forward(xs, inp["w"], eps, off)
                fused_oracle.golden_cast_backward(dys, xs, inp["w"], eps, off)
            elif ln:
                ln_oracle.golden_ln_forward(xs, inp["w"], inp["b"], eps)
                ln_oracle.golden_ln_dx(dys, xs, inp["w"], eps)
                ln_oracle.golden_ln_param_grads(dys, xs, eps)
            else:
                golden.golden_forward(xs, inp["w"], eps, off)
                golden.golden_dx(dys, xs, inp["w"], eps, off)
                golden.golden_dgamma(dys, xs, eps)
            times.append(time.perf_counter() - t)
        torch.set_num_threads(nthreads)
        cpu_s = statistics.median(times)
        sb = sum(alg_bytes(R, N, s, args.op))
        # The same-dtype eager reference (float32 intermediates, PyTorch CPU)
        # on the same rows, with torch's own thread pool.
        rtimes = []
        for _ in range(3):
            t = time.perf_counter()
            if fused:
                hs, _, _ = fused_oracle.reference_add_forward(xs, inp["res"][:R], inp["w"], eps, off)
                fused_oracle.reference_add_backward(dys, inp["dh"][:R], hs, inp["w"], eps, off)
            elif cast:
                fused_oracle.reference_cast_forward(xs, inp["w"], cast_to, eps, off)
                fused_oracle.reference_cast_backward(dys, xs, inp["w"], eps, off)
            elif ln:
                ln_oracle.reference_ln_forward(xs, inp["w"], inp["b"], eps)
                ln_oracle.reference_ln_backward(dys, xs, inp["w"], eps)
            else:
                ref_oracle.reference_forward(xs, inp["w"], eps, off)
                ref_oracle.reference_backward(dys, xs, inp["w"], eps, off)
            rtimes.append(time.perf_counter() - t)
        ref_s = statistics.median(rtimes)
        cpu_baseline = {"value": round(sb / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1,
                        "kind": "oracle",
                        "sample": f"float64 NumPy golden forward+backward over {R} of {M} rows "
                                  f"(all of them by default), median of 3 runs of {cpu_s:.1f} s, "
                                  "one thread",
                        "host_cores_available": len(os.sched_getaffinity(0)),
                        "torch_fp32_reference": {
                            "value": round(sb / ref_s / 1e9, 4), "unit": "GB/s",
                            "threads": nthreads,
                            "sample": f"same rows, float32 torch CPU reference forward+backward, "
                                      f"median of 3 runs of {ref_s:.2f} s"}}

    result = {
        "metric": metric_for(args.op, args.workload),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[T],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl.description}"
                   + (" (LayerNorm inputs)" if ln else " (with res and dh)" if fused
                      else f" (float32 x and gamma, y and dy in {str(cast_to)[6:]})" if cast
                      else ""),
                   "op": args.op, "M": M, "N": N,
                   "eps": eps, "offset_weight": off, "seed": inp["seed"],
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "kernels_us": {k: round(v, 2) for k, v in per_kernel_us.items()},
        "dominant_kernel_us_in_timed_steps": round(dominant_us, 2),
        "fwd": {"us": round(per_kernel_us["fwd"], 2),
                "GBps": round(fb / (per_kernel_us["fwd"] * 1e-6) / 1e9, 1)},
        "bwd": {"us": round(per_kernel_us["bwd_rows"] + per_kernel_us["bwd_reduce"], 2),
                "GBps": round((rb + db) / ((per_kernel_us["bwd_rows"]
                                            + per_kernel_us["bwd_reduce"]) * 1e-6) / 1e9, 1)},
        "cold_cache": cold,
        "rotating_warm": rotating,
        "device_copy_GBps": round(copy_gbs, 1),
        "unfused_step_us": None if unfused_us is None else round(unfused_us, 2),
        "roofline": {"kernel": ("ln_bwd_rows" if ln else "add_bwd_rows" if fused
                                else "cast_bwd_rows" if cast else "bwd_rows"),
                     "bound": "hbm",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if (ln or fused or cast) else measured_traffic(args.workload),
                     "alg_bytes_per_launch": rb},
        "cpu_baseline": cpu_baseline,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
