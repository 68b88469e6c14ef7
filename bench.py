#!/usr/bin/env python3
"""Float8Linear forward + backward benchmark on one MI355X.

A step is one forward + backward (amax -> scale -> fp8 cast + transposed
copy -> three fp8 GEMMs with dequantisation) of every linear in the
workload, through the C ABI (f8lin_forward / f8lin_backward; plus
f8lin_delayed_update for delayed scaling), on seeded synthetic bf16 inputs
already resident in HBM.  Prints ONE JSON line.

Timed region: W untimed warm-up steps, synchronize, K timed steps bracketed
by HIP events on the launch stream, synchronize.  Input sets rotate between
steps (enough copies that a step's inputs are not left in the 256 MB
last-level cache by the previous step).

A second, instrumented pass runs the same K steps through the individual
entry points (amax / cast_transpose / gemm -- the exact launch sequence
f8lin_forward/backward perform) with HIP events between the calls on the same
stream, giving each kernel's average duration for the roofline figures.

The oracle (CPU, test infrastructure) is timed on the host cores on a bounded
sample of the same workload for the cpu_baseline field.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
MALL_BYTES = 256 << 20
# P3 (pytorch/torchtitan PR #778) single-linear table, (4096, 4096) input,
# float8nocompile ATOMIC_MAX on H100: 977.858 (read as microseconds) for
# forward + backward of a 4096->4096 linear -> 6*4096^3 / 977.858 us.
H100_BASELINE_TFLOPS = {"linear4096_m4096": 6 * 4096 ** 3 / 977.858e-6 / 1e12,
                        "linear4096_m16": 6 * 16 * 4096 ** 2 / 386.469e-6 / 1e12,
                        "linear4096_m256": 6 * 256 * 4096 ** 2 / 408.137e-6 / 1e12,
                        "linear4096_m65536_outliers": 6 * 65536 * 4096 ** 2 / 10813.3e-6 / 1e12}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="linear4096_m4096")
    p.add_argument("--algo", default="twopass", choices=["atomic", "twopass"],
                   help="amax algorithm of the timed loop; the other one is timed right after")
    p.add_argument("--rotate", type=int, default=0, help="input sets to rotate (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=4096, help="rows of X/dY in the oracle's timed sample")
    p.add_argument("--only-timed", action="store_true", help="skip the instrumented pass (for profiling)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes three times (counter calibration)")
    return p.parse_args()


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(gemm_src, workload):
    """HBM traffic of the GEMM from rocprofv3 counter runs, if the committed
    record was taken on the current kernel source and on this workload (else
    None)."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha256_of(gemm_src) or rec.get("workload_name") != workload:
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   f"(got {args.gpus}); multi-GPU sharding is design-only"}))
        sys.exit(2)

    import numpy as np
    import torch
    from float8linear_tensorwise_amax_amd import f8lin, inputs

    if args.calibrate_copy:
        # A plain copy of known size: HBM counters of the same profiler run,
        # divided by these bytes, give the counters' scale factors.
        n = args.calibrate_copy
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return

    wl = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    delayed = wl.scaling == "delayed"

    # ---- inputs: R rotating sets, generated on the host, copied once to HBM
    per_set_bytes = sum(2 * (l.M * l.K + l.N * l.K + l.M * l.N) for l in wl.linears)
    R = args.rotate or max(1, min(8, math.ceil(3 * MALL_BYTES / per_set_bytes)))
    sets = []
    for r in range(R):
        step_in = inputs.workload_inputs(wl, r if delayed else 0)
        if r > 0 and not delayed:  # distinct data per set: reseed
            gen = torch.Generator().manual_seed(1000 + r)
            step_in = [(l, *inputs.draw_linear(gen, l, wl.outlier_fraction, wl.outlier_multiplier))
                       for l in wl.linears]
        sets.append([(l, x.to(dev), w.to(dev), dy.to(dev)) for (l, x, w, dy) in step_in])
    bufs = [f8lin.LinearBuffers(l.M, l.N, l.K, dev) for l in wl.linears]
    torch.cuda.synchronize()

    groups = inputs.groups_of(wl)
    assert not (delayed and any(len(g) > 1 for g in groups)), "shared inputs are measured with dynamic scaling"

    def step(t, algo):
        mode = "delayed" if (delayed and t > 0) else "dynamic"
        data = sets[t % R]
        for g in groups:
            if len(g) == 1:
                buf, (l, x, w, dy) = bufs[g[0]], data[g[0]]
                buf.forward(x, w, mode, algo)
                buf.backward(dy, mode, algo)
                continue
            # linears reading one X: X cast once, their forward GEMMs in one launch
            lead = bufs[g[0]]
            x = data[g[0]][1]
            f8lin.forward_shared_x(x, lead.x8, lead.x8t, lead.sx, lead.ws,
                                   [{"w": data[i][2], "y": bufs[i].y, "w8": bufs[i].w8, "w8t": bufs[i].w8t,
                                     "sw": bufs[i].sw} for i in g], mode, algo)
            for i in g:
                b = bufs[i]
                f8lin.backward(data[i][3], lead.x8t, b.w8t, b.dx, b.dw, b.dy8, b.dy8t, lead.sx, b.sw, b.sdy, b.ws,
                               mode, algo)
        if delayed:
            # the history sync after backward: one call for every linear's states
            f8lin.delayed_update([st for b in bufs for st in b.states()])

    def timed_steps(algo):
        for t in range(args.warmup):
            step(t, algo)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t_host0 = time.perf_counter()
        e0.record(stream)
        for t in range(args.steps):
            step(args.warmup + t, algo)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, time.perf_counter() - t_host0

    def step_spread(algo, n=100):
        """Per-step HIP events around n further steps: median and min (the
        events themselves add a little time per step)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for t, (a, b) in enumerate(evs):
            a.record(stream)
            step(args.warmup + args.steps + t, algo)
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return ts[len(ts) // 2], ts[0]

    # ---- timed region (the headline), then the same with the other amax algorithm
    ms_per_step, t_host = timed_steps(args.algo)
    ms_median, ms_min = step_spread(args.algo)
    other = "twopass" if args.algo == "atomic" else "atomic"
    ms_other = None if (delayed or args.only_timed) else timed_steps(other)[0]
    flops = wl.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": "Float8Linear fwd+bwd us & TFLOP/s (frac fp8 peak); cast/amax HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(tflops / H100_BASELINE_TFLOPS[args.workload], 3)
                        if args.workload in H100_BASELINE_TFLOPS else None),
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "shared_input_groups": [list(g) for g in wl.shared_x],
                   "linears": [{"name": l.name, "M": l.M, "K": l.K, "N": l.N} for l in wl.linears],
                   "scaling": wl.scaling, "amax_algo": args.algo, "rotating_input_sets": R,
                   "inputs": "X~N(0,1), W~N(0,1/K), dY~N(0,1e-3) bf16, seeded"},
        "fwd_bwd_us": round(ms_per_step * 1e3, 2),
        "fwd_bwd_us_per_step_events": {"median": round(ms_median * 1e3, 2), "min": round(ms_min * 1e3, 2),
                                       "steps": 100},
        "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
        "host_wall_s_timed": round(t_host, 4),
    }
    if ms_other is not None:
        out["fwd_bwd_us_by_amax_algo"] = {args.algo: round(ms_per_step * 1e3, 2), other: round(ms_other * 1e3, 2)}
    if out["vs_baseline"] is not None:
        out["baseline_note"] = ("pages' H100 float8nocompile ATOMIC_MAX fwd+bwd time for this shape "
                                "(read as microseconds), converted to TFLOP/s; another machine's number")

    if not args.only_timed:
        out.update(instrumented(args, wl, sets, bufs, R, f8lin, torch, stream, delayed))
        # the step's dominant kernel: the backward's dgrad + wgrad launch
        rl = out["kernels"]["gemm_bwd_pair"]
        traffic = load_traffic(os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "csrc", "gemm.hip"),
                               args.workload)
        out["roofline"] = {"kernel": "gemm_fp8_tn_kernel<e5m2,e4m3> (dgrad + wgrad, one launch)",
                           "bound": "mfma", "achieved": rl["tflops"],
                           "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(rl["tflops"] / PEAK_FP8_TFLOPS, 4),
                           "traffic": (traffic["hbm_bytes_per_launch"] if traffic else None),
                           "algorithmic_bytes_per_launch": rl["algorithmic_bytes_per_launch"]}
        if traffic:
            out["roofline"]["traffic_note"] = traffic.get("note", "")
        out["hbm_copy_reference"] = copy_reference(torch, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, wl, sets, np, torch)
    print(json.dumps(out), flush=True)


def copy_reference(torch, stream, nbytes=1 << 30, reps=20):
    """The rate a plain device-to-device copy reaches (the runtime's copy
    kernel, 1 GiB read + 1 GiB written per copy), timed with HIP events on
    the launch stream: what this HBM delivers to a streaming kernel, beside
    the 8 TB/s spec that the roofline fractions use.  Context only: no step
    of the path runs through it."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    return {"what": "device-to-device copy of 1 GiB (read + write), HIP events, average of 20",
            "us_per_copy": round(us, 2), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def instrumented(args, wl, sets, bufs, R, f8lin, torch, stream, delayed):
    """Per-call and per-kernel durations with HIP events on the launch stream:
    each f8lin_forward / f8lin_backward call as the step issues it, and its
    GEMM launch again on its own (f8lin_gemm; f8lin_gemm_batch for the
    backward's dgrad + wgrad pair).  A call's time minus its GEMM's is its
    amax + cast phase, whose algorithmic bytes are 2 B/element for each
    dynamic-mode amax pass and 4 B/element for each cast.  f8lin_gemm_batch
    is the plain shared launch: where f8lin_backward splits a GEMM along K or
    hands out the pair's tiles through its work queue (problems of different
    contraction length), the pair inside the call runs faster than this
    figure and the amax + cast share absorbs the difference; the step time
    above is the real path either way.  At M = N = K the two launches are the
    same."""
    acc = {k: [0.0, 0, 0.0] for k in ("fwd_call", "bwd_call", "gemm_fwd", "gemm_bwd_pair")}  # ms, calls, units
    ew_bytes = {"fwd": 0, "bwd": 0}
    gemm_bytes = {"gemm_fwd": [], "gemm_bwd_pair": []}

    def timed(kind, fn, units):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pending.append((kind, a, b, units))

    # the timed loops ran just before, so the device is warm: fewer rounds
    # suffice.  Everything is queued before one synchronisation, so the host
    # stays ahead of the GPU and no call starts from an idle device.
    warm, steps = min(args.warmup, 10), min(args.steps, 100)
    recorded = []
    for t in range(warm + steps):
        pending = []
        mode = "delayed" if (delayed and t > 0) else "dynamic"
        for buf, (l, x, w, dy) in zip(bufs, sets[t % R]):
            per = 6 if mode == "dynamic" else 4  # amax pass (dynamic) + cast
            timed("fwd_call", lambda: buf.forward(x, w, mode, args.algo), per * (l.M * l.K + l.N * l.K))
            timed("gemm_fwd", lambda: f8lin.gemm(buf.x8, "e4m3", buf.w8, "e4m3", buf.sx.inv_scale,
                                                 buf.sw.inv_scale, buf.y), 2 * l.M * l.N * l.K)
            timed("bwd_call", lambda: buf.backward(dy, mode, args.algo), per * l.M * l.N)
            # dgrad and wgrad in one launch, as f8lin_backward issues them
            timed("gemm_bwd_pair", lambda: f8lin.gemm_batch(
                [(buf.dy8, buf.w8t, buf.sdy.inv_scale, buf.sw.inv_scale, buf.dx),
                 (buf.dy8t, buf.x8t, buf.sdy.inv_scale, buf.sx.inv_scale, buf.dw)], "e5m2", "e4m3"),
                4 * l.M * l.N * l.K)
            if delayed:
                f8lin.delayed_update(buf.states())
            if t == 0:
                gemm_bytes["gemm_fwd"].append(l.M * l.K + l.N * l.K + 2 * l.M * l.N)
                gemm_bytes["gemm_bwd_pair"].append(l.M * l.N + l.N * l.K + 2 * l.M * l.K +
                                                   l.M * l.N + l.M * l.K + 2 * l.N * l.K)
        if t >= warm:
            recorded.extend(pending)
    torch.cuda.synchronize()
    for kind, a, b, units in recorded:
        acc[kind][0] += a.elapsed_time(b)
        acc[kind][1] += 1
        acc[kind][2] += units
    k = {}
    for name in ("gemm_fwd", "gemm_bwd_pair"):
        ms, n, el = acc[name]
        k[name] = {"avg_us": round(ms / n * 1e3, 3), "launches": n,
                   "tflops": round(el / (ms * 1e-3) / 1e12, 2),
                   "algorithmic_bytes_per_launch": int(sum(gemm_bytes[name]) / len(gemm_bytes[name])),
                   "flops_per_launch": int(el / n)}
    for side, gemm in (("fwd", "gemm_fwd"), ("bwd", "gemm_bwd_pair")):
        ms_call, n, by = acc[side + "_call"]
        ms_ew = ms_call - acc[gemm][0]
        k["amax_cast_" + side] = {"avg_us": round(ms_ew / n * 1e3, 3), "calls": n,
                                  "call_avg_us": round(ms_call / n * 1e3, 3),
                                  "gbs": round(by / (ms_ew * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(by / (ms_ew * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "algorithmic_bytes_per_call": int(by / n),
                                  "what": ("amax pass(es) + cast of X and W" if side == "fwd" else
                                           "amax pass + cast of dY") + " = call time minus its GEMM launch"}
    # amax alone, both algorithms, on the step's three tensors
    for algo in ("atomic", "twopass"):
        tot_ms, n, el = 0.0, 0, 0
        kept = []
        for t in range(warm + steps):
            evs = []
            for buf, (l, x, w, dy) in zip(bufs, sets[t % R]):
                for tensor, st in ((x, buf.sx), (w, buf.sw), (dy, buf.sdy)):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    f8lin.amax(tensor, st.amax, buf.ws, algo)
                    b.record(stream)
                    evs.append((a, b, tensor.numel()))
            if t >= warm:
                kept.extend(evs)
        torch.cuda.synchronize()
        for a, b, units in kept:
            tot_ms += a.elapsed_time(b)
            n += 1
            el += units
        k["amax_" + algo] = {"avg_us": round(tot_ms / n * 1e3, 3), "launches": n,
                             "gbs": round(2 * el / (tot_ms * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(2 * el / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "bytes_per_elem": 2}
    return {"kernels": k}


def cpu_baseline(args, wl, sets, np, torch):
    """The oracle (as it stands) on a bounded sample of the workload: the first
    `cpu_rows` rows of X and dY of each linear with the full W -- amax, scale,
    cast + transpose of all three tensors and the three fp64 GEMM references."""
    import oracle
    from threadpoolctl import threadpool_info

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    flops = 0
    secs = 0.0
    rows_used = []
    host = []
    for (l, x, w, dy) in sets[0]:
        ms = min(l.M, args.cpu_rows)
        rows_used.append(ms)
        host.append((l, ms, bits(x[:ms]), bits(w), bits(dy[:ms])))
    reps = 0
    while reps < 30 and (reps == 0 or secs < 10.0):  # about 10 s of CPU work, repeated samples
        for l, ms, xb, wb, dyb in host:
            t0 = time.perf_counter()
            oracle.linear_step(xb, wb, dyb, gemms=True)
            secs += time.perf_counter() - t0
            flops += 6 * ms * l.N * l.K
        reps += 1
    # one more sample, op by op (same oracle functions linear_step calls)
    ops = {"amax": 0.0, "scale": 0.0, "cast_transpose": 0.0, "gemm_refs": 0.0}
    for l, ms, xb, wb, dyb in host:
        q = {}
        for name, t_bits, fmt in (("x", xb, oracle.E4M3), ("w", wb, oracle.E4M3), ("dy", dyb, oracle.E5M2)):
            t0 = time.perf_counter()
            a = oracle.amax(t_bits)
            t1 = time.perf_counter()
            sc, _ = oracle.scale(a, fmt)
            t2 = time.perf_counter()
            q[name] = (oracle.cast(t_bits, fmt, sc)[0], sc)
            t3 = time.perf_counter()
            ops["amax"] += t1 - t0
            ops["scale"] += t2 - t1
            ops["cast_transpose"] += t3 - t2
        t0 = time.perf_counter()
        oracle.forward_ref(q["x"][0], q["w"][0], q["x"][1], q["w"][1])
        oracle.dgrad_ref(q["dy"][0], q["w"][0], q["dy"][1], q["w"][1])
        oracle.wgrad_ref(q["dy"][0], q["x"][0], q["dy"][1], q["x"][1])
        ops["gemm_refs"] += time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(secs, 2),
            "seconds_by_op_one_sample": {k: round(v, 4) for k, v in ops.items()},
            "sample": f"{reps} repetition(s) of one step of {wl.name} on the first {rows_used} rows of X and dY "
                      "per linear (full W): amax, scale, cast+transpose of X, W, dY and the three fp64 GEMM "
                      "references",
            "host_cpus_visible": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
