#!/usr/bin/env python3
"""Float8Linear forward + backward benchmark on one MI355X.

A step is one forward + backward (amax -> scale -> fp8 cast + transposed
copy -> three fp8 GEMMs with dequantisation) of every linear in the
workload, through the C ABI (f8lin_forward / f8lin_backward; plus
f8lin_delayed_update for delayed scaling), on seeded synthetic bf16 inputs
already resident in HBM.  Prints ONE JSON line.

Default workload: the pages' largest single-linear shape, 65536 x 4096 ->
4096 with 0.1% outliers in X (pytorch/torchtitan PR #778, single-linear-layer
table, input (65536, 4096)).

Timed region: steps for --settle-ms of wall clock (the shader clock settles
under load), W untimed warm-up steps, synchronize, K timed steps bracketed by
HIP events on the launch stream, synchronize.  Input sets rotate between
steps (enough copies that a step's inputs are not left in the 256 MB
last-level cache by the previous step).

Then: the two amax algorithms in alternating timed blocks; an instrumented
pass of the same steps with HIP events around every forward / backward call
and the events each call records around its own GEMM launch (the roofline
figure is the backward's dgrad + wgrad launch as f8lin_backward issues it);
both amax algorithms alone; the epilogue amax against the amax pass it
spares; a plain device copy for reference.

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
# The pages' H100 float8nocompile ATOMIC_MAX forward + backward times for a
# 4096 -> 4096 linear (pytorch/torchtitan PR #778, single-linear-layer table,
# read as microseconds), by input rows: another machine's numbers, context only.
H100_US = {"linear4096_m16": 386.469, "linear4096_m256": 408.137, "linear4096_m4096": 977.858,
           "linear4096_m65536_outliers": 10813.3}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="linear4096_m65536_outliers")
    p.add_argument("--algo", default="twopass", choices=["atomic", "twopass"],
                   help="amax algorithm of the headline loop")
    p.add_argument("--settle-ms", type=float, default=1000.0,
                   help="run steps for this long (wall clock) before the warm-up, so the clocks settle")
    p.add_argument("--algo-rounds", type=int, default=3,
                   help="rounds of alternating timed blocks (one per amax algorithm) for the comparison")
    p.add_argument("--rotate", type=int, default=0, help="input sets to rotate (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=4096, help="rows of X/dY in the oracle's timed sample")
    p.add_argument("--only-timed", action="store_true", help="skip everything after the headline (for profiling)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes three times (counter calibration)")
    p.add_argument("--ceilings", action="store_true",
                   help="only measure this GPU's ceilings: HBM streaming (own read / write / copy kernels), "
                        "MFMA issue from registers with its clock, and the GEMM's own K loop at long K")
    return p.parse_args()


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(gemm_src, workload):
    """HBM traffic of the backward GEMM launch from rocprofv3 counter runs, if
    the committed record for this workload was read on the current kernel
    source (else None)."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get("records", {}).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("source_sha256") != sha256_of(gemm_src):
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

    if args.ceilings:
        print(json.dumps(ceilings(torch, f8lin)), flush=True)
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

    def step(t, algo, ev=None):
        """One step; with ev (a list), HIP events around each forward / backward
        call and, from inside the call, around its GEMM launch are appended as
        (kind, begin, end, group) for the instrumented pass."""
        mode = "delayed" if (delayed and t > 0) else "dynamic"
        data = sets[t % R]

        def events(kind, g):
            if ev is None:
                return None, None
            pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            gemm = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev.append((kind, pair, gemm, g))
            return pair, gemm

        for g in groups:
            call, gemm = events("fwd", g)
            if call:
                call[0].record(stream)
            if len(g) == 1:
                buf, (l, x, w, dy) = bufs[g[0]], data[g[0]]
                buf.forward(x, w, mode, algo, gemm_events=gemm)
            else:
                # linears reading one X: X cast once, their forward GEMMs in one launch
                lead = bufs[g[0]]
                f8lin.forward_shared_x(data[g[0]][1], lead.x8, lead.x8t, lead.sx, lead.ws,
                                       [{"w": data[i][2], "y": bufs[i].y, "w8": bufs[i].w8, "w8t": bufs[i].w8t,
                                         "sw": bufs[i].sw} for i in g], mode, algo, gemm_events=gemm)
            if call:
                call[1].record(stream)
            lead = bufs[g[0]]
            for i in g:
                b = bufs[i]
                call, gemm = events("bwd", [i])
                if call:
                    call[0].record(stream)
                f8lin.backward(data[i][3], lead.x8t, b.w8t, b.dx, b.dw, b.dy8, b.dy8t, lead.sx, b.sw, b.sdy, b.ws,
                               mode, algo, gemm_ws=b.gemm_ws, gemm_events=gemm)
                if call:
                    call[1].record(stream)
        if delayed:
            # the history sync after backward: one call for every linear's states
            f8lin.delayed_update([st for b in bufs for st in b.states()])

    t_next = [0]  # step counter across phases (delayed workloads use it for the mode)

    def run(n, algo):
        for _ in range(n):
            step(t_next[0], algo)
            t_next[0] += 1

    def timed(n, algo):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(n, algo)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---- settle: the shader clock takes ~0.1 s of load to reach its sustained
    # level; run steps for settle_ms of wall clock first
    t0 = time.perf_counter()
    settle_steps = 0
    while True:
        run(5, args.algo)
        settle_steps += 5
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= args.settle_ms:
            break
    settle_ms = (time.perf_counter() - t0) * 1e3

    # ---- timed region (the headline): W warm-up steps, then exactly K steps
    run(args.warmup, args.algo)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_host0 = time.perf_counter()
    e0.record(stream)
    run(args.steps, args.algo)
    e1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    ms_per_step = e0.elapsed_time(e1) / args.steps
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
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "shared_input_groups": [list(g) for g in wl.shared_x],
                   "linears": [{"name": l.name, "M": l.M, "K": l.K, "N": l.N} for l in wl.linears],
                   "scaling": wl.scaling, "amax_algo": args.algo, "rotating_input_sets": R,
                   "inputs": "X~N(0,1), W~N(0,1/K), dY~N(0,1e-3) bf16, seeded"
                             + (f"; {wl.outlier_fraction:.1%} of X x{wl.outlier_multiplier:g}"
                                if wl.outlier_fraction else "")},
        "fwd_bwd_us": round(ms_per_step * 1e3, 2),
        "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps,
                   "what": "untimed steps run for this wall-clock time before the warm-up (clock settling)"},
        "host_wall_s_timed": round(t_host, 4),
    }
    if args.workload in H100_US:
        h100_us = H100_US[args.workload]
        out["h100_context"] = {"fwd_bwd_us": h100_us, "tflops": round(flops / (h100_us * 1e-6) / 1e12, 1),
                               "what": "the pages' H100 float8nocompile ATOMIC_MAX figure for this shape (single-"
                                       "linear table, read as microseconds): another machine, context only"}

    if args.only_timed:
        print(json.dumps(out), flush=True)
        return

    # ---- the two amax algorithms, in alternating timed blocks after the same settle
    if not delayed:
        blocks = {"atomic": [], "twopass": []}
        nb = max(args.steps, 10)
        for r in range(args.algo_rounds):
            order = ("twopass", "atomic") if r % 2 == 0 else ("atomic", "twopass")
            for algo in order:
                run(2, algo)  # the first steps after a switch are not timed
                blocks[algo].append(timed(nb, algo) * 1e3)
        out["fwd_bwd_us_by_amax_algo"] = {
            a: {"median_us": round(float(np.median(v)), 2), "blocks_us": [round(x, 2) for x in v]}
            for a, v in blocks.items()}
        out["fwd_bwd_us_by_amax_algo"]["what"] = (f"{args.algo_rounds} rounds of one {nb}-step block per algorithm, "
                                                  "alternating which goes first")

    out.update(instrumented(args, wl, bufs, sets, step, t_next, f8lin, torch, stream, delayed))
    rl = out["kernels"]["gemm_bwd"]
    traffic = load_traffic(os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "csrc", "gemm.hip"),
                           args.workload)
    out["roofline"] = {"kernel": rl["kernel"], "bound": "mfma", "achieved": rl["tflops"],
                       "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(rl["tflops"] / PEAK_FP8_TFLOPS, 4),
                       "traffic": (traffic["hbm_bytes_per_launch"] if traffic else None),
                       "algorithmic_bytes_per_launch": rl["algorithmic_bytes_per_launch"],
                       "flops_per_launch": rl["flops_per_launch"],
                       "timing": "HIP events that f8lin_backward records on its stream around the GEMM launch it "
                                 "issues (ev_gemm_begin / ev_gemm_end), averaged over the instrumented steps"}
    if traffic:
        out["roofline"]["traffic_note"] = traffic.get("note", "")
    if not delayed:
        out["epilogue_amax"] = epilogue_amax(wl, bufs, sets, f8lin, torch, stream)
    out["hbm_copy_reference"] = copy_reference(torch, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, wl, sets, np, torch)
    print(json.dumps(out), flush=True)


def ceilings(torch, f8lin):
    """The chip's ceilings for the path's two bounds, from kernels shaped like
    the path's own (libf8lin_probe.so), each after a settle and timed with HIP
    events: (1) HBM streaming with 128-bit accesses over 1 GiB (larger than the
    256 MB last-level cache), read only, write only and copy, over a few grid
    shapes (the best is the ceiling); (2) fp8 MFMA issue from registers, eight
    waves per CU, with the shader clock each workgroup read, on constant and on
    random operands, and the same MFMAs fed from LDS as the GEMM's K loop feeds
    them (without its global copies); (3) the product GEMM at one tile per CU
    and a long contraction (4096 x 4096 x 65408 and x 16384), where its K loop
    is nearly all of the launch.  Random operand codes are finite, of either
    sign and every exponent."""
    import ctypes
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = torch.cuda.current_stream()
    lib = ctypes.CDLL(os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "libf8lin_probe.so"))
    lib.f8probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.f8probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    lib.f8probe_mfma_lds.argtypes = lib.f8probe_mfma.argtypes
    lib.f8probe_mfma_shape.argtypes = [ctypes.c_int] + lib.f8probe_mfma.argtypes

    def timed(fn, reps):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us

    out = {"what": "ceilings of this GPU, measured by bench.py --ceilings"}
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    red = torch.zeros(4096, dtype=torch.int32, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:  # settle
        assert lib.f8probe_stream(2, src.data_ptr(), dst.data_ptr(), nbytes, 1024, 256, None, s.cuda_stream) == 0
        torch.cuda.synchronize()
    shapes = [(256, 512), (512, 512), (1024, 256), (2048, 256), (4096, 256)]
    stream_res = {}
    for mode, name, moved in ((0, "read", 1), (1, "write", 1), (2, "copy", 2)):
        best = None
        per = {}
        for grid, block in shapes:
            def fn():
                r = lib.f8probe_stream(mode, src.data_ptr(), dst.data_ptr(), nbytes, grid, block,
                                       red.data_ptr(), s.cuda_stream)
                assert r == 0, r
            us = timed(fn, 10)
            gbs = moved * nbytes / (us * 1e-6) / 1e9
            per[f"{grid}x{block}"] = round(gbs, 1)
            best = gbs if best is None else max(best, gbs)
        stream_res[name] = {"best_gbs": round(best, 1), "frac_hbm_peak": round(best / PEAK_HBM_GBS, 4),
                            "by_grid": per}
    out["hbm_stream_1gib"] = stream_res
    del src, dst
    torch.cuda.empty_cache()
    # smaller tensors, as the layer workloads have them: cold data (a pool of
    # buffers larger than the last-level cache, rotated), one launch at a time
    # between HIP events, read and copy with the best grid shape above
    by_size = {}
    for mib in (16, 32, 64, 128, 256):
        nb = mib << 20
        pool = max(4, (1 << 30) // nb)
        srcs = torch.ones(pool * nb, dtype=torch.uint8, device=dev).view(pool, nb)
        dsts = torch.empty(pool * nb, dtype=torch.uint8, device=dev).view(pool, nb)
        row = {}
        for mode, name, moved in ((0, "read", 1), (2, "copy", 2)):
            evs = []
            for rep in range(3 * pool):
                i = rep % pool
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(s)
                assert lib.f8probe_stream(mode, srcs[i].data_ptr(), dsts[i].data_ptr(), nb, 256, 512,
                                          red.data_ptr(), s.cuda_stream) == 0
                e1.record(s)
                if rep >= pool:
                    evs.append((e0, e1))
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / len(evs)
            row[name] = {"us": round(us, 2), "gbs": round(moved * nb / (us * 1e-6) / 1e9, 1)}
        by_size[f"{mib}MiB"] = row
        del srcs, dsts
        torch.cuda.empty_cache()
    out["hbm_stream_by_size_cold"] = by_size

    def codes(n, fmt):
        # finite codes of either sign, every exponent (e4m3: 0x7F is NaN;
        # e5m2: 0x7C-0x7F are Inf and NaN), as scaled real data has them
        top = 0x7F if fmt == "e4m3" else 0x7C
        mag = torch.randint(0, top, (n,), dtype=torch.uint8, device=dev)
        return mag | (torch.randint(0, 2, (n,), dtype=torch.uint8, device=dev) << 7)

    grid, iters = 256, 5000
    sink = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * grid, dtype=torch.int64, device=dev)
    ops = codes(grid * 512 * 48 * 4, "e4m3")
    lds_src = codes(131072, "e4m3")

    def mfma_run(fn, flops, what):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            fn()
            torch.cuda.synchronize()
        us = timed(fn, 10)
        c = clocks.view(grid, 2).cpu().double()
        ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1  # cycles per 100 MHz tick
        tf = flops / (us * 1e-6) / 1e12
        return {"tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                "shader_clock_ghz": round(ghz, 3), "us_per_launch": round(us, 1), "what": what}

    reg_flops = grid * 8 * iters * 8 * 131072
    out["mfma_f8_from_registers"] = mfma_run(
        lambda: lib.f8probe_mfma(grid, iters, None, sink.data_ptr(), clocks.data_ptr(), s.cuda_stream),
        reg_flops, "256 workgroups x 8 waves, 8 independent 32x32x64 MFMA chains per wave, small constant operands")
    out["mfma_f8_from_registers_random"] = mfma_run(
        lambda: lib.f8probe_mfma(grid, iters, ops.data_ptr(), sink.data_ptr(), clocks.data_ptr(), s.cuda_stream),
        reg_flops, "the same, operands random finite e4m3 codes of either sign")
    shape_ops = codes(grid * 256 * 128 * 4, "e4m3")
    sink4 = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    for shape, name, kdepth in ((0, "32x32x64", 64), (1, "16x16x128", 128)):
        out[f"mfma_f8_{name}_one_wave_per_simd_random"] = mfma_run(
            lambda: lib.f8probe_mfma_shape(shape, grid, iters, shape_ops.data_ptr(), sink4.data_ptr(),
                                           clocks.data_ptr(), s.cuda_stream),
            grid * 4 * iters * 2 * 128 * 128 * kdepth,
            f"256 workgroups x 4 waves (one per SIMD), 128 x 128 outputs per wave as {name} MFMAs from registers, "
            "operands random finite e4m3 codes of either sign")
    del shape_ops, sink4
    lds_iters = iters // 2
    out["mfma_f8_from_lds"] = mfma_run(
        lambda: lib.f8probe_mfma_lds(grid, lds_iters, lds_src.data_ptr(), sink.data_ptr(), clocks.data_ptr(),
                                     s.cuda_stream),
        grid * 8 * lds_iters * 16 * 131072,
        "the GEMM's K loop without its global copies: 128 x 64 wave tiles, fragments read from two 64 KB LDS stages "
        "of random codes, one barrier per 128-byte K block")
    del ops, lds_src
    # the GEMM's own K loop: one 256 x 256 tile per CU, long contraction
    loop = {}
    for K in (65408, 16384):
        a = codes(4096 * K, "e5m2").view(4096, K)
        b = codes(4096 * K, "e4m3").view(4096, K)
        cc = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
        one = torch.ones(1, dtype=torch.float32, device=dev)

        def g():
            f8lin.gemm(a, "e5m2", b, "e4m3", one, one, cc)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            g()
            torch.cuda.synchronize()
        us = timed(g, 5)
        loop[f"4096x4096x{K}"] = {"us": round(us, 1), "tflops": round(2 * 4096 * 4096 * K / (us * 1e-6) / 1e12, 1)}
        del a, b, cc
    out["gemm_k_loop"] = loop
    return out


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


def instrumented(args, wl, bufs, sets, step, t_next, f8lin, torch, stream, delayed):
    """Per-call and per-GEMM durations of the real step, with HIP events on
    the launch stream: around each f8lin_forward / f8lin_backward call as the
    step issues it, and the events each call records around its own GEMM
    launch (so the GEMM figures are those of the launches the path issues:
    the backward's work-queue or split launches included).  A call's time
    minus its GEMM's is its amax + cast phase, whose algorithmic bytes are
    2 B/element for each dynamic-mode amax pass and 4 B/element for each
    cast.  Then both amax algorithms alone (f8lin_amax) on the step's
    tensors."""
    lin = wl.linears
    warm, steps = 2, min(max(args.steps, 5), 20)
    recorded = []
    for t in range(warm + steps):
        ev = []
        step(t_next[0], args.algo, ev)
        mode = "delayed" if (delayed and t_next[0] > 0) else "dynamic"
        t_next[0] += 1
        if t >= warm:
            recorded.append((ev, mode))
    torch.cuda.synchronize()
    acc = {k: [0.0, 0, 0.0, 0.0] for k in ("fwd_call", "bwd_call", "gemm_fwd", "gemm_bwd")}  # ms, n, work, bytes
    for ev, mode in recorded:
        per = 6 if mode == "dynamic" else 4  # amax pass (dynamic) + cast, bytes per element
        for kind, call, gemm, g in ev:
            t_call = call[0].elapsed_time(call[1])
            t_gemm = gemm[0].elapsed_time(gemm[1])
            ls = [lin[i] for i in g]
            if kind == "fwd":
                l0 = ls[0]
                cast_b = per * (l0.M * l0.K + sum(l.N * l.K for l in ls))  # X once, each W
                gflop = sum(2 * l.M * l.N * l.K for l in ls)
                gbytes = sum(l.M * l.K + l.N * l.K + 2 * l.M * l.N for l in ls)
                key = "fwd"
            else:
                l = ls[0]
                cast_b = per * l.M * l.N
                gflop = 4 * l.M * l.N * l.K
                gbytes = (l.M * l.N + l.N * l.K + 2 * l.M * l.K) + (l.M * l.N + l.M * l.K + 2 * l.N * l.K)
                key = "bwd"
            a = acc[key + "_call"]
            a[0] += t_call
            a[1] += 1
            a[2] += cast_b
            b = acc["gemm_" + key]
            b[0] += t_gemm
            b[1] += 1
            b[2] += gflop
            b[3] += gbytes
    k = {}
    for name, kern in (("gemm_fwd", "gemm_fp8_tn_kernel<e4m3,e4m3> (forward; one launch per call)"),
                       ("gemm_bwd", "gemm_fp8_tn_kernel<e5m2,e4m3> (dgrad + wgrad, the launch f8lin_backward "
                                    "issues)")):
        ms, n, fl, by = acc[name]
        k[name] = {"kernel": kern, "avg_us": round(ms / n * 1e3, 3), "launches": n,
                   "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                   "algorithmic_bytes_per_launch": int(by / n), "flops_per_launch": int(fl / n)}
    for side in ("fwd", "bwd"):
        ms_call, n, by, _ = acc[side + "_call"]
        ms_ew = ms_call - acc["gemm_" + side][0]
        k["amax_cast_" + side] = {"avg_us": round(ms_ew / n * 1e3, 3), "calls": n,
                                  "call_avg_us": round(ms_call / n * 1e3, 3),
                                  "gbs": round(by / (ms_ew * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(by / (ms_ew * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "algorithmic_bytes_per_call": int(by / n),
                                  "what": ("amax pass(es) + cast of X and W" if side == "fwd" else
                                           "amax pass + cast of dY") + " = call time minus its GEMM launch"}
    # amax alone, both algorithms, alternating, on the step's X, W and dY (first input set)
    per_algo = {"atomic": [0.0, 0, 0], "twopass": [0.0, 0, 0]}
    word = torch.zeros(1, dtype=torch.float32, device=bufs[0].ws.device)
    pend = []
    for rep in range(12):
        for algo in (("atomic", "twopass") if rep % 2 == 0 else ("twopass", "atomic")):
            for b, (_, x, w, dy) in zip(bufs, sets[0]):
                for tensor in (x, w, dy):
                    a = torch.cuda.Event(enable_timing=True)
                    e = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    f8lin.amax(tensor, word, b.ws, algo)
                    e.record(stream)
                    if rep >= 2:
                        pend.append((algo, a, e, tensor.numel()))
    torch.cuda.synchronize()
    for algo, a, e, n in pend:
        v = per_algo[algo]
        v[0] += a.elapsed_time(e)
        v[1] += 1
        v[2] += n
    for algo, (ms, n, el) in per_algo.items():
        k["amax_" + algo] = {"avg_us": round(ms / n * 1e3, 3), "launches": n,
                             "gbs": round(2 * el / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(2 * el / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "bytes_per_elem": 2,
                             "what": "f8lin_amax alone on the step's X, W and dY, the algorithms alternating"}
    return {"kernels": k}


def epilogue_amax(wl, bufs, sets, f8lin, torch, stream, reps=12):
    """The amax taken in the GEMM epilogue (y_amax) against the amax pass it
    spares the next layer, on the workload's first linear: the forward call
    with and without x_amax_given (its X amax already in the state), and the
    forward GEMM launch with and without y_amax.  Alternating, events on the
    launch stream."""
    l, x, w, _ = sets[0][0]
    b = bufs[0]
    word = torch.zeros(1, dtype=torch.float32, device=x.device)
    f8lin.forward(x, w, b.y, b.x8, b.x8t, b.w8, b.w8t, b.sx, b.sw, b.ws, algo="twopass")  # sx.amax = amax(X)
    res = {"call": [], "call_given": [], "gemm": [], "gemm_y_amax": []}
    pend = []
    for r in range(reps):
        for given in ((False, True) if r % 2 == 0 else (True, False)):
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            c0.record(stream)
            f8lin.forward(x, w, b.y, b.x8, b.x8t, b.w8, b.w8t, b.sx, b.sw, b.ws, algo="twopass",
                          x_amax_given=given, gemm_events=g, y_amax=word if given else None)
            c1.record(stream)
            if r >= 2:
                pend.append((given, c0, c1, g))
    torch.cuda.synchronize()
    for given, c0, c1, g in pend:
        res["call_given" if given else "call"].append(c0.elapsed_time(c1) * 1e3)
        res["gemm_y_amax" if given else "gemm"].append(g[0].elapsed_time(g[1]) * 1e3)
    avg = {k: round(sum(v) / len(v), 3) for k, v in res.items()}
    return {"linear": {"name": l.name, "M": l.M, "K": l.K, "N": l.N},
            "fwd_call_us": avg["call"], "fwd_call_us_x_amax_given": avg["call_given"],
            "x_amax_pass_saved_us": round(avg["call"] - avg["call_given"], 3),
            "gemm_fwd_us": avg["gemm"], "gemm_fwd_us_with_y_amax": avg["gemm_y_amax"],
            "what": "forward call with X's amax pass vs with amax(X) handed in (x_amax_given), and its GEMM launch "
                    "without vs with the epilogue amax of Y (y_amax); alternating calls, HIP events"}


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
