#!/usr/bin/env python3
"""Benchmark of the LC-VQ hot path on one MI355X.

Headline: one LC-VQ linear training step -- quantize + folded forward product
(lcvq_linear_fwd) and the straight-through backward (lcvq_linear_bwd: dX, dWp, dA, dB)
-- on the 4096 x 4096 weight with 4096 bf16 tokens and d = 8, reported as TFLOP/s over
the algorithmic 6 M N K flops. Inputs are seeded synthetic tensors already resident in
HBM. Also measured in the same run:
  * per-kernel durations with HIP events (the library's profiling hook), and the roofline
    of the dominant product kernel against the bf16 dense matrix-core peak;
  * the packed 2-bit decode product on {4096x4096, 14336x4096, 4096x14336} x M in
    {1, 4, 16}, cycling over >= 512 MiB of distinct code copies so the 256 MB
    last-level cache cannot serve them, against the HBM peak;
  * the CPU oracle on the same step (the full 4096-token step on the host cores).
Prints one JSON line.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--clock-warmup-s 0.5]

Before the W warmup steps the step runs untimed for --clock-warmup-s seconds of wall
time: the GPU starts from its idle clock state, and the shader clock needs tens of
milliseconds of load to reach its working level (with 5 warmup steps and no clock
warm-up the timed steps ran about 18% slower than sustained back-to-back steps).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
KERNELS = {1: "quantize_prologue", 2: "fwd_product", 6: "bwd_prologue", 3: "dx_product",
           4: "dw_product"}

# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE, WRITE_SIZE, each
# scaled by what it reads for a copy of known size). They are valid only for the kernel
# sources they were taken on; the summary records those sources' SHA-256.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "train_step_4096x4096_m4096_d8_hbm_counters.md")
CSRC = os.path.join(ROOT, "bit_weight_only_lc_amd", "csrc")
KERNEL_SOURCES = {
    "products": ["gemm_kernels.hip", "lcvq_device.h", "lcvq_internal.h"],
    "quantize": ["quant_kernels.hip", "lcvq_device.h", "lcvq_internal.h"],
}
SOURCE_GROUP = {"quantize_prologue": "quantize", "fwd_product": "products",
                "dx_product": "products", "dw_product": "products"}


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    the summary is missing or the kernel's sources changed since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    group = SOURCE_GROUP[kernel]
    if rec.get("sources_sha256", {}).get(group) != source_digest(KERNEL_SOURCES[group]):
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--clock-warmup-s", type=float, default=0.5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--no-copy-probe", action="store_true")
    return ap.parse_args()


def timed_events(torch, n):
    evs = []
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return evs


def clock_warmup(torch, fn, seconds):
    """Runs fn, untimed, until `seconds` of wall time have passed; returns the call count."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    return n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of the path is described, not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_lc_amd as P
    import synth_inputs as SI

    L = P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- training step
    c = SI.CONFIGS["c1_square_4096"]
    (N, K), M, d = c["mats"][0], c["M"], c["d"]
    inp = SI.make_layer(N, K, M, d, seed=1000, device=dev)
    X, Wp, A, B, dY = (inp[k] for k in ("X", "Wp", "A", "B", "dY"))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    mask = torch.empty((N, K // 8), dtype=torch.uint8, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dWp = torch.empty((N, K), dtype=torch.float32, device=dev)
    dA = torch.empty((d, d), dtype=torch.float32, device=dev)
    dB = torch.empty((d,), dtype=torch.float32, device=dev)
    wsf = torch.empty(P.lcvq_linear_fwd_workspace_size(M, N, K, d), dtype=torch.uint8, device=dev)
    wsb = torch.empty(P.lcvq_linear_bwd_workspace_size(M, N, K, d), dtype=torch.uint8, device=dev)

    def step():
        P.lcvq_linear_fwd(X, Wp, A, B, d, Y, packed, mask, None, wsf)
        P.lcvq_linear_bwd(dY, X, packed, mask, A, B, d, dX, dWp, dA, dB, wsb)

    kern_ids = list(KERNELS.items())
    step_evs = timed_events(torch, args.steps)
    clock_steps = clock_warmup(torch, step, args.clock_warmup_s)
    for _ in range(args.warmup):
        step()
    # Per-kernel durations come from the timed steps themselves: step i arms the timing
    # hook for kernel number i mod 5 of KERNELS, whose launch is then bracketed by two
    # events on the library's stream, so they are the durations that make up the measured
    # step time.
    kern_evs = {name: [] for _, name in kern_ids}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        kid, name = kern_ids[i % len(kern_ids)]
        a, b = step_evs[i]
        L.lcvq_profile_next(kid, a.cuda_event, b.cuda_event)
        step()
        kern_evs[name].append((a, b))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / args.steps
    flops = 6.0 * M * N * K

    # The same step captured once in a HIP graph and replayed: it removes the host-side
    # launch path between the eight kernels. Replays are checked against the eager step
    # (the library is deterministic, so the bytes must agree).
    ref = [t.clone() for t in (Y, dX, dWp, dA, dB)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    for a_, b_ in zip(ref, (Y, dX, dWp, dA, dB)):
        if not torch.equal(a_, b_):
            raise RuntimeError("graph replay differs from the eager step")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_graph = (t1 - t0) * 1e3 / args.steps
    ms = min(ms_eager, ms_graph)
    tflops = flops / (ms * 1e-3) / 1e12

    # the same step with the DGE estimator in the backward (sharpness 8)
    def step_dge():
        P.lcvq_linear_fwd(X, Wp, A, B, d, Y, packed, mask, None, wsf)
        P.lcvq_linear_bwd_dge(dY, X, packed, mask, Wp, 8.0, A, B, d, dX, dWp, dA, dB, wsb)

    for _ in range(args.warmup):
        step_dge()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_dge()
    torch.cuda.synchronize()
    ms_dge = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-kernel durations: the timed steps' samples; a kernel that got none (fewer
    # timed steps than kernels) is timed over --profile-steps extra steps
    kern = {}
    for kid, name in KERNELS.items():
        evs = kern_evs[name]
        if not evs:
            evs = timed_events(torch, args.profile_steps)
            for a, b in evs:
                L.lcvq_profile_next(kid, a.cuda_event, b.cuda_event)
                step()
            torch.cuda.synchronize()
        kern[name] = sum(a.elapsed_time(b) for a, b in evs) / len(evs)   # ms
    gemm_flops = 2.0 * M * N * K
    prods = {k: kern[k] for k in ("fwd_product", "dx_product", "dw_product")}
    dom = max(prods, key=prods.get)
    achieved = gemm_flops / (prods[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(dom),
                "per_kernel_ms": {k: round(v, 4) for k, v in kern.items()},
                "per_product_tflops": {k: round(gemm_flops / (v * 1e-3) / 1e12, 1)
                                       for k, v in prods.items()}}
    # one launch: Wp read; packed codes, mask bits, GEMM code words written; X read and
    # X' written (bf16), one float per row
    q_bytes = N * K * (4 + 0.25 + 0.125 + 0.25) + M * K * (2 + 2) + M * 4
    roofline["quantize_prologue_gbs"] = round(q_bytes / (kern["quantize_prologue"] * 1e-3) / 1e9, 1)

    # ---------------------------------------------------------------- decode product
    decode = None
    if not args.no_decode:
        decode = {}
        clock_warmup(torch, step, min(args.clock_warmup_s, 0.2))
        for (n, k) in SI.CONFIGS["c3_decode"]["mats"]:
            wp = SI.make_wp(n, k, seed=3000 + n + k, device=dev)
            pk0 = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
            P.lcvq_quantize(wp, None, pk0, None)
            del wp
            copies = max(2, -(-(512 << 20) // pk0.numel()))
            A16, B16 = (t.half().to(dev) for t in SI.make_ab(8, seed=3000))
            # layout 0: canonical packed codes; layout 1: the decode layout written once by
            # lcvq_gemv2b_shuffle (weight preparation, outside the timed calls)
            for layout in (0, 1):
                pool = [P.gemv2b_shuffle(pk0) if layout else pk0.clone() for _ in range(copies)]
                call = P.lcvq_gemv2b_shuffled if layout else P.lcvq_gemv2b
                for m in SI.CONFIGS["c3_decode"]["Ms"]:
                    Xd = SI.make_act(m, k, seed=3100 + m, device=dev)
                    Yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                    ws = torch.empty(P.lcvq_gemv2b_workspace_size(m, n, k, 8),
                                     dtype=torch.uint8, device=dev)
                    calls = 2 * copies
                    for i in range(copies):
                        call(Xd, pool[i], A16, B16, 8, Yd, ws)
                    evs = timed_events(torch, calls)
                    for i, (a, b) in enumerate(evs):
                        L.lcvq_profile_next(5, a.cuda_event, b.cuda_event)
                        call(Xd, pool[i % copies], A16, B16, 8, Yd, ws)
                    torch.cuda.synchronize()
                    t_k = sum(a.elapsed_time(b) for a, b in evs) / calls * 1e-3
                    w0 = torch.cuda.Event(enable_timing=True)
                    w1 = torch.cuda.Event(enable_timing=True)
                    w0.record()
                    for i in range(calls):
                        call(Xd, pool[i % copies], A16, B16, 8, Yd, ws)
                    w1.record()
                    torch.cuda.synchronize()
                    t_w = w0.elapsed_time(w1) / calls * 1e-3
                    nbytes = n * k // 4 + 2 * m * k + 2 * m * n + 2 * (64 + 8)
                    rec = {"bytes": nbytes, "kernel_us": round(t_k * 1e6, 2),
                           "kernel_gbs": round(nbytes / t_k / 1e9, 1),
                           "frac": round(nbytes / t_k / 1e9 / PEAK_HBM_GBS, 4),
                           "call_us": round(t_w * 1e6, 2),
                           "call_gbs": round(nbytes / t_w / 1e9, 1)}
                    if layout:
                        decode[f"{n}x{k}_M{m}"]["decode_layout"] = rec
                    else:
                        decode[f"{n}x{k}_M{m}"] = rec
            del pool
            torch.cuda.empty_cache()

    # ------------------------------------------------- decode step of an 8B-shaped stack
    # One token through all 7 projections of 32 layers (1.63 GiB of codes, far beyond the
    # last-level cache), as 224 single calls, as 128 calls that group the matrices sharing
    # an input (q, k, v and gate, up) into one launch each, and as the same 128 calls on
    # codes prepared once in the decode layout (lcvq_gemv2b_shuffle, outside the timing).
    decode_stack = None
    if not args.no_decode:
        shapes = SI.CONFIGS["c4_stack_8b_layer"]["mats"]     # q, k, v, o, gate, up, down
        layers = SI.CONFIGS["c4_stack_8b_layer"]["layers"]
        dd = 8
        gen = torch.Generator(device=dev).manual_seed(7000)
        xs = {k: SI.make_act(1, k, seed=7100 + k, device=dev) for k in {k for _, k in shapes}}
        A16, B16 = (t.half().to(dev) for t in SI.make_ab(dd, seed=7200))
        mats = []
        for _ in range(layers):
            mats.append([(torch.randint(0, 256, (n, k // 4), generator=gen, dtype=torch.uint8,
                                        device=dev),
                          torch.empty((1, n), dtype=torch.bfloat16, device=dev), k)
                         for n, k in shapes])
        ws_s = torch.empty(P.lcvq_gemv2b_workspace_size(1, 14336, 14336, dd), dtype=torch.uint8,
                           device=dev)
        groups = [[0, 1, 2], [3], [4, 5], [6]]
        total_bytes = layers * sum(n * k // 4 for n, k in shapes)

        def run_single():
            for lay in mats:
                for pk, y, k in lay:
                    P.lcvq_gemv2b(xs[k], pk, A16, B16, dd, y, ws_s)

        def grouped(stack, layout):
            one = P.lcvq_gemv2b_shuffled if layout else P.lcvq_gemv2b

            def run():
                for lay in stack:
                    for g in groups:
                        k = lay[g[0]][2]
                        if len(g) == 1:
                            pk, y, _ = lay[g[0]]
                            one(xs[k], pk, A16, B16, dd, y, ws_s)
                        else:
                            P.lcvq_gemv2b_batched(
                                xs[k], [(lay[i][0], A16, B16, lay[i][1], layout) for i in g],
                                dd, ws_s)
            return run

        mats_dl = [[(P.gemv2b_shuffle(pk), y, k) for pk, y, k in lay] for lay in mats]
        run_grouped = grouped(mats, 0)

        decode_stack = {"codes_bytes": total_bytes, "layers": layers, "tokens": 1}
        for name, fn, calls in (("single", run_single, layers * 7),
                                ("grouped", run_grouped, layers * len(groups)),
                                ("grouped_decode_layout", grouped(mats_dl, 1),
                                 layers * len(groups))):
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t_s = e0.elapsed_time(e1) / reps * 1e-3
            # the same calls captured once in a HIP graph (no host work per call); the
            # replayed outputs must equal the eager ones
            ref = [y.clone() for lay in mats for _, y, _ in lay]
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for lay in mats:
                for _, y, _ in lay:
                    y.zero_()
            g.replay()
            torch.cuda.synchronize()
            got = [y for lay in mats for _, y, _ in lay]
            if not all(torch.equal(a_, b_) for a_, b_ in zip(ref, got)):
                raise RuntimeError("decode graph replay differs from the eager calls")
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t_g = e0.elapsed_time(e1) / reps * 1e-3
            del g
            decode_stack[name] = {"calls": calls, "ms": round(t_s * 1e3, 3),
                                  "gbs": round(total_bytes / t_s / 1e9, 1),
                                  "frac": round(total_bytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
                                  "graph_ms": round(t_g * 1e3, 3),
                                  "graph_gbs": round(total_bytes / t_g / 1e9, 1),
                                  "graph_frac": round(total_bytes / t_g / 1e9 / PEAK_HBM_GBS, 4)}
        del mats, mats_dl
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- HBM copy ceiling
    # A plain device-to-device copy of 1 GiB: the streaming ceiling measured beside the
    # decode product, and the kernel of known size that scales the HBM byte counters.
    copy_probe = None
    if not args.no_copy_probe:
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev).random_(0, 256)
        dst = torch.empty_like(src)
        dst.copy_(src)
        reps = 10
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(reps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        t_c = c0.elapsed_time(c1) / reps * 1e-3
        copy_probe = {"bytes_read": nb, "bytes_written": nb, "us": round(t_c * 1e6, 1),
                      "gbs": round(2 * nb / t_c / 1e9, 1)}
        del src, dst
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import lcvq_oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max(i.get("num_threads", 1) for i in threadpool_info())
        except Exception:
            cores = os.cpu_count()
        Xh = X.double().cpu().numpy()
        dYh = dY.double().cpu().numpy()
        wph = Wp.cpu().numpy()
        Ah, Bh = A.double().cpu().numpy(), B.double().cpu().numpy()
        reps, tot = 0, 0.0
        while reps < 3 and (reps == 0 or tot < 10.0):
            t = time.perf_counter()
            f = O.linear_fwd(Xh, wph, Ah, Bh, d)
            O.linear_bwd(dYh, Xh, f["z"], f["m"], Ah, Bh, d)
            tot += time.perf_counter() - t
            reps += 1
        cpu = {"value": round(flops / (tot / reps) / 1e12, 4), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"the full step (4096x4096 weight, 4096 tokens, d=8: quantize, "
                         f"decode, forward, dX, dWp, dA, dB) in float64, {reps} run(s), "
                         f"{tot / reps:.2f} s each"}

    out = {
        "metric": "LC-VQ linear fwd+bwd TFLOP/s (4096²×4096 tok); 2-bit decode GEMV HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup": {"seconds": args.clock_warmup_s, "steps": clock_steps},
        "ms_per_step": round(ms, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": round(ms_graph, 4),
        "ms_per_step_dge": round(ms_dge, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Wp ~ U[-0.5,3.5), A = 0.02 I + 0.002 N(0,1) off-diagonal, "
                "B ~ 0.01 N(0,1), X, dY ~ N(0,1) in bf16)",
        "config": {"workload": "LC-VQ linear layer W[4096,4096], d=8, 4096 bf16 tokens, "
                               "quantize + forward + straight-through backward",
                   "M": M, "N": N, "K": K, "d": d},
        "roofline": roofline,
        "decode": decode,
        "decode_stack_8b": decode_stack,
        "hbm_copy_probe": copy_probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
