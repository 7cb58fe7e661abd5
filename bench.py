"""Benchmark of the flash-CCE ORPO head on one MI355X.

One step = cce_forward + orpo_epilogue + cce_backward over one batch of the
Gemma-4B-class head workload (M=8192 rows = 2048 prompt + 3072 chosen + 3072
rejected, D=2560, V=262144, bf16 inputs already resident in HBM).  Throughput
is rows (tokens) per second; the FLOP count is 8*M*V*D (forward 2, recompute 2,
dh 2, dW 2).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload gemma4b_head]
                    [--no-cpu-baseline] [--traffic-json profiles/<file>.json]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gemma4b_head")
    ap.add_argument("--filter-eps", type=float, default=None,
                    help="coefficient filter eps (default: the workload's own setting)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="final-logit softcap c (logits c*tanh(z/c)); 0 = off (the metric's config)")
    ap.add_argument("--quant", type=int, default=0, choices=(0, 4, 8),
                    help="affine-quantised frozen head with 4- or 8-bit codes (forward + dh); "
                         "0 = the bf16 head (the metric's config)")
    ap.add_argument("--group", type=int, default=64, help="quantisation group size (with --quant)")
    ap.add_argument("--block-max", action="store_true",
                    help="the forward saves the per-(vocab block, row) maximum and the backward "
                         "decides its block skip from it before recomputing a tile")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "kernel_traffic.json"))
    ap.add_argument("--no-launch-timing", action="store_true",
                    help="time the steps without the library's per-launch events")
    ap.add_argument("--v-sweep", action="store_true",
                    help="time one step and record workspace / peak device memory at "
                         "V in {32768, 65536, 131072, 262144} (M=8192, D=2560); one JSON line per V")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --calibrate-copy run into --traffic-json; no GPU use")
    return ap.parse_args()


TRAFFIC_KERNELS = ("k_fwd", "k_fwd_tall", "k_bwd_fused", "k_grads", "k_recompute_tall")


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str, workload: str):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the head's GEMM kernels,
    averaged per kernel over its dispatches, each scaled by what the same counter
    reads for the 1 GiB copy kernel of the same run (true bytes per counted
    byte)."""
    import csv
    from linear_cross_entropy_forward_amd import binding as B

    def per_dispatch(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        return acc

    def base_name(kname):
        n = kname.split("(")[0].split("<")[0].strip()
        return n.split("::")[-1].split(" ")[-1]

    out = {"workload": workload, "kernel_source_hash": B.kernel_source_hash(), "kernels": {}}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        d = per_dispatch(path, counter)
        copy = [v for (i, n), v in d.items() if "copyBuffer" in n or "copy" in n.lower()]
        copy = [v for v in copy if v > 1e5]          # the 1 GiB copy, not small transfers
        if not copy:
            raise SystemExit(f"{path}: no copy dispatch with {counter}")
        scale = (1 << 30) / (max(copy) * 1024.0)
        for kn in TRAFFIC_KERNELS:
            vals = [v for (i, n), v in d.items() if base_name(n) == kn]
            if not vals:
                continue
            e = out["kernels"].setdefault(kn, {"dispatches": len(vals)})
            e[counter] = {"kib_per_launch": sum(vals) / len(vals), "copy_kib": max(copy),
                          "scale": scale, "bytes_per_launch": sum(vals) / len(vals) * 1024.0 * scale}
    for e in out["kernels"].values():
        if "FETCH_SIZE" in e and "WRITE_SIZE" in e:
            e["bytes_per_launch"] = e["FETCH_SIZE"]["bytes_per_launch"] + e["WRITE_SIZE"]["bytes_per_launch"]
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def host_description():
    """CPU model name and the BLAS numpy calls (for the CPU baseline)."""
    import numpy as np
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return model, blas


def cpu_baseline(wl, rows: int):
    """The fp64 oracle (as it stands) on a bounded row sample of the workload:
    forward, epilogue and backward over the full V and D for `rows` rows."""
    import numpy as np
    from linear_cross_entropy_forward_amd import workloads as WL
    from oracle import cce_oracle as O

    # a single-pair sample with the workload's span proportions
    kinds = wl.seg & 3
    idx = []
    for k in (WL.KIND_PROMPT, WL.KIND_CHOSEN, WL.KIND_REJECTED):
        sel = np.nonzero(kinds == k)[0]
        take = max(1, int(round(rows * len(sel) / wl.M)))
        idx.append(sel[:take])
    idx = np.concatenate(idx)[:rows]
    seg = np.where((wl.seg[idx] & 3) == WL.KIND_IGNORE, WL.KIND_IGNORE, wl.seg[idx] & 3).astype(np.int32)
    H = WL.bf16_bits_to_f32(wl.h_bits[idx]).astype(np.float64)
    W = wl.W64()
    y = wl.y[idx]
    t0 = time.perf_counter()
    O.step(H, W, y, seg, 1, wl.lam, wl.scope, wl.filter_eps)
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    model, blas = host_description()
    return {"value": len(idx) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"{len(idx)} rows of {wl.name} (one pair, same span mix), full V={wl.V} and "
                      f"D={wl.D}; fp64 forward+epilogue+backward; {dt:.2f} s"}


def v_sweep(steps: int):
    """Workspace and peak device memory against V at the Gemma-4B head's M and D.

    Inputs and outputs grow with V (W, dW); the workspace must not.  Reported per
    V: workspace bytes (what the library needs besides inputs and outputs), the
    torch peak allocated during a step minus the inputs and outputs, and the
    step time."""
    import torch
    from linear_cross_entropy_forward_amd import binding as B
    from linear_cross_entropy_forward_amd import workloads as WL
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.zeros(1, device=dev)  # initialise the context and the caching allocator
    for V in (32768, 65536, 131072, 262144):
        wl = WL.make_workload("gemma4b_head", V=V)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base0 = torch.cuda.memory_allocated(dev)
        h = B.to_device_bits(wl.h_bits, dev)
        W = B.to_device_bits(wl.W_bits, dev)
        y = torch.from_numpy(wl.y).to(dev)
        seg = torch.from_numpy(wl.seg).to(dev)
        dh = torch.empty((wl.M, wl.D), dtype=torch.float32, device=dev)
        dW = torch.empty((wl.V, wl.D), dtype=torch.float32, device=dev)
        logp = torch.empty(wl.M, dtype=torch.float32, device=dev)
        lse = torch.empty_like(logp)
        coef = torch.empty_like(logp)
        out5 = torch.empty(5, dtype=torch.float32, device=dev)
        pst = torch.empty((wl.n_pairs, 8), dtype=torch.float32, device=dev)
        io_bytes = torch.cuda.memory_allocated(dev) - base0
        head = B.Head(wl.M, wl.V, wl.D, dev)

        def one():
            head.forward(h, W, y, logp, lse)
            head.epilogue(logp, y, seg, wl.n_pairs, wl.lam, wl.scope, out5, pst, coef)
            head.backward(h, W, y, lse, coef, 0.0, 0.0, dh, dW)

        for _ in range(2):
            one()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            one()
        e.record()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base0
        rec = {"V": V, "M": wl.M, "D": wl.D, "workspace_bytes": B.workspace_bytes(wl.M, V, wl.D),
               "inputs_outputs_bytes": io_bytes,
               "peak_minus_inputs_outputs_bytes": peak - io_bytes,
               "ms_per_step": round(s.elapsed_time(e) / steps, 3),
               "tflops": round(8.0 * wl.M * V * wl.D / (s.elapsed_time(e) / steps * 1e-3) / 1e12, 1),
               "status": head.read_status()}
        print(json.dumps(rec), flush=True)
        del h, W, y, seg, dh, dW, logp, lse, coef, out5, pst, head
        torch.cuda.empty_cache()


def filter_deviation(head, h, W, y, lse, coef, feps, dh, dW, bwd_ms, softcap, bmax, stream):
    """How far the filtered gradient of the timed steps (in dh, dW) is from the
    exact one, both from the library (relative L2 over every entry), and the
    backward's effective speed-up (exact backward time over the filtered one,
    medians of a few backward calls each, outside the timed region)."""
    import numpy as np
    import torch
    dh_x, dW_x = head.backward(h, W, y, lse, coef, 0.0, 0.0, stream=stream, softcap=softcap)
    torch.cuda.synchronize()

    def rl2(a, b):
        return float(torch.linalg.vector_norm((a - b).double()) / torch.linalg.vector_norm(b.double()))

    dev = {"eps": feps, "dh_rel_l2_vs_exact": rl2(dh, dh_x), "dW_rel_l2_vs_exact": rl2(dW, dW_x),
           "reference": "the library's own exact backward (filter and block skip off) on the same inputs"}
    del dW_x
    torch.cuda.empty_cache()
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        head.backward(h, W, y, lse, coef, 0.0, 0.0, dh_x, dW, stream=stream, softcap=softcap)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    dev["backward_ms_exact"] = round(float(np.median(times)), 4)
    dev["backward_ms_filtered"] = round(bwd_ms, 4)
    dev["speedup"] = round(dev["backward_ms_exact"] / bwd_ms, 4)
    return dev


def head_bytes_per_step(V, D, bits, group):
    """Algorithmic bytes of the head moved per step (each pass reads it once).
    bf16: the forward, the recompute and the dh contraction each read V x D bf16.
    Quantised: the forward and the backward each dequantise the head once (codes,
    bf16 scales and biases read; a bf16 chunk buffer written), and the three
    contractions read the chunk buffers; the frozen head has no dW."""
    bf16 = V * D * 2
    if not bits:
        return {"bf16_head_read": 3 * bf16, "total": 3 * bf16}
    packed = V * D * bits // 8 + V * (D // group) * 2 * 2
    out = {"packed_read": 2 * packed, "chunk_buffer_write": 2 * bf16,
           "chunk_buffer_read": 3 * bf16}
    out["total"] = sum(out.values())
    out["bf16_head_equivalent"] = 3 * bf16
    return out


def main():
    args = parse()
    if args.v_sweep:
        v_sweep(max(1, min(args.steps, 5)))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.traffic_json, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the head is built and "
              f"measured on a single MI355X, with no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from linear_cross_entropy_forward_amd import binding as B
    from linear_cross_entropy_forward_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WL.make_workload(args.workload)
    feps = wl.filter_eps if args.filter_eps is None else args.filter_eps
    print(f"[bench] workload {wl.name} M={wl.M} V={wl.V} D={wl.D} filter_eps={feps}",
          file=sys.stderr, flush=True)
    quant = args.quant != 0
    head = B.Head(wl.M, wl.V, wl.D, dev, quantized=quant)
    h = B.to_device_bits(wl.h_bits, dev)
    if quant:
        print(f"[bench] quantising the head to {args.quant}-bit codes, group {args.group} (host)",
              file=sys.stderr, flush=True)
        qh = WL.quantize_affine(WL.bf16_bits_to_f32(wl.W_bits), args.quant, args.group)
        Wq = torch.from_numpy(qh.Wq.view(np.int32)).to(dev)
        Ws = B.to_device_bits(qh.scale_bits, dev)
        Wb = B.to_device_bits(qh.bias_bits, dev)
        del qh
        W = None
    else:
        W = B.to_device_bits(wl.W_bits, dev)
    y = torch.from_numpy(wl.y).to(dev)
    seg = torch.from_numpy(wl.seg).to(dev)
    logp = torch.empty(wl.M, dtype=torch.float32, device=dev)
    lse = torch.empty_like(logp)
    coef = torch.empty_like(logp)
    out5 = torch.empty(5, dtype=torch.float32, device=dev)
    pst = torch.empty((wl.n_pairs, 8), dtype=torch.float32, device=dev)
    dh = torch.empty((wl.M, wl.D), dtype=torch.float32, device=dev)
    dW = None if quant else torch.empty((wl.V, wl.D), dtype=torch.float32, device=dev)
    bmax = (torch.empty(B.block_max_shape(wl.M, wl.V), dtype=torch.float32, device=dev)
            if args.block_max else None)
    stream = torch.cuda.current_stream()

    def one_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if quant:
            head.forward_q(h, Wq, Ws, Wb, args.quant, args.group, y, logp, lse, stream=stream,
                           softcap=args.softcap, block_max=bmax)
        else:
            head.forward(h, W, y, logp, lse, stream=stream, softcap=args.softcap, block_max=bmax)
        if ev is not None:
            ev[1].record(stream)
        head.epilogue(logp, y, seg, wl.n_pairs, wl.lam, wl.scope, out5, pst, coef, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if quant:
            head.backward_q(h, Wq, Ws, Wb, args.quant, args.group, y, lse, coef, feps, feps, dh,
                            stream=stream, softcap=args.softcap, block_max=bmax)
        else:
            head.backward(h, W, y, lse, coef, feps, feps, dh, dW, stream=stream,
                          softcap=args.softcap, block_max=bmax)
        if ev is not None:
            ev[3].record(stream)

    head.clear_status()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    status = head.read_status()
    print(f"[bench] warmup done, status={status}", file=sys.stderr, flush=True)

    # pass 1 (the headline): K steps, each bracketed by events on the stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        one_step(evs[k])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # pass 2: the same K steps with every library launch bracketed by its own events
    # (recording them between launches adds a few microseconds a launch, so the
    # headline comes from pass 1)
    timer = None if args.no_launch_timing else B.LaunchTimer(capacity=96 * args.steps)
    if timer is not None:
        with timer:
            for k in range(args.steps):
                one_step()
        torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    ms_step = float(np.median(step_ms))
    fwd_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    epi_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    bwd_ms = float(np.median([e[2].elapsed_time(e[3]) for e in evs]))
    print(f"[bench] {args.steps} steps: median {ms_step:.3f} ms/step, mean {ms_total / args.steps:.3f} "
          f"(fwd {fwd_ms:.3f}, epi {epi_ms:.3f}, bwd {bwd_ms:.3f}); wall {wall:.2f} s",
          file=sys.stderr, flush=True)

    # contractions per step: forward logits, recomputed logits, dh, and dW (bf16 head
    # only: the quantised head is frozen)
    n_contr = 3 if quant else 4
    flops = 2.0 * n_contr * wl.M * wl.V * wl.D
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens_s = wl.M / (ms_step * 1e-3)
    fwd_flops = 2.0 * wl.M * wl.V * wl.D
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tflops = (n_contr - 1) * fwd_flops / (bwd_ms * 1e-3) / 1e12

    # per-kernel figures from the library's launch events over the timed steps
    kernels = {}
    if timer is not None:
        for name, ms, fl in timer.launches():
            k = kernels.setdefault(name, {"launches": 0, "ms": 0.0, "flops": 0.0})
            k["launches"] += 1
            k["ms"] += ms
            k["flops"] += fl
        for name, k in kernels.items():
            k["launches_per_step"] = k["launches"] / args.steps
            k["avg_launch_us"] = round(k["ms"] / k["launches"] * 1e3, 2)
            k["share_of_step"] = round(k["ms"] / args.steps / ms_step, 4)
            k["tflops"] = round(k["flops"] / (k["ms"] * 1e-3) / 1e12, 2) if k["flops"] else None
            k["flops_per_launch"] = k["flops"] / k["launches"]
            k["ms"] = round(k["ms"], 3)
        tsum = sum(k["ms"] for k in kernels.values()) / args.steps
        print(f"[bench] launches: {sum(k['launches'] for k in kernels.values()) // args.steps} per "
              f"step, {tsum:.3f} ms of kernel time per step", file=sys.stderr, flush=True)
        for name, k in sorted(kernels.items(), key=lambda kv: -kv[1]["ms"]):
            print(f"[bench]   {name:18s} {k['launches_per_step']:5.1f}/step  {k['avg_launch_us']:9.2f} us"
                  f"  {k['tflops'] or 0:8.1f} TFLOP/s  {100 * k['share_of_step']:5.1f} %",
                  file=sys.stderr, flush=True)
    traffic = {}
    if args.traffic_json and os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("workload") == wl.name and tj.get("kernel_source_hash") == B.kernel_source_hash():
                traffic = {n: e.get("bytes_per_launch") for n, e in tj.get("kernels", {}).items()}
        except Exception:
            traffic = {}

    def roof(name):
        k = kernels[name]
        ach = k["flops"] / (k["ms"] * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic.get(name),
                "avg_launch_us": k["avg_launch_us"], "algorithmic_flops_per_launch": k["flops_per_launch"],
                "launches_per_step": k["launches_per_step"]}

    gemm = {n: k for n, k in kernels.items() if k["flops"] > 0 and n != "k_target_logit"}
    dominant = max(gemm, key=lambda n: gemm[n]["ms"]) if gemm else None
    fwd_kernel = next((n for n in ("k_fwd", "k_fwd_tall") if n in kernels), None)

    metric = "fused CCE fwd+bwd tokens/s and % bf16 MFMA peak (8*M*V*D FLOPs)"
    workload = wl.name
    if quant:
        metric = "fused CCE fwd+bwd(dh) tokens/s over a quantised frozen head (6*M*V*D FLOPs)"
        workload = f"{wl.name}_q{args.quant}g{args.group}"
    result = {
        "metric": metric,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_mean": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden, N(0,0.02^2) head, Zipf(1.1) targets"
                + (", token-frequency prior -1.1 ln(1+v) on the logits)" if wl.name == "gemma4b_peaked"
                   else ")"),
        "config": {"workload": workload, "M": wl.M, "V": wl.V, "D": wl.D, "n_pairs": wl.n_pairs,
                   "lambda": wl.lam, "scope": "full" if wl.scope == 0 else "response",
                   "filter_eps": feps, "softcap": args.softcap,
                   "quant": {"bits": args.quant, "group": args.group} if quant else None,
                   "block_max": bool(args.block_max),
                   "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "phase_ms": {"forward": round(fwd_ms, 4), "epilogue": round(epi_ms, 4),
                     "backward": round(bwd_ms, 4)},
        "workspace_bytes": (B.workspace_bytes_q if quant else B.workspace_bytes)(wl.M, wl.V, wl.D),
        "head_bytes_per_step": head_bytes_per_step(wl.V, wl.D, args.quant if quant else 0, args.group),
        "device_status": status,
        # the dominant kernel (largest share of the step), timed live per launch with the
        # library's events on the stream it runs on (bench pass 2, the same K steps); FLOPs
        # per launch as the library counts them (2 per multiply-add at the nominal sizes of
        # the launch's contractions)
        "roofline": roof(dominant) if dominant else None,
        "roofline_forward": roof(fwd_kernel) if fwd_kernel else None,
        # the whole backward (cce_backward: all of its launches) timed per step
        "roofline_backward": {"kernels": "cce_backward", "bound": "mfma",
                              "achieved": round(bwd_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(bwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        "forward_phase_tflops": round(fwd_tflops, 2),
        "kernels": kernels,
    }
    if feps > 0 and not quant:
        result["filter_deviation"] = filter_deviation(head, h, W, y, lse, coef, feps, dh, dW, bwd_ms,
                                                      args.softcap, bmax, stream)
    del dh, dW
    torch.cuda.empty_cache()
    if args.calibrate_copy:
        a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not quant:
        print(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
