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
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "k_fwd_traffic.json"))
    ap.add_argument("--v-sweep", action="store_true",
                    help="time one step and record workspace / peak device memory at "
                         "V in {32768, 65536, 131072, 262144} (M=8192, D=2560); one JSON line per V")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --calibrate-copy run into --traffic-json; no GPU use")
    return ap.parse_args()


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str, workload: str):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the forward kernel, scaled by
    what the same counters read for the 1 GiB copy kernel of the same run."""
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

    res = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        d = per_dispatch(path, counter)
        fwd = [v for (i, n), v in d.items() if "k_fwd<" in n or "k_fwd_tall<" in n]
        kname = "k_fwd_tall" if any("k_fwd_tall<" in n for (i, n) in d) else "k_fwd"
        copy = [v for (i, n), v in d.items() if "copyBuffer" in n or "copy" in n.lower()]
        copy = [v for v in copy if v > 1e5]          # the 1 GiB copy, not small transfers
        if not fwd or not copy:
            raise SystemExit(f"{path}: no forward or copy dispatch with {counter}")
        scale = (1 << 30) / (max(copy) * 1024.0)      # true bytes per counted byte
        res[counter] = {"kib_per_launch": sum(fwd) / len(fwd), "copy_kib": max(copy),
                        "scale": scale, "bytes_per_launch": sum(fwd) / len(fwd) * 1024.0 * scale}
    out = {"workload": workload, "kernel": kname, "kernel_source_hash": B.kernel_source_hash(),
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


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
    return {"value": len(idx) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
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
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    epi_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (fwd {fwd_ms:.3f}, epi {epi_ms:.3f}, "
          f"bwd {bwd_ms:.3f}); wall {wall:.2f} s", file=sys.stderr, flush=True)

    # contractions per step: forward logits, recomputed logits, dh, and dW (bf16 head
    # only: the quantised head is frozen)
    n_contr = 3 if quant else 4
    flops = 2.0 * n_contr * wl.M * wl.V * wl.D
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens_s = wl.M / (ms_step * 1e-3)
    # the longest single launch, timed live: the forward GEMM + online-LSE kernel
    # (cce_forward = k_fwd + target-logit and merge kernels of a few microseconds)
    fwd_flops = 2.0 * wl.M * wl.V * wl.D
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tflops = (n_contr - 1) * fwd_flops / (bwd_ms * 1e-3) / 1e12
    # the forward runs 256 x 256 tiles with 64-wide K-slices (k_fwd) when D % 64 == 0
    # and each workgroup runs >= 32 vocab tiles, else 384 x 256 tiles (k_fwd_tall)
    # when D % 32 == 0 and no block maximum is saved, else k_fwd; the recompute
    # runs k_recompute_tall when D % 32 == 0 and no tile is skipped
    n_mt = (wl.M + 255) // 256
    full = wl.V // 256
    smax = max(1, min(256 // n_mt, full)) if full > 0 else 1
    tiles_per_wg = (full + smax - 1) // smax if full > 0 else 0
    if wl.D % 64 == 0 and tiles_per_wg >= 32:
        fwd_kernel = "k_fwd"
    else:
        fwd_kernel = "k_fwd_tall" if (wl.D % 32 == 0 and not args.block_max) else "k_fwd"
    rec_kernel = "k_recompute_tall" if (wl.D % 32 == 0 and not feps > 0) else "k_recompute"
    # the bf16 head with tall recompute tiles runs the pipelined backward: chunk 0's
    # recompute alone, one fused launch per later chunk (dh / dW of chunk c and the
    # recompute of c + 1), the last chunk's dh / dW alone
    bwd_kernels = ("k_recompute_tall + k_bwd_fused + k_grads (cce_backward)"
                   if rec_kernel == "k_recompute_tall" else f"{rec_kernel} + k_grads (cce_backward)")
    traffic = None
    if args.traffic_json and os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("workload") == wl.name and tj.get("kernel_source_hash") == B.kernel_source_hash():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

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
        "device_status": status,
        "roofline": {"kernel": f"cce_forward_q (k_dequant + {fwd_kernel} per chunk)" if quant
                     else f"{fwd_kernel} (cce_forward)", "bound": "mfma",
                     "achieved": round(fwd_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if quant else traffic},
        # the backward's kernels (per vocab chunk: recompute, then dh + dW) timed
        # together live around cce_backward: 3 contractions of 2*M*V*D FLOPs
        "roofline_backward": {"kernels": f"k_dequant + {rec_kernel} + k_grads (dh) (cce_backward_q)"
                              if quant else bwd_kernels,
                              "bound": "mfma", "achieved": round(bwd_tflops, 2),
                              "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(bwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
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
