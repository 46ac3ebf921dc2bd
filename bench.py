"""Benchmark of one fine-grained MoE layer step (route + forward + backward) on
one MI355X through the C ABI.

Prints one JSON line: whole-step TFLOPS (useful FLOPs 18*P*d*n per step, P =
routed rows; the timed steps run with nothing recorded between launches) and
its fraction of the bf16 MFMA peak, the roofline position of the dominant
kernel (per-launch durations from HIP events the library records on its
stream during a second pass of as many steps), every kernel's time and roofline
fraction, and the fp64 CPU oracle timed on a bounded sample of the same
workload as a reported baseline.  Also reported: single steps timed after a
1 GiB write that evicts the caches ("flushed"), the bytes kept between forward
and backward ("memory") and the realised expert loads ("routing").

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload fg7b_bf16]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16
MFMA_PEAK_F32 = 157.3     # TFLOP/s, MI355X fp32 (MFMA fp32 reuses this figure)
MFMA_PEAK_FP8 = 5000.0    # TFLOP/s, MI355X dense fp8 (the MXFP8 forward GEMMs)
HBM_PEAK = 8000.0         # GB/s
CPU_FLOP_BUDGET = 4.0e12  # useful FLOPs of the default CPU oracle sample


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fg7b_bf16")
    ap.add_argument("--round-mode", type=int, default=0)
    ap.add_argument("--tile", type=int, default=128,
                    help="token-rounding tile (128 or 256; 256 matches the bf16 GEMMs' row tile)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the unfused layer (separate gather / SwiGLU kernels, X_g H A Y cached, "
                         "dS = <dO_g, Y>) instead of the fused one, for comparison")
    ap.add_argument("--mxfp8", action="store_true",
                    help="run the forward GEMMs and the dH and dXt GEMMs in MXFP8 (moe_fwd_mxfp8, "
                         "moe_bwd_mxfp8); the weight-gradient GEMMs stay bf16")
    ap.add_argument("--mxfp8-wgrad", action="store_true",
                    help="with --mxfp8: the two weight-gradient GEMMs in MXFP8 too, on operands "
                         "quantized along each expert's rows (MOE_FLAG_MXFP8_WGRAD)")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the oracle's CPU baseline sample (0 = skip, -1 = as many as "
                         "fit a 4 TFLOP budget, about 20 s of fp64 work, capped at the workload's T)")
    ap.add_argument("--flushed-steps", type=int, default=5,
                    help="after the timed steps, time this many single steps one by one, each "
                         "after writing a 1 GiB buffer so that no input or weight is still in the "
                         "L2 / MALL caches (reported as 'flushed'; 0 = skip)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many bytes "
                         "(calibration dispatch for HBM counter passes)")
    return ap.parse_args()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter passes, or
    None when they are missing or were taken on different kernel sources."""
    from fine_grained_mixture_top_amd import hbm_traffic
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != hbm_traffic.source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else round(k["bytes"])


def kernel_work(name, w, P, es, mx=False):
    """Algorithmic work of one launch: (amount, kind) with kind 'flop' or 'byte'."""
    T, d, E, n = w.T, w.d, w.E, w.n
    flops = {
        "router_logits": 2.0 * T * d * E, "up": 4.0 * P * d * n, "down": 2.0 * P * n * d,
        "dh": 2.0 * P * d * n, "dxt": 4.0 * P * d * n, "dw1": 4.0 * P * d * n,
        "dw2": 2.0 * P * n * d, "dwr": 2.0 * T * d * E, "da": 2.0 * P * d * n,
        "up_mx": 4.0 * P * d * n, "down_mx": 2.0 * P * n * d, "dxt_mx": 4.0 * P * d * n, "dh_mx": 2.0 * P * d * n,
        "dw1_mx": 4.0 * P * d * n, "dw2_mx": 2.0 * P * n * d,
    }
    if name in flops:
        return flops[name], "flop"
    # bandwidth-bound kernels: bytes that must cross HBM once
    bytes_ = {
        "agg_o": P * d * es + T * d * es + P * 8 + (T + 1) * 4,
        # dXt rows (each with its router term) in, dX out, the token CSR
        "agg_dx": P * d * es + T * d * es + P * 4 + (T + 1) * 4,
        "route_select": T * E * 4 + T * w.K * 8 + P * 16 + T * E * (1 + 1 + 4),
        # router backward: dS (one partial per row counted), gate, expert and
        # the token CSR in; dS and dz per row and the dense dz rows out
        "router_grad": P * (4 + 4 + 4 + 4) + (T + 1) * 4 + P * (4 + 4) + T * E * es,
        "wr_t": 2 * E * d * es, "db": P * 4,
        # unfused layer: row gather (read + write), SwiGLU, dS = <dO_g, Y>, SwiGLU backward
        "gather": 2 * P * d * es + P * 4, "swiglu": 3 * P * n * es, "row_dot": 2 * P * d * es + P * 4,
        "swiglu_bwd": P * (n + 2 * n + n) * es + P * 4 + P * (2 * n + n) * es,
        # MXFP8 quantizers (bf16 in, codes + 1/32 scale bytes out), averaged
        # over their four launches per step: x, A, dO and dH rows; w1 and w2
        # along their forward reductions, w2 along d for dH, w1 along 2n for dXt
        "mx_quant_rows": (T * d + P * n + T * d + P * 2 * n) * (es + 1 + 1 / 32) / 4,
        "mx_quant_w": 6 * E * d * n * (es + 1 + 1 / 32) / 4,
        # weight-gradient operands along the segments, averaged over the four
        # launches: x and dO rows gathered (d columns each), dH (2n), A_s (n)
        "mx_quant_seg": (2 * d + 2 * n + n) * P * (es + 1 + 1 / 32) / 4,
        "mx_pad_offsets": (E + 1) * 4 * 2,
    }
    return float(bytes_.get(name, 0)), "byte"


def memory_report(w, L, es):
    """Bytes the layer keeps between forward and backward (the cached H plus the
    routing metadata), the transient workspaces, and what a layer that caches
    the usual backward activations (gathered X, H, A and Y per routed row)
    would keep instead."""
    from fine_grained_mixture_top_amd import binding as B
    P = w.P
    cap = int(L.routing.cap)
    routing = sum(t.numel() * t.element_size() for t in L.routing.tensors())
    if L.unfused:
        cache = B.moe_unfused_cache_bytes(L.desc)
        return {"cached_bytes": cache + routing, "activation_cache_bytes": cache, "workspace_fwd_bytes": 0,
                "workspace_bwd_bytes": B.moe_workspace_bytes(L.desc, B.MOE_WS_BWD_UNFUSED)}
    return {
        "cached_bytes": cap * 2 * w.n * es + routing,
        "h_cache_bytes": cap * 2 * w.n * es,
        "workspace_fwd_bytes": B.moe_workspace_bytes(L.desc, B.MOE_WS_FWD),
        "workspace_bwd_bytes": B.moe_workspace_bytes(L.desc, B.MOE_WS_BWD),
        "naive_cache_bytes": P * (w.d + 2 * w.n + w.n + w.d) * es,
    }


def routing_report(L, tile=128):
    """Realised expert loads of the last routed batch: rows before / after
    token rounding, max / min / median load, experts below one tile and
    experts whose last tile is partial."""
    import numpy as np
    raw = L.routing.counts_raw.cpu().numpy().astype(np.int64)
    cnt = L.routing.counts.cpu().numpy().astype(np.int64)
    return {"rows_raw": int(raw.sum()), "rows": int(cnt.sum()), "max": int(raw.max()), "min": int(raw.min()),
            "median": float(np.median(raw)), "below_tile": int((raw < tile).sum()),
            "partial_tile": int((raw % tile != 0).sum()), "tile": tile}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(w, a, tokens, repeats=1):
    """fp64 oracle (as it stands) on the first `tokens` tokens of the workload:
    routing + forward and the backward timed separately; with repeats > 1 the
    median of that many runs of each."""
    import numpy as np
    from oracle import moe_oracle as O
    tk = min(tokens, w.T)
    x64, wr64 = O.to_f64(a["x"][:tk], w.dtype), O.to_f64(a["w_r"], w.dtype)
    w1, w2 = O.to_f64(a["w1"], w.dtype), O.to_f64(a["w2"], w.dtype)
    dO = O.to_f64(a["d_o"][:tk], w.dtype)
    fwd_s, bwd_s = [], []
    for _ in range(repeats):
        t0 = time.perf_counter()
        rt = O.route(x64, wr64, a["bias"], w.K)
        f = O.forward(x64, w1, w2, rt)
        t1 = time.perf_counter()
        O.backward(x64, wr64, w1, w2, rt, f["H"], dO)
        t2 = time.perf_counter()
        fwd_s.append(t1 - t0)
        bwd_s.append(t2 - t1)
    fwd, bwd = float(np.median(fwd_s)), float(np.median(bwd_s))
    dt = fwd + bwd
    rows = int(rt["n_rows"])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    med = f", median of {repeats} runs" if repeats > 1 else ""
    return {"value": 18.0 * rows * w.d * w.n / dt / 1e12, "unit": "TFLOPS", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "fwd_s": round(fwd, 6), "bwd_s": round(bwd, 6),
            "fwd_tflops": 6.0 * rows * w.d * w.n / fwd / 1e12, "bwd_tflops": 12.0 * rows * w.d * w.n / bwd / 1e12,
            "sample": f"route+fwd ({fwd:.3g} s) and bwd ({bwd:.3g} s) of {tk} of {w.T} tokens ({rows} rows), "
                      f"same weights, fp64 numpy{med}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    if args.unfused and args.mxfp8:
        print("--unfused and --mxfp8 are separate comparisons; pick one", file=sys.stderr)
        sys.exit(2)
    if args.mxfp8_wgrad and not args.mxfp8:
        print("--mxfp8-wgrad goes with --mxfp8", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fine_grained_mixture_top_amd import binding as B
    from fine_grained_mixture_top_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    a = I.draw_all(w)
    dt = B.TORCH_DTYPE[B.DTYPE_CODE[w.dtype]]

    def dev(v):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()

    x, wr, w1, w2, do = (dev(a[k]) for k in ("x", "w_r", "w1", "w2", "d_o"))
    bias = None if a["bias"] is None else torch.from_numpy(a["bias"]).cuda()
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, w.dtype, round_mode=args.round_mode, tile=args.tile,
                       flags=B.MOE_FLAG_MXFP8_WGRAD if args.mxfp8_wgrad else 0)
    L = B.Layer(desc, unfused=args.unfused)

    def step():
        L.route(x, wr, bias)
        if args.mxfp8:
            L.forward_mxfp8(x, w1, w2)
            L.backward_mxfp8(x, wr, w1, w2, do)
        else:
            L.forward(x, w1, w2)
            L.backward(x, wr, w1, w2, do)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # headline: the timed steps with nothing recorded between the launches
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # per-kernel times: the same number of steps again, with the library
    # recording a HIP event pair around every launch on its stream
    prof = B.Profiler(capacity=(B.MOE_K_COUNT + 2) * args.steps)
    prof.attach(L.desc)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    B.Profiler.detach(L.desc)
    ms_step_profiled = t0.elapsed_time(t1) / args.steps
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flushed = None
    if args.flushed_steps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(args.flushed_steps):
            flush.zero_()
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del flush
        times.sort()
        flushed = {"steps": args.flushed_steps, "flush_bytes": 1 << 30,
                   "ms_per_step_median": round(times[len(times) // 2], 4), "ms_per_step_min": round(times[0], 4)}

    P = int(L.routing.offsets[-1].item())
    es = 2 if w.dtype == "bf16" else 4
    peak_mfma = MFMA_PEAK_BF16 if w.dtype == "bf16" else MFMA_PEAK_F32
    per = {}
    for kid, ms in prof.records():
        per.setdefault(B.KERNEL_NAMES[kid], []).append(ms)
    prof.close()
    kernels = {}
    for name, lst in per.items():
        avg = sum(lst) / len(lst)
        work, kind = kernel_work(name, w, P, es, args.mxfp8)
        if kind == "flop":
            ach = work / (avg * 1e-3) / 1e12
            pk = MFMA_PEAK_FP8 if name.endswith("_mx") else peak_mfma
            kernels[name] = {"ms": round(avg, 4), "bound": "mfma", "achieved": round(ach, 1),
                             "peak": pk, "unit": "TFLOP/s", "frac": round(ach / pk, 4),
                             "work": work}
        else:
            ach = work / (avg * 1e-3) / 1e9
            kernels[name] = {"ms": round(avg, 4), "bound": "hbm", "achieved": round(ach, 1),
                             "peak": HBM_PEAK, "unit": "GB/s", "frac": round(ach / HBM_PEAK, 4),
                             "work": work}
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    useful = w.flops_fwd_bwd(P if args.round_mode else None)
    tflops = useful / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "MoE layer fwd+bwd TFLOPS and % of bf16 MFMA peak, 7B fine-grained shape, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8 (all six GEMMs) + bf16" if args.mxfp8_wgrad else
                  "mxfp8 (fwd, dH, dXt GEMMs) + bf16") if args.mxfp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "n": w.n, "K": w.K,
                   "round_mode": args.round_mode, "tile": args.tile, "rows": P, "parallelism": "single GPU",
                   "layer": "unfused" if args.unfused else "fused",
                   "forward_gemms": "mxfp8" if args.mxfp8 else w.dtype,
                   "weight_grad_gemms": "mxfp8" if args.mxfp8_wgrad else w.dtype},
        "mfma_peak_frac": round(tflops / peak_mfma, 4),
        # the per-kernel pass (event pair around every launch) timed on its own
        "ms_per_step_profiled": round(ms_step_profiled, 4),
        "tokens_per_s": round(w.T / (ms_step * 1e-3), 1),
        "roofline": {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"],
                     "unit": dk["unit"], "frac": dk["frac"], "traffic": None if (args.unfused or args.mxfp8) else measured_traffic(w.name, dom)},
        "kernels": {k: {kk: v for kk, v in d.items() if kk != "work"} for k, d in kernels.items()},
        "memory": memory_report(w, L, es),
        "routing": routing_report(L, args.tile),
    }
    if flushed is not None:
        flushed["tflops_median"] = round(useful / (flushed["ms_per_step_median"] * 1e-3) / 1e12, 2)
        out["flushed"] = flushed
    cpu_tokens = args.cpu_tokens
    if cpu_tokens < 0:
        cpu_tokens = max(1, min(w.T, int(CPU_FLOP_BUDGET // (18.0 * w.K * w.d * w.n))))
    if cpu_tokens > 0:
        # the tiny workload runs in well under a second: median of 5
        out["cpu_baseline"] = cpu_baseline(w, a, cpu_tokens, repeats=5 if w.T * w.d * w.n < (1 << 24) else 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
