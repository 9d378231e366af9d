"""Benchmark of the fused MoE layer forward on one MI355X.

A step is one moe_forward (router GEMM, top-k, alignment, gate|up GEMM with the
SiLU*up epilogue, down GEMM, weighted combine) over one batch of synthetic
tokens of the decode layer E=8, top-2, d=4096, d_ff=14336, bf16, with weights
and tokens already resident in HBM.  Prints one JSON line.

Infinity-Cache guard: MI355X keeps up to 256 MB of recently read lines in its
memory-side cache, so a layer whose active weights are small would be timed
from that cache when the same weights are read step after step.  Timed loops
therefore cycle through R copies of the weights, R chosen so that one cycle
reads at least 1 GiB of layer bytes.

  python bench.py [--steps K] [--warmup W] [--tokens T] [--config C]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=None,
                    help="batch size (default: the largest decode batch of the config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs that capture one forward each")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-qk", action="store_true", help="skip the QK-norm measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run a plain device copy of MB megabytes (counter calibration)")
    return ap.parse_args()


GUARD_BYTES = 1 << 30
MAX_REPLICAS = 32


def guarded_forwards(B, roof, layer, bias, sh, x, T):
    """Forward objects over R copies of the layer's weights (R >= 1 chosen so
    that one cycle reads >= GUARD_BYTES), the routing of the first call, and
    the number of active experts."""
    import torch
    f0 = B.Forward(layer.w_router, bias, layer.w_gate_up, layer.w_down, sh.k,
                   layer.scale_gate_up, layer.scale_down)
    rb = f0.routing_buffers(T)
    f0(x, routing=rb)
    torch.cuda.synchronize()
    active = int((rb["counts"].cpu().numpy() > 0).sum())
    work = roof.layer_work(T, sh.d, sh.d_ff, sh.E, sh.k, sh.act, sh.wdt, active)
    reps = max(1, min(MAX_REPLICAS, -(-GUARD_BYTES // max(int(work.bytes_total), 1))))
    fwds = [f0]
    for _ in range(reps - 1):
        c = (lambda t: None if t is None else t.clone())
        fwds.append(B.Forward(c(layer.w_router), bias, c(layer.w_gate_up), c(layer.w_down), sh.k,
                              c(layer.scale_gate_up), c(layer.scale_down)))
    torch.cuda.synchronize()
    return fwds, rb, active, work


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer is built and measured on a single "
              "MI355X (no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_align_amd import _binding as B
    from mixture_experts_layer_align_amd import roofline as R
    from workloads import LAYERS, make_bias, make_layer, make_tokens

    sh = LAYERS[args.config]
    decode_T = [t for t in sh.tokens if t <= 256]
    T = args.tokens if args.tokens is not None else (max(decode_T) if decode_T else max(sh.tokens))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = make_layer(sh, None, dev, zipf=None)
    bias = make_bias(sh, sh.zipf_for(T), dev)
    stream = torch.cuda.current_stream()

    def timed(fwds, x, steps, warmup):
        out = torch.empty_like(x)
        for i in range(max(warmup, len(fwds))):
            fwds[i % len(fwds)](x, out)
        torch.cuda.synchronize()
        run = [lambda f=f: f(x, out) for f in fwds]
        if args.graph:
            # one graph per weight copy, each capturing one whole forward
            graphs = []
            for f in fwds:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    f(x, out)
                graphs.append(g)
            torch.cuda.synchronize()
            run = [g.replay for g in graphs]
            for i in range(warmup):
                run[i % len(run)]()
            torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            run[i % len(run)]()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, out

    x = make_tokens(sh, T, dev)
    fwds, rb, active, work = guarded_forwards(B, R, layer, bias, sh, x, T)
    ms, out = timed(fwds, x, args.steps, args.warmup)

    # per-kernel durations, HIP events recorded on the launch stream between
    # the kernels of each forward
    _, bm, names = fwds[0](x, routing=rb, events=[])
    torch.cuda.synchronize()
    nk = len(names)
    ev = B.HipEvents(nk + 1)
    per = np.zeros(nk)
    reps = max(args.steps, 10)
    for i in range(reps):
        fwds[i % len(fwds)](x, out, events=ev.handles)
        torch.cuda.synchronize()
        per += [ev.elapsed_ms(i, i + 1) for i in range(nk)]
    per /= reps
    kern = {n: float(v) for n, v in zip(names, per)}
    # the roofline is taken for the longer of the two expert GEMMs (the
    # layer's dominant kernels by design; the others have no fixed roofline)
    dom = max((n for n in kern if n in ("gate_up", "down")), key=kern.get)
    dom_bytes = {"gate_up": work.bytes_gate_up, "down": work.bytes_down}.get(dom)
    dom_flops = {"gate_up": work.flops_gate_up, "down": work.flops_down}.get(dom)
    prefill = T * sh.k / sh.E > 256
    if prefill:
        achieved = dom_flops / (kern[dom] * 1e-3) / 1e12
        peak = R.MFMA_BF16_FLOPS / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    else:
        achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
        peak = R.HBM_BYTES_PER_S / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": peak, "unit": "GB/s"}
    roof.update({"frac": achieved / peak, "traffic": measured_traffic(dom, sh, T), "kernel": dom,
                 "kernel_ms": kern[dom], "algorithmic_bytes_per_launch": dom_bytes,
                 "algorithmic_flops_per_launch": dom_flops})

    # other batch sizes of the same layer (same process, same weights)
    sweep = {}
    if not args.no_sweep:
        nrep_main = len(fwds)
        del fwds
        for t2 in sh.tokens:
            if t2 == T:
                continue
            x2 = make_tokens(sh, t2, dev)
            f2, _, _, _ = guarded_forwards(B, R, layer, make_bias(sh, sh.zipf_for(t2), dev), sh,
                                           x2, t2)
            m2, _ = timed(f2, x2, max(args.steps // 2, 5), 3)
            sweep[str(t2)] = {"ms": m2, "tokens_per_s": t2 / (m2 * 1e-3),
                              "weight_replicas": len(f2)}
            del f2
            torch.cuda.empty_cache()
    else:
        nrep_main = len(fwds)

    line = {
        "metric": "MoE layer tokens/s; decode HBM GB/s, prefill MFMA TFLOP/s as % of peak",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "bf16-act/fp8-weight",
                  "mxfp4": "bf16-act/mxfp4-weight", "mxfp8": "bf16-act/mxfp8-weight"}[sh.wdt],
        "data": "synthetic",
        "config": {"workload": f"fused MoE layer forward, {sh.name}: E={sh.E} top-{sh.k} "
                               f"d={sh.d} d_ff={sh.d_ff} {sh.act} x / {sh.wdt} experts, T={T}",
                   "tokens": T, "E": sh.E, "k": sh.k, "d": sh.d, "d_ff": sh.d_ff,
                   "active_experts": active, "block_m": bm, "parallelism": "single GPU"},
        "launch": "hip graph replay" if args.graph else "eager",
        "cache_guard": {"weight_replicas": nrep_main,
                        "layer_bytes": int(work.bytes_total),
                        "min_bytes_per_cycle": GUARD_BYTES},
        "layer_hbm_GBps": work.bytes_total / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": work.bytes_total / (ms * 1e-3) / R.HBM_BYTES_PER_S,
        "kernels_ms": kern,
        "roofline": roof,
        "sweep": sweep,
    }

    if not args.no_qk:
        line["qk_norm"] = qk_norm_bench(B, R, dev, args.steps)

    if args.copy_calibration:
        # a plain copy of known size, so hardware byte counters can be scaled
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layer, bias, x, sh)
    print(json.dumps(line), flush=True)


def qk_norm_bench(B, roof, dev, steps):
    """In-place QK-norm of the attention shape of the E=128 top-8 layer's model
    class (32 query and 4 key heads of 128, bf16) over an 8192-token batch:
    HBM-bound, algorithmic bytes = q and k read once and written once (+ the
    two weight vectors).  Launches cycle through copies of q and k so that one
    cycle moves >= 1 GiB (Infinity-Cache guard)."""
    import torch
    from workloads.qk import make_qk
    T, nq, nk, hd = 8192, 32, 4, 128
    nbytes = 2 * T * (nq + nk) * hd * 2 + 2 * hd * 2
    copies = max(1, min(MAX_REPLICAS, -(-GUARD_BYTES // nbytes)))
    sets = [make_qk(T, nq, nk, hd, "bf16", seed=i, device=dev) for i in range(copies)]
    for i in range(max(3, copies)):
        q, k, wq, wk = sets[i % copies]
        B.qk_norm(q, k, wq, wk, eps=1e-6)
    torch.cuda.synchronize()
    n = max(steps, 20) * copies
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n):
        q, k, wq, wk = sets[i % copies]
        B.qk_norm(q, k, wq, wk, eps=1e-6)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / n
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"QK-norm in place, bf16, T={T}, {nq} q + {nk} k heads of {hd}",
            "us_per_launch": us, "algorithmic_bytes_per_launch": nbytes, "GB/s": gbs,
            "frac_of_hbm_peak": gbs * 1e9 / roof.HBM_BYTES_PER_S, "cache_guard_copies": copies}


def measured_traffic(kernel, sh, T):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record for this workload (FETCH_SIZE and WRITE_SIZE scaled by a plain copy
    of known size), or None when there is none or any source the kernel is
    compiled from changed since the counters were taken."""
    import glob
    import hashlib
    want = f"E={sh.E} top-{sh.k} d={sh.d} d_ff={sh.d_ff} {sh.wdt} T={T}"
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")):
        with open(path) as f:
            rec = json.load(f)
        if rec.get("kernel") != kernel or rec.get("workload") != want:
            continue
        # every source the kernel is compiled from, as at measurement (a
        # record without them cannot be matched to the code: stale)
        if not rec.get("sources"):
            return None
        for src, sha in rec["sources"].items():
            with open(os.path.join(ROOT, src), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != sha:
                    return None
        return rec["traffic_bytes_per_launch"]
    return None


def cpu_baseline(layer, bias, x, sh):
    """The oracle (float64 NumPy, as it stands) on the host cores, on the same
    batch; tokens/s over its full forward including the decode of the stored
    weights it reads."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe_oracle as O

    cores = min(len(os.sched_getaffinity(0)), 16)

    def bits(t):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).cpu().numpy()
        return t.cpu().numpy()

    fmt = {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}[sh.wdt]
    gu = [bits(layer.w_gate_up[e]) for e in range(sh.E)]
    dn = [bits(layer.w_down[e]) for e in range(sh.E)]
    sgu = layer.scale_gate_up.cpu().numpy() if layer.scale_gate_up is not None else None
    sdn = layer.scale_down.cpu().numpy() if layer.scale_down is not None else None
    xb, wrb = bits(x), bits(layer.w_router)
    b64 = None if bias is None else bias.cpu().numpy().astype(np.float64)
    T = x.shape[0]
    # whole oracle forwards (weight decode included) repeated until at least
    # MIN_S seconds of CPU work, at most MAX_RUNS of them
    MIN_S, MAX_RUNS = 10.0, 50
    runs = 0
    with threadpool_limits(limits=cores):
        used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        t0 = time.perf_counter()
        while True:
            efn = O.expert_weights_from_raw(gu, dn, fmt, sgu, sdn)
            O.moe_forward(O.decode(xb, sh.act), O.decode(wrb, sh.act), b64, efn, sh.E, sh.k, 32)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= MIN_S or runs >= MAX_RUNS:
                break
    return {"value": runs * T / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{runs} full oracle forwards of the benchmarked T={T} batch "
                      f"({dt:.1f} s, float64 NumPy incl. weight decode each time)"}


if __name__ == "__main__":
    main()
