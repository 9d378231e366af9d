"""Benchmark of the fused MoE layer forward on one MI355X.

A step is one moe_forward (router GEMM, top-k, alignment, gate|up GEMM with the
SiLU*up epilogue, down GEMM, weighted combine) over one batch of synthetic
tokens, with weights and tokens already resident in HBM.  The headline
workload is the largest layer, E=256 top-8 d=7168 d_ff=2048 with fp8 e4m3
expert weights (fp32 per-column scales), bf16 tokens, 16384 tokens under a
Zipf(1.2) router skew: the prefill half of the metric, reported against the
dense MFMA peak.  The same JSON line carries every other layer and batch size
of the workload set (decode batches against the HBM roofline), each timed the
same way in the same process.

Infinity-Cache guard: MI355X keeps up to 256 MB of recently read lines in its
memory-side cache, so a layer whose active weights are small would be timed
from that cache when the same weights are read step after step.  Timed loops
therefore cycle through R copies of the weights, R chosen so that one cycle
reads at least 1 GiB of layer bytes.

  python bench.py [--steps K] [--warmup W] [--config C --tokens T] [--only]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEAD_CONFIG, HEAD_TOKENS = 4, 16384


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEAD_CONFIG)
    ap.add_argument("--tokens", type=int, default=None,
                    help="batch size of the headline (default: the config's largest)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload only (no per-layer block, no extras)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs that capture one forward each")
    ap.add_argument("--no-qk", action="store_true",
                    help="skip the QK-norm, RMSNorm and MXFP8-quantiser measurements")
    ap.add_argument("--norms", "--aux", dest="norms", action="store_true",
                    help="only the QK-norm, RMSNorm and MXFP8-quantiser measurements "
                         "(one JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run a plain device copy of MB megabytes (counter calibration)")
    return ap.parse_args()


GUARD_BYTES = 1 << 30
MAX_REPLICAS = 32
# MFMA-bound when a layer's flops per weight byte exceed the bf16 ridge
# (dense MFMA peak / HBM bandwidth)
RIDGE = 2.5e15 / 8.0e12


def guarded_forwards(B, roof, layer, bias, sh, x, T):
    """Forward objects over R copies of the layer's weights (R >= 1 chosen so
    that one cycle reads >= GUARD_BYTES), the routing of the first call, and
    the number of active experts."""
    import torch
    f0 = B.Forward(layer.w_router, bias, layer.w_gate_up, layer.w_down, sh.k,
                   layer.scale_gate_up, layer.scale_down)
    rb = f0.routing_buffers(T)
    _, bm, _ = f0(x, routing=rb)
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
    return fwds, rb, active, work, bm


def timed(fwds, x, steps, warmup, graph=False):
    """Average ms per forward over `steps` forwards (cycling the weight
    copies), bracketed by device synchronisations."""
    import torch
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for i in range(max(warmup, len(fwds))):
        fwds[i % len(fwds)](x, out)
    torch.cuda.synchronize()
    run = [lambda f=f: f(x, out) for f in fwds]
    if graph:
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
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        run[i % len(run)]()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, out


def kernel_times(B, fwds, x, reps):
    """Average duration of each kernel of the forward: HIP events recorded on
    the launch stream between the kernels (the stream the kernels run on)."""
    import numpy as np
    import torch
    out = torch.empty_like(x)
    _, _, names = fwds[0](x, out, events=[])
    torch.cuda.synchronize()
    nk = len(names)
    ev = B.HipEvents(nk + 1)
    per = np.zeros(nk)
    for i in range(reps):
        fwds[i % len(fwds)](x, out, events=ev.handles)
        torch.cuda.synchronize()
        per += [ev.elapsed_ms(j, j + 1) for j in range(nk)]
    per /= reps
    return {n: float(v) for n, v in zip(names, per)}


def measure(B, R, sh, layer, T, steps, warmup, graph=False):
    """One workload (layer, batch): time per forward, per-kernel times and the
    roofline of the dominant expert GEMM."""
    import torch
    from workloads import make_bias, make_tokens
    dev = layer.device
    bias = make_bias(sh, sh.zipf_for(T), dev)
    x = make_tokens(sh, T, dev)
    fwds, rb, active, work, bm = guarded_forwards(B, R, layer, bias, sh, x, T)
    ms, _ = timed(fwds, x, steps, warmup, graph)
    kern = kernel_times(B, fwds, x, max(steps, 10))
    # the layer's bound: flops per byte of expert weights against the ridge
    w_bytes = work.bytes_total - 2 * T * sh.d * R.ELEM_BYTES[sh.act]
    mfma = work.flops_total / max(w_bytes, 1) > RIDGE
    # the roofline is taken for the longer of the two expert GEMMs (the
    # layer's dominant kernels by design; the others have no fixed roofline)
    dom = max((n for n in kern if n in ("gate_up", "down")), key=kern.get)
    dom_bytes = {"gate_up": work.bytes_gate_up, "down": work.bytes_down}[dom]
    dom_flops = {"gate_up": work.flops_gate_up, "down": work.flops_down}[dom]
    gemm_flops = work.flops_gate_up + work.flops_down
    if mfma:
        achieved = dom_flops / (kern[dom] * 1e-3) / 1e12
        peak = R.MFMA_BF16_FLOPS / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak,
                # the expert math runs on bf16/fp16 MFMA (weights widened
                # exactly); the fp8 MFMA peak, for reference
                "frac_of_fp8_peak": achieved * 1e12 / R.MFMA_FP8_FLOPS}
        layer_frac = gemm_flops / (ms * 1e-3) / R.MFMA_BF16_FLOPS
    else:
        achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
        peak = R.HBM_BYTES_PER_S / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": peak, "unit": "GB/s",
                "frac": achieved / peak}
        layer_frac = work.bytes_total / (ms * 1e-3) / R.HBM_BYTES_PER_S
    roof.update({"traffic": measured_traffic(dom, sh, T), "kernel": dom,
                 "kernel_ms": kern[dom], "algorithmic_bytes_per_launch": dom_bytes,
                 "algorithmic_flops_per_launch": dom_flops})
    res = {"workload": workload_name(sh, T), "tokens": T, "ms": ms,
           "tokens_per_s": T / (ms * 1e-3), "active_experts": active, "block_m": bm,
           "weight_replicas": len(fwds), "layer_bytes": int(work.bytes_total),
           "layer_flops": int(work.flops_total),
           "layer_frac": layer_frac, "kernels_ms": kern, "roofline": roof}
    del fwds
    torch.cuda.empty_cache()
    return res, x, bias


def workload_name(sh, T):
    return (f"fused MoE layer forward, {sh.name}: E={sh.E} top-{sh.k} d={sh.d} d_ff={sh.d_ff} "
            f"{sh.act} x / {sh.wdt} experts, T={T}")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer is built and measured on a single "
              "MI355X (no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_align_amd import _binding as B
    from mixture_experts_layer_align_amd import roofline as R
    from workloads import LAYERS, make_layer

    if args.norms:
        dev = torch.device("cuda:0")
        print(json.dumps({"qk_norm": qk_norm_bench(B, R, dev, args.steps),
                          "rms_norm": rms_norm_bench(B, R, dev, args.steps),
                          "mx_quant": mx_quant_bench(B, R, dev, args.steps)}), flush=True)
        return

    hc = args.config
    hsh = LAYERS[hc]
    hT = args.tokens if args.tokens is not None else max(hsh.tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    head = None
    per_layer = {}
    # the headline's layer first, then (unless --only) every layer of the
    # workload set; one layer's weights are resident at a time
    order = [hc] + ([] if args.only else [c for c in sorted(LAYERS) if c != hc])
    for c in order:
        sh = LAYERS[c]
        layer = make_layer(sh, None, dev, zipf=None)
        tokens = [hT] if c == hc else []
        if not args.only:
            tokens += [t for t in sh.tokens if not (c == hc and t == hT)]
        for T in tokens:
            print(f"# layer {c} ({sh.name}) T={T}", file=sys.stderr, flush=True)
            is_head = c == hc and T == hT
            steps = args.steps if is_head else max(args.steps // 2, 5)
            warmup = args.warmup if is_head else 3
            res, x, bias = measure(B, R, sh, layer, T, steps, warmup, args.graph)
            per_layer[f"cfg{c} T={T}"] = res
            if is_head:
                head = res
                if not args.no_cpu_baseline:
                    cpu = cpu_baseline(layer, bias, x, sh)
            del x
        del layer
        torch.cuda.empty_cache()

    line = {
        "metric": "MoE layer tokens/s; decode HBM GB/s, prefill MFMA TFLOP/s as % of peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "tokens": hT, "E": hsh.E, "k": hsh.k,
                   "d": hsh.d, "d_ff": hsh.d_ff, "activations": hsh.act,
                   "expert_weights": hsh.wdt, "active_experts": head["active_experts"],
                   "block_m": head["block_m"], "parallelism": "single GPU"},
        "launch": "hip graph replay" if args.graph else "eager",
        "cache_guard": {"weight_replicas": head["weight_replicas"],
                        "layer_bytes": head["layer_bytes"],
                        "min_bytes_per_cycle": GUARD_BYTES},
        "layer_frac": head["layer_frac"],
        "kernels_ms": head["kernels_ms"],
        "roofline": head["roofline"],
        "per_layer": per_layer,
    }
    if not args.only and not args.no_qk:
        line["qk_norm"] = qk_norm_bench(B, R, dev, args.steps)
        line["rms_norm"] = rms_norm_bench(B, R, dev, args.steps)
        line["mx_quant"] = mx_quant_bench(B, R, dev, args.steps)
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
        line["cpu_baseline"] = cpu
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


def rms_norm_bench(B, roof, dev, steps):
    """Row RMSNorm of an 8192-token batch at the E=256 top-8 layer's hidden
    size (d = 7168, bf16), out of place: HBM-bound, algorithmic bytes = x read
    once, y written once (+ the gain).  Launches cycle through copies of x and
    y so that one cycle moves >= 1 GiB (Infinity-Cache guard)."""
    import torch
    from workloads.norm import make_rows
    T, d = 8192, 7168
    nbytes = 2 * T * d * 2 + d * 2
    copies = max(1, min(MAX_REPLICAS, -(-GUARD_BYTES // nbytes)))
    sets = []
    for i in range(copies):
        x, g = make_rows(T, d, "bf16", seed=i, device=dev)
        sets.append((x, g, torch.empty_like(x)))
    for i in range(max(3, copies)):
        x, g, y = sets[i % copies]
        B.rms_norm(x, g, out=y, eps=1e-6)
    torch.cuda.synchronize()
    n = max(steps, 20) * copies
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n):
        x, g, y = sets[i % copies]
        B.rms_norm(x, g, out=y, eps=1e-6)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / n
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"row RMSNorm, bf16, T={T}, d={d}, out of place",
            "us_per_launch": us, "algorithmic_bytes_per_launch": nbytes, "GB/s": gbs,
            "frac_of_hbm_peak": gbs * 1e9 / roof.HBM_BYTES_PER_S, "cache_guard_copies": copies}


def mx_quant_bench(B, roof, dev, steps):
    """MXFP8 quantisation of the E=256 top-8 layer's activations at prefill
    (16384 tokens x d = 7168, bf16): HBM-bound, algorithmic bytes = x read
    once, the codes and scale bytes written once.  Launches cycle through
    copies so that one cycle moves >= 1 GiB (Infinity-Cache guard)."""
    import torch
    from workloads.mxq import make_mx_rows
    rows, n = 16384, 7168
    nbytes = rows * n * 2 + rows * n + rows * n // 32
    copies = max(1, min(MAX_REPLICAS, -(-GUARD_BYTES // nbytes)))
    sets = []
    for i in range(copies):
        x = make_mx_rows(rows, n, "bf16", seed=i, device=dev)
        sets.append((x, torch.empty((rows, n), dtype=torch.uint8, device=dev),
                     torch.empty((rows, n // 32), dtype=torch.uint8, device=dev)))
    for i in range(max(3, copies)):
        B.quantize_mxfp8(*sets[i % copies])
    torch.cuda.synchronize()
    cnt = max(steps, 20) * copies
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(cnt):
        B.quantize_mxfp8(*sets[i % copies])
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / cnt
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"MXFP8 quantisation (32-element blocks), bf16 in, rows={rows}, n={n}",
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


def host_cores():
    """Cores available to this process: its CPU affinity, capped by a cgroup
    CPU quota when one is set."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return n


CPU_SAMPLE_TOKENS = 2048


def cpu_baseline(layer, bias, x, sh):
    """The oracle (float64 NumPy, as it stands) on the host cores: one oracle
    forward (routing, alignment, every expert's SwiGLU, combine, including the
    decode of the stored weights it reads) over the first CPU_SAMPLE_TOKENS
    tokens of the benchmarked batch (all of them if fewer); tokens/s of that
    sample."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe_oracle as O

    cores = host_cores()

    def bits(t):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).cpu().numpy()
        return t.cpu().numpy()

    class PerExpert:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return bits(self.t[e])

    fmt = {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}.get(sh.wdt)
    if fmt is None:
        return None  # microscaled experts: no baseline leg for them here
    sgu = layer.scale_gate_up.cpu().numpy() if layer.scale_gate_up is not None else None
    sdn = layer.scale_down.cpu().numpy() if layer.scale_down is not None else None
    Ts = min(x.shape[0], CPU_SAMPLE_TOKENS)
    xb, wrb = bits(x[:Ts]), bits(layer.w_router)
    b64 = None if bias is None else bias.cpu().numpy().astype(np.float64)
    with threadpool_limits(limits=cores):
        used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        t0 = time.perf_counter()
        efn = O.expert_weights_from_raw(PerExpert(layer.w_gate_up), PerExpert(layer.w_down), fmt,
                                        sgu, sdn)
        O.moe_forward(O.decode(xb, sh.act), O.decode(wrb, sh.act), b64, efn, sh.E, sh.k, 32)
        dt = time.perf_counter() - t0
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"one oracle forward of the first {Ts} of the {x.shape[0]} benchmarked "
                      f"tokens ({dt:.1f} s, float64 NumPy on {used} threads, including the "
                      f"decode of every expert weight it reads and their device-to-host copy)"}


if __name__ == "__main__":
    main()
