"""MoE-layer benchmark on one MI355X.

A step is one pass of the whole layer -- topK routing, gather, shared expert,
routed experts (NVFP4 up -> relu^2 / SwiGLU -> down), WeightedRowSum -- over
one batch of seeded synthetic input (bit_block_scaled_topk_amd.synth), with
every input and weight resident in HBM before the timed region starts.

The parsed line is the largest workload, the 4314-token prefill layer (d_model
2688, 128 experts, topK 6, relu^2 d_ff 1856, shared d_ff 3712, bf16
activations): every expert takes the bf16 MFMA GEMM.  Exactly --steps eager
steps are timed between two device synchronisations; `value` is tokens per
second of wall time over them.

Fields beyond the contract:
  roofline      the dominant kernel, k_dq_gemm (one up and one down launch
                per step), against the dense bf16 matrix-core peak: the step's
                algorithmic flops (2 per multiply-add over real rows, no tile
                padding) over the two launches' durations, which the library
                brackets with HIP events recorded on the launch stream
                (moe_layer_forward_profiled).  Median over --kernel-steps
                steps after the timed region; the timed region's own mean is
                reported beside it.  `traffic` is the HBM bytes per launch
                rocprofv3 counted (FETCH_SIZE + WRITE_SIZE, scaled by what the
                counters read for a plain copy), taken from profiles/ only
                while the kernel's sources are the ones that were counted.
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  router        the router step fused with routing (moe_router_topk: logits
                x . W_r^T on the matrix cores, top-K, softmax) at 4314 and at 1
                token (graph replays of 20 calls, so host launch latency is
                not counted), next to moe_route_topk on given logits
  decode        the three decode workloads (1 token; 32 tokens with a skewed
                router; 2 tokens with SwiGLU experts), each timed as the median
                of --decode-replays replays of a HIP graph of 16 steps that
                walk 16 device copies of the weights (as 16 layers would, so no
                step finds its weights in the 256 MB Infinity Cache), with its
                own HBM roofline: the touched NVFP4 weights' bytes over the
                duration of the step's weight-streaming kernels.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_COPIES = 16
SETTLE_STEPS = 20  # untimed steps before the warmup steps (see bench_main)
METRIC = "MoE-layer tokens/s; decode HBM GB/s & prefill TFLOPS as % of MI355X peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill4314")
    p.add_argument("--kernel-steps", type=int, default=50, help="profiled steps for the kernel medians")
    p.add_argument("--decode", default="decode1,decode32_zipf,gated2",
                   help="decode workloads benchmarked beside the main line ('' for none)")
    p.add_argument("--decode-replays", type=int, default=50)
    p.add_argument("--no-router", action="store_true")
    p.add_argument("--copies", type=int, default=N_COPIES)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB, 5 times (the "
                        "reference for scaling FETCH_SIZE / WRITE_SIZE), then exit")
    return p.parse_args()


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_bandwidth_gbs(mib: int = 1024, reps: int = 5) -> float:
    """Measured HBM bandwidth of a plain device-to-device copy of `mib` MiB
    (bytes read + bytes written over the best of `reps` event-timed copies):
    context for the 8 TB/s spec peak, outside the timed region."""
    import torch
    src = torch.empty((mib << 20,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None or ms < best else best
    del src, dst
    return round(2 * (mib << 20) / (best * 1e-3) / 1e9, 1)


def copy_probe(mb: int):
    import torch
    src = torch.empty((mb << 20,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mb << 20, "launches": 5}))


DECODE_KERNEL_SOURCES = ("dq_layer.hip", "nvfp4_device.hpp", "launch.hpp")
PREFILL_KERNEL_SOURCES = ("dq_gemm.hip", "nvfp4_device.hpp", "launch.hpp")
GEMV_KERNEL_SOURCES = ("dq_gemv.hip", "nvfp4_device.hpp", "launch.hpp")


def kernel_source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_block_scaled_topk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str, sources):
    """HBM bytes per launch of `kernel` from the committed counter summary for
    this workload, if it was taken from the current sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_source_digest(sources):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def weight_bytes(t) -> int:
    return int(t.codes.nbytes + t.scales.nbytes + t.globals_.nbytes)


def per_expert_bytes(t) -> int:
    return weight_bytes(t) // t.n_experts


def decode_step_bytes(inp, ids) -> dict:
    """Algorithmic HBM bytes of one decode step: each picked expert's and the
    shared expert's NVFP4 weights once (codes + scales + global), x, the
    logits, the output written.  The intermediates (h, the expert outputs)
    pass between workgroups through the caches and are not counted."""
    import numpy as np
    distinct = len(np.unique(ids))
    xb = 4 if inp.x_dtype == "f32" else 2
    w = distinct * (per_expert_bytes(inp.up) + per_expert_bytes(inp.down))
    if inp.fs > 0:
        w += weight_bytes(inp.shared_up) + weight_bytes(inp.shared_down)
    act = inp.n * inp.d * xb + inp.n * inp.E * 4 + inp.n * inp.d * 4
    return dict(weights=w, activations=act, total=w + act, distinct_experts=distinct)


def layer_ffn_flops(inp) -> dict:
    """2 flops per multiply-add over real rows (no tile padding): the up and the
    down launch, shared + routed."""
    R = inp.n * inp.K
    up_rows = 2 * inp.f if inp.act == "swiglu" else inp.f
    up = 2 * R * inp.d * up_rows
    down = 2 * R * inp.f * inp.d
    if inp.fs > 0:
        up += 2 * inp.n * inp.d * inp.fs
        down += 2 * inp.n * inp.fs * inp.d
    return {"up": up, "down": down, "total": up + down}


def cpu_baseline(inp, budget_s: float) -> dict:
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    if inp.n <= 64:
        calls = 0
        while True:
            oracle.layer(inp, threads=threads)
            calls += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        tokens = calls * inp.n
        sample = f"{calls} full oracle layer calls on the {inp.name} inputs ({tokens} tokens)"
    else:
        ids, w = oracle.route_topk(inp.logits, inp.K)
        rng = np.random.default_rng(0)
        tokens = 0
        while time.perf_counter() - t0 < budget_s:
            t = int(rng.integers(0, inp.n))
            oracle.layer_sampled(inp, [t], ids, w, threads=threads)
            tokens += 1
        dt = time.perf_counter() - t0
        sample = (f"{tokens} tokens of the {inp.name} layer drawn at random, one oracle call each "
                  f"(shared expert + {inp.K} picked experts + WeightedRowSum; routing once for the batch)")
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def median(v):
    import numpy as np
    return float(np.median(np.asarray(v, dtype=np.float64)))


# ---------------------------------------------------------------------------
# the main line: eager steps of one layer (prefill)
# ---------------------------------------------------------------------------

def bench_main(args, ops, synth):
    import numpy as np
    import torch

    dev = "cuda:0"
    t_gen = time.perf_counter()
    inp = synth.make_layer(args.workload)
    gen_s = time.perf_counter() - t_gen
    layer = ops.MoELayer(inp, device=dev)
    x = torch.from_numpy(np.ascontiguousarray(inp.x.view(np.int16) if inp.x.dtype == np.uint16 else inp.x)).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    stream = torch.cuda.Stream()
    E8 = ops.PROFILE_EVENTS
    torch.cuda.synchronize()
    # Settle steps before the warmup: after the set-up the GPU's first
    # launches run slow (the prefill GEMM launches take up to 40 % longer over
    # the first ~15 steps, as the clocks come up), so that few warmup steps
    # would leave part of that ramp inside the timed region.
    log(f"{inp.name}: inputs in {gen_s:.1f} s; {SETTLE_STEPS} settle + {args.warmup} warmup steps")
    with torch.cuda.stream(stream):
        for _ in range(SETTLE_STEPS + max(1, args.warmup)):
            layer.forward_fused(x, logits, stream=stream, check=False)
    torch.cuda.synchronize()

    # ---- timed region: exactly args.steps steps, the library recording HIP
    # events between its launches on the launch stream ----
    K = args.steps
    ev = ops.HipEvents(E8 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(K):
            layer.forward_profiled(x, logits, ev.slice(E8 * i), stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region = [[ev.elapsed_ms(E8 * i + j, E8 * i + j + 1) * 1e3 for j in range(E8 - 1)] for i in range(K)]
    ev.close()
    log(f"{inp.name}: {K} timed steps in {elapsed * 1e3:.1f} ms")

    # ---- kernel medians: a further profiled pass ----
    KS = max(1, args.kernel_steps)
    ev = ops.HipEvents(E8 * KS)
    with torch.cuda.stream(stream):
        for i in range(KS):
            layer.forward_profiled(x, logits, ev.slice(E8 * i), stream=stream)
    torch.cuda.synchronize()
    prof = [[ev.elapsed_ms(E8 * i + j, E8 * i + j + 1) * 1e3 for j in range(E8 - 1)] for i in range(KS)]
    ev.close()
    names = ["route_gather", "split", "decode_up", "gemm_up", "decode_down", "gemm_down", "combine"]
    phase_med = {nm: median([r[j] for r in prof]) for j, nm in enumerate(names)}
    step_med = median([sum(r) for r in prof])

    fl = layer_ffn_flops(inp)
    gemm_us = [r[3] + r[5] for r in prof]
    g_med = median(gemm_us)
    tf = fl["total"] / (g_med * 1e-6) / 1e12
    region_gemm = float(np.mean([r[3] + r[5] for r in region]))
    roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("k_dq_gemm", inp.name, PREFILL_KERNEL_SOURCES),
                "kernel": "k_dq_gemm (grouped bf16 MFMA GEMM with the NVFP4 unpack fused; one up and one down "
                          "launch per step, shared + routed experts)",
                "flops_per_launch": fl["total"] // 2, "flops": fl,
                "us_per_launch": round(g_med / 2, 3),
                "us_up_down_median": [round(phase_med["gemm_up"], 2), round(phase_med["gemm_down"], 2)],
                "timed_region_us_per_launch_mean": round(region_gemm / 2, 3),
                "kernel_steps": KS, "timing": "HIP events recorded by the library on the launch stream"}
    ids = layer.views()["ids"].cpu().numpy()
    counts = np.diff(layer.views()["offsets"].cpu().numpy())
    return inp, gen_s, elapsed, roofline, {k: round(v, 2) for k, v in phase_med.items()}, step_med, counts, ids


# ---------------------------------------------------------------------------
# decode workloads: HIP-graph replays over 16 weight copies
# ---------------------------------------------------------------------------

def bench_decode(name, args, ops, synth):
    import numpy as np
    import torch

    dev = "cuda:0"
    inp = synth.make_layer(name)
    layer = ops.MoELayer(inp, device=dev, single_launch=True)
    copies = [layer.weights()]
    for _ in range(args.copies - 1):
        copies.append(tuple(None if w is None else w.clone() for w in layer.weights()))
    x = torch.from_numpy(np.ascontiguousarray(inp.x.view(np.int16) if inp.x.dtype == np.uint16 else inp.x)).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    L = len(copies)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(2 * L):
            layer.forward_fused(x, logits, weights=copies[i % L], stream=stream, check=False)
    torch.cuda.synchronize()
    layer.check_wait_error()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in copies:
            layer.forward_fused(x, logits, weights=c, stream=stream, check=False)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    v = layer.views()
    launches0 = int(v["decode_launch"].cpu()[0])
    R = max(1, args.decode_replays)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            graph.replay()
            b.record(stream)
    torch.cuda.synchronize()
    layer.check_wait_error()
    rep_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    single = int(v["decode_launch"].cpu()[0]) - launches0 == R * L
    step_us = median(rep_us) / L
    ids = v["ids"].cpu().numpy()
    b = decode_step_bytes(inp, ids)
    out = {"tokens": inp.n, "d_model": inp.d, "experts": inp.E, "top_k": inp.K, "d_ff": inp.f,
           "shared_d_ff": inp.fs, "activation": inp.act, "weight_copies": L, "replays": R,
           "tokens_per_s": round(inp.n / (step_us * 1e-6), 1), "us_per_step_median": round(step_us, 3)}
    if single:
        # one launch per step: the graph replay's event time over its launches
        ach = b["total"] / (step_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("k_decode_step", name, DECODE_KERNEL_SOURCES),
                           "kernel": "k_decode_step (the whole decode step in one persistent launch)",
                           "bytes_per_launch": b["total"], "us_per_launch": round(step_us, 3), "bytes": b}
    else:
        # the weight-streaming launches of k_dq_gemv (one up, one down), timed
        # with the library's events in an eager pass over the same copies
        E8 = ops.PROFILE_EVENTS
        n = 2 * L
        ev = ops.HipEvents(E8 * n)
        with torch.cuda.stream(stream):
            for i in range(n):
                layer.forward_profiled(x, logits, ev.slice(E8 * i), weights=copies[i % L], stream=stream)
        torch.cuda.synchronize()
        up = median([ev.elapsed_ms(E8 * i + 2, E8 * i + 3) * 1e3 for i in range(n)])
        dn = median([ev.elapsed_ms(E8 * i + 4, E8 * i + 5) * 1e3 for i in range(n)])
        ev.close()
        ach = b["weights"] / ((up + dn) * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("k_dq_gemv", name, GEMV_KERNEL_SOURCES),
                           "kernel": "k_dq_gemv (decode dequant-GEMV: one up and one down launch per step, "
                                     "shared + routed experts)",
                           "bytes_per_launch": b["weights"] // 2, "us_per_launch": round((up + dn) / 2, 3),
                           "us_up_down_median": [round(up, 2), round(dn, 2)], "bytes": b}
    del copies, layer, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bench_router(ops, synth, reps=10, per_graph=20):
    """GPU time of moe_router_topk (and of moe_route_topk on the same logits)
    for the prefill and the batch-1 decode workloads: each call captured
    per_graph times into a HIP graph, the median replay time over `reps`
    replays divided by per_graph (so host launch latency is not counted)."""
    import numpy as np
    import torch

    out = {}
    for name in ("prefill4314", "decode1"):
        cfg = synth.WORKLOADS[name]
        x = synth.draw_activations(name)
        x = torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).to("cuda:0")
        wr = torch.from_numpy(synth.draw_router(name).view(np.int16)).to("cuda:0")
        n, E, K, d = cfg["n"], cfg["E"], cfg["K"], cfg["d"]
        ws = torch.empty((ops.moe_router_workspace_size(n, E),), dtype=torch.uint8, device="cuda:0")
        ops.moe_router_workspace_init(ws, n)
        logits = torch.empty((n, E), dtype=torch.float32, device="cuda:0")
        ids = torch.empty((n, K), dtype=torch.int32, device="cuda:0")
        w = torch.empty((n, K), dtype=torch.float32, device="cuda:0")
        stream = torch.cuda.Stream()
        med = {}
        for key, fn in (("router_topk", lambda: ops.moe_router_topk(x, wr, K, ws, ids, w, logits, stream=stream)),
                        ("route_topk", lambda: ops.moe_route_topk(logits, K, ids, w, stream=stream))):
            with torch.cuda.stream(stream):
                for _ in range(3):
                    fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(per_graph):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            with torch.cuda.stream(stream):
                for a, b in ev:
                    a.record(stream)
                    g.replay()
                    b.record(stream)
            torch.cuda.synchronize()
            med[key] = round(median([a.elapsed_time(b) * 1e3 for a, b in ev]) / per_graph, 2)
        flops = 2 * n * E * d
        out[name] = {"tokens": n, "experts": E, "top_k": K, "d_model": d, "router_weights": "bf16",
                     "us_router_topk_median": med["router_topk"], "us_route_topk_only_median": med["route_topk"],
                     "router_gemm_tflops": round(flops / (med["router_topk"] * 1e-6) / 1e12, 2),
                     "router_weight_gbs": round(E * d * 2 / (med["router_topk"] * 1e-6) / 1e9, 1),
                     "timing": f"median of {reps} replays of a graph of {per_graph} calls"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 (sharding the "
                                   "layer across GPUs is not built)"}))
        sys.exit(2)
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb)
        return
    import torch

    from bit_block_scaled_topk_amd import ops, synth

    torch.cuda.set_device(0)
    inp, gen_s, elapsed, roofline, phases, step_med, counts, ids = bench_main(args, ops, synth)
    roofline["copy_gbs"] = copy_bandwidth_gbs()
    decode = {}
    for name in [w for w in args.decode.split(",") if w]:
        log(f"decode workload {name}")
        decode[name] = bench_decode(name, args, ops, synth)
    router = None
    if not args.no_router:
        log("router")
        router = bench_router(ops, synth)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cpu = cpu_baseline(inp, args.cpu_seconds)
    K = args.steps
    line = {
        "metric": METRIC,
        "value": round(inp.n * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": SETTLE_STEPS,
        "ms_per_step": round(elapsed / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": inp.name, "tokens": inp.n, "d_model": inp.d, "experts": inp.E, "top_k": inp.K,
                   "d_ff": inp.f, "shared_d_ff": inp.fs, "activation": inp.act,
                   "activations_dtype": inp.x_dtype, "weights": "nvfp4 (e2m1, e4m3/16, fp32 global)",
                   "routed_rows": int(counts.sum()), "rows_per_expert": [int(counts.min()), int(counts.max())],
                   "launch": "eager", "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_median_us": round(step_med, 2),
        "step_breakdown_us_median": phases,
        "input_gen_s": round(gen_s, 1),
        "decode": decode,
        "router": router,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
