"""MoE-layer benchmark on one MI355X.

A step is one pass of the whole layer -- topK routing, gather, shared expert,
routed experts (NVFP4 up -> relu^2 -> down), WeightedRowSum -- over one batch
of seeded synthetic input (bit_block_scaled_topk_amd.synth), all inputs and
weights resident in HBM before the timed region starts.

The default workload is the batch-1 decode layer (1 token, d_model 2688, 128
experts, topK 6, relu^2 d_ff 1856, shared d_ff 3712, bf16 activations).  The
timed loop walks 16 device-resident copies of the layer's weights, one per
step, as consecutive MoE layers of a model would, so no step finds its
weights in the 256 MB Infinity Cache.  Steps are replayed from a HIP graph
(the layer allocates and synchronises nothing, so it captures whole).

Prints ONE JSON line with the contract fields plus:
  roofline      the routed-expert FFN of a step (its two decode GEMV launches,
                timed with HIP events on the launch stream in an eager pass
                over the same copies): algorithmic bytes / duration vs 8 TB/s
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3200)
    p.add_argument("--warmup", type=int, default=320)
    p.add_argument("--workload", default="decode1")
    p.add_argument("--copies", type=int, default=N_COPIES)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    p.add_argument("--traffic", default=None,
                   help="JSON file with measured HBM bytes per routed-FFN call (from rocprofv3 --pmc)")
    return p.parse_args()


def weight_bytes(t) -> int:
    return int(t.codes.nbytes + t.scales.nbytes + t.globals_.nbytes)


def per_expert_bytes(t) -> int:
    return weight_bytes(t) // t.n_experts


def routed_ffn_bytes(inp, ids) -> dict:
    """Algorithmic bytes of one routed nvfp4_expert_ffn call: every picked
    expert's up and down NVFP4 weights once (codes + scales + global), the
    gathered activations read, h written and read once at fp32, y written."""
    import numpy as np
    distinct = len(np.unique(ids))
    R = inp.n * inp.K
    xb = 4 if inp.x_dtype == "f32" else 2
    w = distinct * (per_expert_bytes(inp.up) + per_expert_bytes(inp.down))
    act = R * inp.d * xb + 2 * R * inp.f * 4 + R * inp.d * 4
    return dict(weights=w, activations=act, total=w + act, distinct_experts=distinct)


def routed_ffn_flops(inp, ids) -> int:
    R = inp.n * inp.K
    up_rows = 2 * inp.f if inp.act == "swiglu" else inp.f
    return 2 * R * inp.d * up_rows + 2 * R * inp.f * inp.d


def cpu_baseline(inp, budget_s: float) -> dict:
    import oracle
    threads = oracle.default_threads()
    sample_tokens = list(range(inp.n))
    t0 = time.perf_counter()
    calls = 0
    if inp.n <= 64:
        while True:
            oracle.layer(inp, threads=threads)
            calls += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        tokens = calls * inp.n
        sample = f"{calls} full oracle layer calls on the {inp.name} inputs ({tokens} tokens)"
    else:
        import numpy as np
        ids, w = oracle.route_topk(inp.logits, inp.K)
        rng = np.random.default_rng(0)
        tokens = 0
        sample_tokens = []
        while time.perf_counter() - t0 < budget_s:
            t = int(rng.integers(0, inp.n))
            oracle.layer_sampled(inp, [t], ids, w, threads=threads)
            tokens += 1
            sample_tokens.append(t)
        dt = time.perf_counter() - t0
        sample = f"{tokens} sampled tokens of the {inp.name} layer (routing, shared + 6 experts each)"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sample": sample,
            "seconds": round(dt, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(the sharded design is described, not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    from bit_block_scaled_topk_amd import ops, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    inp = synth.make_layer(args.workload)
    gen_s = time.perf_counter() - t_gen
    layer = ops.MoELayer(inp, device=dev)
    copies = [layer.weights()]
    for _ in range(args.copies - 1):
        copies.append(tuple(None if w is None else ops.DeviceNVFP4(w.codes.clone(), w.scales.clone(),
                                                                   w.globals_.clone(), w.rows, w.cols)
                            for w in layer.weights()))
    xs = inp.x.view(np.int16) if inp.x.dtype == np.uint16 else inp.x
    x = torch.from_numpy(np.ascontiguousarray(xs)).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    L = len(copies)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def one_pass():
        for c in copies:
            layer.forward(x, logits, weights=c)

    # warmup (eager) on the bench stream
    with torch.cuda.stream(stream):
        for i in range(max(1, args.warmup)):
            layer.forward(x, logits, weights=copies[i % L])
    torch.cuda.synchronize()

    steps = max(L, (args.steps // L) * L)
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            one_pass()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` layer steps ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if graph is not None:
            for _ in range(steps // L):
                graph.replay()
        else:
            for i in range(steps):
                layer.forward(x, logits, weights=copies[i % L])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tokens_per_s = inp.n * steps / elapsed

    # ---- kernel timing: HIP events around each call, eager, same copies ----
    timing = {}
    k_steps = min(steps, 20 * L)
    with torch.cuda.stream(stream):
        for i in range(k_steps):
            layer.forward(x, logits, weights=copies[i % L], timing=timing)
    torch.cuda.synchronize()
    breakdown = {k: float(np.mean([a.elapsed_time(b) for a, b in v]) * 1e3) for k, v in timing.items()}
    ids = layer.ids.cpu().numpy()
    b = routed_ffn_bytes(inp, ids)
    ffn_us = breakdown["routed_ffn"]
    achieved = b["total"] / (ffn_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "routed nvfp4_expert_ffn (k_dq_gemv up + down)",
                "bytes_per_call": b["total"], "us_per_call": round(ffn_us, 3)}
    counts = np.diff(layer.offsets.cpu().numpy())
    if counts.max() > 32:
        flops = routed_ffn_flops(inp, ids)
        tf = flops / (ffn_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "routed nvfp4_expert_ffn (k_dq_gemm up + down)",
                    "flops_per_call": flops, "us_per_call": round(ffn_us, 3)}
    if args.traffic and os.path.exists(args.traffic):
        with open(args.traffic) as fh:
            roofline["traffic"] = json.load(fh).get("bytes_per_call")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    line = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s & prefill TFLOPS as % of MI355X peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": inp.name, "tokens": inp.n, "d_model": inp.d, "experts": inp.E, "top_k": inp.K,
                   "d_ff": inp.f, "shared_d_ff": inp.fs, "activation": inp.act,
                   "activations_dtype": inp.x_dtype, "weights": "nvfp4 (e2m1, e4m3/16, fp32 global)",
                   "weight_copies": L, "launch": "hipgraph" if graph is not None else "eager",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_breakdown_us": {k: round(v, 2) for k, v in breakdown.items()},
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
