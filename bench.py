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
  roofline      the step's dominant kernel against its roofline.  A decode
                step of one or two tokens is one launch (k_decode_layer):
                its average duration is the timed region measured with HIP
                events on the launch stream, divided by the launches in it,
                and it is held against 8 TB/s with the step's algorithmic
                bytes (the picked experts' and the shared expert's NVFP4
                weights once, x, the logits, the output).  A prefill step's
                dominant kernel is the grouped GEMM (k_dq_gemm: one up and one
                down launch), timed with HIP events between the library's
                launch phases, against the dense bf16 matrix-core peak.
                `traffic` is the HBM bytes per launch that rocprofv3 counted
                (FETCH_SIZE + WRITE_SIZE, scaled by what the counters read for
                a plain copy), taken from profiles/ only while the kernel's
                sources are the ones that were counted (else null).
                `copy_gbs` is the HBM bandwidth a plain 1 GiB device copy
                reaches on the same GPU (read + write bytes), for context.
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
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB, 5 times (the "
                        "reference for scaling FETCH_SIZE / WRITE_SIZE), then exit")
    return p.parse_args()


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


def kernel_source_digest(files=DECODE_KERNEL_SOURCES) -> str:
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


def layer_ffn_flops(inp) -> int:
    """2 flops per multiply-add over real rows (no tile padding), shared + routed."""
    R = inp.n * inp.K
    up_rows = 2 * inp.f if inp.act == "swiglu" else inp.f
    fl = 2 * R * inp.d * up_rows + 2 * R * inp.f * inp.d
    if inp.fs > 0:
        fl += 2 * inp.n * inp.d * inp.fs * 2
    return fl


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
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb)
        return
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
    # the one-time scale repack of each copy (the prefill GEMM reads it), timed
    # apart from the steps
    torch.cuda.synchronize()
    t_pack = time.perf_counter()
    for c in copies[1:]:
        for w in c:
            if w is not None:
                w.pack()
    torch.cuda.synchronize()
    prepack_ms = (time.perf_counter() - t_pack) * 1e3 / max(1, len(copies) - 1)
    xs = inp.x.view(np.int16) if inp.x.dtype == np.uint16 else inp.x
    x = torch.from_numpy(np.ascontiguousarray(xs)).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    L = len(copies)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def one_pass():
        for c in copies:
            layer.forward_fused(x, logits, weights=c)

    # warmup (eager) on the bench stream
    with torch.cuda.stream(stream):
        for i in range(max(1, args.warmup)):
            layer.forward_fused(x, logits, weights=copies[i % L])
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
    launches0 = int(layer.views()["decode_launch"].cpu()[0])
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev_start.record()  # on `stream`, the launch stream
        if graph is not None:
            for _ in range(steps // L):
                graph.replay()
        else:
            for i in range(steps):
                layer.forward_fused(x, logits, weights=copies[i % L])
        ev_end.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_us = ev_start.elapsed_time(ev_end) * 1e3
    single_launch = int(layer.views()["decode_launch"].cpu()[0]) - launches0 == steps
    tokens_per_s = inp.n * steps / elapsed

    # ---- kernel timing: HIP events recorded by the library between its launch
    # phases (moe_layer_forward_profiled), on the launch stream, same copies ----
    k_steps = min(steps, 20 * L)
    ev = ops.HipEvents(6 * k_steps)
    with torch.cuda.stream(stream):
        for i in range(k_steps):
            layer.forward_profiled(x, logits, ev.slice(6 * i), weights=copies[i % L])
    torch.cuda.synchronize()
    names = ["route_gather", "split", "up", "down", "combine"]
    phase = {nm: [ev.elapsed_ms(6 * i + j, 6 * i + j + 1) * 1e3 for i in range(k_steps)]
             for j, nm in enumerate(names)}
    ev.close()
    breakdown = {k: float(np.mean(v)) for k, v in phase.items()}
    v = layer.views()
    ids = v["ids"].cpu().numpy()
    if single_launch:
        # one launch per step: the timed region's event time over its launches
        us = region_us / steps
        b = decode_step_bytes(inp, ids)
        achieved = b["total"] / (us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("k_decode_layer", inp.name, DECODE_KERNEL_SOURCES),
                    "kernel": "k_decode_layer (the whole decode step in one persistent launch)",
                    "bytes_per_launch": b["total"], "us_per_launch": round(us, 3), "bytes": b}
        breakdown = {"decode_layer_eager": breakdown["route_gather"]}
    elif np.diff(v["offsets"].cpu().numpy()).max() <= layer.gemv_max_rows:
        # every expert on the decode GEMV: one up and one down launch of k_dq_gemv
        ffn_us = breakdown["up"] + breakdown["down"]
        b = decode_step_bytes(inp, ids)
        achieved = b["weights"] / (ffn_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("k_dq_gemv", inp.name, GEMV_KERNEL_SOURCES),
                    "kernel": "k_dq_gemv (decode dequant-GEMV: one up and one down launch per step, "
                              "shared + routed experts)",
                    "bytes_per_launch": b["weights"] // 2, "us_per_launch": round(ffn_us / 2, 3), "bytes": b}
    else:
        flops = layer_ffn_flops(inp)
        ffn_us = breakdown["up"] + breakdown["down"]
        tf = flops / (ffn_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic("k_dq_gemm", inp.name, PREFILL_KERNEL_SOURCES),
                    "kernel": "k_dq_gemm (prefill grouped bf16 GEMM: one up and one down launch per step, "
                              "shared + routed experts)",
                    "flops_per_launch": flops // 2, "us_per_launch": round(ffn_us / 2, 3)}

    roofline["copy_gbs"] = copy_bandwidth_gbs()

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
        "prepack_ms_per_weight_set": round(prepack_ms, 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
