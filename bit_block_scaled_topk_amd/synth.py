"""Seeded synthetic inputs for the NVFP4 MoE expert-FFN layer.

This module only *draws* inputs: router logits, activations and NVFP4-encoded
expert weights.  It holds none of the layer's arithmetic (no routing, gather,
dequantisation, matmul or combine), so both the HIP path and the CPU oracle can
take their inputs from it without sharing any of the computation under test.

Workloads (the five layer shapes the method is exercised on):

    tiny16        16 tokens, d_model 64, 8 experts, topK 2, relu^2 d_ff 128,
                  shared expert d_ff 128, fp32 activations
    decode1       1 token, d_model 2688, 128 experts, topK 6, relu^2 d_ff 1856,
                  shared d_ff 3712, bf16 activations
    decode32_zipf 32 tokens, shapes of decode1, Zipf(1.1)-skewed router logits
    prefill4314   4314 tokens, shapes of decode1
    gated2        2 tokens, d_model 2048, 256 experts, topK 8, SwiGLU experts with
                  fused gate-up [2*1024, 2048] and down [2048, 1024], no shared
                  expert, bf16 activations

Recipe (every tensor has its own child stream of ``numpy.random.SeedSequence``,
so tensors can be drawn in parallel and each is reproducible on its own):

    stream 0          router logits [n, E], float32 N(0, 1); for the Zipf
                      workload logit[t, e] = -1.1 * ln(rank_e) + N(0, 1) with
                      rank a seeded permutation of 1..E (drawn first)
    stream 1          activations [n, d] float32 N(0, 1), rounded to bfloat16
                      (round to nearest even) for the bf16 workloads
    streams 2+2e, 3+2e  expert e's up and down weights, float32 N(0, 0.02)
    streams 2+2E, 3+2E  shared expert's up and down weights
    stream 4+2E       router weights W_r [E, d], float32 N(0, 0.02) rounded to
                      bfloat16 (for the router GEMM x . W_r^T; with d in the
                      thousands its logits are about N(0, 1), like stream 0's)

NVFP4 encoding of a weight W [rows, cols] (cols along the input axis):

    global g  = max|W| / (6 * 448)           (1 when W is all zero)
    per 16-element block b of a row:  scale s_b = e4m3(min(max|W_b| / 6 / g, 448))
                                      (cast with torch.float8_e4m3fn after clamping)
    per element:  code = nearest e2m1 value to  w / (s_b * g), ties to the even code,
                  saturating at +-6; sign bit set for negative w
    codes   uint8 [rows, cols/2], element 2i in the low nibble of byte i
    scales  uint8 [rows, cols/16]

The e2m1 nearest-value search uses the midpoints of the E2M1 value grid; the
decoding side of the format is not implemented here.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

WORKLOADS: Dict[str, dict] = {
    "tiny16": dict(n=16, d=64, E=8, K=2, f=128, fs=128, act="relu2", x_dtype="f32",
                   seed=1, logits="normal"),
    "decode1": dict(n=1, d=2688, E=128, K=6, f=1856, fs=3712, act="relu2", x_dtype="bf16",
                    seed=2, logits="normal"),
    "decode32_zipf": dict(n=32, d=2688, E=128, K=6, f=1856, fs=3712, act="relu2",
                          x_dtype="bf16", seed=3, logits="zipf"),
    "prefill4314": dict(n=4314, d=2688, E=128, K=6, f=1856, fs=3712, act="relu2",
                        x_dtype="bf16", seed=4, logits="normal"),
    "gated2": dict(n=2, d=2048, E=256, K=8, f=1024, fs=0, act="swiglu", x_dtype="bf16",
                   seed=5, logits="normal"),
}

WEIGHT_STD = 0.02
E4M3_MAX = 448.0
E2M1_MAX = 6.0


@dataclasses.dataclass
class NVFP4Tensor:
    """NVFP4 weights for ``n_experts`` experts of shape [rows, cols]."""
    codes: np.ndarray    # uint8 [E, rows, cols // 2]
    scales: np.ndarray   # uint8 [E, rows, cols // 16]
    globals_: np.ndarray  # float32 [E]
    rows: int
    cols: int

    @property
    def n_experts(self) -> int:
        return int(self.codes.shape[0])

    def nbytes(self) -> int:
        return int(self.codes.nbytes + self.scales.nbytes + self.globals_.nbytes)


@dataclasses.dataclass
class LayerInputs:
    name: str
    n: int
    d: int
    E: int
    K: int
    f: int
    fs: int
    act: str
    x_dtype: str
    logits: np.ndarray          # float32 [n, E]
    x: np.ndarray               # float32 [n, d] or uint16 bf16 bits [n, d]
    up: NVFP4Tensor             # rows = f (relu2) or 2f (swiglu), cols = d
    down: NVFP4Tensor           # rows = d, cols = f
    shared_up: Optional[NVFP4Tensor]
    shared_down: Optional[NVFP4Tensor]


# ----------------------------------------------------------------------------
# encoding helpers (input side only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Non-negative float32 (already clamped to <= 448) -> E4M3FN bytes, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _e4m3_value(b: np.ndarray) -> np.ndarray:
    """E4M3FN bytes -> float32 through torch's own cast (used to place codes)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().copy()


# Midpoints between consecutive E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}.  At a tie
# the even code (0, 2, 4, 6 -> magnitudes 0, 1, 2, 4) wins: '>' keeps the lower
# code at the tie, '>=' takes the upper one.
_E2M1_MIDPOINTS = ((0.25, ">"), (0.75, ">="), (1.25, ">"), (1.75, ">="),
                   (2.5, ">"), (3.5, ">="), (5.0, ">"))


def _e2m1_encode(q: np.ndarray) -> np.ndarray:
    a = np.abs(q)
    idx = np.zeros(a.shape, dtype=np.uint8)
    for mid, op in _E2M1_MIDPOINTS:
        idx += (a > mid) if op == ">" else (a >= mid)
    sign = (q < 0).astype(np.uint8) << 3
    return idx | sign


def quantize_nvfp4(w: np.ndarray):
    """float32 [rows, cols] -> (codes [rows, cols/2], scales [rows, cols/16], global)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    g = np.float32(amax / (E2M1_MAX * E4M3_MAX)) if amax > 0 else np.float32(1.0)
    blocks = w.reshape(rows, cols // 16, 16)
    bmax = np.max(np.abs(blocks), axis=2)
    s_req = np.minimum(bmax / np.float32(E2M1_MAX) / g, np.float32(E4M3_MAX)).astype(np.float32)
    s_bytes = _e4m3_encode(s_req)
    s_val = _e4m3_value(s_bytes)
    denom = (s_val * g)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(denom > 0, blocks / np.where(denom > 0, denom, 1), 0).astype(np.float32)
    codes = _e2m1_encode(q).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_bytes.reshape(rows, cols // 16), g


def _draw_weight(seedseq, rows, cols):
    rng = np.random.default_rng(seedseq)
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(WEIGHT_STD)
    return quantize_nvfp4(w)


def _draw_tensor(seqs, rows, cols, pool) -> NVFP4Tensor:
    E = len(seqs)
    codes = np.empty((E, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((E, rows, cols // 16), dtype=np.uint8)
    globals_ = np.empty((E,), dtype=np.float32)

    def one(e):
        c, s, g = _draw_weight(seqs[e], rows, cols)
        codes[e] = c
        scales[e] = s
        globals_[e] = g

    list(pool.map(one, range(E)))
    return NVFP4Tensor(codes, scales, globals_, rows, cols)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cfg(name: str, overrides) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return cfg


def _streams(cfg):
    # child i depends only on (seed, i), so adding the router's stream at the
    # end left every other stream unchanged
    return np.random.SeedSequence(cfg["seed"]).spawn(5 + 2 * cfg["E"])


def draw_logits(name: str, **overrides) -> np.ndarray:
    """Router logits [n, E] float32 of workload ``name`` (stream 0)."""
    cfg = _cfg(name, overrides)
    n, E = cfg["n"], cfg["E"]
    rng_l = np.random.default_rng(_streams(cfg)[0])
    if cfg["logits"] == "zipf":
        rank = rng_l.permutation(E).astype(np.float64) + 1.0
        noise = rng_l.standard_normal((n, E), dtype=np.float32)
        return (-1.1 * np.log(rank)[None, :] + noise).astype(np.float32)
    return rng_l.standard_normal((n, E), dtype=np.float32)


def draw_activations(name: str, **overrides) -> np.ndarray:
    """Activations [n, d] of workload ``name`` (stream 1): float32, or bfloat16
    bit patterns (uint16) for the bf16 workloads."""
    cfg = _cfg(name, overrides)
    rng_x = np.random.default_rng(_streams(cfg)[1])
    x = rng_x.standard_normal((cfg["n"], cfg["d"]), dtype=np.float32)
    if cfg["x_dtype"] == "bf16":
        x = f32_to_bf16_bits(x)
    return x


def draw_router(name: str, **overrides) -> np.ndarray:
    """Router weights W_r [E, d] of workload ``name`` (stream 4 + 2E) as
    bfloat16 bit patterns (uint16)."""
    cfg = _cfg(name, overrides)
    rng = np.random.default_rng(_streams(cfg)[4 + 2 * cfg["E"]])
    w = rng.standard_normal((cfg["E"], cfg["d"]), dtype=np.float32) * np.float32(WEIGHT_STD)
    return f32_to_bf16_bits(w)


def make_layer(name: str, **overrides) -> LayerInputs:
    """Draw the seeded inputs of workload ``name`` (see module docstring)."""
    cfg = _cfg(name, overrides)
    n, d, E, K, f, fs = cfg["n"], cfg["d"], cfg["E"], cfg["K"], cfg["f"], cfg["fs"]
    up_rows = 2 * f if cfg["act"] == "swiglu" else f
    kids = _streams(cfg)
    logits = draw_logits(name, **overrides)
    x = draw_activations(name, **overrides)
    with _cf.ThreadPoolExecutor(_threads()) as pool:
        up = _draw_tensor([kids[2 + 2 * e] for e in range(E)], up_rows, d, pool)
        down = _draw_tensor([kids[3 + 2 * e] for e in range(E)], d, f, pool)
        if fs > 0:
            sh_up = _draw_tensor([kids[2 + 2 * E]], fs, d, pool)
            sh_dn = _draw_tensor([kids[3 + 2 * E]], d, fs, pool)
        else:
            sh_up = sh_dn = None
    return LayerInputs(name=name, n=n, d=d, E=E, K=K, f=f, fs=fs, act=cfg["act"],
                       x_dtype=cfg["x_dtype"], logits=logits, x=x, up=up, down=down,
                       shared_up=sh_up, shared_down=sh_dn)


def random_nvfp4(seed: int, n_experts: int, rows: int, cols: int, std: float = WEIGHT_STD) -> NVFP4Tensor:
    """A stand-alone seeded NVFP4 tensor (for unit-level tests)."""
    kids = np.random.SeedSequence(seed).spawn(n_experts)
    codes = np.empty((n_experts, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((n_experts, rows, cols // 16), dtype=np.uint8)
    globals_ = np.empty((n_experts,), dtype=np.float32)
    for e in range(n_experts):
        rng = np.random.default_rng(kids[e])
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
        codes[e], scales[e], globals_[e] = quantize_nvfp4(w)
    return NVFP4Tensor(codes, scales, globals_, rows, cols)


def random_bytes_nvfp4(seed: int, n_experts: int, rows: int, cols: int,
                       allow_nan_scale: bool = False) -> NVFP4Tensor:
    """NVFP4 tensor with uniformly random code and scale bytes (every code, every
    finite scale), and random positive globals: exercises the whole format."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n_experts, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(n_experts, rows, cols // 16), dtype=np.uint8)
    if not allow_nan_scale:
        nan = (scales & 0x7F) == 0x7F
        scales[nan] = scales[nan] & 0xF0  # replace NaN bytes by finite ones
    globals_ = (rng.random(n_experts, dtype=np.float32) * np.float32(0.01) +
                np.float32(1e-4)).astype(np.float32)
    return NVFP4Tensor(codes, scales, globals_, rows, cols)
