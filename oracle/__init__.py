"""CPU oracle for the NVFP4 MoE expert-FFN layer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
fixed summation orders; see that file for the passages each function follows)
and composes the layer from its pieces in plain Python.  Two arithmetics are
offered: IEEE double (the exact values, up to rounding far below binary32's;
the default) and binary32 with fused multiply-adds in one fixed order (the
``*_f32`` functions, ``layer(..., arith="f32")``).

It shares no code with the HIP library: bf16 decoding of activations, the
NVFP4 decode and every sum are its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT_RELU2 = 0
ACT_SWIGLU = 1


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", "-pthread", "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_e2m1.argtypes = [ctypes.c_uint]; L.orc_e2m1.restype = ctypes.c_double
        L.orc_e4m3.argtypes = [ctypes.c_uint]; L.orc_e4m3.restype = ctypes.c_double
        L.orc_round_bf16.argtypes = [ctypes.c_double]; L.orc_round_bf16.restype = ctypes.c_double
        L.orc_dequant.argtypes = [P, P, ctypes.c_float, I, I, I, P]; L.orc_dequant.restype = I
        L.orc_route_topk.argtypes = [P, I, I, I, P, P]; L.orc_route_topk.restype = I
        L.orc_gather_layout.argtypes = [P, I, I, I, P, P, P]; L.orc_gather_layout.restype = I
        L.orc_gather_copy.argtypes = [P, I, I, I, P, I, P]; L.orc_gather_copy.restype = I
        L.orc_expert_ffn.argtypes = [P, I, I, P, I, P, P, P, P, P, P, I, I, I, I, I, P]
        L.orc_expert_ffn.restype = I
        L.orc_linear.argtypes = [P, I, I, P, I, P, P, P, I, I, P]; L.orc_linear.restype = I
        L.orc_weighted_row_sum.argtypes = [P, P, I, P, P, I, I, I]; L.orc_weighted_row_sum.restype = I
        L.orc_expert_ffn_f32.argtypes = [P, I, I, P, I, P, P, P, P, P, P, I, I, I, I, P]
        L.orc_expert_ffn_f32.restype = I
        L.orc_linear_f32.argtypes = [P, I, I, P, I, P, P, P, I, I, P]; L.orc_linear_f32.restype = I
        L.orc_weighted_row_sum_f32.argtypes = [P, P, I, P, P, I, I, I]
        L.orc_weighted_row_sum_f32.restype = I
        L.orc_router_logits.argtypes = [P, I, I, P, I, P]; L.orc_router_logits.restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == 1:
        raise OracleError(f"{what}: invalid argument")
    if rc == 2:
        raise OracleError(f"{what}: index out of range")
    if rc != 0:
        raise OracleError(f"{what}: error {rc}")


def default_threads() -> int:
    # at most 16: the share of host cores one GPU's job gets on a shared machine
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------

def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def e4m3(byte: int) -> float:
    return lib().orc_e4m3(byte)


def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(v)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (a bf16 value is the top half of a binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def activations_f64(x: np.ndarray, x_dtype: str) -> np.ndarray:
    if x_dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)


def dequant(codes: np.ndarray, scales: np.ndarray, global_: float, with_global: bool = True) -> np.ndarray:
    """One NVFP4 tensor [rows, cols] -> float64 values."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = half * 2
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequant(_p(codes), _p(scales), ctypes.c_float(global_), rows, cols,
                             1 if with_global else 0, _p(out)), "dequant")
    return out


# ----------------------------------------------------------------------------
# the steps of the layer
# ----------------------------------------------------------------------------

def route_topk(logits: np.ndarray, K: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n, E = logits.shape
    ids = np.empty((n, K), dtype=np.int32)
    w = np.empty((n, K), dtype=np.float64)
    _check(lib().orc_route_topk(_p(logits), n, E, K, _p(ids), _p(w)), "route_topk")
    return ids, w


def router_logits(x64: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """Router logits x . W_r^T in double, for activations x (double [n, d]) and
    bf16 router weights W_r (bit patterns [E, d]).  Returns [n, E] float64."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    wr = bf16_bits_to_f64(wr_bits)
    n, d = x64.shape
    E = wr.shape[0]
    out = np.empty((n, E), dtype=np.float64)
    _check(lib().orc_router_logits(_p(x64), n, d, _p(np.ascontiguousarray(wr)), E, _p(out)), "router_logits")
    return out


def router_topk(x: np.ndarray, x_dtype: str, wr_bits: np.ndarray, K: int):
    """The router step: logits = x . W_r^T (double, rounded once to binary32, the
    logits' dtype), then route_topk on them.  Returns (ids, weights, logits
    float64 before rounding)."""
    lg = router_logits(activations_f64(x, x_dtype), wr_bits)
    ids, w = route_topk(lg.astype(np.float32), K)
    return ids, w, lg


def gather_layout(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, K = ids.shape
    offsets = np.empty((E + 1,), dtype=np.int32)
    row_token = np.empty((n * K,), dtype=np.int32)
    rows = np.empty((n, K), dtype=np.int32)
    _check(lib().orc_gather_layout(_p(ids), n, K, E, _p(offsets), _p(row_token), _p(rows)),
           "gather_layout")
    return offsets, row_token, rows


def gather_copy(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    n, d = x.shape
    row_token = np.ascontiguousarray(row_token, dtype=np.int32)
    R = row_token.shape[0]
    xg = np.empty((R, d), dtype=x.dtype)
    _check(lib().orc_gather_copy(_p(x), x.itemsize, n, d, _p(row_token), R, _p(xg)), "gather_copy")
    return xg


def expert_ffn(x64: np.ndarray, offsets: np.ndarray, up, down, f: int, act: str,
               bf16_act: bool = False, threads: Optional[int] = None) -> np.ndarray:
    """Packed rows grouped by expert -> y [n_rows, d_out] (float64).

    ``up``/``down`` are objects with ``codes``, ``scales``, ``globals_`` laid out
    [E, rows, ...] (see bit_block_scaled_topk_amd.synth.NVFP4Tensor)."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    n_rows, d = x64.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = offsets.shape[0] - 1
    d_out = down.rows
    out = np.zeros((n_rows, d_out), dtype=np.float64)
    a = ACT_SWIGLU if act == "swiglu" else ACT_RELU2
    uc, us, ug = (np.ascontiguousarray(up.codes), np.ascontiguousarray(up.scales),
                  np.ascontiguousarray(up.globals_, dtype=np.float32))
    dc, ds, dg = (np.ascontiguousarray(down.codes), np.ascontiguousarray(down.scales),
                  np.ascontiguousarray(down.globals_, dtype=np.float32))
    _check(lib().orc_expert_ffn(_p(x64), n_rows, d, _p(offsets), E, _p(uc), _p(us), _p(ug),
                                _p(dc), _p(ds), _p(dg), f, d_out, a, 1 if bf16_act else 0,
                                threads or default_threads(), _p(out)), "expert_ffn")
    return out


def linear(a64: np.ndarray, offsets: np.ndarray, w, threads: Optional[int] = None) -> np.ndarray:
    """One NVFP4 projection per expert group: y = a . W^T (global included)."""
    a64 = np.ascontiguousarray(a64, dtype=np.float64)
    n_rows, k = a64.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = offsets.shape[0] - 1
    out = np.zeros((n_rows, w.rows), dtype=np.float64)
    c, s, g = (np.ascontiguousarray(w.codes), np.ascontiguousarray(w.scales),
               np.ascontiguousarray(w.globals_, dtype=np.float32))
    _check(lib().orc_linear(_p(a64), n_rows, k, _p(offsets), E, _p(c), _p(s), _p(g), w.rows,
                            threads or default_threads(), _p(out)), "linear")
    return out


def weighted_row_sum(dst: np.ndarray, src: np.ndarray, rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Returns dst + sum_j w[i,j] * src[rows[i,j]] (float64; dst is not modified)."""
    out = np.array(dst, dtype=np.float64, order="C", copy=True)
    src = np.ascontiguousarray(src, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n, K = rows.shape
    d = out.shape[1] if out.ndim == 2 else 0
    _check(lib().orc_weighted_row_sum(_p(out), _p(src), src.shape[0], _p(rows), _p(w), n, K, d),
           "weighted_row_sum")
    return out


def activations_f32(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Activations as binary32 (a bf16 value is exact in binary32)."""
    if x_dtype == "bf16":
        b = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return b.view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def expert_ffn_f32(x32: np.ndarray, offsets: np.ndarray, up, down, f: int, act: str,
                   threads: Optional[int] = None) -> np.ndarray:
    """expert_ffn in binary32: each dot product a chain of fmaf in k order, the
    global applied after it, relu^2 / SwiGLU in binary32.  Returns float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    n_rows, d = x32.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = offsets.shape[0] - 1
    d_out = down.rows
    out = np.zeros((n_rows, d_out), dtype=np.float32)
    a = ACT_SWIGLU if act == "swiglu" else ACT_RELU2
    uc, us, ug = (np.ascontiguousarray(up.codes), np.ascontiguousarray(up.scales),
                  np.ascontiguousarray(up.globals_, dtype=np.float32))
    dc, ds, dg = (np.ascontiguousarray(down.codes), np.ascontiguousarray(down.scales),
                  np.ascontiguousarray(down.globals_, dtype=np.float32))
    _check(lib().orc_expert_ffn_f32(_p(x32), n_rows, d, _p(offsets), E, _p(uc), _p(us), _p(ug),
                                    _p(dc), _p(ds), _p(dg), f, d_out, a, threads or default_threads(),
                                    _p(out)), "expert_ffn_f32")
    return out


def linear_f32(a32: np.ndarray, offsets: np.ndarray, w, threads: Optional[int] = None) -> np.ndarray:
    """linear in binary32 (fmaf chain in k order, then times the global)."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    n_rows, k = a32.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = offsets.shape[0] - 1
    out = np.zeros((n_rows, w.rows), dtype=np.float32)
    c, s, g = (np.ascontiguousarray(w.codes), np.ascontiguousarray(w.scales),
               np.ascontiguousarray(w.globals_, dtype=np.float32))
    _check(lib().orc_linear_f32(_p(a32), n_rows, k, _p(offsets), E, _p(c), _p(s), _p(g), w.rows,
                                threads or default_threads(), _p(out)), "linear_f32")
    return out


def weighted_row_sum_f32(dst: np.ndarray, src: np.ndarray, rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """WeightedRowSum in binary32: per element a chain of fmaf over j from a zero
    accumulator, then one add onto dst.  Returns a new float32 array."""
    out = np.array(dst, dtype=np.float32, order="C", copy=True)
    src = np.ascontiguousarray(src, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, K = rows.shape
    d = out.shape[1] if out.ndim == 2 else 0
    _check(lib().orc_weighted_row_sum_f32(_p(out), _p(src), src.shape[0], _p(rows), _p(w), n, K, d),
           "weighted_row_sum_f32")
    return out


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def layer(inp, bf16_act: bool = False, threads: Optional[int] = None, routing=None,
          arith: str = "f64") -> dict:
    """The whole layer: route -> gather -> experts -> shared expert -> combine.

    ``routing`` (ids, weights) may be supplied to run the experts and combine on
    a given routing; by default the oracle routes itself.  ``arith`` is "f64"
    (exact values) or "f32" (binary32, fixed-order fmaf chains; the routing
    weights are then rounded to binary32 before the combine, and ``bf16_act``
    is not available).  Returns every intermediate in a dict."""
    if routing is None:
        ids, w = route_topk(inp.logits, inp.K)
    else:
        ids, w = routing
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
    offsets, row_token, rows = gather_layout(ids, inp.E)
    xg = gather_copy(inp.x, row_token)
    if arith == "f32":
        if bf16_act:
            raise ValueError("the bf16-activation mode is a double-precision mode")
        w32 = w.astype(np.float32)
        yg = expert_ffn_f32(activations_f32(xg, inp.x_dtype), offsets, inp.up, inp.down, inp.f, inp.act,
                            threads)
        if inp.fs > 0:
            shared = expert_ffn_f32(activations_f32(inp.x, inp.x_dtype), np.array([0, inp.n], dtype=np.int32),
                                    inp.shared_up, inp.shared_down, inp.fs, "relu2", threads)
        else:
            shared = np.zeros((inp.n, inp.d), dtype=np.float32)
        out = weighted_row_sum_f32(shared, yg, rows, w32)
        return dict(ids=ids, weights=w, offsets=offsets, row_token=row_token, rows=rows, xg=xg,
                    yg=yg, shared=shared, out=out)
    if arith != "f64":
        raise ValueError(f"unknown arithmetic {arith!r}")
    x64 = activations_f64(inp.x, inp.x_dtype)
    xg64 = activations_f64(xg, inp.x_dtype)
    yg = expert_ffn(xg64, offsets, inp.up, inp.down, inp.f, inp.act, bf16_act, threads)
    if inp.fs > 0:
        shared = expert_ffn(x64, np.array([0, inp.n], dtype=np.int32), inp.shared_up,
                            inp.shared_down, inp.fs, "relu2", bf16_act, threads)
    else:
        shared = np.zeros((inp.n, inp.d), dtype=np.float64)
    out = weighted_row_sum(shared, yg, rows, w)
    return dict(ids=ids, weights=w, offsets=offsets, row_token=row_token, rows=rows, xg=xg,
                yg=yg, shared=shared, out=out)


def layer_sampled(inp, tokens, ids: np.ndarray, w: np.ndarray, bf16_act_of_expert=None,
                  threads: Optional[int] = None) -> np.ndarray:
    """Layer output (double) for a few tokens only, on a given routing (ids, w).

    The same steps as ``layer`` restricted to the sampled tokens: the shared
    expert over their rows, each picked expert over the rows of the sampled
    tokens that picked it (expert by expert, so each expert's weights are
    decoded once), then WeightedRowSum in slot order onto the shared output.
    Every output row is computed alone, so the values equal ``layer``'s rows.
    ``bf16_act_of_expert(e)`` (optional) says which experts run in the
    bf16-activation mode; e = -1 is the shared expert.  Returns
    [len(tokens), d] float64."""
    tokens = [int(t) for t in tokens]
    m = len(tokens)
    x64 = activations_f64(inp.x, inp.x_dtype)[tokens]
    if inp.fs > 0:
        shared = expert_ffn(x64, np.array([0, m], dtype=np.int32), inp.shared_up, inp.shared_down, inp.fs,
                            "relu2", bool(bf16_act_of_expert and bf16_act_of_expert(-1)), threads)
    else:
        shared = np.zeros((m, inp.d), dtype=np.float64)
    sub_ids = np.ascontiguousarray(np.asarray(ids)[tokens], dtype=np.int32)
    src = np.zeros((m * inp.K, inp.d), dtype=np.float64)  # row i*K + j: token i's pick j
    for e in sorted(set(sub_ids.ravel().tolist())):
        picks = [(i, j) for i in range(m) for j in range(inp.K) if sub_ids[i, j] == e]
        mode = bool(bf16_act_of_expert and bf16_act_of_expert(e))
        y = expert_ffn(x64[[i for i, _ in picks]], np.array([0, len(picks)], dtype=np.int32),
                       _one_expert(inp.up, e), _one_expert(inp.down, e), inp.f, inp.act, mode, threads)
        for (i, j), row in zip(picks, y):
            src[i * inp.K + j] = row
    rows = np.arange(m * inp.K, dtype=np.int32).reshape(m, inp.K)
    return weighted_row_sum(shared, src, rows, np.asarray(w, dtype=np.float64)[tokens])


class _Slice:
    def __init__(self, codes, scales, globals_, rows, cols):
        self.codes, self.scales, self.globals_, self.rows, self.cols = codes, scales, globals_, rows, cols


def _one_expert(t, e: int):
    return _Slice(t.codes[e:e + 1], t.scales[e:e + 1], t.globals_[e:e + 1], t.rows, t.cols)


def naive_layer(inp, threads: Optional[int] = None, routing=None) -> np.ndarray:
    """The pre-gather algorithm ([gllm#91] "What the profile showed"): every expert
    runs over every token, weighted zero where the token did not pick it.
    out[t] = shared[t] + sum_{e=0..E-1} W[t,e] * FFN_e(x[t]), e ascending."""
    if routing is None:
        ids, w = route_topk(inp.logits, inp.K)
    else:
        ids, w = routing
    n, E = inp.n, inp.E
    dense = np.zeros((n, E), dtype=np.float64)
    for t in range(n):
        for j in range(inp.K):
            dense[t, ids[t, j]] = w[t, j]
    x64 = activations_f64(inp.x, inp.x_dtype)
    if inp.fs > 0:
        out = expert_ffn(x64, np.array([0, n], dtype=np.int32), inp.shared_up, inp.shared_down,
                         inp.fs, "relu2", False, threads)
    else:
        out = np.zeros((n, inp.d), dtype=np.float64)
    per_expert = []
    for e in range(E):
        per_expert.append(expert_ffn(x64, np.array([0, n], dtype=np.int32), _one_expert(inp.up, e),
                                     _one_expert(inp.down, e), inp.f, inp.act, False, threads))
    acc = np.zeros((n, inp.d), dtype=np.float64)
    for t in range(n):
        for e in range(E):
            acc[t] += dense[t, e] * per_expert[e][t]
    return out + acc
