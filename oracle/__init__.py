"""CPU oracle for the NVFP4 MoE expert-FFN layer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
IEEE double, fixed summation orders; see that file for the passages each
function follows) and composes the layer from its pieces in plain Python.

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
    return max(1, min(64, os.cpu_count() or 1))


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


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def layer(inp, bf16_act: bool = False, threads: Optional[int] = None, routing=None) -> dict:
    """The whole layer: route -> gather -> experts -> shared expert -> combine.

    ``routing`` (ids, weights) may be supplied to run the experts and combine on
    a given routing; by default the oracle routes itself.  Returns every
    intermediate in a dict."""
    if routing is None:
        ids, w = route_topk(inp.logits, inp.K)
    else:
        ids, w = routing
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
    offsets, row_token, rows = gather_layout(ids, inp.E)
    xg = gather_copy(inp.x, row_token)
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
    """Layer output for a few tokens only, on a given routing (ids, w).

    Each sampled token's picked experts run over that token's activation row;
    ``bf16_act_of_expert(e)`` (optional) says which experts are evaluated in the
    bf16-activation mode.  Returns [len(tokens), d] float64."""
    tokens = list(tokens)
    x64 = activations_f64(inp.x, inp.x_dtype)
    out = np.zeros((len(tokens), inp.d), dtype=np.float64)
    for i, t in enumerate(tokens):
        if inp.fs > 0:
            s = expert_ffn(x64[t:t + 1], np.array([0, 1], dtype=np.int32), inp.shared_up,
                           inp.shared_down, inp.fs, "relu2",
                           bool(bf16_act_of_expert and bf16_act_of_expert(-1)), threads)[0]
        else:
            s = np.zeros((inp.d,), dtype=np.float64)
        ys = []
        for j in range(inp.K):
            e = int(ids[t, j])
            sub_up = _one_expert(inp.up, e)
            sub_dn = _one_expert(inp.down, e)
            mode = bool(bf16_act_of_expert and bf16_act_of_expert(e))
            ys.append(expert_ffn(x64[t:t + 1], np.array([0, 1], dtype=np.int32), sub_up, sub_dn,
                                 inp.f, inp.act, mode, threads)[0])
        src = np.stack(ys)
        out[i] = weighted_row_sum(s[None, :], src, np.arange(inp.K, dtype=np.int32)[None, :],
                                  np.asarray(w[t:t + 1], dtype=np.float64))[0]
    return out


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
