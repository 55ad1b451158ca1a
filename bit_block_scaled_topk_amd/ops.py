"""Python binding of libmoe_nvfp4.so (argument marshalling only).

Each function has the name of the C entry point it calls and passes torch
tensors' device pointers and the current HIP stream.  Every step of the layer
runs in the library's HIP kernels; there is no fallback: importing this module
raises if the library is not built, and every call raises on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_nvfp4.so")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_HIP_ERROR, MOE_WORKSPACE_TOO_SMALL = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16 = 0, 1
MOE_RELU2, MOE_SWIGLU = 0, 1
MOE_DEVERR_EXPERT_ID, MOE_DEVERR_ROW = 1, 2
MAX_GEMV_ROWS = 32

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run bit_block_scaled_topk_amd/build.py "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.moe_status_string(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class NVFP4Weights(ctypes.Structure):
    """moe_nvfp4_weights: device pointers of one projection for E experts."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_", ctypes.c_void_p),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int), ("scales_packed", ctypes.c_void_p),
                ("codes_packed", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_lib.moe_status_string.argtypes = [_I]
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_route_topk.argtypes = [_P, _I, _I, _I, _P, _P, _P]
_lib.moe_route_topk.restype = _I
_lib.moe_router_workspace_size.argtypes = [_I, _I]
_lib.moe_router_workspace_size.restype = _SZ
_lib.moe_router_workspace_init.argtypes = [_P, _SZ, _I, _P]
_lib.moe_router_workspace_init.restype = _I
_lib.moe_router_topk.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]
_lib.moe_router_topk.restype = _I
_lib.moe_gather_workspace_size.argtypes = [_I, _I]
_lib.moe_gather_workspace_size.restype = _SZ
_lib.moe_gather_rows.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]
_lib.moe_gather_rows.restype = _I
_lib.nvfp4_expert_ffn_workspace_size.argtypes = [_I, _I, _I, _I]
_lib.nvfp4_expert_ffn_workspace_size.restype = _SZ
_lib.nvfp4_grouped_linear_workspace_size.argtypes = [_I, _I, _I]
_lib.nvfp4_grouped_linear_workspace_size.restype = _SZ
_lib.nvfp4_expert_ffn.argtypes = [_P, _I, _I, _I, _P, _I, ctypes.POINTER(NVFP4Weights),
                                  ctypes.POINTER(NVFP4Weights), _I, _I, _P, _SZ, _P, _P]
_lib.nvfp4_expert_ffn.restype = _I
_lib.moe_weighted_row_sum.argtypes = [_P, _P, _I, _P, _P, _I, _I, _I, _P, _P]
_lib.moe_weighted_row_sum.restype = _I
_lib.moe_weighted_row_sum_into.argtypes = [_P, _P, _I, _P, _P, _I, _I, _I, _P, _P]
_lib.moe_weighted_row_sum_into.restype = _I
_lib.moe_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
_lib.moe_workspace_size.restype = _SZ
_lib.moe_error_word_clear.argtypes = [_P, _P]
_lib.moe_error_word_clear.restype = _I
_lib.moe_error_word_read.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), _P]
_lib.moe_error_word_read.restype = _I
_lib.nvfp4_unpack_bf16.argtypes = [_P, _P, _I, _I, _P, _P]
_lib.nvfp4_unpack_bf16.restype = _I
_lib.nvfp4_grouped_linear.argtypes = [_P, _I, _I, _I, _P, _I, ctypes.POINTER(NVFP4Weights), _I, _P, _SZ,
                                      _P, _P]
_lib.nvfp4_grouped_linear.restype = _I
_lib.nvfp4_packed_scales_bytes.argtypes = [_I, _I, _I]
_lib.nvfp4_packed_scales_bytes.restype = _SZ
_lib.nvfp4_pack_scales.argtypes = [ctypes.POINTER(NVFP4Weights), _I, _P, _SZ, _P]
_lib.nvfp4_pack_scales.restype = _I
_lib.nvfp4_packed_codes_bytes.argtypes = [_I, _I, _I]
_lib.nvfp4_packed_codes_bytes.restype = _SZ
_lib.nvfp4_pack_codes.argtypes = [ctypes.POINTER(NVFP4Weights), _I, _P, _SZ, _P]
_lib.nvfp4_pack_codes.restype = _I

class LayerDesc(ctypes.Structure):
    """moe_layer_desc."""
    _fields_ = [("n_tokens", ctypes.c_int), ("d_model", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("x_dtype", ctypes.c_int), ("act", ctypes.c_int),
                ("gemv_max_rows", ctypes.c_int), ("up", NVFP4Weights), ("down", NVFP4Weights),
                ("shared_up", NVFP4Weights), ("shared_down", NVFP4Weights), ("flags", ctypes.c_int)]


MOE_LAYER_SINGLE_LAUNCH = 1
MOE_LAYER_FUSED_COMBINE = 2
PROFILE_EVENTS = 8  # events moe_layer_forward_profiled records per call


class LayerViews(ctypes.Structure):
    """moe_layer_views."""
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("row_token", ctypes.c_void_p), ("rows", ctypes.c_void_p),
                ("yg", ctypes.c_void_p), ("wait_error", ctypes.c_void_p),
                ("decode_launch", ctypes.c_void_p)]


_lib.moe_layer_workspace_size.argtypes = [ctypes.POINTER(LayerDesc)]
_lib.moe_layer_workspace_size.restype = _SZ
_lib.moe_layer_workspace_init.argtypes = [ctypes.POINTER(LayerDesc), _P, _SZ, _P]
_lib.moe_layer_workspace_init.restype = _I
_lib.moe_layer_get_views.argtypes = [ctypes.POINTER(LayerDesc), _P, ctypes.POINTER(LayerViews)]
_lib.moe_layer_get_views.restype = _I
_lib.moe_layer_forward.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _SZ, _P]
_lib.moe_layer_forward.restype = _I
_lib.moe_layer_forward_profiled.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _SZ, _P, _P]
_lib.moe_layer_forward_profiled.restype = _I
_lib.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P]
_lib.moe_layer_forward_noalloc.restype = _I
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("moe_route_topk", "moe_router_workspace_size", "moe_router_workspace_init", "moe_router_topk",
            "moe_gather_workspace_size", "moe_gather_rows",
            "nvfp4_expert_ffn_workspace_size", "nvfp4_grouped_linear_workspace_size",
            "nvfp4_expert_ffn", "moe_weighted_row_sum", "moe_weighted_row_sum_into", "moe_workspace_size",
            "moe_error_word_clear", "moe_error_word_read", "nvfp4_unpack_bf16",
            "nvfp4_grouped_linear", "nvfp4_packed_scales_bytes", "nvfp4_pack_scales",
            "nvfp4_packed_codes_bytes", "nvfp4_pack_codes", "moe_status_string",
            "moe_layer_workspace_size",
            "moe_layer_workspace_init", "moe_layer_get_views",
            "moe_layer_forward", "moe_layer_forward_profiled", "moe_layer_forward_noalloc")


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        return MOE_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


@dataclass
class DeviceNVFP4:
    """One NVFP4 projection for E experts resident on the device: the canonical
    codes and scales, the repacked copies, or both (see drop_canonical)."""
    codes: Optional[torch.Tensor]    # uint8 [E, rows, cols/2]
    scales: Optional[torch.Tensor]   # uint8 [E, rows, cols/16]
    globals_: torch.Tensor  # float32 [E]
    rows: int
    cols: int
    scales_packed: Optional[torch.Tensor] = None  # uint8, nvfp4_pack_scales order (optional)
    codes_packed: Optional[torch.Tensor] = None   # uint8, nvfp4_pack_codes order (optional)

    @classmethod
    def from_host(cls, t, device="cuda") -> "DeviceNVFP4":
        return cls(torch.from_numpy(t.codes).to(device), torch.from_numpy(t.scales).to(device),
                   torch.from_numpy(t.globals_).to(device), int(t.rows), int(t.cols))

    def struct(self) -> NVFP4Weights:
        return NVFP4Weights(None if self.codes is None else self.codes.data_ptr(),
                            None if self.scales is None else self.scales.data_ptr(), self.globals_.data_ptr(),
                            self.rows, self.cols,
                            None if self.scales_packed is None else self.scales_packed.data_ptr(),
                            None if self.codes_packed is None else self.codes_packed.data_ptr())

    def pack(self, stream=None) -> "DeviceNVFP4":
        """Repack the scales and codes once (nvfp4_pack_scales, nvfp4_pack_codes);
        the prefill GEMM then reads them.  Returns self."""
        self.scales_packed = nvfp4_pack_scales(self, stream=stream)
        self.codes_packed = nvfp4_pack_codes(self, stream=stream)
        return self

    def drop_canonical(self) -> "DeviceNVFP4":
        """Free the canonical codes and scales once the repacked copies exist:
        one copy of the weights stays on the device.  Returns self."""
        if self.codes_packed is None or self.scales_packed is None:
            raise ValueError("pack() first: the repacked copies are the only copy left")
        self.codes = None
        self.scales = None
        return self

    def clone(self) -> "DeviceNVFP4":
        """A second device copy of whatever this projection holds."""
        c = lambda t: None if t is None else t.clone()
        return DeviceNVFP4(c(self.codes), c(self.scales), self.globals_.clone(), self.rows, self.cols,
                           c(self.scales_packed), c(self.codes_packed))

    @property
    def n_experts(self) -> int:
        return int(self.globals_.shape[0])


# ----------------------------------------------------------------------------
# the C entry points, one to one
# ----------------------------------------------------------------------------

def moe_route_topk(logits: torch.Tensor, top_k: int, ids: Optional[torch.Tensor] = None,
                   weights: Optional[torch.Tensor] = None, stream=None):
    n, E = logits.shape
    if ids is None:
        ids = torch.empty((n, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((n, top_k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", _lib.moe_route_topk(_ptr(logits), n, E, top_k, _ptr(ids), _ptr(weights),
                                                 _stream(stream)))
    return ids, weights


def moe_router_workspace_size(n_tokens: int, n_experts: int) -> int:
    return int(_lib.moe_router_workspace_size(n_tokens, n_experts))


def moe_router_workspace_init(workspace: torch.Tensor, n_tokens: int, stream=None) -> None:
    _check("moe_router_workspace_init", _lib.moe_router_workspace_init(
        _ptr(workspace), workspace.numel() * workspace.element_size(), n_tokens, _stream(stream)))


def moe_router_topk(x: torch.Tensor, router_w: torch.Tensor, top_k: int, workspace: torch.Tensor,
                    ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None,
                    logits: Optional[torch.Tensor] = None, stream=None):
    """x [n, d] (float32, or bf16 bits as int16), router_w [E, d] bf16 bits
    (int16).  Returns (ids, weights, logits or None)."""
    n, d = x.shape
    E = router_w.shape[0]
    if ids is None:
        ids = torch.empty((n, top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((n, top_k), dtype=torch.float32, device=x.device)
    _check("moe_router_topk", _lib.moe_router_topk(
        _ptr(x), _dtype_code(x), n, d, _ptr(router_w), E, top_k, _ptr(ids), _ptr(weights), _ptr(logits),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return ids, weights, logits


def moe_gather_workspace_size(n_tokens: int, n_experts: int) -> int:
    return int(_lib.moe_gather_workspace_size(n_tokens, n_experts))


def moe_gather_rows(x: torch.Tensor, topk_ids: torch.Tensor, n_experts: int, workspace: torch.Tensor,
                    xg=None, offsets=None, row_token=None, rows=None, stream=None):
    n, d = x.shape
    K = topk_ids.shape[1]
    dev = x.device
    if xg is None:
        xg = torch.empty((n * K, d), dtype=x.dtype, device=dev)
    if offsets is None:
        offsets = torch.empty((n_experts + 1,), dtype=torch.int32, device=dev)
    if row_token is None:
        row_token = torch.empty((n * K,), dtype=torch.int32, device=dev)
    if rows is None:
        rows = torch.empty((n, K), dtype=torch.int32, device=dev)
    _check("moe_gather_rows", _lib.moe_gather_rows(
        _ptr(x), _dtype_code(x), n, d, _ptr(topk_ids), K, n_experts, _ptr(xg), _ptr(offsets),
        _ptr(row_token), _ptr(rows), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return xg, offsets, row_token, rows


def nvfp4_expert_ffn_workspace_size(n_rows: int, d_model: int, d_ff: int, act_dtype: int) -> int:
    return int(_lib.nvfp4_expert_ffn_workspace_size(n_rows, d_model, d_ff, act_dtype))


def nvfp4_grouped_linear_workspace_size(n_rows: int, k: int, a_dtype: int) -> int:
    return int(_lib.nvfp4_grouped_linear_workspace_size(n_rows, k, a_dtype))


def nvfp4_expert_ffn(xg: torch.Tensor, offsets: torch.Tensor, up: DeviceNVFP4, down: DeviceNVFP4,
                     act: int, max_rows_per_expert: int, workspace: torch.Tensor, out: torch.Tensor,
                     gemv_max_rows: int = MAX_GEMV_ROWS, stream=None) -> torch.Tensor:
    n_rows = xg.shape[0]
    u, dn = up.struct(), down.struct()
    _check("nvfp4_expert_ffn", _lib.nvfp4_expert_ffn(
        _ptr(xg), _dtype_code(xg), n_rows, max_rows_per_expert, _ptr(offsets), up.n_experts,
        ctypes.byref(u), ctypes.byref(dn), act, gemv_max_rows, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))
    return out


def moe_weighted_row_sum(dst: torch.Tensor, src: torch.Tensor, rows: torch.Tensor, weights: torch.Tensor,
                         error_word: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n, K = rows.shape
    _check("moe_weighted_row_sum", _lib.moe_weighted_row_sum(
        _ptr(dst), _ptr(src), src.shape[0], _ptr(rows), _ptr(weights), n, K, dst.shape[1], _ptr(error_word),
        _stream(stream)))
    return dst


def moe_weighted_row_sum_into(dst: torch.Tensor, src: torch.Tensor, rows: torch.Tensor, weights: torch.Tensor,
                              error_word: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n, K = rows.shape
    _check("moe_weighted_row_sum_into", _lib.moe_weighted_row_sum_into(
        _ptr(dst), _ptr(src), src.shape[0], _ptr(rows), _ptr(weights), n, K, dst.shape[1], _ptr(error_word),
        _stream(stream)))
    return dst


def moe_workspace_size(n_tokens: int, top_k: int, n_experts: int, d_model: int, d_ff_max: int, act: int) -> int:
    return int(_lib.moe_workspace_size(n_tokens, top_k, n_experts, d_model, d_ff_max, act))


def moe_error_word_clear(word: torch.Tensor, stream=None) -> None:
    """``word``: an int32 device tensor whose first element is the error word
    (e.g. a workspace viewed as int32)."""
    _check("moe_error_word_clear", _lib.moe_error_word_clear(_ptr(word), _stream(stream)))


def moe_error_word_read(word: torch.Tensor, stream=None) -> int:
    """Test and debugging helper: waits for the stream, returns the word."""
    v = ctypes.c_int32(0)
    _check("moe_error_word_read", _lib.moe_error_word_read(_ptr(word), ctypes.byref(v), _stream(stream)))
    return int(v.value)


def nvfp4_unpack_bf16(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.int16, device=codes.device)
    _check("nvfp4_unpack_bf16", _lib.nvfp4_unpack_bf16(_ptr(codes), _ptr(scales), rows, cols, _ptr(out),
                                                       _stream(stream)))
    return out


def nvfp4_packed_scales_bytes(n_experts: int, rows: int, cols: int) -> int:
    return int(_lib.nvfp4_packed_scales_bytes(n_experts, rows, cols))


def nvfp4_pack_scales(w: DeviceNVFP4, dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    nbytes = nvfp4_packed_scales_bytes(w.n_experts, w.rows, w.cols)
    if dst is None:
        dst = torch.empty(nbytes, dtype=torch.uint8, device=w.scales.device)
    s = w.struct()
    _check("nvfp4_pack_scales", _lib.nvfp4_pack_scales(ctypes.byref(s), w.n_experts, _ptr(dst), dst.numel(),
                                                       _stream(stream)))
    return dst


def nvfp4_packed_codes_bytes(n_experts: int, rows: int, cols: int) -> int:
    return int(_lib.nvfp4_packed_codes_bytes(n_experts, rows, cols))


def nvfp4_pack_codes(w: DeviceNVFP4, dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    nbytes = nvfp4_packed_codes_bytes(w.n_experts, w.rows, w.cols)
    if dst is None:
        dst = torch.empty(nbytes, dtype=torch.uint8, device=w.codes.device)
    s = w.struct()
    _check("nvfp4_pack_codes", _lib.nvfp4_pack_codes(ctypes.byref(s), w.n_experts, _ptr(dst), dst.numel(),
                                                     _stream(stream)))
    return dst


def nvfp4_grouped_linear(a: torch.Tensor, offsets: torch.Tensor, w: DeviceNVFP4, max_rows_per_expert: int,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         gemv_max_rows: int = MAX_GEMV_ROWS, stream=None) -> torch.Tensor:
    n_rows = a.shape[0]
    if out is None:
        out = torch.empty((n_rows, w.rows), dtype=torch.float32, device=a.device)
    need = nvfp4_grouped_linear_workspace_size(n_rows, w.cols, _dtype_code(a))
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws = w.struct()
    _check("nvfp4_grouped_linear", _lib.nvfp4_grouped_linear(
        _ptr(a), _dtype_code(a), n_rows, max_rows_per_expert, _ptr(offsets), w.n_experts, ctypes.byref(ws),
        gemv_max_rows, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))
    return out


def moe_layer_workspace_size(desc: LayerDesc) -> int:
    return int(_lib.moe_layer_workspace_size(ctypes.byref(desc)))


def moe_layer_workspace_init(desc: LayerDesc, workspace: torch.Tensor, stream=None) -> None:
    _check("moe_layer_workspace_init", _lib.moe_layer_workspace_init(
        ctypes.byref(desc), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_layer_get_views(desc: LayerDesc, workspace: torch.Tensor) -> LayerViews:
    v = LayerViews()
    _check("moe_layer_get_views", _lib.moe_layer_get_views(ctypes.byref(desc), _ptr(workspace), ctypes.byref(v)))
    return v


def moe_layer_forward(desc: LayerDesc, x: torch.Tensor, logits: torch.Tensor, out: torch.Tensor,
                      workspace: torch.Tensor, stream=None) -> torch.Tensor:
    _check("moe_layer_forward", _lib.moe_layer_forward(
        ctypes.byref(desc), _ptr(x), _ptr(logits), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def moe_layer_forward_noalloc(desc: LayerDesc, x: torch.Tensor, logits: torch.Tensor, out: torch.Tensor,
                              stream=None) -> torch.Tensor:
    _check("moe_layer_forward_noalloc", _lib.moe_layer_forward_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(logits), _ptr(out), _stream(stream)))
    return out


def moe_layer_forward_profiled(desc: LayerDesc, x: torch.Tensor, logits: torch.Tensor, out: torch.Tensor,
                               workspace: torch.Tensor, events, stream=None) -> torch.Tensor:
    """``events``: PROFILE_EVENTS hipEvent_t handles (see HipEvents.slice)."""
    _check("moe_layer_forward_profiled", _lib.moe_layer_forward_profiled(
        ctypes.byref(desc), _ptr(x), _ptr(logits), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), events, _stream(stream)))
    return out


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (for the
    profiled layer entry point); elapsed times in milliseconds."""

    def __init__(self, count: int):
        self._hip = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * count)()
        for i in range(count):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = h

    def slice(self, start: int):
        return ctypes.cast(ctypes.byref(self.handles, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.c_void_p)

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = (ctypes.c_void_p * 0)()


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


# ----------------------------------------------------------------------------
# the layer: the four calls composed on one stream
# ----------------------------------------------------------------------------

class MoELayer:
    """Device-resident weights and preallocated buffers of one NVFP4 MoE layer.

    ``forward(x, logits)`` runs route -> gather -> shared expert -> routed
    experts -> WeightedRowSum on the current stream and returns the [n, d]
    float32 output (gllm PR #91, "What changes").  Buffers are allocated once
    at construction for n_tokens tokens, so a forward pass allocates nothing.
    ``single_launch`` sets MOE_LAYER_SINGLE_LAUNCH in the layer description:
    only for callers that run nothing else on the device during a step.
    ``fused_combine`` sets MOE_LAYER_FUSED_COMBINE (WeightedRowSum inside the
    prefill down projection).  The weights are repacked once when the layer is
    built; every kernel of the layer reads the repacked copies, so the
    canonical copy is freed unless ``keep_canonical``: one copy of the weights
    stays on the device.
    """

    def __init__(self, inp, device="cuda", gemv_max_rows: int = MAX_GEMV_ROWS, n_tokens: Optional[int] = None,
                 single_launch: bool = False, fused_combine: bool = False, keep_canonical: bool = False):
        self.n = int(n_tokens if n_tokens is not None else inp.n)
        self.d, self.E, self.K, self.f, self.fs = inp.d, inp.E, inp.K, inp.f, inp.fs
        self.act = MOE_SWIGLU if inp.act == "swiglu" else MOE_RELU2
        self.x_dtype = MOE_F32 if inp.x_dtype == "f32" else MOE_BF16
        self.gemv_max_rows = gemv_max_rows
        self.flags = (MOE_LAYER_SINGLE_LAUNCH if single_launch else 0) | \
            (MOE_LAYER_FUSED_COMBINE if fused_combine else 0)
        self.up = DeviceNVFP4.from_host(inp.up, device)
        self.down = DeviceNVFP4.from_host(inp.down, device)
        self.shared_up = DeviceNVFP4.from_host(inp.shared_up, device) if inp.fs > 0 else None
        self.shared_down = DeviceNVFP4.from_host(inp.shared_down, device) if inp.fs > 0 else None
        for w in self.weights():
            if w is not None:
                w.pack()  # the one-time repack every kernel of the layer reads
                if not keep_canonical:
                    w.drop_canonical()
        self.device = device
        self.layer_ws = None
        self._alloc(self.n)

    def _alloc(self, n):
        dev, K, d = self.device, self.K, self.d
        xdt = torch.float32 if self.x_dtype == MOE_F32 else torch.int16
        R = n * K
        self.ids = torch.empty((n, K), dtype=torch.int32, device=dev)
        self.w = torch.empty((n, K), dtype=torch.float32, device=dev)
        self.xg = torch.empty((R, d), dtype=xdt, device=dev)
        self.offsets = torch.empty((self.E + 1,), dtype=torch.int32, device=dev)
        self.shared_offsets = torch.tensor([0, n], dtype=torch.int32, device=dev)
        self.row_token = torch.empty((R,), dtype=torch.int32, device=dev)
        self.rows = torch.empty((n, K), dtype=torch.int32, device=dev)
        self.yg = torch.empty((R, d), dtype=torch.float32, device=dev)
        self.out = torch.empty((n, d), dtype=torch.float32, device=dev)
        ws = max(moe_gather_workspace_size(n, self.E),
                 nvfp4_expert_ffn_workspace_size(R, d, self.f, self.x_dtype),
                 nvfp4_expert_ffn_workspace_size(n, d, max(self.fs, 32), self.x_dtype))
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
        moe_error_word_clear(self.workspace.view(torch.int32))  # the gather's error word
        self.layer_ws = torch.empty((moe_layer_workspace_size(self.desc(None, n)),), dtype=torch.uint8, device=dev)
        moe_layer_workspace_init(self.desc(None, n), self.layer_ws)

    def weights(self):
        return (self.up, self.down, self.shared_up, self.shared_down)

    def desc(self, weights=None, n_tokens: Optional[int] = None) -> LayerDesc:
        up, down, sup, sdn = weights if weights is not None else self.weights()
        empty = NVFP4Weights(None, None, None, 0, 0, None, None)
        return LayerDesc(self.n if n_tokens is None else n_tokens, self.d, self.E, self.K, self.x_dtype, self.act,
                         self.gemv_max_rows, up.struct(), down.struct(),
                         sup.struct() if sup is not None else empty, sdn.struct() if sdn is not None else empty,
                         self.flags)

    def forward_fused(self, x: torch.Tensor, logits: torch.Tensor, stream=None, weights=None,
                      check: bool = True) -> torch.Tensor:
        """The whole layer through moe_layer_forward (the fewest launches);
        intermediates stay in the layer workspace (see views()).  With
        ``check`` (and outside graph capture) the call waits for the stream and
        raises if a bounded wait of the single-launch step expired, i.e. the
        output is invalid; pass check=False in timed or captured loops and call
        check_wait_error() afterwards."""
        d = self.desc(weights, x.shape[0])
        need = moe_layer_workspace_size(d)
        if self.layer_ws is None or self.layer_ws.numel() < need:
            raise MoeError("moe_layer_forward", MOE_WORKSPACE_TOO_SMALL)
        out = moe_layer_forward(d, x, logits, self.out, self.layer_ws, stream=stream)
        if check and (self.flags & MOE_LAYER_SINGLE_LAUNCH) and not torch.cuda.is_current_stream_capturing():
            self.check_wait_error(stream)
        return out

    def check_wait_error(self, stream=None) -> None:
        """Raise if the single-launch step's wait_error word is set (waits for
        the stream)."""
        v = moe_layer_get_views(self.desc(None, self.n), self.layer_ws)
        word = self.layer_ws[v.wait_error - self.layer_ws.data_ptr():][:4].view(torch.int32)
        if moe_error_word_read(word, stream) != 0:
            raise RuntimeError("moe_layer_forward: a bounded wait of the single-launch decode step expired; "
                               "the output of that call is invalid (was another kernel running on the device?)")

    def gather_error(self, stream=None) -> int:
        """The gather workspace's error word (MOE_DEVERR_* bits; waits for the stream)."""
        return moe_error_word_read(self.workspace.view(torch.int32), stream)

    def forward_profiled(self, x: torch.Tensor, logits: torch.Tensor, events, stream=None,
                         weights=None) -> torch.Tensor:
        d = self.desc(weights, x.shape[0])
        return moe_layer_forward_profiled(d, x, logits, self.out, self.layer_ws, events, stream=stream)

    def views(self, n_tokens: Optional[int] = None) -> dict:
        """The fused path's intermediates as tensors viewing the workspace."""
        n = self.n if n_tokens is None else n_tokens
        v = moe_layer_get_views(self.desc(None, n), self.layer_ws)
        base = self.layer_ws.data_ptr()
        R = n * self.K

        def view(addr, numel, dtype):
            off = addr - base
            esz = torch.tensor([], dtype=dtype).element_size()
            return self.layer_ws[off:off + numel * esz].view(dtype)

        xdt = torch.float32 if self.x_dtype == MOE_F32 else torch.int16
        return dict(ids=view(v.topk_ids, R, torch.int32).view(n, self.K),
                    w=view(v.topk_weights, R, torch.float32).view(n, self.K),
                    offsets=view(v.expert_offsets, self.E + 1, torch.int32),
                    row_token=view(v.row_token, R, torch.int32),
                    rows=view(v.rows, R, torch.int32).view(n, self.K),
                    yg=view(v.yg, R * self.d, torch.float32).view(R, self.d),
                    wait_error=view(v.wait_error, 1, torch.int32),
                    decode_launch=view(v.decode_launch, 1, torch.int32))

    def forward(self, x: torch.Tensor, logits: torch.Tensor, stream=None, weights=None,
                timing: Optional[dict] = None) -> torch.Tensor:
        """x [n, d] (float32 or bf16 bits as int16), logits [n, E] float32.
        ``weights`` optionally overrides the projections: (up, down, shared_up,
        shared_down) DeviceNVFP4 tuples, e.g. another layer's copy.  ``timing``
        (a dict of step name -> list) collects (start, end) HIP events recorded
        on the stream around each call."""
        up, down, sup, sdn = weights if weights is not None else self.weights()
        n = x.shape[0]

        def mark(name, fn):
            if timing is None:
                return fn()
            s = torch.cuda.current_stream() if stream is None else stream
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            r = fn()
            b.record(s)
            timing.setdefault(name, []).append((a, b))
            return r

        mark("route", lambda: moe_route_topk(logits, self.K, self.ids, self.w, stream=stream))
        mark("gather", lambda: moe_gather_rows(x, self.ids, self.E, self.workspace, self.xg, self.offsets,
                                               self.row_token, self.rows, stream=stream))
        if self.fs > 0:
            mark("shared_ffn", lambda: nvfp4_expert_ffn(x, self.shared_offsets, sup, sdn, MOE_RELU2, n,
                                                        self.workspace, self.out, self.gemv_max_rows,
                                                        stream=stream))
        mark("routed_ffn", lambda: nvfp4_expert_ffn(self.xg, self.offsets, up, down, self.act, n,
                                                    self.workspace, self.yg, self.gemv_max_rows, stream=stream))
        if self.fs > 0:
            mark("combine", lambda: moe_weighted_row_sum(self.out, self.yg, self.rows, self.w, stream=stream))
        else:
            mark("combine", lambda: moe_weighted_row_sum_into(self.out, self.yg, self.rows, self.w,
                                                              stream=stream))
        return self.out
