"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any HIP call (no GPU needed for any of these)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")
LIB = os.path.join(ROOT, "bit_block_scaled_topk_amd", "libmoe_nvfp4.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from bit_block_scaled_topk_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:moe_status|size_t|const char \*)\s*\**\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_layer_calls():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_gather_rows", "nvfp4_expert_ffn", "moe_weighted_row_sum"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in include/moe_nvfp4.h but not exported"


def test_binding_names_match_header():
    from bit_block_scaled_topk_amd import ops
    assert sorted(ops.EXPORTED) == declared_functions()
    for n in ops.EXPORTED:
        if not n.endswith("status_string"):
            assert hasattr(ops, n)


class W(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_", ctypes.c_void_p),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int), ("scales_packed", ctypes.c_void_p),
                ("codes_packed", ctypes.c_void_p)]


FAKE = ctypes.c_void_p(1 << 20)  # an aligned non-null address: never dereferenced on the host


class Desc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int), ("d_model", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("x_dtype", ctypes.c_int), ("act", ctypes.c_int),
                ("gemv_max_rows", ctypes.c_int), ("up", W), ("down", W), ("shared_up", W), ("shared_down", W),
                ("flags", ctypes.c_int)]


def _setup(lib):
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_route_topk.argtypes = [P, I, I, I, P, P, P]
    lib.moe_gather_rows.argtypes = [P, I, I, I, P, I, I, P, P, P, P, P, SZ, P]
    lib.moe_gather_workspace_size.argtypes = [I, I]
    lib.moe_gather_workspace_size.restype = SZ
    lib.nvfp4_expert_ffn_workspace_size.argtypes = [I, I, I, I]
    lib.nvfp4_expert_ffn_workspace_size.restype = SZ
    lib.nvfp4_expert_ffn.argtypes = [P, I, I, I, P, I, ctypes.POINTER(W), ctypes.POINTER(W), I, I, P, SZ, P, P]
    lib.moe_weighted_row_sum.argtypes = [P, P, I, P, P, I, I, I, P, P]
    lib.moe_weighted_row_sum_into.argtypes = [P, P, I, P, P, I, I, I, P, P]
    lib.moe_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.moe_workspace_size.restype = SZ
    lib.moe_error_word_clear.argtypes = [P, P]
    lib.moe_error_word_read.argtypes = [P, P, P]
    lib.moe_layer_workspace_size.argtypes = [ctypes.POINTER(Desc)]
    lib.moe_layer_workspace_size.restype = SZ
    lib.nvfp4_unpack_bf16.argtypes = [P, P, I, I, P, P]
    lib.nvfp4_grouped_linear.argtypes = [P, I, I, I, P, I, ctypes.POINTER(W), I, P, SZ, P, P]
    lib.moe_status_string.argtypes = [I]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.nvfp4_packed_scales_bytes.argtypes = [I, I, I]
    lib.nvfp4_packed_scales_bytes.restype = SZ
    lib.nvfp4_pack_scales.argtypes = [ctypes.POINTER(W), I, P, SZ, P]
    lib.nvfp4_packed_codes_bytes.argtypes = [I, I, I]
    lib.nvfp4_packed_codes_bytes.restype = SZ
    lib.nvfp4_pack_codes.argtypes = [ctypes.POINTER(W), I, P, SZ, P]


def test_status_strings(lib):
    _setup(lib)
    assert lib.moe_status_string(0) == b"ok"
    for s in (1, 2, 3, 4):
        assert lib.moe_status_string(s) not in (b"ok", b"unknown status")
    assert lib.moe_status_string(99) == b"unknown status"


def test_route_argument_errors(lib):
    _setup(lib)
    assert lib.moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == 1       # top_k > E
    assert lib.moe_route_topk(FAKE, 4, 8, 0, FAKE, FAKE, None) == 1       # top_k < 1
    assert lib.moe_route_topk(FAKE, -1, 8, 2, FAKE, FAKE, None) == 1
    assert lib.moe_route_topk(FAKE, 4, 2048, 2, FAKE, FAKE, None) == 2    # too many experts
    assert lib.moe_route_topk(FAKE, 4, 64, 33, FAKE, FAKE, None) == 2     # top_k above 32
    assert lib.moe_route_topk(None, 4, 8, 2, FAKE, FAKE, None) == 1       # null logits
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == 0       # empty: nothing launched


def test_gather_argument_errors(lib):
    _setup(lib)
    ws = lib.moe_gather_workspace_size(16, 8)
    assert ws > 0 and ws % 256 == 0
    assert lib.moe_gather_workspace_size(16, 0) == 0
    assert lib.moe_gather_rows(FAKE, 1, 16, 24, FAKE, 2, 8, ctypes.c_void_p(2 << 20), FAKE, FAKE, FAKE, FAKE,
                               ws, None) == 2   # d_model % 16
    assert lib.moe_gather_rows(FAKE, 1, 16, 64, FAKE, 2, 8, ctypes.c_void_p(2 << 20), FAKE, FAKE, FAKE, FAKE,
                               ws - 1, None) == 4  # workspace too small
    assert lib.moe_gather_rows(FAKE, 1, 16, 64, FAKE, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 1  # xg == x
    assert lib.moe_gather_rows(FAKE, 7, 16, 64, FAKE, 2, 8, ctypes.c_void_p(2 << 20), FAKE, FAKE, FAKE, FAKE,
                               ws, None) == 1   # bad dtype
    assert lib.moe_gather_rows(ctypes.c_void_p((1 << 20) + 8), 1, 16, 64, FAKE, 2, 8, ctypes.c_void_p(2 << 20),
                               FAKE, FAKE, FAKE, FAKE, ws, None) == 1  # misaligned x


def _w(rows, cols, codes=FAKE):
    return W(codes, FAKE, FAKE, rows, cols)


def test_ffn_argument_errors(lib):
    _setup(lib)
    up, dn = _w(128, 64), _w(64, 128)
    ws = lib.nvfp4_expert_ffn_workspace_size(32, 64, 128, 0)
    assert ws >= 3 * 32 * 128 * 2 + 3 * 32 * 64 * 2
    assert lib.nvfp4_expert_ffn_workspace_size(32, 64, 128, 1) < ws
    args = lambda **k: dict(dict(xg=FAKE, dt=0, n=32, mx=16, off=FAKE, E=8, up=up, dn=dn, act=0, gm=32,
                                 ws=FAKE, wsb=ws, out=FAKE), **k)

    def call(a):
        return lib.nvfp4_expert_ffn(a["xg"], a["dt"], a["n"], a["mx"], a["off"], a["E"], ctypes.byref(a["up"]),
                                    ctypes.byref(a["dn"]), a["act"], a["gm"], a["ws"], a["wsb"], a["out"], None)

    assert call(args(gm=33)) == 2                      # gemv_max_rows above 32
    assert call(args(gm=-1)) == 2
    assert call(args(wsb=ws - 1)) == 4                 # workspace too small
    assert call(args(act=5)) == 1                      # unknown activation
    assert call(args(act=1)) == 1                      # swiglu needs up rows = 2 f
    assert call(args(up=_w(128, 48), dn=_w(48, 128))) == 2   # cols not a multiple of 32
    assert call(args(up=_w(128, 64, codes=ctypes.c_void_p((1 << 20) + 4)))) == 1  # misaligned codes
    assert call(args(E=2000)) == 2
    assert call(args(xg=None)) == 1
    assert call(args(n=0, xg=None, off=None, out=None, ws=None)) == 0   # empty: nothing launched
    # the prefill GEMM addresses each activation matrix with 32-bit offsets:
    # 2^24 rows x 64 bf16 = 2 GiB is refused on the host before any launch
    big = 1 << 24
    big_ws = lib.nvfp4_expert_ffn_workspace_size(big, 64, 128, 1)
    assert call(args(n=big, mx=big, dt=1, wsb=big_ws)) == 2


def test_wrs_and_unpack_and_linear_argument_errors(lib):
    _setup(lib)
    assert lib.moe_weighted_row_sum(FAKE, FAKE, 4, FAKE, FAKE, 2, 2, 8, None, None) == 1      # dst aliases src
    assert lib.moe_weighted_row_sum(FAKE, ctypes.c_void_p(2 << 20), 4, FAKE, FAKE, 2, 0, 8, None, None) == 1
    assert lib.moe_weighted_row_sum_into(None, FAKE, 4, FAKE, FAKE, 2, 2, 8, None, None) == 1
    assert lib.moe_weighted_row_sum(None, None, 0, None, None, 0, 2, 8, None, None) == 0    # empty
    # a misaligned error word
    assert lib.moe_weighted_row_sum(FAKE, ctypes.c_void_p(2 << 20), 4, FAKE, FAKE, 2, 2, 8,
                                    ctypes.c_void_p((3 << 20) + 2), None) == 1
    assert lib.nvfp4_unpack_bf16(FAKE, FAKE, 4, 48, FAKE, None) == 2                    # cols % 32
    assert lib.nvfp4_unpack_bf16(FAKE, FAKE, -1, 64, FAKE, None) == 1
    assert lib.nvfp4_unpack_bf16(ctypes.c_void_p((1 << 20) + 1), FAKE, 4, 64, FAKE, None) == 1
    w = _w(64, 64)
    assert lib.nvfp4_grouped_linear(FAKE, 0, 8, 8, FAKE, 2, ctypes.byref(w), 32, None, 0, FAKE, None) == 1
    assert lib.nvfp4_grouped_linear(FAKE, 1, 8, 8, FAKE, 2, ctypes.byref(w), 40, None, 0, FAKE, None) == 2
    # prefill path over a 2^25 x 64 bf16 activation matrix (4 GiB): refused
    assert lib.nvfp4_grouped_linear(FAKE, 1, 1 << 25, 64, FAKE, 2, ctypes.byref(w), 32, None, 0, FAKE, None) == 2


def test_packed_scales_size_and_pack_argument_errors(lib):
    """The repacked scale layout's size is n_experts * ceil(rows/16) *
    ceil(cols/128) * 128 bytes (whole 16-row blocks and 128-wide chunks, 8 scale
    bytes per row and chunk); bad arguments are refused before any launch."""
    _setup(lib)
    assert lib.nvfp4_packed_scales_bytes(128, 1856, 2688) == 128 * 116 * 21 * 128
    assert lib.nvfp4_packed_scales_bytes(128, 2688, 1856) == 128 * 168 * 15 * 128
    assert lib.nvfp4_packed_scales_bytes(3, 17, 32) == 3 * 2 * 1 * 128
    assert lib.nvfp4_packed_scales_bytes(0, 16, 32) == 0
    w = _w(64, 256)
    need = lib.nvfp4_packed_scales_bytes(2, 64, 256)
    assert lib.nvfp4_pack_scales(ctypes.byref(w), 2, FAKE, need - 1, None) == 1   # dst too small
    assert lib.nvfp4_pack_scales(ctypes.byref(w), 0, FAKE, need, None) == 1       # no experts
    assert lib.nvfp4_pack_scales(ctypes.byref(_w(64, 48)), 2, FAKE, need, None) == 1  # cols % 32
    assert lib.nvfp4_pack_scales(ctypes.byref(w), 2, None, need, None) == 1       # null dst
    assert lib.nvfp4_pack_scales(None, 2, FAKE, need, None) == 1                  # null weights


def test_packed_codes_size_and_pack_argument_errors(lib):
    """The repacked code layout's size: n_experts * ceil(rows/16) *
    ceil(cols/128) * 1024 bytes (64 code bytes per row and 128-wide chunk)."""
    _setup(lib)
    assert lib.nvfp4_packed_codes_bytes(128, 1856, 2688) == 128 * 116 * 21 * 1024
    assert lib.nvfp4_packed_codes_bytes(3, 17, 160) == 3 * 2 * 2 * 1024
    assert lib.nvfp4_packed_codes_bytes(1, 0, 64) == 0
    w = _w(64, 256)
    need = lib.nvfp4_packed_codes_bytes(2, 64, 256)
    assert lib.nvfp4_pack_codes(ctypes.byref(w), 2, FAKE, need - 1, None) == 1   # dst too small
    assert lib.nvfp4_pack_codes(ctypes.byref(_w(64, 40)), 2, FAKE, need, None) == 1  # cols % 32
    assert lib.nvfp4_pack_codes(ctypes.byref(w), 2, None, need, None) == 1       # null dst


def test_workspace_size_serves_gather_and_both_expert_calls(lib):
    """moe_workspace_size is the largest of the gather's and the two expert
    calls' sizes (routed rows n*K, shared rows n; fp32 activations, the larger
    dtype); 0 for invalid arguments.  Every workspace of these calls starts
    with the 256 bytes of its error word."""
    _setup(lib)
    for n, K, E, d, f in ((4314, 6, 128, 2688, 3712), (1, 6, 128, 2688, 3712), (2, 8, 256, 2048, 1024),
                          (0, 2, 8, 64, 128)):
        got = lib.moe_workspace_size(n, K, E, d, f, 0)
        parts = (lib.moe_gather_workspace_size(n, E), lib.nvfp4_expert_ffn_workspace_size(n * K, d, f, 0),
                 lib.nvfp4_expert_ffn_workspace_size(n, d, f, 0), lib.nvfp4_expert_ffn_workspace_size(n * K, d, f, 1))
        assert got == max(parts) and got % 256 == 0
        assert lib.moe_workspace_size(n, K, E, d, f, 1) == got
    assert lib.nvfp4_expert_ffn_workspace_size(0, 64, 128, 1) == 256
    assert lib.moe_gather_workspace_size(0, 8) >= 256
    assert lib.moe_workspace_size(4, 9, 8, 64, 128, 0) == 0      # top_k > E
    assert lib.moe_workspace_size(4, 2, 8, 64, 128, 7) == 0      # unknown activation
    assert lib.moe_workspace_size(-1, 2, 8, 64, 128, 0) == 0
    assert lib.moe_workspace_size(4, 2, 2000, 64, 128, 0) == 0   # too many experts


def test_error_word_helpers_reject_bad_pointers(lib):
    _setup(lib)
    v = ctypes.c_int32(0)
    assert lib.moe_error_word_clear(None, None) == 1
    assert lib.moe_error_word_clear(ctypes.c_void_p((1 << 20) + 2), None) == 1
    assert lib.moe_error_word_read(None, ctypes.byref(v), None) == 1
    assert lib.moe_error_word_read(FAKE, None, None) == 1


def test_repacked_weights_are_both_or_neither_aligned_and_addressable(lib):
    """A projection's repacked copies are checked on the host: both present or
    both absent, 16-byte aligned, and one expert's repacked codes under 2 GiB
    (the GEMM's 32-bit offsets)."""
    _setup(lib)
    dn = _w(64, 128)
    ws = lib.nvfp4_expert_ffn_workspace_size(32, 64, 128, 1)

    def call(up):
        return lib.nvfp4_expert_ffn(FAKE, 1, 32, 16, FAKE, 8, ctypes.byref(up), ctypes.byref(dn), 0, 32,
                                    FAKE, ws, FAKE, None)

    ok = W(FAKE, FAKE, FAKE, 128, 64, ctypes.c_void_p(4 << 20), ctypes.c_void_p(5 << 20))
    assert call(W(FAKE, FAKE, FAKE, 128, 64, ctypes.c_void_p(4 << 20), None)) == 1     # scales only
    assert call(W(FAKE, FAKE, FAKE, 128, 64, None, ctypes.c_void_p(5 << 20))) == 1     # codes only
    assert call(W(FAKE, FAKE, FAKE, 128, 64, ctypes.c_void_p((4 << 20) + 8), ctypes.c_void_p(5 << 20))) == 1
    assert call(W(FAKE, FAKE, FAKE, 128, 64, ctypes.c_void_p(4 << 20), ctypes.c_void_p((5 << 20) + 4))) == 1
    # 65536 rows x 32768 cols: 4096 blocks x 256 chunks x 1 KB = 1 GiB -> fine;
    # 131072 rows: 2 GiB of repacked codes per expert -> refused
    assert lib.nvfp4_packed_codes_bytes(1, 131072, 32768) == 1 << 31
    big_up = W(FAKE, FAKE, FAKE, 131072, 32768, ctypes.c_void_p(4 << 20), ctypes.c_void_p(5 << 20))
    big_dn = W(FAKE, FAKE, FAKE, 32768, 131072)
    ws_big = lib.nvfp4_expert_ffn_workspace_size(1, 32768, 131072, 1)
    assert lib.nvfp4_expert_ffn(FAKE, 1, 1, 1, FAKE, 1, ctypes.byref(big_up), ctypes.byref(big_dn), 0, 32,
                                FAKE, ws_big, FAKE, None) == 1
    # the well-formed pair passes the weight checks: with a too-small workspace
    # the call gets as far as the workspace check (and launches nothing)
    assert lib.nvfp4_expert_ffn(FAKE, 1, 32, 16, FAKE, 8, ctypes.byref(ok), ctypes.byref(dn), 0, 32,
                                FAKE, ws - 1, FAKE, None) == 4


def test_layer_description_flags_are_checked(lib):
    """moe_layer_desc.flags takes only MOE_LAYER_SINGLE_LAUNCH and
    MOE_LAYER_FUSED_COMBINE; any other bit makes the description invalid."""
    _setup(lib)
    up, dn = W(FAKE, FAKE, FAKE, 128, 64), W(FAKE, FAKE, FAKE, 64, 128)
    none = W(None, None, None, 0, 0)
    d = Desc(16, 64, 8, 2, 0, 0, 32, up, dn, none, none, 0)
    base = lib.moe_layer_workspace_size(ctypes.byref(d))
    assert base > 0
    d.flags = 1
    assert lib.moe_layer_workspace_size(ctypes.byref(d)) == base
    d.flags = 3
    assert lib.moe_layer_workspace_size(ctypes.byref(d)) == base
    d.flags = 4
    assert lib.moe_layer_workspace_size(ctypes.byref(d)) == 0


def test_noalloc_refuses_descriptions_beyond_its_scratch(lib):
    """moe_layer_forward_noalloc checks the description's workspace size against
    its static array before touching the device: the 4314-token layer (about
    0.6 GB of intermediates) is refused with MOE_UNSUPPORTED, an invalid
    description with MOE_INVALID_ARG."""
    _setup(lib)
    lib.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
    up, dn = W(FAKE, FAKE, FAKE, 1856, 2688), W(FAKE, FAKE, FAKE, 2688, 1856)
    sup, sdn = W(FAKE, FAKE, FAKE, 3712, 2688), W(FAKE, FAKE, FAKE, 2688, 3712)
    d = Desc(4314, 2688, 128, 6, 1, 0, 32, up, dn, sup, sdn, 0)
    assert lib.moe_layer_workspace_size(ctypes.byref(d)) > 64 << 20
    assert lib.moe_layer_forward_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None) == 2
    d.flags = 8
    assert lib.moe_layer_forward_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None) == 1


def test_router_argument_errors(lib):
    """moe_router_topk and its workspace calls check their arguments on the host."""
    _setup(lib)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_router_workspace_size.argtypes = [I, I]
    lib.moe_router_workspace_size.restype = SZ
    lib.moe_router_workspace_init.argtypes = [P, SZ, I, P]
    lib.moe_router_topk.argtypes = [P, I, I, I, P, I, I, P, P, P, P, SZ, P]
    ws = lib.moe_router_workspace_size(4314, 128)
    assert ws >= 4314 * 128 * 4 + 270 * 64 and ws % 256 == 0
    assert lib.moe_router_workspace_size(16, 0) == 0
    assert lib.moe_router_workspace_size(16, 2048) == 0
    assert lib.moe_router_workspace_init(None, ws, 16, None) == 1
    assert lib.moe_router_workspace_init(ctypes.c_void_p((1 << 20) + 16), ws, 16, None) == 1
    assert lib.moe_router_workspace_init(FAKE, 0, 16, None) == 4
    call = lambda **k: lib.moe_router_topk(*[dict(dict(x=FAKE, dt=1, n=16, d=64, w=FAKE, E=8, K=2, ids=FAKE,
                                                       wt=FAKE, lg=None, ws=FAKE, wsb=ws), **k)[a]
                                             for a in ("x", "dt", "n", "d", "w", "E", "K", "ids", "wt", "lg",
                                                       "ws", "wsb")], None)
    assert call(d=48) == 2                       # d_model % 32
    assert call(K=9) == 1                        # top_k > E
    assert call(E=2048) == 2
    assert call(K=33, E=64) == 2
    assert call(dt=3) == 1
    assert call(w=None) == 1
    assert call(x=ctypes.c_void_p((1 << 20) + 8)) == 1     # misaligned x
    assert call(wsb=lib.moe_router_workspace_size(16, 8) - 1) == 4
    assert call(n=0, x=None, w=None, ids=None, wt=None, ws=None) == 0


def test_weights_given_only_as_repacked_copies(lib):
    """Without the canonical codes and scales a projection needs both repacked
    copies and whole 16-row blocks (32 for a SwiGLU up projection); one
    canonical array without the other is refused."""
    _setup(lib)
    pk = dict(scales_packed=ctypes.c_void_p(4 << 20), codes_packed=ctypes.c_void_p(5 << 20))

    def call(up, dn, act=0):
        return lib.nvfp4_expert_ffn(FAKE, 1, 32, 16, FAKE, 8, ctypes.byref(up), ctypes.byref(dn), act, 32,
                                    FAKE, 255, FAKE, None)   # too small a workspace: nothing launches

    up, dn = W(None, None, FAKE, 128, 64, **pk), W(None, None, FAKE, 64, 128, **pk)
    assert call(up, dn) == 4                                       # accepted up to the workspace check
    assert call(W(None, None, FAKE, 120, 64, **pk), W(None, None, FAKE, 64, 120, **pk)) in (1, 2)  # rows % 16
    assert call(W(None, None, FAKE, 128, 64), dn) == 1             # no copy at all
    assert call(W(FAKE, None, FAKE, 128, 64, **pk), dn) == 1       # codes without scales
    sw_up = W(None, None, FAKE, 2 * 48, 64, **pk)                  # 2f rows, f = 48: halves not whole blocks
    sw_dn = W(None, None, FAKE, 64, 48, **pk)
    assert call(sw_up, sw_dn, act=1) in (1, 2)
    assert call(W(None, None, FAKE, 2 * 64, 64, **pk), W(None, None, FAKE, 64, 64, **pk), act=1) == 4
