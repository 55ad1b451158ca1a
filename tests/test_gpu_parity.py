"""Parity of every HIP entry point with the CPU oracle, on seeded inputs.

Bars: bit-exact for routing ids, gather layouts and the unpacked weights;
normwise relative max-error max|gpu - ref| / max|ref| <= 1e-5 for the decode
(fp32-accurate) path and <= 2e-2 for the prefill (bf16-activation MFMA) path;
WeightedRowSum within its rigorous fp32 rounding bound.  All inputs come from
bit_block_scaled_topk_amd.synth; every expected value comes from oracle/.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_block_scaled_topk_amd import synth
from conftest import cached_layer

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_DECODE = 1e-5
TOL_PREFILL = 2e-2


@pytest.fixture(scope="module")
def ops():
    from bit_block_scaled_topk_amd import ops as _ops
    return _ops


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def normwise(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def bf16_bits_to_f64(b):
    return oracle.bf16_bits_to_f64(np.asarray(b).view(np.uint16))


def ulps_f32(got, ref):
    """|got - ref| in units of the binary32 spacing at ref (ref exact, float64)."""
    ref = np.asarray(ref, dtype=np.float64)
    spacing = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return np.abs(np.asarray(got, dtype=np.float64) - ref) / spacing


def route_weight_ulps_bound(K):
    """Routing weights w_j = e_j / S on the GPU: each e_j = expf(l_j - l_0) is
    within about 2 ulp of exp of the rounded difference (one rounding of the
    difference, the device expf's error), S sums K of them in binary32 (K - 1
    roundings) and the divide rounds once: a relative error below
    (K + 4) * 2^-24, i.e. at most K + 4 units of the binary32 spacing."""
    return K + 4


def check_route_weights(got, ref, K):
    u = ulps_f32(got, ref)
    assert np.max(u) <= route_weight_ulps_bound(K), f"routing weights off by {np.max(u):.1f} ulp"


# ----------------------------------------------------------------------------
# unpack
# ----------------------------------------------------------------------------

def test_unpack_every_code_with_every_scale(ops):
    """Every (e2m1 code, e4m3 scale byte) pair, NaN scales included, unpacks
    bit-exactly to the oracle's value (which PIN tests tie to torch's casts)."""
    rows, cols = 256, 32
    codes = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8), (rows, 2))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)
    out = ops.nvfp4_unpack_bf16(dev(codes), dev(scales), rows, cols)
    got = bf16_bits_to_f64(host(out))
    ref = oracle.dequant(codes, scales, 1.0, with_global=False)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 32
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_unpack_random_multi_expert(ops):
    t = synth.random_bytes_nvfp4(101, 3, 96, 224)
    rows = 3 * 96
    out = ops.nvfp4_unpack_bf16(dev(t.codes.reshape(rows, -1)), dev(t.scales.reshape(rows, -1)), rows, 224)
    got = bf16_bits_to_f64(host(out))
    ref = oracle.dequant(t.codes.reshape(rows, -1), t.scales.reshape(rows, -1), 1.0, with_global=False)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def _route_case(ops, logits, K):
    ids, w = ops.moe_route_topk(dev(logits), K)
    rids, rw = oracle.route_topk(logits, K)
    assert np.array_equal(host(ids), rids)
    check_route_weights(host(w), rw, K)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_route_workloads(ops, name):
    cfg = synth.WORKLOADS[name]
    _route_case(ops, synth.draw_logits(name), cfg["K"])


def test_route_edge_cases(ops):
    rng = np.random.default_rng(3)
    _route_case(ops, np.zeros((5, 10), dtype=np.float32), 4)                        # all tied
    _route_case(ops, rng.standard_normal((7, 6)).astype(np.float32), 6)             # K = E
    _route_case(ops, rng.standard_normal((3, 1)).astype(np.float32), 1)             # E = 1
    lg = rng.standard_normal((9, 1024)).astype(np.float32)
    _route_case(ops, lg, 32)                                                        # max E, max K
    lg = np.round(rng.standard_normal((33, 200)) * 2).astype(np.float32)            # many ties
    _route_case(ops, lg, 8)
    lg = rng.standard_normal((4, 77)).astype(np.float32)
    lg[:, ::3] = -np.inf                                                            # masked experts
    _route_case(ops, lg, 5)
    lg = np.zeros((6, 40), dtype=np.float32)                                       # +0 and -0 tie
    lg[:, 1::2] = np.float32(-0.0)
    lg[1, 7] = 0.5
    lg[2, 30] = -1.0
    lg[3, ::5] = np.float32(-0.0)
    _route_case(ops, lg, 7)
    ids, w = ops.moe_route_topk(torch.empty((0, 8), device=DEV), 2)                 # no tokens
    assert ids.shape == (0, 2)


# ----------------------------------------------------------------------------
# gather
# ----------------------------------------------------------------------------

def gather_ws(ops, n, E):
    ws = torch.empty((ops.moe_gather_workspace_size(n, E),), dtype=torch.uint8, device=DEV)
    ops.moe_error_word_clear(ws.view(torch.int32))
    return ws


def _gather_case(ops, x, ids, E):
    n, K = ids.shape
    ws = gather_ws(ops, n, E)
    xg, off, row_token, rows = ops.moe_gather_rows(dev(x), dev(ids), E, ws)
    assert ops.moe_error_word_read(ws.view(torch.int32)) == 0
    r_off, r_rt, r_rows = oracle.gather_layout(ids, E)
    assert np.array_equal(host(off), r_off)
    assert np.array_equal(host(rows), r_rows)
    assert np.array_equal(host(row_token), r_rt)
    r_xg = oracle.gather_copy(x, r_rt)
    assert np.array_equal(host(xg).view(np.uint8), r_xg.view(np.uint8))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_gather_workloads(ops, name):
    cfg = synth.WORKLOADS[name]
    ids, _ = oracle.route_topk(synth.draw_logits(name), cfg["K"])
    _gather_case(ops, synth.draw_activations(name), ids, cfg["E"])


def test_gather_edge_cases(ops):
    rng = np.random.default_rng(5)
    # one expert takes every token; ragged token count; fp32 rows
    ids = np.zeros((45, 1), dtype=np.int32)
    _gather_case(ops, rng.standard_normal((45, 32)).astype(np.float32), ids, 3)
    # many tokens, large E (global-memory bitmap path), bf16 rows
    E, n, K = 256, 3001, 8
    ids = np.stack([rng.permutation(E)[:K] for _ in range(n)]).astype(np.int32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((n, 64)).astype(np.float32))
    _gather_case(ops, x, ids, E)


@pytest.mark.parametrize("n, K, E", [(10, 3, 5), (700, 4, 40)])
def test_gather_drops_invalid_ids_and_sets_the_error_word(ops, n, K, E):
    """Out-of-range ids are dropped (rows -1, not counted, tail rows untouched)
    and set MOE_DEVERR_EXPERT_ID in the workspace's error word; the word is
    sticky across a following valid call and cleared by moe_error_word_clear.
    Both the one-workgroup path (10 tokens) and the multi-workgroup path (700)."""
    rng = np.random.default_rng(6)
    d = 16
    ids = np.stack([rng.permutation(E)[:K] for _ in range(n)]).astype(np.int32)
    ids[2, 1] = E
    ids[7, 0] = -3
    x = rng.standard_normal((n, d)).astype(np.float32)
    ws = gather_ws(ops, n, E)
    word = ws.view(torch.int32)
    canary = torch.full((n * K, d), float("nan"), device=DEV)
    xg, off, row_token, rows = ops.moe_gather_rows(dev(x), dev(ids), E, ws, xg=canary)
    assert ops.moe_error_word_read(word) == ops.MOE_DEVERR_EXPERT_ID
    valid = (ids >= 0) & (ids < E)
    got_rows = host(rows)
    assert np.all(got_rows[~valid] == -1)
    got_off = host(off)
    assert got_off[-1] == valid.sum()
    assert np.array_equal(np.diff(got_off), np.bincount(ids[valid], minlength=E))
    rt = host(row_token)
    assert np.all(rt[valid.sum():] == -1)
    xgh = host(xg)
    for t in range(n):
        for j in range(K):
            if valid[t, j]:
                assert rt[got_rows[t, j]] == t
                assert np.array_equal(xgh[got_rows[t, j]], x[t])
    assert np.all(np.isnan(xgh[valid.sum():]))
    good = np.stack([rng.permutation(E)[:K] for _ in range(n)]).astype(np.int32)
    ops.moe_gather_rows(dev(x), dev(good), E, ws)
    assert ops.moe_error_word_read(word) == ops.MOE_DEVERR_EXPERT_ID   # sticky
    ops.moe_error_word_clear(word)
    ops.moe_gather_rows(dev(x), dev(good), E, ws)
    assert ops.moe_error_word_read(word) == 0


# ----------------------------------------------------------------------------
# WeightedRowSum
# ----------------------------------------------------------------------------

def _wrs_bound(dst, src, rows, w):
    """|fl(dst + sum_j w*src) - exact| <= (K+1) * 2^-24 * (|dst| + sum_j |w*src|):
    K fused multiply-adds and one add, each rounding once."""
    K = rows.shape[1]
    mag = np.abs(dst).astype(np.float64)
    for j in range(K):
        r = rows[:, j]
        ok = (r >= 0) & (r < src.shape[0])
        mag += np.where(ok[:, None], np.abs(w[:, j:j + 1] * src[np.clip(r, 0, src.shape[0] - 1)]), 0)
    return (K + 1) * 2.0 ** -24 * mag


@pytest.mark.parametrize("K", [6, 12])
@pytest.mark.parametrize("d", [100, 33])
def test_weighted_row_sum(ops, d, K):
    """Bit for bit equal to the oracle's binary32 WeightedRowSum (a fixed-order
    fmaf chain over j, then one add onto dst), with repeated source rows and a
    pre-filled dst; within the rigorous bound of the exact sum; deterministic.
    d = 100 takes the 16-byte kernel (K = 6 its all-rows-first form, K = 12 the
    per-row loop), d = 33 the element kernel.  Row 1 is the case where an
    unfused multiply-add or the other j order gives other bits."""
    rng = np.random.default_rng(d + K)
    n, ns = 37, 50
    src = rng.standard_normal((ns, d)).astype(np.float32)
    rows = rng.integers(0, ns, size=(n, K)).astype(np.int32)
    rows[0] = rows[0, 0]                       # repeated source rows
    w = rng.standard_normal((n, K)).astype(np.float32)
    t = np.float32(1.0 + 2.0 ** -12)
    src[0, 0], src[1, 0] = -1.0, t
    rows[1, :2], w[1, :2], w[1, 2:] = [0, 1], [1.0, t], 0.0
    dst = rng.standard_normal((n, d)).astype(np.float32) * 10   # pre-filled dst
    dst[1, 0] = 0.0
    word = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = ops.moe_weighted_row_sum(dev(dst), dev(src), dev(rows), dev(w), error_word=word)
    got = host(out)
    ref32 = oracle.weighted_row_sum_f32(dst, src, rows, w)
    assert np.array_equal(got.view(np.uint32), ref32.view(np.uint32))
    assert got[1, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)
    ref = oracle.weighted_row_sum(dst, src, rows, w)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= _wrs_bound(dst, src, rows, w))
    assert int(host(word)[0]) == 0
    out2 = ops.moe_weighted_row_sum(dev(dst), dev(src), dev(rows), dev(w))
    assert np.array_equal(host(out2), got)   # deterministic
    into = ops.moe_weighted_row_sum_into(torch.full((n, d), 7.0, device=DEV), dev(src), dev(rows), dev(w))
    zero = np.zeros_like(dst)
    assert np.array_equal(host(into).view(np.uint32), oracle.weighted_row_sum_f32(zero, src, rows, w).view(np.uint32))


def test_weighted_row_sum_skips_out_of_range_rows_and_sets_the_error_word(ops):
    """An out-of-range row contributes nothing (the oracle's binary32 sum with
    that weight zeroed, bit for bit) and sets MOE_DEVERR_ROW in the error word."""
    rng = np.random.default_rng(8)
    n, K, ns, d = 6, 3, 4, 8
    src = rng.standard_normal((ns, d)).astype(np.float32)
    rows = rng.integers(0, ns, size=(n, K)).astype(np.int32)
    rows[1, 2], rows[4, 0] = 4, -1
    w = rng.standard_normal((n, K)).astype(np.float32)
    dst = rng.standard_normal((n, d)).astype(np.float32)
    word = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    ops.moe_error_word_clear(word)
    got = host(ops.moe_weighted_row_sum(dev(dst), dev(src), dev(rows), dev(w), error_word=word))
    assert ops.moe_error_word_read(word) == ops.MOE_DEVERR_ROW
    w0 = w.copy()
    w0[1, 2] = w0[4, 0] = 0
    rows0 = np.clip(rows, 0, ns - 1)
    assert np.array_equal(got.view(np.uint32), oracle.weighted_row_sum_f32(dst, src, rows0, w0).view(np.uint32))
    # without a word the call still skips the entry
    got2 = host(ops.moe_weighted_row_sum(dev(dst), dev(src), dev(rows), dev(w)))
    assert np.array_equal(got2, got)


# ----------------------------------------------------------------------------
# one grouped projection
# ----------------------------------------------------------------------------

def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("a_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_grouped_linear(ops, a_dtype, path):
    """The prefill case is gllm #91's NVFP4Exact test: bf16-exact activations on
    the bf16 MFMA path are held to the fp32 tolerance (a lossy unpack, or a
    missing or doubled global, fails it)."""
    rng = np.random.default_rng(11)
    if path == "decode":
        counts = [3, 0, 32, 1, 17, 16, 5]
        gmax = 32
    else:
        counts = [33, 0, 130, 1, 257, 64]
        gmax = 0
    k, n_out = 96, 200
    w = synth.random_bytes_nvfp4(12, len(counts), n_out, k)
    n_rows = int(sum(counts))
    a32 = rng.standard_normal((n_rows, k)).astype(np.float32)
    if a_dtype == "bf16":
        a = synth.f32_to_bf16_bits(a32)
        a64 = oracle.bf16_bits_to_f64(a)
    else:
        a = a32
        a64 = a32.astype(np.float64)
    off = _offsets(counts)
    dw = ops.DeviceNVFP4.from_host(w)
    out = ops.nvfp4_grouped_linear(dev(a), dev(off), dw, max(counts), gemv_max_rows=gmax)
    got = host(out)
    if path == "prefill" and a_dtype == "f32":
        # the prefill path rounds fp32 activations to bf16
        a64 = np.vectorize(oracle.round_bf16)(a64)
    ref = oracle.linear(a64, off, w)
    assert normwise(got, ref) <= TOL_DECODE


def test_pack_scales_layout(ops):
    """nvfp4_pack_scales against the layout written out on the host: 16-row
    blocks, 128-wide k chunks, each in two 64-wide halves of 4 scale bytes per
    row, zeros past the rows (40 = 2.5 blocks) and past the row's 14 scale
    bytes (224 columns: the second chunk's second half is half empty)."""
    E, rows, cols = 3, 40, 224
    w = synth.random_bytes_nvfp4(41, E, rows, cols)
    got = host(ops.nvfp4_pack_scales(ops.DeviceNVFP4.from_host(w)))
    kb, nrb, nch = cols // 16, (rows + 15) // 16, (cols + 127) // 128
    sc = np.asarray(w.scales).reshape(E, rows, kb)
    ref = np.zeros((E, nrb, nch, 2, 16, 4), dtype=np.uint8)
    for b in range(nrb):
        for r in range(16):
            if 16 * b + r >= rows:
                continue
            for c in range(nch):
                for h in range(2):
                    lo = 8 * c + 4 * h
                    n = min(4, kb - lo)
                    if n > 0:
                        ref[:, b, c, h, r, :n] = sc[:, 16 * b + r, lo:lo + n]
    assert got.size == ops.nvfp4_packed_scales_bytes(E, rows, cols) == ref.size
    assert np.array_equal(got.reshape(ref.shape), ref)


def test_pack_codes_layout(ops):
    """nvfp4_pack_codes against the layout written out on the host: 16-row
    blocks, 128-wide k chunks, each in two 64-wide halves of 32 code bytes per
    row, zeros past the rows (40) and past the row's 112 code bytes (224
    columns: the second chunk's second half is half empty)."""
    E, rows, cols = 3, 40, 224
    w = synth.random_bytes_nvfp4(42, E, rows, cols)
    got = host(ops.nvfp4_pack_codes(ops.DeviceNVFP4.from_host(w)))
    kc, nrb, nch = cols // 2, (rows + 15) // 16, (cols + 127) // 128
    cd = np.asarray(w.codes).reshape(E, rows, kc)
    ref = np.zeros((E, nrb, nch, 2, 16, 32), dtype=np.uint8)
    for b in range(nrb):
        for r in range(16):
            if 16 * b + r >= rows:
                continue
            for c in range(nch):
                for h in range(2):
                    lo = 64 * c + 32 * h
                    n = min(32, kc - lo)
                    if n > 0:
                        ref[:, b, c, h, r, :n] = cd[:, 16 * b + r, lo:lo + n]
    assert got.size == ops.nvfp4_packed_codes_bytes(E, rows, cols) == ref.size
    assert np.array_equal(got.reshape(ref.shape), ref)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_repacked_weights_give_identical_results(ops, path):
    """The repacked codes and scales are the same bytes in another order, and
    the kernels do the same arithmetic on them: the GEMV (decode) and GEMM
    (prefill) results with and without the repacked copies are bit-identical."""
    rng = np.random.default_rng(43)
    counts = [3, 0, 32, 1, 17, 16, 5] if path == "decode" else [33, 0, 130, 1, 257, 64]
    k, n_out = 256, 208
    w = synth.random_bytes_nvfp4(44, len(counts), n_out, k)
    a = synth.f32_to_bf16_bits(rng.standard_normal((sum(counts), k)).astype(np.float32))
    off = _offsets(counts)
    gmax = 32 if path == "decode" else 0
    plain = ops.DeviceNVFP4.from_host(w)
    packed = ops.DeviceNVFP4.from_host(w).pack()
    got_plain = host(ops.nvfp4_grouped_linear(dev(a), dev(off), plain, max(counts), gemv_max_rows=gmax))
    got_packed = host(ops.nvfp4_grouped_linear(dev(a), dev(off), packed, max(counts), gemv_max_rows=gmax))
    assert np.array_equal(got_plain.view(np.uint32), got_packed.view(np.uint32))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("n_out", [96, 90])
@pytest.mark.parametrize("counts", [[120, 128, 40, 200], [33, 202, 190, 215, 4]])
def test_grouped_linear_prefill_row_mixes(ops, counts, n_out, packed):
    """The prefill GEMM over row counts around one and two 128-row m-tiles
    (prefill4314 has about 202 rows per expert), with a k of 160 (a partial
    128-wide chunk) and an expert of a few rows, against the oracle.  An
    output width that is not a multiple of 4 takes the element stores instead
    of the 16-byte ones; with repacked scales and codes (and 96 rows) the
    GEMM reads those."""
    rng = np.random.default_rng(31)
    k = 160
    w = synth.random_nvfp4(32, len(counts), n_out, k)
    a = synth.f32_to_bf16_bits(rng.standard_normal((sum(counts), k)).astype(np.float32))
    off = _offsets(counts)
    dw = ops.DeviceNVFP4.from_host(w)
    if packed:  # read by the GEMM when the row count is a whole number of 16-row blocks
        dw.pack()
    got = host(ops.nvfp4_grouped_linear(dev(a), dev(off), dw, max(counts), gemv_max_rows=0))
    ref = oracle.linear(oracle.bf16_bits_to_f64(a), off, w)
    assert normwise(got, ref) <= TOL_DECODE


def test_grouped_linear_mixed_paths(ops):
    """Experts on both sides of the 32-row threshold in one call."""
    rng = np.random.default_rng(13)
    counts = [32, 33, 1, 0, 70, 31]
    k, n_out = 128, 64
    w = synth.random_nvfp4(14, len(counts), n_out, k)
    a = synth.f32_to_bf16_bits(rng.standard_normal((sum(counts), k)).astype(np.float32))
    off = _offsets(counts)
    got = host(ops.nvfp4_grouped_linear(dev(a), dev(off), ops.DeviceNVFP4.from_host(w), max(counts)))
    ref = oracle.linear(oracle.bf16_bits_to_f64(a), off, w)
    assert normwise(got, ref) <= TOL_DECODE


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def _run_layer(ops, inp, gemv_max_rows=32, stream=None):
    layer = ops.MoELayer(inp, gemv_max_rows=gemv_max_rows)
    out = layer.forward(dev(inp.x), dev(inp.logits), stream=stream)
    torch.cuda.synchronize()
    return layer, host(out).astype(np.float64)


@pytest.mark.parametrize("name", ["tiny16", "decode1", "decode32_zipf", "gated2"])
def test_layer_decode_workloads(ops, name):
    inp = cached_layer(name)
    layer, got = _run_layer(ops, inp)
    ref = oracle.layer(inp)
    assert np.array_equal(host(layer.ids), ref["ids"])
    assert np.array_equal(host(layer.offsets), ref["offsets"])
    assert np.array_equal(host(layer.rows), ref["rows"])
    counts = np.diff(ref["offsets"])
    assert counts.max() <= 32   # every expert on the decode path
    assert normwise(got, ref["out"]) <= TOL_DECODE
    # routed expert outputs row by row (the packed yg buffer)
    R = inp.n * inp.K
    assert normwise(host(layer.yg)[:R], ref["yg"]) <= TOL_DECODE
    # and against the oracle's binary32 fixed-order evaluation (another
    # summation order than the kernels', so to the same tolerance, not bits)
    ref32 = oracle.layer(inp, arith="f32")
    assert normwise(got, ref32["out"]) <= TOL_DECODE


# Every expert forced onto the prefill GEMM: a k that is not a whole number of
# 64-wide steps (d 96, d_ff 160, shared 224) and the gated FFN (SwiGLU gate
# and up rows side by side in the weight tile).
FORCED_PREFILL_CASES = [("tiny16", dict()), ("tiny16", dict(n=24, d=96, f=160, fs=224, seed=21)),
                        ("gated2", dict(n=40, seed=22)),
                        # about 128 rows per expert, shared expert over four m-tiles
                        ("tiny16", dict(n=512, seed=24))]


@pytest.mark.parametrize("case", range(len(FORCED_PREFILL_CASES)))
def test_layer_forced_onto_prefill_path(ops, case):
    name, ov = FORCED_PREFILL_CASES[case]
    inp = cached_layer(name, **ov)
    print(f"forced prefill case {name} {ov}", flush=True)
    _, got = _run_layer(ops, inp, gemv_max_rows=0)
    assert normwise(got, oracle.layer(inp)["out"]) <= TOL_PREFILL
    # against the oracle's bf16-activation mode the only differences are
    # accumulation order and rare bf16 rounding flips of h
    assert normwise(got, oracle.layer(inp, bf16_act=True)["out"]) <= 2e-3


def _whole_expert_checks(ops, inp, layer, off, row_token, experts):
    """Every routed output row (yg) of the given experts against the oracle's
    expert FFN over those rows: 2e-2 against the exact values, 2e-3 against
    the bf16-activation mode (the path's own rounding of x and h)."""
    yg = host(layer.yg)
    x64 = oracle.activations_f64(inp.x, inp.x_dtype)
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        rows_x = x64[row_token[r0:r1]]
        one = np.array([0, r1 - r0], dtype=np.int32)
        sub_up, sub_dn = oracle._one_expert(inp.up, e), oracle._one_expert(inp.down, e)
        ref = oracle.expert_ffn(rows_x, one, sub_up, sub_dn, inp.f, inp.act)
        ref_bf = oracle.expert_ffn(rows_x, one, sub_up, sub_dn, inp.f, inp.act, bf16_act=True)
        got = yg[r0:r1].astype(np.float64)
        print(f"  expert {e}: rows {r1 - r0}, err {normwise(got, ref):.2e} / bf16 mode {normwise(got, ref_bf):.2e}",
              flush=True)
        assert normwise(got, ref) <= TOL_PREFILL
        assert normwise(got, ref_bf) <= 2e-3


def _pick_experts(counts, k=8):
    """The smallest and largest experts plus others spread over the row counts
    (prefill4314: 160-250 rows, i.e. one full 128-row m-tile and a partial one)."""
    order = np.argsort(counts, kind="stable")
    idx = np.unique(np.linspace(0, len(order) - 1, k).round().astype(int))
    return [int(order[i]) for i in idx]


def _spread_tokens(n, m=64):
    return sorted(set(np.linspace(0, n - 1, m).round().astype(int).tolist()))


def test_layer_prefill_4314_tokens(ops):
    """The largest workload (every expert on the bf16 MFMA GEMM): routing and
    layout bit for bit; every yg row of 8 whole experts (smallest, largest and
    six between); the layer output of 64 tokens spread over the batch (which
    between them pick most experts) against the sampled oracle."""
    inp = cached_layer("prefill4314")
    print("prefill4314 layer", flush=True)
    layer, got = _run_layer(ops, inp)
    ids, w = oracle.route_topk(inp.logits, inp.K)
    assert np.array_equal(host(layer.ids), ids)
    check_route_weights(host(layer.w), w, inp.K)
    off, row_token, rows = oracle.gather_layout(ids, inp.E)
    assert np.array_equal(host(layer.offsets), off)
    assert np.array_equal(host(layer.rows), rows)
    assert np.array_equal(host(layer.row_token), row_token)
    counts = np.diff(off)
    assert counts.min() > 32    # every expert on the prefill path
    experts = _pick_experts(counts)
    assert len(experts) >= 8 and counts[experts].min() == counts.min() and counts[experts].max() == counts.max()
    _whole_expert_checks(ops, inp, layer, off, row_token, experts)
    tokens = _spread_tokens(inp.n)
    assert len(tokens) >= 64
    assert len(np.unique(ids[tokens])) >= 100
    ref = oracle.layer_sampled(inp, tokens, ids, w)
    assert normwise(got[tokens], ref) <= TOL_PREFILL
    ref_bf = oracle.layer_sampled(inp, tokens, ids, w, bf16_act_of_expert=lambda e: True)
    assert normwise(got[tokens], ref_bf) <= 2e-3
    assert np.all(np.isfinite(got))


def test_layer_gated_prefill_scale(ops):
    """SwiGLU experts at prefill scale on the bf16 MFMA GEMM: 2048 tokens over
    64 experts with topK 8 give about 256 rows per expert, so every expert spans
    two or three 128-row m-tiles and each weight tile carries gate and up rows
    side by side.  Sampled tokens against the oracle."""
    inp = cached_layer("gated2", n=2048, E=64, seed=23)
    print("gated prefill-scale case: n 2048, E 64, K 8, SwiGLU f 1024", flush=True)
    layer, got = _run_layer(ops, inp)
    ids, w = oracle.route_topk(inp.logits, inp.K)
    assert np.array_equal(host(layer.ids), ids)
    off, row_token, rows = oracle.gather_layout(ids, inp.E)
    assert np.array_equal(host(layer.offsets), off)
    assert np.array_equal(host(layer.rows), rows)
    counts = np.diff(off)
    assert counts.min() > 32 and counts.max() > 128   # GEMM path, several m-tiles
    tokens = [0, 5, 1023, 2047]
    ref = oracle.layer_sampled(inp, tokens, ids, w)
    assert normwise(got[tokens], ref) <= TOL_PREFILL
    ref_bf = oracle.layer_sampled(inp, tokens, ids, w, bf16_act_of_expert=lambda e: True)
    assert normwise(got[tokens], ref_bf) <= 2e-3


def test_layer_is_deterministic_and_stream_independent(ops):
    inp = cached_layer("decode32_zipf")
    layer = ops.MoELayer(inp)
    x, lg = dev(inp.x), dev(inp.logits)
    a = layer.forward(x, lg).clone()
    b = layer.forward(x, lg).clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = layer.forward(x, lg, stream=s).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_expert_ffn_writes_only_its_rows(ops):
    """A canary-filled output: the FFN writes rows [0, offsets[E]) and nothing
    else (gllm #91 "Testing": a product written into a row range of a larger
    buffer must change those rows and no others)."""
    inp = cached_layer("tiny16")
    counts = np.array([3, 0, 9, 1, 0, 4, 2, 1], dtype=np.int64)
    off = _offsets(counts)
    n_rows = int(off[-1]) + 5
    rng = np.random.default_rng(17)
    xg = rng.standard_normal((n_rows, inp.d)).astype(np.float32)
    out = torch.full((n_rows, inp.d), float("nan"), device=DEV)
    ws = torch.empty((ops.nvfp4_expert_ffn_workspace_size(n_rows, inp.d, inp.f, ops.MOE_F32),),
                     dtype=torch.uint8, device=DEV)
    up, dn = ops.DeviceNVFP4.from_host(inp.up), ops.DeviceNVFP4.from_host(inp.down)
    ops.nvfp4_expert_ffn(dev(xg), dev(off), up, dn, ops.MOE_RELU2, int(counts.max()), ws, out)
    got = host(out)
    assert np.all(np.isnan(got[off[-1]:]))
    ref = oracle.expert_ffn(xg[:off[-1]].astype(np.float64), off, inp.up, inp.down, inp.f, "relu2")
    assert normwise(got[:off[-1]], ref) <= TOL_DECODE


# ----------------------------------------------------------------------------
# the fused layer entry point
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny16", "decode1", "decode32_zipf", "gated2", "prefill4314"])
def test_layer_forward_fused(ops, name):
    """moe_layer_forward matches the oracle at the path's tolerance, leaves the
    same intermediates, and gives the same bits as the four calls in order.
    One- and two-token steps run as the single launch (the flag is set), and
    without the flag as the per-step launches."""
    inp = cached_layer(name)
    layer = ops.MoELayer(inp, single_launch=True)
    x, lg = dev(inp.x), dev(inp.logits)
    fused = layer.forward_fused(x, lg).clone()
    v = layer.views()
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(inp.logits, inp.K)
    off, row_token, rows = oracle.gather_layout(ids, inp.E)
    assert np.array_equal(host(v["ids"]), ids)
    check_route_weights(host(v["w"]), w, inp.K)
    assert np.array_equal(host(v["offsets"]), off)
    assert np.array_equal(host(v["rows"]), rows)
    assert np.array_equal(host(v["row_token"]), row_token)
    got = host(fused).astype(np.float64)
    if name == "prefill4314":
        tokens = _spread_tokens(inp.n, 64)[::2]
        ref = oracle.layer_sampled(inp, tokens, ids, w)
        assert normwise(got[tokens], ref) <= TOL_PREFILL
    else:
        ref = oracle.layer(inp)
        assert normwise(got, ref["out"]) <= TOL_DECODE
    assert int(host(v["wait_error"])[0]) == 0
    single = inp.n <= 2
    # calls since the workspace was prepared that ran the single-launch step
    assert int(host(v["decode_launch"])[0]) == (1 if single else 0)
    unfused = layer.forward(x, lg).clone()
    torch.cuda.synchronize()
    if name == "prefill4314":  # and with the combine fused into the down GEMM
        layer.flags |= ops.MOE_LAYER_FUSED_COMBINE
        assert torch.equal(layer.forward_fused(x, lg), unfused)
        layer.flags &= ~ops.MOE_LAYER_FUSED_COMBINE
    if single:  # fp32 dot products on the vector ALUs: equal to fp32 rounding
        assert normwise(host(fused).astype(np.float64), host(unfused).astype(np.float64)) <= 2e-6
    else:
        assert torch.equal(fused, unfused)
    layer.flags = 0   # without the flag: the per-step launches, bit for bit the four calls
    plain = layer.forward_fused(x, lg).clone()
    torch.cuda.synchronize()
    assert int(host(v["decode_launch"])[0]) == (1 if single else 0)
    assert torch.equal(plain, unfused)


# Decode steps the single-launch layer takes (one or two tokens): tiny shapes
# (fp32 x) with every expert holding both rows, one expert, k-slices that leave
# wavefronts empty; realistic shapes with a skewed router, without a shared
# expert and with the gated FFN (bf16 x); the gated FFN with fp32 x, also with
# a ragged last chunk (d 160) and a half-filled last unit (d_ff 96).  The last
# case (seven tokens) falls back to the per-step launches.
SINGLE_LAUNCH_CASES = [
    ("tiny16", dict(n=1, seed=11), True),
    ("tiny16", dict(n=2, E=4, K=4, seed=12), True),
    ("tiny16", dict(n=1, E=1, K=1, seed=13), True),
    ("tiny16", dict(n=2, d=96, f=160, fs=224, seed=14), True),
    ("decode1", dict(n=2, K=2, E=32, fs=1856, logits="zipf", seed=15), True),
    ("decode1", dict(n=1, E=32, fs=0, seed=16), True),
    ("gated2", dict(n=1, seed=17), True),
    ("tiny16", dict(n=2, act="swiglu", fs=0, seed=19), True),
    ("tiny16", dict(n=1, act="swiglu", fs=0, d=160, f=96, seed=20), True),
    # gated units whose up pieces go chunk-fastest (d_model a multiple of 1024
    # or just under): shared experts and a half-filled last unit; fp32 x with a
    # ragged last chunk
    ("gated2", dict(n=2, E=8, K=4, f=992, seed=21), True),
    ("tiny16", dict(n=2, act="swiglu", fs=0, d=960, f=96, seed=22), True),
    # more than 128 experts (two ranking passes), and more than 8 picks
    ("tiny16", dict(n=2, E=200, K=6, seed=23), True),
    ("tiny16", dict(n=1, E=48, K=12, seed=24), True),
    ("decode1", dict(n=7, E=32, fs=0, seed=18), False),
]


@pytest.mark.parametrize("case", range(len(SINGLE_LAUNCH_CASES)))
def test_layer_single_launch_decode(ops, case):
    """Back-to-back fused calls with different routings: each matches the
    oracle, leaves no expired wait, agrees with the four-call path (bit for bit
    where the per-step launches run) and repeats bit for bit; the last call's
    routing and layout views match the oracle's."""
    name, ov, single = SINGLE_LAUNCH_CASES[case]
    inp = cached_layer(name, **ov)
    print(f"single-launch case {name} {ov}", flush=True)
    layer = ops.MoELayer(inp, single_launch=True)
    x = dev(inp.x)
    logit_sets = [inp.logits, np.ascontiguousarray(np.roll(inp.logits, 1, axis=1))]
    lgs = [dev(l) for l in logit_sets]
    outs = [layer.forward_fused(x, lg).clone() for lg in lgs + lgs[:1]]
    v = layer.views()
    errs = host(v["wait_error"]).copy()
    ran = host(v["decode_launch"]).copy()
    torch.cuda.synchronize()
    assert int(errs[0]) == 0
    assert int(ran[0]) == (3 if single else 0)
    assert torch.equal(outs[0], outs[2])
    ids, w = oracle.route_topk(inp.logits, inp.K)
    off, row_token, rows = oracle.gather_layout(ids, inp.E)
    assert np.array_equal(host(v["ids"]), ids)
    check_route_weights(host(v["w"]), w, inp.K)
    assert np.array_equal(host(v["offsets"]), off)
    assert np.array_equal(host(v["rows"]), rows)
    assert np.array_equal(host(v["row_token"]), row_token)
    for lg_host, lg, got in zip(logit_sets, lgs, outs):
        ref = oracle.layer(inp, routing=oracle.route_topk(lg_host, inp.K))
        assert normwise(host(got).astype(np.float64), ref["out"]) <= TOL_DECODE
        unfused = layer.forward(x, lg).clone()
        torch.cuda.synchronize()
        if single:
            assert normwise(host(got).astype(np.float64), host(unfused).astype(np.float64)) <= 2e-6
        else:
            assert torch.equal(got, unfused)


def test_layer_single_launch_token_counts(ops):
    """One workspace, prepared once, serves single-launch steps of one and of
    two tokens in any order (its flags and counters carry over between
    calls of different sizes)."""
    inp = cached_layer("decode1", n=2, K=3, E=32, fs=1856, seed=19)
    layer = ops.MoELayer(inp, single_launch=True)
    x, lg = dev(inp.x), dev(inp.logits)
    order = [2, 1, 1, 2, 1, 2, 2]
    outs = [layer.forward_fused(x[:m], lg[:m]).clone()[:m] for m in order]
    v = layer.views(1)
    errs = host(v["wait_error"]).copy()
    ran = host(v["decode_launch"]).copy()
    torch.cuda.synchronize()
    assert int(errs[0]) == 0
    assert int(ran[0]) == len(order)
    full = oracle.layer(inp)["out"]
    for m, got in zip(order, outs):
        assert normwise(host(got).astype(np.float64), full[:m]) <= TOL_DECODE


@pytest.mark.parametrize("name", ["decode1", "decode32_zipf"])
def test_layer_forward_fused_repeat_and_graph(ops, name):
    """Captured in a HIP graph and replayed, the fused layer gives the eager
    bits on every replay (the layer neither allocates nor synchronises)."""
    inp = cached_layer(name)
    layer = ops.MoELayer(inp, single_launch=True)
    x, lg = dev(inp.x), dev(inp.logits)
    eager = layer.forward_fused(x, lg).clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward_fused(x, lg)
    for _ in range(3):
        layer.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager)


def test_layers_on_two_streams_concurrent_equal_alone_equal_serial(ops):
    """Without the single-launch flag no kernel of a layer waits on another
    workgroup, so layers may run concurrently: two layers (a 32-token and a
    one-token decode step) launched on two streams at once, ten rounds, give
    the bits each gives alone and the bits of running them one after the
    other on one stream."""
    a_inp, b_inp = cached_layer("decode32_zipf"), cached_layer("decode1")
    la, lb = ops.MoELayer(a_inp), ops.MoELayer(b_inp)
    xa, ga, xb, gb = dev(a_inp.x), dev(a_inp.logits), dev(b_inp.x), dev(b_inp.logits)
    alone_a = la.forward_fused(xa, ga).clone()
    torch.cuda.synchronize()
    alone_b = lb.forward_fused(xb, gb).clone()
    torch.cuda.synchronize()
    serial_a = la.forward_fused(xa, ga).clone()
    serial_b = lb.forward_fused(xb, gb).clone()
    torch.cuda.synchronize()
    assert torch.equal(serial_a, alone_a) and torch.equal(serial_b, alone_b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for _ in range(10):
        with torch.cuda.stream(s1):
            la.forward_fused(xa, ga, stream=s1)
            oa = la.out.clone()
        with torch.cuda.stream(s2):
            lb.forward_fused(xb, gb, stream=s2)
            ob = lb.out.clone()
        outs.append((oa, ob))
        s1.wait_stream(s2)   # the next round's writes of la.out / lb.out wait for the clones
        s2.wait_stream(s1)
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa, alone_a) and torch.equal(ob, alone_b)
    ref = oracle.layer(b_inp)["out"]
    assert normwise(host(alone_b).astype(np.float64), ref) <= TOL_DECODE


def test_single_launch_200_graph_replayed_steps(ops):
    """The single-launch decode step, captured as 8 steps over two alternating
    routings and replayed 25 times (200 steps): after every replay no bounded
    wait has expired and every step's output equals the eager output of its
    routing bit for bit.  Stops at the first mismatch or error word."""
    inp = cached_layer("decode1")
    layer = ops.MoELayer(inp, single_launch=True)
    x = dev(inp.x)
    lgs = [dev(inp.logits), dev(np.ascontiguousarray(np.roll(inp.logits, 5, axis=1)))]
    eager = [layer.forward_fused(x, lg).clone() for lg in lgs]
    torch.cuda.synchronize()
    assert not torch.equal(eager[0], eager[1])
    wait = layer.views()["wait_error"]
    slots = torch.empty((8,) + tuple(layer.out.shape), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(8):
            layer.forward_fused(x, lgs[i % 2], check=False)
            slots[i].copy_(layer.out)
    for rep in range(25):
        slots.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(wait.cpu()[0]) == 0, f"a bounded wait expired in replay {rep}"
        for i in range(8):
            assert torch.equal(slots[i], eager[i % 2]), f"replay {rep}, step {i} differs"


# ----------------------------------------------------------------------------
# the router GEMM fused with routing
# ----------------------------------------------------------------------------

def router_ws(ops, n, E):
    ws = torch.empty((ops.moe_router_workspace_size(n, E),), dtype=torch.uint8, device=DEV)
    ops.moe_router_workspace_init(ws, n)
    return ws


def _router_case(ops, x, x_dtype, wr, K, min_separated=0.5):
    """moe_router_topk against the oracle in three stages: its logits within the
    fp32 accumulation bound of the exact x . W_r^T; its ids and weights those
    of the routing rule applied to its own logits (ids bit for bit, weights
    within the routing bound, and the same bits as moe_route_topk on them);
    and the oracle's ids wherever the exact top K + 1 logits are separated by
    more than twice the bound."""
    n, d = x.shape
    E = wr.shape[0]
    ws = router_ws(ops, n, E)
    logits = torch.full((n, E), float("nan"), device=DEV)
    ids, w, _ = ops.moe_router_topk(dev(x), dev(wr), K, ws, logits=logits)
    lg = host(logits).astype(np.float64)
    x64 = oracle.activations_f64(x, x_dtype)
    exact = oracle.router_logits(x64, wr)
    bound = (d + 8) * 2.0 ** -24 * (np.abs(x64) @ np.abs(oracle.bf16_bits_to_f64(wr)).T)
    assert np.all(np.abs(lg - exact) <= bound), f"router logits off by {np.max(np.abs(lg - exact) / bound):.2f} x bound"
    rid, rw = oracle.route_topk(lg.astype(np.float32), K)
    assert np.array_equal(host(ids), rid)
    check_route_weights(host(w), rw, K)
    ids2, w2 = ops.moe_route_topk(logits, K)
    assert np.array_equal(host(ids2), host(ids)) and np.array_equal(host(w2), host(w))
    oid, ow, _ = oracle.router_topk(x, x_dtype, wr, K)
    srt = -np.sort(-exact, axis=1)[:, :min(K + 1, E)]
    # the smallest gap between neighbours of the exact top K + 1 (the minus sign
    # goes on the differences, before the min)
    gaps = (-np.diff(srt, axis=1)).min(axis=1) if srt.shape[1] > 1 else np.full(n, np.inf)
    sep = gaps > 2 * bound.max(axis=1)
    assert sep.mean() >= min_separated, f"only {sep.mean():.2f} of the tokens are separated"
    assert np.array_equal(host(ids)[sep], oid[sep])
    # the counters were left at zero: a second call, without a logits output,
    # gives the same bits
    ids3, w3, _ = ops.moe_router_topk(dev(x), dev(wr), K, ws)
    assert np.array_equal(host(ids3), host(ids)) and np.array_equal(host(w3), host(w))
    return host(ids), sep


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_router_topk_workloads(ops, name):
    """Each workload's activations through its seeded bf16 router (d_model 64
    with fp32 activations for the small workload; 1 to 4314 tokens)."""
    cfg = synth.WORKLOADS[name]
    print(f"router case {name}", flush=True)
    _router_case(ops, synth.draw_activations(name), cfg["x_dtype"], synth.draw_router(name), cfg["K"])


def test_router_topk_edge_cases(ops):
    """Ragged token tiles and expert groups (37 tokens, 77 experts), the largest
    E and K (1024, 32), one expert, ties (a zero router: experts 0..K-1 with
    weight 1/K), a long fp32 row, each workgroup shape of the large batches
    (16 and 32 tokens, routed in place or through the counters), and no
    tokens."""
    rng = np.random.default_rng(95)

    def bf(a):
        return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))

    x = bf(rng.standard_normal((37, 96)))
    _router_case(ops, x, "bf16", bf(rng.standard_normal((77, 96)) * 0.1), 5)
    x = bf(rng.standard_normal((9, 64)))
    _router_case(ops, x, "bf16", bf(rng.standard_normal((1024, 64)) * 0.1), 32, min_separated=0.0)
    _router_case(ops, x, "bf16", bf(rng.standard_normal((1, 64))), 1)
    ids, _ = _router_case(ops, x, "bf16", np.zeros((12, 64), dtype=np.uint16), 4, min_separated=0.0)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (9, 1)))
    xf = rng.standard_normal((20, 4096)).astype(np.float32)
    # at d = 4096 the worst-case accumulation bound (about 0.013 here) is a fair
    # part of the gaps between neighbouring logits: fewer rows are separated
    _router_case(ops, xf, "f32", bf(rng.standard_normal((64, 4096)) * 0.02), 6, min_separated=0.3)
    # many token tiles: 128-expert groups per workgroup, routed in place (up to
    # 128 experts, bf16 and fp32 x) or through the counters (256 experts)
    _router_case(ops, bf(rng.standard_normal((1500, 256))), "bf16", bf(rng.standard_normal((128, 256)) * 0.06), 6)
    _router_case(ops, bf(rng.standard_normal((700, 128))), "bf16", bf(rng.standard_normal((256, 128)) * 0.09), 8)
    xf = rng.standard_normal((2100, 96)).astype(np.float32)
    _router_case(ops, xf, "f32", bf(rng.standard_normal((64, 96)) * 0.1), 4)
    # more 16-token tiles (times expert groups) than a 256-CU device has CUs:
    # 32-token workgroups, ragged in tokens and experts, routed in place or
    # through the counters (200 experts: two groups)
    _router_case(ops, bf(rng.standard_normal((4130, 64))), "bf16", bf(rng.standard_normal((96, 64)) * 0.12), 6)
    _router_case(ops, bf(rng.standard_normal((2100, 64))), "bf16", bf(rng.standard_normal((200, 64)) * 0.12), 7)
    xf = rng.standard_normal((4130, 64)).astype(np.float32)
    _router_case(ops, xf, "f32", bf(rng.standard_normal((96, 64)) * 0.12), 6)
    _router_case(ops, xf[:2100], "f32", bf(rng.standard_normal((200, 64)) * 0.12), 7)
    ws = router_ws(ops, 0, 8)
    ids, w, _ = ops.moe_router_topk(torch.empty((0, 64), dtype=torch.int16, device=DEV),
                                    dev(np.zeros((8, 64), dtype=np.uint16)), 2, ws)
    assert ids.shape == (0, 2)


# ----------------------------------------------------------------------------
# WeightedRowSum fused into the prefill down projection
# ----------------------------------------------------------------------------

FUSED_COMBINE_CASES = [
    # a skewed router: experts on both paths (some at most 32 rows, on the
    # decode GEMV, whose rows the GEMM's combine reads but does not count)
    ("tiny16", dict(n=100, logits="zipf", seed=31)),
    # every expert on the GEMM; one and several 128-row m-tiles per expert
    ("tiny16", dict(n=512, seed=32)),
    # the workload's widths: 11 column tiles of 256 (the last one of 128)
    ("decode1", dict(n=200, E=16, seed=33)),
]


@pytest.mark.parametrize("case", range(len(FUSED_COMBINE_CASES)))
def test_fused_combine_equals_the_separate_weighted_row_sum(ops, case):
    """With MOE_LAYER_FUSED_COMBINE and a shared expert, a prefill step's
    WeightedRowSum runs in the down
    GEMM's epilogue (the last producer of a token's column tile sums its rows
    in slot order): the output equals the four calls' (separate
    moe_weighted_row_sum launch) bit for bit, twice in a row (the counters are
    prepared by the up launch each call), and matches the oracle."""
    name, ov = FUSED_COMBINE_CASES[case]
    inp = cached_layer(name, **ov)
    print(f"fused combine case {name} {ov}", flush=True)
    layer = ops.MoELayer(inp, fused_combine=True)
    x, lg = dev(inp.x), dev(inp.logits)
    unfused = layer.forward(x, lg).clone()
    yg_unfused = layer.yg.clone()
    a = layer.forward_fused(x, lg).clone()
    b = layer.forward_fused(x, lg).clone()
    v = layer.views()
    torch.cuda.synchronize()
    counts = np.diff(host(v["offsets"]))
    assert counts.max() > 32
    assert torch.equal(a, unfused) and torch.equal(b, unfused)
    R = inp.n * inp.K
    assert torch.equal(v["yg"][:R], yg_unfused[:R])
    ref = oracle.layer(inp)
    assert normwise(host(a).astype(np.float64), ref["out"]) <= TOL_PREFILL
    assert normwise(host(a).astype(np.float64), oracle.layer(inp, bf16_act=True)["out"]) <= 2e-3


# ----------------------------------------------------------------------------
# one copy of the weights
# ----------------------------------------------------------------------------

ONE_COPY_CASES = [("decode32_zipf", {}, 32), ("decode1", {}, 32), ("tiny16", dict(n=512, seed=32), 32),
                  ("gated2", dict(n=40, seed=22), 0)]


@pytest.mark.parametrize("case", range(len(ONE_COPY_CASES)))
def test_one_weight_copy_gives_the_same_bits(ops, case):
    """A layer that keeps only the repacked copies of its weights (the canonical
    codes and scales freed) gives the bits of one that keeps both, on the
    decode GEMV, the relu^2 GEMM and the SwiGLU GEMM; the single-launch step
    (which reads only the repacked copies) runs for the one-token step and
    agrees to fp32 rounding."""
    name, ov, gmax = ONE_COPY_CASES[case]
    inp = cached_layer(name, **ov)
    print(f"one-copy case {name} {ov}", flush=True)
    both = ops.MoELayer(inp, gemv_max_rows=gmax, keep_canonical=True)
    one = ops.MoELayer(inp, gemv_max_rows=gmax, single_launch=True, keep_canonical=False)
    assert all(w is None or (w.codes is None and w.codes_packed is not None) for w in one.weights())
    x, lg = dev(inp.x), dev(inp.logits)
    a = both.forward(x, lg).clone()
    b = one.forward(x, lg).clone()
    c = one.forward_fused(x, lg).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    single = inp.n <= min(2, gmax)
    assert int(host(one.views()["decode_launch"])[0]) == (1 if single else 0)
    if single:
        assert normwise(host(c).astype(np.float64), host(a).astype(np.float64)) <= 2e-6
    else:
        assert torch.equal(a, c)
