"""Pins of the CPU oracle against facts fixed outside it.

Each test compares the oracle with something it does not contain: torch's own
float8/bfloat16 casts, closed forms of the OCP formats, hand-worked fixtures
under tests/golden/, numpy float64 matmuls, invariants of the gather, and the
naive dense-masked algorithm the gather replaced.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_block_scaled_topk_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------

def test_e4m3_all_bytes_match_torch(oracle_lib):
    """PIN: all 256 E4M3FN bytes decode as torch.float8_e4m3fn does."""
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _e2m1_from_bits(code):
    """E2M1 from its bit fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m / 2.0) * 2.0 ** (1 - 1) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def test_e2m1_table_matches_bit_fields(oracle_lib):
    """PIN: the oracle's e2m1 table equals the E2M1 bit-field definition, the
    magnitudes of codes 0..7 rise strictly, max is 6 and code 8 is -0."""
    got = [oracle.e2m1(c) for c in range(16)]
    assert got == [_e2m1_from_bits(c) for c in range(16)]
    mags = got[:8]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    assert mags[-1] == 6.0
    assert got[8] == 0.0 and np.signbit(got[8])


def test_every_e2m1_times_e4m3_is_exact_in_bf16(oracle_lib):
    """PIN (gllm #91, "bf16 NVFP4 GEMM (CUDA)"): the product of an e2m1 value and
    an e4m3 scale is representable in bf16, so the unpack loses nothing.  Checked over
    all 16 x 254 finite products with torch's own float64 -> bfloat16 cast."""
    prods = []
    for c in range(16):
        for s in range(256):
            sv = oracle.e4m3(s)
            if np.isnan(sv):
                continue
            prods.append(oracle.e2m1(c) * sv)
    p = np.array(prods)
    assert p.size == 16 * 254
    rt = torch.from_numpy(p).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, p)
    nz = p[p != 0]
    mant, _ = np.frexp(np.abs(nz))
    sig = mant * 2.0 ** 6
    assert np.all(sig == np.round(sig))  # no more than 6 significant bits


def test_round_bf16_matches_torch(oracle_lib):
    """PIN: the oracle's round-to-bf16 equals torch's float32 -> bfloat16 cast on
    float32-representable values, including exact ties."""
    rng = np.random.default_rng(7)
    v = rng.standard_normal(2000).astype(np.float32) * np.float32(30)
    bits = v.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)   # halfway cases
    vals = np.concatenate([v, ties, np.float32([0, -0.0, 1e-30, 3e38])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(x)) for x in vals])
    assert np.array_equal(got, ref)


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        lines = [ln.strip() for ln in fh if ln.strip() and not ln.startswith("#")]
    return lines


def test_dequant_hand_fixture(oracle_lib):
    """PIN: hand-encoded NVFP4 rows (tests/golden/nvfp4_hand.txt)."""
    lines = _read_golden("nvfp4_hand.txt")
    g = float(lines[0].split()[1])
    codes = np.zeros((2, 16), dtype=np.uint8)
    scales = np.zeros((2, 2), dtype=np.uint8)
    values = np.zeros((2, 32))
    for ln in lines[1:]:
        tok = ln.split()
        r = int(tok[1])
        if tok[0] == "codes":
            codes[r] = [int(t, 16) for t in tok[2:]]
        elif tok[0] == "scales":
            scales[r] = [int(t, 16) for t in tok[2:]]
        elif tok[0] == "values":
            values[r] = [float(t) for t in tok[2:]]
    got = oracle.dequant(codes, scales, g)
    assert np.array_equal(got, values)
    # negative zeros are where the fixture says
    assert np.array_equal(np.signbit(got), np.signbit(values))
    # dropping the global halves every value (global = 0.5)
    assert np.array_equal(oracle.dequant(codes, scales, g, with_global=False), values / g)


def test_dequant_matches_torch_decoders_and_nibble_order(oracle_lib):
    """PIN: random bytes decoded by the oracle equal a decode written from torch's
    float8_e4m3fn cast, the E2M1 bit fields and the low-nibble-first order."""
    t = synth.random_bytes_nvfp4(11, 1, 24, 96)
    c, s, g = t.codes[0], t.scales[0], float(t.globals_[0])
    lo = (c & 15).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    code = np.empty((24, 96), dtype=np.int64)
    code[:, 0::2] = lo
    code[:, 1::2] = hi
    e2 = np.vectorize(_e2m1_from_bits)(code).astype(np.float64)
    sc = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = np.float64(np.float32(g)) * np.repeat(sc, 16, axis=1) * e2
    got = oracle.dequant(c, s, g)
    assert np.array_equal(got, ref)


def test_quantized_weights_decode_close_to_source(oracle_lib):
    """PIN: weights encoded by the input generator and decoded by the oracle stay
    within the format's rounding bound of the float32 source: per element, half
    the local e2m1 gap times the block's scale and global (plus the scale's own
    rounding, absorbed by a 2x margin).  A wrong nibble order, a transposed scale
    or a dropped global breaks it by orders of magnitude."""
    rng = np.random.default_rng(3)
    w = rng.standard_normal((40, 128), dtype=np.float32) * np.float32(0.02)
    codes, scales, g = synth.quantize_nvfp4(w)
    deq = oracle.dequant(codes, scales, float(g))
    block_scale = np.repeat(np.array([[oracle.e4m3(b) for b in row] for row in scales]), 16, axis=1)
    step = block_scale * float(g)  # value of e2m1 1.0 in this block
    err = np.abs(deq - w.astype(np.float64))
    # the largest e2m1 gap is 2 (between 4 and 6): |err| <= 1 * step at worst
    assert np.all(err <= 1.0 * step + 1e-12)
    rel = np.linalg.norm(deq - w) / np.linalg.norm(w)
    assert rel < 0.12


# ----------------------------------------------------------------------------
# WeightedRowSum
# ----------------------------------------------------------------------------

def _golden_wrs():
    lines = _read_golden("weighted_row_sum_hand.txt")
    data = {}
    i = 0
    while i < len(lines):
        name, r, c = lines[i].split()
        r, c = int(r), int(c)
        data[name] = np.array([[float(v) for v in lines[i + 1 + k].split()] for k in range(r)])
        i += 1 + r
    return data


def test_weighted_row_sum_hand_values(oracle_lib):
    """PIN (gllm #91, "What changes" / "Testing"): hand-computed WeightedRowSum with
    repeated source rows and a pre-filled dst."""
    g = _golden_wrs()
    out = oracle.weighted_row_sum(g["dst"], g["src"], g["rows"].astype(np.int32), g["weights"])
    assert np.array_equal(out, g["expected"])


def test_weighted_row_sum_special_cases(oracle_lib):
    """PIN: K = 1 with w = 1 is a row add; w = 0 leaves dst unchanged; an
    out-of-range row is rejected (bounds are checked)."""
    rng = np.random.default_rng(5)
    src = rng.standard_normal((7, 5))
    dst = rng.standard_normal((4, 5))
    rows = np.array([[3], [0], [6], [3]], dtype=np.int32)
    out = oracle.weighted_row_sum(dst, src, rows, np.ones((4, 1)))
    assert np.array_equal(out, dst + src[[3, 0, 6, 3]])
    rows2 = rng.integers(0, 7, size=(4, 3)).astype(np.int32)
    assert np.array_equal(oracle.weighted_row_sum(dst, src, rows2, np.zeros((4, 3))), dst)
    with pytest.raises(oracle.OracleError):
        oracle.weighted_row_sum(dst, src, np.array([[7], [0], [0], [0]], dtype=np.int32), np.ones((4, 1)))
    with pytest.raises(oracle.OracleError):
        oracle.weighted_row_sum(dst, src, np.array([[-1], [0], [0], [0]], dtype=np.int32), np.ones((4, 1)))


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def test_route_matches_torch_topk_softmax(oracle_lib):
    """PIN: on tie-free logits, ids equal torch.topk (descending) and the weights
    equal torch.softmax of the picked logits in float64."""
    for name in ("tiny16", "decode32_zipf", "gated2"):
        cfg = synth.WORKLOADS[name]
        logits = synth.draw_logits(name)
        ids, w = oracle.route_topk(logits, cfg["K"])
        tl = torch.from_numpy(logits)
        vals, idx = torch.topk(tl, cfg["K"], dim=1, largest=True, sorted=True)
        assert np.array_equal(ids, idx.numpy().astype(np.int32))
        ref = torch.softmax(vals.to(torch.float64), dim=1).numpy()
        assert np.max(np.abs(w - ref)) < 1e-15
        assert np.max(np.abs(w.sum(1) - 1)) < 1e-15


def test_route_full_softmax_and_ties(oracle_lib):
    """PIN: K = E is a full softmax in descending order; all-equal logits pick
    experts 0..K-1 with weight 1/K (ties go to the lower index)."""
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((5, 6)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 6)
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    assert np.array_equal(ids, order.astype(np.int32))
    full = torch.softmax(torch.from_numpy(logits).to(torch.float64), 1).numpy()
    assert np.max(np.abs(np.take_along_axis(full, order, 1) - w)) < 1e-15
    eq = np.zeros((3, 10), dtype=np.float32)
    ids, w = oracle.route_topk(eq, 4)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (3, 1)))
    assert np.array_equal(w, np.full((3, 4), 0.25))
    # partial ties: the tied pair keeps index order
    lg = np.array([[0.5, 2.0, 0.5, 2.0, -1.0]], dtype=np.float32)
    ids, _ = oracle.route_topk(lg, 4)
    assert ids.tolist() == [[1, 3, 0, 2]]


# ----------------------------------------------------------------------------
# gather
# ----------------------------------------------------------------------------

def _check_gather_invariants(ids, E, offsets, row_token, rows):
    n, K = ids.shape
    R = n * K
    assert offsets[0] == 0 and offsets[E] == R
    assert np.array_equal(np.diff(offsets), np.bincount(ids.ravel(), minlength=E))
    assert np.array_equal(np.sort(rows.ravel()), np.arange(R))
    for t in range(n):
        for j in range(K):
            r = rows[t, j]
            assert row_token[r] == t
            assert offsets[ids[t, j]] <= r < offsets[ids[t, j] + 1]
    for e in range(E):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending tokens inside an expert


def test_gather_invariants(oracle_lib):
    """PIN: offsets are the exclusive scan of the expert counts, rows is a
    permutation of 0..R-1, row_token[rows[t,j]] = t, rows of an expert are in
    ascending token order, and xg[rows[t,j]] == x[t] bit for bit."""
    for name in ("tiny16", "decode32_zipf", "gated2"):
        cfg = synth.WORKLOADS[name]
        ids, _ = oracle.route_topk(synth.draw_logits(name), cfg["K"])
        offsets, row_token, rows = oracle.gather_layout(ids, cfg["E"])
        _check_gather_invariants(ids, cfg["E"], offsets, row_token, rows)
        x = synth.draw_activations(name)
        xg = oracle.gather_copy(x, row_token)
        for t in range(cfg["n"]):
            for j in range(cfg["K"]):
                assert np.array_equal(xg[rows[t, j]].view(np.uint8), x[t].view(np.uint8))


def test_gather_prefill_row_counts(oracle_lib):
    """PIN (gllm #91, "What the profile showed"): at 4314 tokens with 128 experts
    and topK 6 the gather packs 4314 * 6 = 25,884 rows where the dense-masked
    loop ran 4314 * 128 = 552,192; nearly all experts are picked."""
    cfg = synth.WORKLOADS["prefill4314"]
    ids, _ = oracle.route_topk(synth.draw_logits("prefill4314"), cfg["K"])
    offsets, row_token, rows = oracle.gather_layout(ids, cfg["E"])
    assert offsets[-1] == 25884
    assert cfg["n"] * cfg["E"] == 552192
    assert np.count_nonzero(np.diff(offsets)) >= 120
    _check_gather_invariants(ids[:64], cfg["E"], *oracle.gather_layout(ids[:64], cfg["E"]))


def test_gather_rejects_bad_expert_id(oracle_lib):
    with pytest.raises(oracle.OracleError):
        oracle.gather_layout(np.array([[0, 8]], dtype=np.int32), 8)


# ----------------------------------------------------------------------------
# expert FFN and the layer
# ----------------------------------------------------------------------------

def _np_dequant(t, e):
    """Independent decode for the tests: torch's e4m3 cast + E2M1 bit fields."""
    c = t.codes[e]
    code = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.int64)
    code[:, 0::2] = c & 15
    code[:, 1::2] = c >> 4
    e2 = np.vectorize(_e2m1_from_bits)(code).astype(np.float64)
    sc = torch.from_numpy(t.scales[e].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return float(t.globals_[e]) * np.repeat(sc, 16, axis=1) * e2


def _np_ffn(x, wu, wd, act, f):
    u = x @ wu.T
    if act == "swiglu":
        a, b = u[:, :f], u[:, f:]
        h = a / (1 + np.exp(-a)) * b
    else:
        h = np.maximum(u, 0) ** 2
    return h @ wd.T


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_expert_ffn_matches_numpy_matmul(oracle_lib, act):
    """PIN: the oracle FFN over grouped rows equals numpy float64 matmuls on
    independently decoded weights, expert by expert (normwise 1e-13)."""
    E, d, f, n = 5, 64, 48, 23
    up_rows = 2 * f if act == "swiglu" else f
    up = synth.random_nvfp4(21, E, up_rows, d)
    dn = synth.random_nvfp4(22, E, d, f)
    rng = np.random.default_rng(23)
    x = rng.standard_normal((n, d))
    counts = np.array([4, 0, 11, 1, 7])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    got = oracle.expert_ffn(x, offsets, up, dn, f, act)
    ref = np.zeros_like(got)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ref[r0:r1] = _np_ffn(x[r0:r1], _np_dequant(up, e), _np_dequant(dn, e), act, f)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_linear_matches_numpy(oracle_lib):
    """PIN: one grouped NVFP4 projection equals numpy a @ W^T per expert."""
    w = synth.random_bytes_nvfp4(31, 3, 40, 64)
    rng = np.random.default_rng(32)
    a = rng.standard_normal((9, 64))
    offsets = np.array([0, 2, 2, 9], dtype=np.int32)
    got = oracle.linear(a, offsets, w)
    ref = np.zeros_like(got)
    for e in range(3):
        ref[offsets[e]:offsets[e + 1]] = a[offsets[e]:offsets[e + 1]] @ _np_dequant(w, e).T
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_ffn_thread_count_invariance(oracle_lib):
    """Each output element comes from one thread in one order: 1 vs 7 threads
    give identical bits."""
    up = synth.random_nvfp4(41, 3, 64, 64)
    dn = synth.random_nvfp4(42, 3, 64, 64)
    x = np.random.default_rng(43).standard_normal((30, 64))
    off = np.array([0, 10, 25, 30], dtype=np.int32)
    a = oracle.expert_ffn(x, off, up, dn, 64, "relu2", threads=1)
    b = oracle.expert_ffn(x, off, up, dn, 64, "relu2", threads=7)
    assert np.array_equal(a, b)


def test_layer_equals_naive_dense_loop(oracle_lib):
    """PIN (gllm #91, "What the profile showed" / "What changes"): gather +
    per-expert FFN + WeightedRowSum equals running every expert over every token
    with weight zero where the token did not pick it."""
    for name in ("tiny16", "gated2"):
        inp = synth.make_layer(name)
        r = oracle.layer(inp)
        nv = oracle.naive_layer(inp)
        assert np.max(np.abs(r["out"] - nv)) <= 1e-13 * np.max(np.abs(nv))


def test_layer_equals_naive_loop_bitwise_on_dyadic_inputs(oracle_lib):
    """PIN: on inputs whose every product and sum is exact in float64 (small
    dyadic activations, dyadic routing weights), the gather path and the naive
    loop agree bit for bit."""
    inp = synth.make_layer("tiny16")
    rng = np.random.default_rng(51)
    inp.x = (rng.integers(-4, 5, size=inp.x.shape) / 4.0).astype(np.float32)
    ids, _ = oracle.route_topk(inp.logits, inp.K)
    w = np.tile(np.array([0.75, 0.25]), (inp.n, 1))
    r = oracle.layer(inp, routing=(ids, w))
    nv = oracle.naive_layer(inp, routing=(ids, w))
    assert np.array_equal(r["out"], nv)


def test_single_expert_layer_is_a_dense_ffn(oracle_lib):
    """PIN: E = 1, K = 1 (weight 1) reduces to relu(x W_u^T)^2 W_d^T plus the
    shared expert's FFN, checked with numpy float64."""
    inp = synth.make_layer("tiny16", E=1, K=1)
    r = oracle.layer(inp)
    assert np.all(r["weights"] == 1.0)
    x = inp.x.astype(np.float64)
    ref = _np_ffn(x, _np_dequant(inp.up, 0), _np_dequant(inp.down, 0), "relu2", inp.f)
    ref += _np_ffn(x, _np_dequant(inp.shared_up, 0), _np_dequant(inp.shared_down, 0), "relu2", inp.fs)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_bf16_mode_rounds_activations(oracle_lib):
    """The bf16-activation mode equals numpy matmuls on bf16-rounded x with h
    rounded to bf16 (the rounding itself is pinned to torch above)."""
    E, d, f, n = 2, 32, 32, 6
    up = synth.random_nvfp4(61, E, f, d)
    dn = synth.random_nvfp4(62, E, d, f)
    x = np.random.default_rng(63).standard_normal((n, d))
    off = np.array([0, 2, 6], dtype=np.int32)
    got = oracle.expert_ffn(x, off, up, dn, f, "relu2", bf16_act=True)

    ref = np.zeros_like(got)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        xb = np.array([[oracle.round_bf16(v) for v in row] for row in x[r0:r1]])
        u = xb @ _np_dequant(up, e).T
        h = np.array([[oracle.round_bf16(v) for v in row] for row in np.maximum(u, 0) ** 2])
        ref[r0:r1] = h @ _np_dequant(dn, e).T
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


# ----------------------------------------------------------------------------
# activation decode, and the sampled layer
# ----------------------------------------------------------------------------

def test_bf16_bits_decode_matches_torch_on_every_pattern(oracle_lib):
    """PIN: the oracle's bf16 activation decode equals torch's bfloat16 -> float64
    cast on all 65,536 bit patterns (NaNs where torch has NaNs, signed zeros and
    subnormals included); the binary32 decode agrees with it."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127   # exponent all ones, non-zero mantissa, both signs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    g32 = oracle.activations_f32(bits, "bf16").astype(np.float64)
    assert np.array_equal(np.isnan(g32), nan)
    assert np.array_equal(g32[~nan], ref[~nan])


@pytest.mark.parametrize("name, ov", [("tiny16", {}), ("gated2", {}),
                                      ("decode1", dict(n=3, E=16, seed=71))])
def test_layer_sampled_equals_layer(oracle_lib, name, ov):
    """The sampled layer (the reference for the largest workload, where the whole
    layer is too slow on a CPU) gives the full layer's rows bit for bit, in
    both the exact and the bf16-activation mode, for any token subset and
    order."""
    inp = synth.make_layer(name, **ov)
    full = oracle.layer(inp)
    ids, w = full["ids"], full["weights"]
    toks = list(range(inp.n))[::-1]
    got = oracle.layer_sampled(inp, toks, ids, w)
    assert np.array_equal(got, full["out"][toks])
    sub = toks[: max(1, inp.n // 2)]
    assert np.array_equal(oracle.layer_sampled(inp, sub, ids, w), full["out"][sub])
    bf = oracle.layer(inp, bf16_act=True)["out"]
    assert np.array_equal(oracle.layer_sampled(inp, toks, ids, w, bf16_act_of_expert=lambda e: True),
                          bf[toks])


# ----------------------------------------------------------------------------
# the binary32 fixed-order arithmetic
# ----------------------------------------------------------------------------

from fractions import Fraction  # noqa: E402

_F32_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)


def _round_f32(q: Fraction) -> float:
    """Exact rational -> nearest binary32, ties to even (written from the
    IEEE 754 definition: 24 significant bits, quantum 2^-149 at the bottom)."""
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    qe = max(e - 23, -149)
    scaled = a / Fraction(2) ** qe
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    v = Fraction(m) * Fraction(2) ** qe
    out = float("inf") if v > _F32_MAX else float(v)
    return -out if neg else out


def _fmaf(a, b, c) -> float:
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _mul32(a, b) -> float:
    return _round_f32(Fraction(float(a)) * Fraction(float(b)))


def _add32(a, b) -> float:
    return _round_f32(Fraction(float(a)) + Fraction(float(b)))


def test_round_f32_helper_matches_numpy():
    """The test's own rational rounding agrees with numpy's float64 -> float32
    cast wherever that cast is a single rounding (every double input)."""
    rng = np.random.default_rng(81)
    v = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-40, 38, 500),
                        [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150]])
    for x in v:
        assert _round_f32(Fraction(float(x))) == float(np.float32(x))


def test_weighted_row_sum_f32_is_a_fixed_order_fma_chain(oracle_lib):
    """PIN: the binary32 WeightedRowSum equals a chain of correctly rounded fmaf
    over j from a zero accumulator followed by one rounded add onto dst,
    evaluated here with exact rationals.  The first row is built so that an
    unfused multiply-add, or the j-sum in the other order, gives another
    value: fmaf(1, -1, 0) = -1, then fmaf(1+2^-12, 1+2^-12, -1) = 2^-11 + 2^-24
    exactly, where rounding the product first loses the 2^-24."""
    t = 1.0 + 2.0 ** -12
    src = np.array([[-1.0, 3.0], [t, 0.5], [0.1, -7.25]], dtype=np.float32)
    rows = np.array([[0, 1], [2, 2], [1, 0]], dtype=np.int32)
    w = np.array([[1.0, t], [0.3, -0.7], [1e-3, 2.5]], dtype=np.float32)
    dst = np.array([[0.0, 1.0], [5.0, -5.0], [1e8, 3.0]], dtype=np.float32)
    got = oracle.weighted_row_sum_f32(dst, src, rows, w)
    assert got[0, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)
    ref = np.zeros_like(dst)
    for i in range(3):
        for c in range(2):
            acc = 0.0
            for j in range(2):
                acc = _fmaf(w[i, j], src[rows[i, j], c], acc)
            ref[i, c] = _add32(dst[i, c], acc)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the hand fixture (every value exact in binary32) and a random case
    g = _golden_wrs()
    out = oracle.weighted_row_sum_f32(g["dst"], g["src"], g["rows"].astype(np.int32), g["weights"])
    assert np.array_equal(out, g["expected"].astype(np.float32))
    rng = np.random.default_rng(82)
    src = rng.standard_normal((5, 3)).astype(np.float32)
    rows = rng.integers(0, 5, size=(4, 6)).astype(np.int32)
    w = rng.standard_normal((4, 6)).astype(np.float32)
    dst = rng.standard_normal((4, 3)).astype(np.float32)
    got = oracle.weighted_row_sum_f32(dst, src, rows, w)
    for i in range(4):
        for c in range(3):
            acc = 0.0
            for j in range(6):
                acc = _fmaf(w[i, j], src[rows[i, j], c], acc)
            assert got[i, c] == np.float32(_add32(dst[i, c], acc))
    with pytest.raises(oracle.OracleError):
        oracle.weighted_row_sum_f32(dst, src, np.full((4, 6), 5, dtype=np.int32), w)


def _dot_chain(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc = _fmaf(x, y, acc)
    return acc


def test_linear_and_ffn_f32_are_fixed_order_fma_chains(oracle_lib):
    """PIN: the binary32 projection is global * (fmaf chain over k ascending)
    on weights decoded independently (torch's e4m3 cast, E2M1 bit fields), and
    the binary32 FFN rounds relu^2 as max(u, 0) * max(u, 0): checked bit for bit
    with exact rationals on a small case of two experts."""
    d, f = 32, 16
    up = synth.random_nvfp4(83, 2, f, d)
    dn = synth.random_nvfp4(84, 2, d, f)
    x = np.random.default_rng(85).standard_normal((3, d)).astype(np.float32)
    off = np.array([0, 1, 3], dtype=np.int32)
    lin = oracle.linear_f32(x, off, up)
    ffn = oracle.expert_ffn_f32(x, off, up, dn, f, "relu2")
    for e in range(2):
        wu = _np_dequant(up, e) / float(up.globals_[e])
        wd = _np_dequant(dn, e) / float(dn.globals_[e])
        gu, gd = float(up.globals_[e]), float(dn.globals_[e])
        for r in range(off[e], off[e + 1]):
            u = [_mul32(gu, _dot_chain(x[r], wu[n])) for n in range(f)]
            assert np.array_equal(lin[r], np.array(u, dtype=np.float32))
            h = [_mul32(max(v, 0.0), max(v, 0.0)) for v in u]
            y = [_mul32(gd, _dot_chain(h, wd[c])) for c in range(d)]
            assert np.array_equal(ffn[r], np.array(y, dtype=np.float32))


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_ffn_f32_within_its_error_bound_of_the_exact_values(oracle_lib, act):
    """The binary32 FFN stays within the forward error bound of a k-term fmaf
    chain of the exact (double) FFN: per projection |err| <= (k+2) * 2^-24 *
    (sum_k |a_k * b_k| * |g|), propagated through the activation; checked
    here in the normwise form the layer tolerance uses (<= 1e-5)."""
    E, d, f, n = 3, 256, 128, 17
    up_rows = 2 * f if act == "swiglu" else f
    up = synth.random_nvfp4(86, E, up_rows, d)
    dn = synth.random_nvfp4(87, E, d, f)
    x = np.random.default_rng(88).standard_normal((n, d)).astype(np.float32)
    off = np.array([0, 5, 5, n], dtype=np.int32)
    got = oracle.expert_ffn_f32(x, off, up, dn, f, act).astype(np.float64)
    ref = oracle.expert_ffn(x.astype(np.float64), off, up, dn, f, act)
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert 0 < err <= 1e-5
    lin = oracle.linear_f32(x, off, up).astype(np.float64)
    lref = oracle.linear(x.astype(np.float64), off, up)
    bound = (d + 2) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(
        np.concatenate([_np_dequant(up, 0)]).T))
    assert np.all(np.abs(lin[:5] - lref[:5]) <= bound[:5])


def test_layer_f32_close_to_exact_layer(oracle_lib):
    """The binary32 layer (fixed-order fmaf chains, binary32 routing weights)
    agrees with the exact layer to the decode path's tolerance on the small
    workload and on a gated shape."""
    for name, ov in (("tiny16", {}), ("gated2", dict(n=3, E=16, seed=89))):
        inp = synth.make_layer(name, **ov)
        a = oracle.layer(inp, arith="f32")
        b = oracle.layer(inp)
        assert a["out"].dtype == np.float32
        err = np.max(np.abs(a["out"].astype(np.float64) - b["out"])) / np.max(np.abs(b["out"]))
        assert err <= 1e-5


# ----------------------------------------------------------------------------
# the router GEMM before routing
# ----------------------------------------------------------------------------

def test_router_logits_match_numpy_on_torch_decoded_weights(oracle_lib):
    """PIN: the oracle's router logits equal numpy float64 x @ W_r^T with W_r
    decoded by torch's bfloat16 cast (normwise 1e-13; another summation
    order), for bf16 and fp32 activations."""
    for name, ov in (("tiny16", {}), ("gated2", dict(n=5, E=32, seed=91))):
        cfg = dict(synth.WORKLOADS[name], **ov)
        wr = synth.draw_router(name, **ov)
        assert wr.shape == (cfg["E"], cfg["d"]) and wr.dtype == np.uint16
        x = synth.draw_activations(name, **ov)
        x64 = oracle.activations_f64(x, cfg["x_dtype"])
        wt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        ref = x64 @ wt.T
        got = oracle.router_logits(x64, wr)
        assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_router_logits_special_cases(oracle_lib):
    """PIN: one-hot router rows pick columns of x exactly; a zero router gives
    zero logits, i.e. all-tied routing to experts 0..K-1 with weights 1/K."""
    rng = np.random.default_rng(92)
    n, d, E = 6, 64, 8
    x = rng.standard_normal((n, d))
    onehot = np.zeros((E, d), dtype=np.float32)
    cols = rng.permutation(d)[:E]
    onehot[np.arange(E), cols] = 1.0
    got = oracle.router_logits(x, synth.f32_to_bf16_bits(onehot))
    assert np.array_equal(got, x[:, cols])
    ids, w, lg = oracle.router_topk(x.astype(np.float32), "f32", np.zeros((E, d), dtype=np.uint16), 3)
    assert np.all(lg == 0)
    assert np.array_equal(ids, np.tile(np.arange(3, dtype=np.int32), (n, 1)))
    assert np.allclose(w, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_router_topk_matches_torch_on_the_workload_router(oracle_lib):
    """PIN: routing the router's logits equals torch.topk + softmax on numpy's
    float64 logits rounded to binary32 (tie-free at these sizes); the logits
    of a d = 2688 layer are about N(0, 1), like the workloads' drawn logits."""
    name, ov = "decode1", dict(n=24, seed=93)
    wr = synth.draw_router(name, **ov)
    x = synth.draw_activations(name, **ov)
    ids, w, lg = oracle.router_topk(x, "bf16", wr, 6)
    assert 0.8 < float(np.std(lg)) < 1.3
    wt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref = (oracle.bf16_bits_to_f64(x) @ wt.T).astype(np.float32)
    vals, idx = torch.topk(torch.from_numpy(ref), 6, dim=1)
    assert np.array_equal(ids, idx.numpy().astype(np.int32))
    assert np.max(np.abs(w - torch.softmax(vals.to(torch.float64), 1).numpy())) < 1e-15


def test_router_stream_leaves_the_other_streams_unchanged():
    """Adding the router's seed stream at the end keeps every earlier stream:
    a SeedSequence child depends on its index only, not on how many are spawned."""
    a = np.random.SeedSequence(2).spawn(4 + 2 * 128)
    b = np.random.SeedSequence(2).spawn(5 + 2 * 128)
    for i in (0, 1, 2, 257, 259):
        assert np.array_equal(np.random.default_rng(a[i]).integers(0, 2 ** 31, 4),
                              np.random.default_rng(b[i]).integers(0, 2 ** 31, 4))
