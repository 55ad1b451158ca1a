"""Host-side checks of bench.py (CPU only): its refusal of several GPUs and
the algorithmic accounting behind its roofline figures, against values worked
out by hand from the workload shapes."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    """--gpus N with N > 1 exits non-zero with a message (one GPU only)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def _shape(**kw):
    return types.SimpleNamespace(**kw)


def test_prefill_flops_count_real_rows_only(bench):
    """2 flops per multiply-add over the real rows: prefill4314 routes
    4314 x 6 = 25,884 rows through d 2688 -> f 1856 -> d 2688 and 4314 rows
    through the shared d 2688 -> 3712 -> 2688, i.e. 688,711,532,544 flops."""
    inp = _shape(n=4314, K=6, d=2688, f=1856, fs=3712, act="relu2")
    fl = bench.layer_ffn_flops(inp)
    routed = 2 * 25884 * 2688 * 1856
    shared = 2 * 4314 * 2688 * 3712
    assert fl["up"] == routed + shared and fl["down"] == routed + shared
    assert fl["total"] == 688_711_532_544
    # SwiGLU: the up projection carries the gate rows too
    g = bench.layer_ffn_flops(_shape(n=2, K=8, d=2048, f=1024, fs=0, act="swiglu"))
    assert g["up"] == 2 * 16 * 2048 * 2048 and g["down"] == 2 * 16 * 1024 * 2048


def _nvfp4(n_experts, rows, cols):
    """A stand-in with the byte counts of an NVFP4 tensor: e2m1 codes (half a
    byte per weight), one e4m3 scale per 16 weights, one fp32 global per
    expert."""
    codes = types.SimpleNamespace(nbytes=n_experts * rows * cols // 2)
    scales = types.SimpleNamespace(nbytes=n_experts * rows * cols // 16)
    globals_ = types.SimpleNamespace(nbytes=n_experts * 4)
    return types.SimpleNamespace(codes=codes, scales=scales, globals_=globals_, n_experts=n_experts)


def test_decode_step_bytes_decode1(bench):
    """decode1: 6 picked experts x (up + down) at 2,806,276 bytes each plus the
    shared expert's 2 x 5,612,548, plus x (bf16), the logits and the output:
    44,917,048 bytes per step."""
    inp = _shape(n=1, d=2688, E=128, f=1856, fs=3712, x_dtype="bf16",
                 up=_nvfp4(128, 1856, 2688), down=_nvfp4(128, 2688, 1856),
                 shared_up=_nvfp4(1, 3712, 2688), shared_down=_nvfp4(1, 2688, 3712))
    assert bench.per_expert_bytes(inp.up) == 1856 * 2688 * 9 // 16 + 4 == 2_806_276
    ids = np.array([[3, 17, 40, 41, 99, 127]])
    b = bench.decode_step_bytes(inp, ids)
    assert b["distinct_experts"] == 6
    assert b["weights"] == 6 * 2 * 2_806_276 + 2 * 5_612_548
    assert b["activations"] == 2688 * 2 + 128 * 4 + 2688 * 4 == 16_640
    assert b["total"] == 44_917_048
    # an expert picked twice is read once
    assert bench.decode_step_bytes(inp, np.array([[3, 3, 40, 41, 99, 127]]))["distinct_experts"] == 5
