"""moe_layer_forward_noalloc (the layer on the library's own static device
scratch, for callers that cannot allocate) against moe_layer_forward with a
caller-allocated workspace: the same kernels, so the same bits."""
import numpy as np
import pytest
import torch

from conftest import cached_layer

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    from bit_block_scaled_topk_amd import ops as _ops
    return _ops


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def _pair(ops, layer, x, lg):
    """(no-alloc output, output of moe_layer_forward with the layer's workspace)."""
    n = x.shape[0]
    d = layer.desc(None, n)
    out_na = torch.full((n, layer.d), float("nan"), device=DEV)
    ops.moe_layer_forward_noalloc(d, x, lg, out_na)
    out_ws = torch.full((n, layer.d), float("nan"), device=DEV)
    ops.moe_layer_forward(d, x, lg, out_ws, layer.layer_ws)
    torch.cuda.synchronize()
    return out_na, out_ws


@pytest.mark.parametrize("single", [False, True])
def test_noalloc_matches_the_workspace_entry_point_twice(ops, single):
    """Two calls in a row, the second with fewer tokens (per-step launches:
    32 then 5 tokens of the skewed-router decode layer; single launch: 2 then
    1 tokens), each bit for bit the workspace entry point's output; then a
    repeat of the first size, since the array keeps the last call's data."""
    inp = cached_layer("decode32_zipf")
    layer = ops.MoELayer(inp, single_launch=single)
    x, lg = dev(inp.x), dev(inp.logits)
    sizes = [2, 1, 2] if single else [32, 5, 32]
    for m in sizes:
        print(f"no-alloc call: {m} tokens, single launch {single}", flush=True)
        a, b = _pair(ops, layer, x[:m], lg[:m])
        assert not torch.isnan(a).any()
        assert torch.equal(a, b), f"{m} tokens: the no-alloc output differs"
    if single:
        assert int(layer.views()["wait_error"].cpu()[0]) == 0


def test_noalloc_refuses_a_layer_beyond_its_scratch(ops):
    """The 4314-token layer needs more than the static array holds: refused
    before anything runs, nothing written."""
    inp = cached_layer("decode32_zipf")
    layer = ops.MoELayer(inp)
    n = 4314
    d = layer.desc(None, n)
    assert ops.moe_layer_workspace_size(d) > ops.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n, inp.d), dtype=torch.int16, device=DEV)
    lg = torch.zeros((n, inp.E), dtype=torch.float32, device=DEV)
    out = torch.full((n, inp.d), 3.0, device=DEV)
    with pytest.raises(ops.MoeError) as ei:
        ops.moe_layer_forward_noalloc(d, x, lg, out)
    assert ei.value.status == ops.MOE_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
