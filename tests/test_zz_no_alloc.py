"""moe_forward_noalloc (the library's fixed device scratch, no workspace
argument) against moe_forward with a caller workspace, through the C ABI."""
import pytest
import torch

import sparse_moe_routed_amd as moe
from sparse_moe_routed_amd import synth

pytestmark = pytest.mark.gpu


def _largest_t(ld, fmt):
    # the largest batch whose workspace fits the fixed scratch
    T = 1
    while moe.workspace_size(ld, fmt, T + 1) <= moe.NOALLOC_SCRATCH_BYTES:
        T += 1
    return T


@pytest.fixture(scope="module")
def layer():
    ld = moe.LayerDims()
    w_r, b = synth.make_router(0)
    up, down = synth.make_experts(0)
    router = moe.pack_router(w_r.cuda(), b.cuda(), ld)
    return ld, router, up.cuda(), down.cuda()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_noalloc_equals_forward(layer, fmt):
    ld, router, up, down = layer
    bank = moe.quantize_experts(up, down, fmt, ld)
    t_max = _largest_t(ld, fmt)
    assert t_max >= 64
    print(f"{fmt}: largest batch for the fixed scratch {t_max}", flush=True)
    # two calls in a row, the second smaller; then the largest batch, then one token
    for T, seed in ((64, 1), (5, 2), (t_max, 3), (1, 4)):
        x = synth.make_tokens_device(T, seed=8000 + seed)
        ids, g = moe.route(x, router, ld)
        y_ref = moe.forward(x, ids, g, bank, ld)
        y = moe.forward_noalloc(x, ids, g, bank, ld)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (fmt, T)
    yb = moe.forward_noalloc(x, ids, g, bank, ld, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(yb, y_ref.to(torch.bfloat16))
    # one token past the scratch: rejected before any launch
    T = t_max + 1
    x = synth.make_tokens_device(T, seed=8100)
    ids, g = moe.route(x, router, ld)
    with pytest.raises(moe.MoeError) as err:
        moe.forward_noalloc(x, ids, g, bank, ld)
    assert err.value.status == moe.EWORKSPACE
    torch.cuda.synchronize()
