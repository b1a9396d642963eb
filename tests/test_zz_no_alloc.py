"""hybrid_moe_forward_static (the forward that allocates nothing, scratch from the
library's per-GPU static array) against hybrid_moe_forward on a caller scratch, through
the C ABI: two calls in a row on the same layer, the second with a smaller batch, in both
the prefill and the decode path; outputs must be bit-identical (same kernels, fixed-order
sums)."""
import numpy as np
import pytest

import synth
from hmoe_testlib import make_layer, scratch_for, to_dev, to_dev_bits, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_moe_amd as m
    m.load_library()
    return m


def test_static_forward_matches_caller_scratch(hm):
    torch = torch_mod()
    w = synth.qwen_decode(8)
    packed = synth.packed_layer(w)
    wts = hm.DeviceWeights(packed)
    layer = make_layer(packed, 64, 32)
    assert hm.moe_scratch_bytes(layer) <= (64 << 20)
    scratch = scratch_for(layer)
    for M in (48, 5):                       # prefill, then a smaller decode batch
        x = to_dev_bits(synth.activations_bf16(w, M))
        lg = to_dev(synth.router_logits(w, M))
        y_ref = torch.empty((M, w.H), dtype=torch.int16, device="cuda")
        y = torch.full((M, w.H), 0x7FC0, dtype=torch.int16, device="cuda")
        hm.hybrid_moe_forward(layer, wts, x, lg, y_ref, scratch)
        hm.hybrid_moe_forward_static(layer, wts, x, lg, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"M={M}: static-scratch forward differs"


def test_static_single_launch_decode_after_another_layer(hm):
    """The static array keeps the last call's contents: a prefill forward of one layer
    fills it, then a single-launch decode layer (whose counters must start at zero, and
    sit where the first layer kept other data) runs through it twice. Its outputs must
    equal the same layer's forward on a zeroed caller scratch, bit for bit."""
    torch = torch_mod()
    w = synth.qwen_decode(8)
    packed = synth.packed_layer(w)
    wts = hm.DeviceWeights(packed)
    big = make_layer(packed, 64, 32)
    fused = make_layer(packed, 8, 0, decode_launch=hm.DECODE_SINGLE_LAUNCH)
    if not hm.moe_layer_query(fused)["single_launch_available"]:
        pytest.skip("no single-launch tiling for this shape")
    scratch = scratch_for(fused)
    M0 = 48
    x0 = to_dev_bits(synth.activations_bf16(w, M0))
    lg0 = to_dev(synth.router_logits(w, M0))
    y0 = torch.empty((M0, w.H), dtype=torch.int16, device="cuda")
    hm.hybrid_moe_forward_static(big, wts, x0, lg0, y0)     # leaves prefill data in the array
    for M in (8, 5):
        x = to_dev_bits(synth.activations_bf16(w, M))
        lg = to_dev(synth.router_logits(w, M))
        y_ref = torch.empty((M, w.H), dtype=torch.int16, device="cuda")
        y = torch.full((M, w.H), 0x7FC0, dtype=torch.int16, device="cuda")
        hm.hybrid_moe_forward(fused, wts, x, lg, y_ref, scratch)
        hm.hybrid_moe_forward_static(fused, wts, x, lg, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"M={M}: static single-launch decode differs"
    assert int(hm.moe_decode_view(fused, scratch)["sync_timeouts"][0]) == 0
