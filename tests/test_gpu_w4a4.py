"""GPU parity of the W4A4 kept tier (MXFP4 kept tier with MXFP4 activations, NF3 tail
W4A16) through the C ABI: the activation quantiser bit for bit against the oracle's
OCP MX conversion, and the layer output against the oracle's W4A4 forward to the
layer tolerance, on tiny layers at every M and tile class, on a layer whose K is a
multiple of 512, and on the GLM-class MXFP4 layer at M = 512 (probed tokens)."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as OL
from hmoe_testlib import check_output, make_layer, run_forward, scratch_for, tiny_packed, to_dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_moe_amd as m
    m.load_library()
    return m


def test_activation_quantiser_bit_exact(hm):
    torch = torch_mod()
    rng = np.random.default_rng(41)
    a = (rng.standard_normal((64, 512)) * np.exp(rng.standard_normal((64, 1)) * 4)).astype(np.float32)
    a[0, :32] = 0.0
    a[1, :32] = np.float32(2.0 ** -130)
    a[2, :32] = np.float32(3.0e38)
    a[3, :16] = np.array([4, 1, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, 6.5, -7, 0.125, 3],
                         np.float32)
    a[4, :] = -0.0
    q_ref, s_ref = F.mxfp4_quantize(a)
    x = to_dev(a)
    q = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((64, 16), dtype=torch.uint8, device="cuda")
    hm.moe_quantize_mxfp4(x, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("M", [1, 4, 8, 9, 37, 200])
@pytest.mark.parametrize("block_m", [16, 64])
def test_w4a4_tiny_layer(hm, M, block_m):
    packed, w = tiny_packed("mxfp4", "prefix")
    layer = make_layer(packed, 256, block_m, 0, hm.ACT_MXFP4)
    wts = hm.DeviceWeights(packed)
    x = synth.activations_bf16(w, M)
    lg = synth.router_logits(w, M)
    y, s = run_forward(layer, wts, x, lg)
    ref = OL.forward(packed, x, lg, act_format="mxfp4")["y"]
    check_output(y, ref, f"W4A4 tiny M={M} bm={block_m}")
    # the bar separates the formats: where the kept tier is used, the W4A16 result is
    # far outside it (the NF3 tail is W4A16 in both)
    tier, _ = OL.tier_map(packed["bit_map"], packed["E"])
    if np.any(tier[OL.route(lg, packed["top_k"])[0]] == OL.KEPT):
        w16 = OL.forward(packed, x, lg)["y"]
        assert np.abs(w16 - ref).max() > 0.1 * np.sqrt(np.mean(ref ** 2))
    y2, _ = run_forward(layer, wts, x, lg, s)
    assert np.array_equal(y, y2), "W4A4 forward not bitwise reproducible"


@pytest.mark.parametrize("block_m", [32, 128])
def test_w4a4_tile_classes_k512(hm, block_m):
    """E = 16 (8 MXFP4 kept, 8 NF3), H = 1024, I = 512, top-4, slot counts across every
    block boundary in both tiers; every output checked."""
    counts = [16, 17, 32, 33, 64, 65, 128, 129, 129, 128, 65, 64, 33, 32, 17, 20]
    E, k = 16, 4
    w = synth.Workload("w4a4k", E, 1024, 512, k, 256, "mxfp4", 8, "prefix", seed=9)
    packed = OL.quantize_layer(w.E, w.H, w.I, k, synth.bit_map(w), "mxfp4",
                               lambda e: synth.master_weights(w, e))
    slots = np.repeat(np.arange(E), counts)
    M = slots.size // k
    rng = np.random.default_rng([17, block_m])
    lg = (rng.standard_normal((M, E)) * 0.1 - 4.0).astype(np.float32)
    t = np.arange(M)
    for r in range(k):
        lg[t, slots[r * M:(r + 1) * M]] = (3.0 - r + rng.standard_normal(M) * 0.05).astype(np.float32)
    assert np.array_equal(np.bincount(OL.route(lg, k)[0].ravel(), minlength=E), counts)
    layer = make_layer(packed, M, block_m, 0, hm.ACT_MXFP4)
    wts = hm.DeviceWeights(packed)
    x = synth.activations_bf16(w, M)
    y, _ = run_forward(layer, wts, x, lg)
    check_output(y, OL.forward(packed, x, lg, act_format="mxfp4")["y"], f"W4A4 K512 bm={block_m}")


def test_w4a4_glm_mxfp4_m512_probed(hm):
    from test_gpu_layer import probe_tokens
    w = synth.glm_mxfp4(512)
    packed = synth.packed_layer(w)
    wts = hm.DeviceWeights(packed)
    layer = make_layer(packed, w.M, 0, 0, hm.ACT_MXFP4)
    x = synth.activations_bf16(w, w.M)
    lg = synth.router_logits(w, w.M)
    y, _ = run_forward(layer, wts, x, lg)
    ids, _ = OL.route(lg, w.top_k)
    tier, _ = OL.tier_map(packed["bit_map"], w.E)
    tokens = probe_tokens(ids, tier, hm.moe_layer_query(layer)["block_m"], 64, 3)
    ref = OL.forward(packed, x, lg, tokens=tokens, threads=16, act_format="mxfp4")
    check_output(y[ref["tokens"]], ref["y"], f"W4A4 GLM MXFP4 M=512 ({len(tokens)} tokens)")
    del wts
    torch_mod().cuda.empty_cache()
