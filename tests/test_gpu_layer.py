"""GPU parity of the whole layer (hybrid_moe_forward through the C ABI) against
the oracle on the same seeded inputs, to the layer tolerance: max |err| <=
2e-2 * RMS and at most 1e-3 of the elements above 1e-2 * RMS. Covers the decode
path (M <= 8) and the prefill path (M > 8) in both kept formats and the uniform
NVFP4 control, the Qwen-shaped decode sweep at full size, determinism, HIP graph
replay, and the GLM-class layer at full size on sampled tokens."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as OL
from hmoe_testlib import (check_output, make_layer, run_forward, scratch_for, tiny_packed,
                          to_dev, to_dev_bits, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_moe_amd as m
    m.load_library()
    return m


# ---------------------------------------------------------------- tiny layer

@pytest.mark.parametrize("fmt,bitmap", [("nvfp4", "prefix"), ("mxfp4", "prefix"), ("nvfp4", None)])
@pytest.mark.parametrize("M", [1, 4, 8, 9, 37, 200])
@pytest.mark.parametrize("block_m", [16, 64])
def test_tiny_layer(hm, fmt, bitmap, M, block_m):
    packed, w = tiny_packed(fmt, bitmap)
    layer = make_layer(packed, 256, block_m)
    wts = hm.DeviceWeights(packed)
    x = synth.activations_bf16(w, M)
    lg = synth.router_logits(w, M)
    y, _ = run_forward(layer, wts, x, lg)
    ref = OL.forward(packed, x, lg)
    check_output(y, ref["y"], f"tiny {fmt} {bitmap} M={M} bm={block_m}")


# Expert slot counts on both sides of every prefill tile-class boundary (the GEMM
# runs an align block's real slots as a 16-, 32-, 64- or block_m-row tile), in both
# tiers: token t takes experts order[t] and order[t + M] of the sorted slot list, so
# each expert ends up with exactly its count.
@pytest.mark.parametrize("fmt,counts", [
    ("nvfp4", [16, 17, 32, 33, 64, 65, 128, 129]),
    ("mxfp4", [129, 128, 65, 64, 33, 32, 17, 16])])
@pytest.mark.parametrize("block_m", [64, 128])
def test_prefill_tile_class_boundaries(hm, fmt, counts, block_m):
    packed, w = tiny_packed(fmt, "prefix")
    slots = np.repeat(np.arange(8), counts)
    M = slots.size // 2
    assert slots.size == 2 * M and max(counts) < M
    rng = np.random.default_rng([11, block_m])
    lg = (rng.standard_normal((M, 8)) * 0.1 - 2.0).astype(np.float32)
    t = np.arange(M)
    lg[t, slots[:M]] = (3.0 + rng.standard_normal(M) * 0.1).astype(np.float32)
    lg[t, slots[M:]] = (2.0 + rng.standard_normal(M) * 0.1).astype(np.float32)
    ids, _ = OL.route(lg, 2)
    assert np.array_equal(np.bincount(np.asarray(ids).ravel(), minlength=8), counts)
    layer = make_layer(packed, 256, block_m)
    wts = hm.DeviceWeights(packed)
    x = synth.activations_bf16(w, M)
    y, _ = run_forward(layer, wts, x, lg)
    check_output(y, OL.forward(packed, x, lg)["y"], f"tile classes {fmt} bm={block_m}")


def test_tiny_layer_wider_topk_and_experts(hm):
    packed, w = tiny_packed("nvfp4", "prefix", E=16, H=384, I=256, k=4, seed=3)
    # experts 0-3 kept; make the map irregular
    for M in (2, 8, 50):
        layer = make_layer(packed, 64, 32)
        wts = hm.DeviceWeights(packed)
        x = synth.activations_bf16(w, M)
        lg = synth.router_logits(w, M)
        y, _ = run_forward(layer, wts, x, lg)
        check_output(y, OL.forward(packed, x, lg)["y"], f"E16 k4 M={M}")


@pytest.mark.parametrize("kept,bit_map", [("nvfp4", "prefix"), ("mxfp4", "prefix"),
                                           ("nvfp4", None)])
def test_decode_shared_experts(hm, kept, bit_map):
    """Decode with K a multiple of 512 (the matrix-core W13 path) in every kept format:
    ordinary routing at M = 1, 3, 8, and routing forced onto the same four experts for
    every token (each expert then serves all M = 8 tokens at once)."""
    packed, w = tiny_packed(kept, bit_map, E=16, H=512, I=256, k=4, seed=5)
    wts = hm.DeviceWeights(packed)
    layer = make_layer(packed, 8)
    # M = 1 has only 512 outputs, too few for the 1e-3 fraction bar on its own: the
    # fraction is taken over the three batches together, the max bar per batch
    ys, refs = [], []
    for M in (1, 3, 8):
        x = synth.activations_bf16(w, M)
        lg = synth.router_logits(w, M)
        y, _ = run_forward(layer, wts, x, lg)
        ys.append(y.ravel())
        refs.append(OL.forward(packed, x, lg)["y"].ravel())
        yv = F.bf16_value(y.ravel()).astype(np.float64)
        assert np.abs(yv - refs[-1]).max() <= 2e-2 * np.sqrt(np.mean(refs[-1] ** 2)), M
    check_output(np.concatenate(ys), np.concatenate(refs), f"{kept} {bit_map} M=1,3,8")
    x = synth.activations_bf16(w, 8)
    lg = synth.router_logits(w, 8)
    lg[:, [2, 5, 9, 12]] += 20.0  # experts 2 (kept) and 5, 9, 12 (tail) take every token
    y, _ = run_forward(layer, wts, x, lg)
    assert set(OL.route(lg, 4)[0].ravel().tolist()) == {2, 5, 9, 12}
    check_output(y, OL.forward(packed, x, lg)["y"], f"{kept} {bit_map} shared experts")


# ---------------------------------------------------------------- Qwen-shaped decode, full size

@pytest.fixture(scope="module")
def qwen(hm):
    w = synth.qwen_decode(8)
    packed = synth.packed_layer(w)
    return w, packed, hm.DeviceWeights(packed)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_qwen_decode_full(hm, qwen, M):
    w, packed, wts = qwen
    layer = make_layer(packed, 8)
    x = synth.activations_bf16(w, M)
    lg = synth.router_logits(w, M)
    y, _ = run_forward(layer, wts, x, lg)
    check_output(y, OL.forward(packed, x, lg)["y"], f"qwen decode M={M}")


def test_qwen_prefill_small(hm, qwen):
    w, packed, wts = qwen
    M = 48
    layer = make_layer(packed, M, 32)
    x = synth.activations_bf16(w, M)
    lg = synth.router_logits(w, M)
    y, _ = run_forward(layer, wts, x, lg)
    check_output(y, OL.forward(packed, x, lg)["y"], "qwen prefill M=48")


def test_determinism_and_m0(hm, qwen):
    torch = torch_mod()
    w, packed, wts = qwen
    for M in (8, 40):
        layer = make_layer(packed, 64, 32)
        x = synth.activations_bf16(w, M)
        lg = synth.router_logits(w, M)
        y1, s = run_forward(layer, wts, x, lg)
        y2, _ = run_forward(layer, wts, x, lg, s)
        assert np.array_equal(y1, y2), f"M={M} not bitwise reproducible"
    y0 = torch.full((0, w.H), 7, dtype=torch.int16, device="cuda")
    hm.hybrid_moe_forward(layer, wts, y0, to_dev(np.zeros((0, w.E), np.float32)), y0,
                          scratch_for(layer))


def test_hip_graph_replay(hm, qwen):
    torch = torch_mod()
    w, packed, wts = qwen
    for M in (4, 24):
        layer = make_layer(packed, 32, 32)
        scratch = scratch_for(layer)
        x = to_dev_bits(synth.activations_bf16(w, M))
        lg = to_dev(synth.router_logits(w, M))
        y_eager = torch.empty((M, w.H), dtype=torch.int16, device="cuda")
        hm.hybrid_moe_forward(layer, wts, x, lg, y_eager, scratch)
        torch.cuda.synchronize()
        y = torch.zeros((M, w.H), dtype=torch.int16, device="cuda")
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                hm.hybrid_moe_forward(layer, wts, x, lg, y, scratch)
        torch.cuda.synchronize()
        for rep in range(4):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_eager), f"M={M} replay {rep} differs from eager"
            # eager work between replays
            hm.hybrid_moe_forward(layer, wts, x, lg, y_eager, scratch)
            torch.cuda.synchronize()


# ---------------------------------------------------------------- GLM-class, full size

def _glm_case(hm, workload, tokens):
    w = workload
    packed = synth.packed_layer(w)
    wts = hm.DeviceWeights(packed)
    layer = make_layer(packed, w.M, 32)
    x = synth.activations_bf16(w, w.M)
    lg = synth.router_logits(w, w.M)
    y, scratch = run_forward(layer, wts, x, lg)
    ref = OL.forward(packed, x, lg, tokens=tokens)
    check_output(y[tokens], ref["y"], w.name)
    tids, _ = hm.moe_topk_view(layer, scratch, w.M)
    assert np.array_equal(tids.cpu().numpy(), ref["ids"]), f"{w.name}: top-k ids"
    del wts
    torch_mod().cuda.empty_cache()


def test_glm_decode_m8(hm):
    _glm_case(hm, synth.glm_decode(8), [0, 5])


def test_glm_prefill_m4096_sampled(hm):
    _glm_case(hm, synth.glm_prefill(4096), [0, 1234, 4095])


def test_glm_mxfp4_m512_and_uniform_control(hm):
    _glm_case(hm, synth.glm_mxfp4(512), [0, 511])
    _glm_case(hm, synth.glm_uniform(512), [7])


# ---------------------------------------------------------------- maximum sizes, empty tier

@pytest.mark.parametrize("rule,n_kept", [("random", 300), ("prefix", 0)])
def test_max_experts_and_topk(hm, rule, n_kept):
    """The library's largest expert count (1024) and top-k (16) through decode (M = 1, 8)
    and prefill (M = 9, 64), with a random 300-expert kept tier, and with the kept tier
    empty (every expert NF3: the kept arrays are NULL)."""
    w = synth.Workload("max", 1024, 256, 128, 16, 64, "nvfp4", n_kept, rule, seed=11)
    packed = synth.packed_layer(w)
    assert packed["kept"]["w13_q"].shape[0] == n_kept
    wts = hm.DeviceWeights(packed)
    layer = make_layer(packed, 64)
    for M in (1, 8, 9, 64):
        x = synth.activations_bf16(w, M)
        lg = synth.router_logits(w, M)
        y, _ = run_forward(layer, wts, x, lg)
        check_output(y, OL.forward(packed, x, lg)["y"], f"E=1024 k=16 {rule} M={M}")
