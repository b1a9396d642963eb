"""GPU parity of the integer/byte work and the dequantisation, bit for bit:
the dequant hook against the oracle's canonical fp32 / bf16 values (edge codes
included), routing ids (weights to 1e-6 relative), the decode grouping and the
per-tier align tables."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as OL
from hmoe_testlib import (check_output, make_layer, run_forward, scratch_for, tiny_packed,
                          to_dev, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_moe_amd as m
    m.load_library()
    return m


# ---------------------------------------------------------------- dequant

def _edge_layer(kept_format):
    """A 2-expert layer (expert 0 kept, expert 1 NF3) whose bytes sweep the edge
    codes: every FP4 code with every non-NaN E4M3 (or E8M0) scale byte, NVFP4
    per-tensor scales that force rounding, NF3 fp16 scales from subnormal to max,
    zero and negative."""
    E, H, I, k = 2, 256, 128, 1
    bm = np.array([4, 3], np.uint8)
    lay = synth.empty_packed_layer(E, H, I, k, kept_format, bm)
    r = np.random.default_rng(99)
    kq = lay["kept"]
    kq["w13_q"][:] = r.integers(0, 256, kq["w13_q"].shape, dtype=np.uint8)
    kq["w2_q"][:] = r.integers(0, 256, kq["w2_q"].shape, dtype=np.uint8)
    kq["w13_q"][0, 0, :] = np.arange(128, dtype=np.uint8)          # all code pairs
    kq["w13_q"][0, 1, :] = np.arange(128, 256, dtype=np.uint8)
    if kept_format == "nvfp4":
        scales = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
        flat = kq["w13_s"].reshape(-1)
        flat[:] = np.resize(scales, flat.size)
        kq["w2_s"].reshape(-1)[:] = np.resize(scales[::-1], kq["w2_s"].size)
        kq["w13_g"][:] = np.float32(1.0 / 3.0)
        kq["w2_g"][:] = np.float32(3.0e-5)
    else:
        scales = np.arange(255, dtype=np.uint8)                      # 0 .. 254 (255 is NaN)
        kq["w13_s"].reshape(-1)[:] = np.resize(scales, kq["w13_s"].size)
        kq["w2_s"].reshape(-1)[:] = np.resize(scales[::-1], kq["w2_s"].size)
    nq = lay["nf3"]
    nq["w13_q"][:] = r.integers(0, 256, nq["w13_q"].shape, dtype=np.uint8)
    nq["w2_q"][:] = r.integers(0, 256, nq["w2_q"].shape, dtype=np.uint8)
    fp16_edges = np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xBC00,
                           0x2E66, 0x1234], np.uint16)
    nq["w13_s"].reshape(-1)[:] = np.resize(fp16_edges, nq["w13_s"].size)
    nq["w2_s"].reshape(-1)[:] = np.resize(fp16_edges[::-1], nq["w2_s"].size)
    return lay


@pytest.mark.parametrize("case", ["tiny_nvfp4", "tiny_mxfp4", "tiny_uniform", "edge_nvfp4", "edge_mxfp4"])
def test_dequant_bit_exact(hm, case):
    torch = torch_mod()
    if case.startswith("tiny"):
        fmt = "mxfp4" if case.endswith("mxfp4") else "nvfp4"
        packed, _ = tiny_packed(fmt, None if case.endswith("uniform") else "prefix")
    else:
        packed = _edge_layer(case.split("_")[1])
    layer = make_layer(packed, 4)
    wts = hm.DeviceWeights(packed)
    for e in range(packed["E"]):
        w13, w2 = OL.expert_weights(packed, e)
        for tensor, ref in ((hm.TENSOR_W13, w13), (hm.TENSOR_W2, w2)):
            out = torch.empty(ref.shape, dtype=torch.float32, device="cuda")
            outb = torch.empty(ref.shape, dtype=torch.int16, device="cuda")
            hm.moe_dequant(layer, wts, e, tensor, out, outb)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
                f"{case} expert {e} tensor {tensor}: " \
                f"{np.sum(got.view(np.uint32) != ref.view(np.uint32))} fp32 mismatches"
            gotb = outb.cpu().numpy().view(np.uint16)
            assert np.array_equal(gotb, F.bf16_bits(ref)), f"{case} expert {e} tensor {tensor}: bf16"


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("M,E,k,kind", [
    (1, 8, 2, "normal"), (7, 128, 8, "normal"), (64, 256, 8, "normal"), (1000, 1000, 16, "normal"),
    (300, 256, 8, "ties"), (33, 64, 64 // 4, "ties"), (5, 3, 3, "normal"), (20, 256, 1, "zeros"),
    (40, 128, 8, "specials"), (9, 64, 16, "specials"),
])
def test_route_matches_oracle(hm, M, E, k, kind):
    torch = torch_mod()
    r = np.random.default_rng(M * 1000 + E)
    if kind == "normal":
        lg = r.standard_normal((M, E)).astype(np.float32)
    elif kind == "ties":
        lg = r.integers(-2, 3, (M, E)).astype(np.float32)
        lg[:, ::3] *= -1.0   # introduces -0.0 next to +0.0
    elif kind == "zeros":
        lg = np.zeros((M, E), np.float32)
        lg[:, 1::2] = -0.0
    else:
        # NaN (ranks below every number), -inf, and +-0, with the selection reaching down
        # into the -inf and zero logits but not the NaNs
        lg = r.standard_normal((M, E)).astype(np.float32)
        lg[:, : E // 2] = -np.abs(lg[:, : E // 2]) - 1.0
        lg[:, E // 2:] = np.nan
        ninf = np.arange(E // 2) % 4 != 0 if k > 8 else np.arange(E // 2) % 7 == 1
        lg[:, : E // 2][:, ninf] = -np.inf
        lg[:, 2 : E // 2 : 9] = 0.0
        lg[:, 4 : E // 2 : 9] = -0.0
        lg[:, E - 1] = 0.5
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    hm.moe_route(to_dev(lg), k, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = OL.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    got = w.cpu().numpy().astype(np.float64)
    nz = ref_w > 0          # -inf logits weigh exactly 0
    assert np.all(got[~nz] == 0.0)
    rel = np.abs(got[nz] - ref_w[nz]) / ref_w[nz]
    assert rel.max() <= 1e-6, rel.max()


# ---------------------------------------------------------------- decode grouping

@pytest.mark.parametrize("M", [1, 3, 8])
def test_decode_grouping_bit_exact(hm, M):
    torch = torch_mod()
    w = synth.qwen_decode(M)
    packed = synth.packed_layer(w)
    layer = make_layer(packed, 8)
    wts = hm.DeviceWeights(packed)
    x = synth.activations_bf16(w, M)
    lg = synth.router_logits(w, M)
    _, scratch = run_forward(layer, wts, x, lg)
    v = hm.moe_decode_view(layer, scratch)
    tier, local = OL.tier_map(packed["bit_map"], w.E)
    ids, _ = OL.route(lg, w.top_k)
    groups = OL.decode_groups(ids, tier, local)
    counts = v["counts"].cpu().numpy()
    assert counts[0] == len(groups) and counts[1] == sum(1 for g in groups if g[1] == 0)
    experts = v["experts"].cpu().numpy()[: len(groups)]
    nslots = v["num_slots"].cpu().numpy()
    slots = v["slots"].cpu().numpy()
    for d, (e, t, l, sl) in enumerate(groups):
        assert experts[d] == e and nslots[d] == len(sl) and list(slots[d, : len(sl)]) == sl
    et = v["expert_tier"].cpu().numpy()
    assert np.array_equal(et >> 16, tier) and np.array_equal(et & 0xFFFF, local)
    tids, tw = hm.moe_topk_view(layer, scratch, M)
    assert np.array_equal(tids.cpu().numpy(), ids)
    # pass records: one per slot, in slot order: slot, tier code of its expert, token,
    # expert
    passes = v["passes"].cpu().numpy()[: M * w.top_k]
    want = [(s, (int(tier[e]) << 16) | int(local[e]), s // w.top_k, int(e))
            for s, e in enumerate(ids.reshape(-1))]
    assert [tuple(int(c) for c in r) for r in passes] == want


# ---------------------------------------------------------------- align

@pytest.mark.parametrize("E,k,M,bm,n_kept", [
    (8, 2, 9, 16, 4), (8, 2, 100, 32, 4), (256, 8, 64, 32, 64), (256, 8, 4096, 32, 64),
    (256, 8, 512, 128, 64), (128, 8, 300, 64, 32), (256, 8, 700, 16, None), (64, 4, 1, 64, 16),
    # 40,000 slots: 2,560 per wave, two and a half batches of 16 steps, the last wave's
    # chunk ending inside its second batch
    (256, 8, 5000, 64, 64),
])
def test_align_bit_exact(hm, E, k, M, bm, n_kept):
    torch = torch_mod()
    r = np.random.default_rng(E + M + bm)
    bit_map = None
    if n_kept is not None:
        bit_map = np.full(E, 3, np.uint8)
        bit_map[r.permutation(E)[:n_kept]] = 4
    lg = (r.standard_normal((M, E)) + 1.5 * r.standard_normal(E)[None, :]).astype(np.float32)
    ids, _ = OL.route(lg, k)
    layer = hm.moe_layer_create(E, 256, 128, k, M, hm.KEPT_NVFP4, bit_map, bm)
    scratch = scratch_for(layer)
    scratch.fill_(0xAB)     # stale contents must not leak into the defined entries
    hm.moe_align(layer, to_dev(ids), M, scratch)
    torch.cuda.synchronize()
    tier, local = OL.tier_map(bit_map, E)
    ref = OL.align(ids, tier, local, bm)
    for t in (0, 1):
        v = hm.moe_align_view(layer, scratch, t)
        npad = int(v["num_padded"].cpu().numpy()[0])
        assert npad == ref[t]["num_padded"]
        assert np.array_equal(v["sorted_slots"].cpu().numpy()[:npad], ref[t]["sorted_slots"])
        assert np.array_equal(v["block_expert"].cpu().numpy()[: npad // bm], ref[t]["block_expert"])
        assert np.array_equal(v["expert_off"].cpu().numpy(), ref[t]["expert_off"])


# ---------------------------------------------------------------- load-time demux / repack

def _repack_case(kept, rule, E, H, I, k, n_kept, seed):
    w = synth.Workload("repack", E, H, I, k, 4, kept, n_kept, rule, seed=seed)
    bm = synth.bit_map(w)
    packed = OL.quantize_layer(E, H, I, k, bm, kept, lambda e: synth.master_weights(w, e))
    return packed, w


@pytest.mark.parametrize("kept,rule,E,H,I,k,n_kept", [
    ("nvfp4", "prefix", 8, 256, 128, 2, 4),
    ("mxfp4", "prefix", 8, 256, 128, 2, 4),
    ("nvfp4", "none", 8, 256, 128, 2, None),
    ("mxfp4", "random", 16, 512, 256, 4, 5),
    ("nvfp4", "random", 16, 512, 256, 4, 11),
])
def test_repack_bit_exact(hm, kept, rule, E, H, I, k, n_kept):
    """moe_repack of checkpoint-style per-expert tensors (NF3 codes as two planes)
    reproduces the oracle's tier-local arrays byte for byte, and a forward on the
    repacked weights equals the forward on the original ones bit for bit."""
    torch = torch_mod()
    packed, w = _repack_case(kept, rule, E, H, I, k, n_kept, seed=9)
    ckpt = OL.checkpoint_experts(packed)
    dev = []
    for ex in ckpt:
        dev.append({n: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                        else np.ascontiguousarray(a).reshape(-1)).cuda()
                    for n, a in ex.items()})
    empty = synth.empty_packed_layer(E, H, I, k, packed["kept_format"], packed["bit_map"])
    dst = hm.DeviceWeights(empty)
    layer = make_layer(packed, 32)
    hm.moe_repack(layer, dev, dst)
    torch.cuda.synchronize()
    for tier, keys in hm.DeviceWeights.KEYS.items():
        for key in keys:
            t = dst.tensors[f"{tier}_{key}"]
            ref = packed[tier][key]
            if t is None:
                assert ref.size == 0
                continue
            got = t.cpu().numpy()
            if ref.dtype == np.uint16:
                got = got.view(np.uint16)
            assert np.array_equal(got.reshape(ref.shape), ref), (tier, key)
    orig = hm.DeviceWeights(packed)
    for M in (3, 20):
        x = synth.activations_bf16(w, M)
        lg = synth.router_logits(w, M)
        y1, _ = run_forward(layer, orig, x, lg)
        y2, _ = run_forward(layer, dst, x, lg)
        assert np.array_equal(y1, y2), M
