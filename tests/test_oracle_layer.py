"""Pins of the oracle's layer arithmetic: routing against library softmax and
brute-force ranking, align and grouping against the invariants that fix them
uniquely, and the expert MLP / layer against a dense textbook SwiGLU MLP,
tier additivity, relabelling invariance and an explicit-loop brute force."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as L


# ---------------------------------------------------------------- routing

def test_route_weights_match_torch_softmax_at_k_equals_E():
    r = np.random.default_rng(10)
    lg = r.standard_normal((16, 12)).astype(np.float32)
    ids, w = L.route(lg, 12)
    ref = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    assert np.allclose(np.take_along_axis(ref, ids, 1), w, rtol=1e-13, atol=0)


def test_route_topk_renormalised_softmax():
    r = np.random.default_rng(11)
    lg = r.standard_normal((32, 64)).astype(np.float32)
    ids, w = L.route(lg, 6)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(p, ids, 1)
    assert np.allclose(sel / sel.sum(1, keepdims=True), w, rtol=1e-12, atol=0)
    assert np.allclose(w.sum(1), 1.0)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_ids_brute_force_with_ties():
    r = np.random.default_rng(12)
    lg = r.integers(-3, 4, (50, 20)).astype(np.float32)   # many exact ties
    lg[0] = 0.0
    lg[1, ::2] = -0.0
    ids, _ = L.route(lg, 5)
    for t in range(lg.shape[0]):
        want = sorted(range(20), key=lambda e: (-float(lg[t, e]), e))[:5]
        assert ids[t].tolist() == want


# ---------------------------------------------------------------- tier map

def test_tier_map_local_ids():
    bm = np.array([3, 4, 4, 3, 3, 4], np.uint8)
    tier, local = L.tier_map(bm, 6)
    assert tier.tolist() == [1, 0, 0, 1, 1, 0]
    assert local.tolist() == [0, 0, 1, 1, 2, 2]
    t0, l0 = L.tier_map(None, 4)
    assert t0.tolist() == [0] * 4 and l0.tolist() == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        L.tier_map(np.array([4, 5], np.uint8), 2)


# ---------------------------------------------------------------- grouping / align

def _ids(M, E, k, seed):
    lg = np.random.default_rng(seed).standard_normal((M, E)).astype(np.float32)
    return L.route(lg, k)[0]


def test_decode_groups_invariants():
    bm = np.where(np.arange(16) % 3 == 0, 4, 3).astype(np.uint8)
    tier, local = L.tier_map(bm, 16)
    ids = _ids(8, 16, 4, 13)
    groups = L.decode_groups(ids, tier, local)
    keys = [(g[1], g[2]) for g in groups]
    assert keys == sorted(keys) and len(set(g[0] for g in groups)) == len(groups)
    seen = []
    for e, t, l, slots in groups:
        assert t == tier[e] and l == local[e]
        assert slots == sorted(slots) and all(ids.reshape(-1)[s] == e for s in slots)
        seen += slots
    assert sorted(seen) == list(range(ids.size))


@pytest.mark.parametrize("block_m", [1, 4, 16])
def test_align_invariants_fix_the_output(block_m):
    E, k, M = 12, 3, 40
    bm = np.array([4, 3, 3, 4, 3, 3, 3, 4, 3, 4, 3, 3], np.uint8)
    tier, local = L.tier_map(bm, E)
    ids = _ids(M, E, k, 14)
    flat = ids.reshape(-1)
    out = L.align(ids, tier, local, block_m)
    for t in (0, 1):
        a = out[t]
        members = [e for e in range(E) if tier[e] == t]
        offs = a["expert_off"]
        assert offs[0] == 0 and offs[-1] == a["num_padded"] == a["sorted_slots"].size
        assert a["num_padded"] % block_m == 0 and len(offs) == len(members) + 1
        real = a["sorted_slots"][a["sorted_slots"] != M * k]
        assert sorted(real.tolist()) == [s for s in range(M * k) if tier[flat[s]] == t]
        for j, e in enumerate(members):
            seg = a["sorted_slots"][offs[j]:offs[j + 1]]
            n = int(np.sum(flat == e))
            assert seg.size == -(-n // block_m) * block_m
            assert seg[:n].tolist() == [s for s in range(M * k) if flat[s] == e]
            assert np.all(seg[n:] == M * k)
            assert np.all(a["block_expert"][offs[j] // block_m:offs[j + 1] // block_m] == j)


# ---------------------------------------------------------------- MLP / layer

def _dense_swiglu(x, w13, w2):
    """Textbook SwiGLU MLP with torch: down(silu(gate x) * up x)."""
    I = w2.shape[1]
    xt = torch.from_numpy(x).double()
    g = xt @ torch.from_numpy(w13[:I]).double().T
    u = xt @ torch.from_numpy(w13[I:]).double().T
    return (torch.nn.functional.silu(g) * u) @ torch.from_numpy(w2).double().T


def _tiny_layer(bit_map, fmt="nvfp4", E=8):
    w = synth.Workload("t", E, 256, 128, 2, 4)
    return L.quantize_layer(E, 256, 128, 2, bit_map, fmt, lambda e: synth.master_weights(w, e)), w


def test_single_expert_layer_is_dense_swiglu():
    lay, w = _tiny_layer(None, E=1)
    lay["top_k"] = 1
    x = synth.activations_bf16(w, 5)
    lg = np.zeros((5, 1), np.float32)
    out = L.forward(lay, x, lg)
    w13, w2 = L.expert_weights(lay, 0)
    ref = _dense_swiglu(F.bf16_value(x).astype(np.float64), w13, w2).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["w"], 1.0)


def test_layer_brute_force_loops():
    bm = np.array([4, 4, 4, 4, 3, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm)
    x = synth.activations_bf16(w, 2)
    lg = synth.router_logits(w, 2)
    out = L.forward(lay, x, lg)
    xs = F.bf16_value(x).astype(np.float64)
    for t in range(2):
        order = sorted(range(8), key=lambda e: (-float(lg[t, e]), e))[:2]
        ex = [np.exp(float(lg[t, e]) - float(lg[t, order[0]])) for e in order]
        y = np.zeros(256)
        for j, e in enumerate(order):
            w13, w2 = L.expert_weights(lay, e)
            h = np.zeros(128)
            for i in range(128):
                a = float(np.dot(w13[i].astype(np.float64), xs[t]))
                b = float(np.dot(w13[128 + i].astype(np.float64), xs[t]))
                h[i] = a / (1.0 + np.exp(-a)) * b
            for n in range(256):
                y[n] += ex[j] / sum(ex) * float(np.dot(w2[n].astype(np.float64), h))
        assert np.allclose(out["y"][t], y, rtol=1e-10, atol=1e-13)


def test_forward_threads_do_not_change_the_result():
    """Running experts on a thread pool adds their outputs in the same ascending
    expert order: bit-identical y and h, for all tokens and for a token subset."""
    bm = np.array([4, 3, 4, 3, 4, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm)
    x = synth.activations_bf16(w, 12)
    lg = synth.router_logits(w, 12)
    for tokens in (None, [0, 5, 11]):
        a = L.forward(lay, x, lg, tokens=tokens)
        b = L.forward(lay, x, lg, tokens=tokens, threads=4)
        assert np.array_equal(a["y"], b["y"])
        assert a["h"].keys() == b["h"].keys()
        assert all(np.array_equal(a["h"][s], b["h"][s]) for s in a["h"])


def test_tier_additivity():
    bm = np.array([4, 3, 4, 3, 4, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm)
    x = synth.activations_bf16(w, 4)
    lg = synth.router_logits(w, 4)
    full = L.forward(lay, x, lg)["y"]
    no_nf3 = {**lay, "nf3": {**lay["nf3"], "w13_s": np.zeros_like(lay["nf3"]["w13_s"])}}
    no_kept = {**lay, "kept": {**lay["kept"], "w13_s": np.zeros_like(lay["kept"]["w13_s"])}}
    y_a = L.forward(no_nf3, x, lg)["y"]
    y_b = L.forward(no_kept, x, lg)["y"]
    assert np.allclose(full, y_a + y_b, rtol=1e-12, atol=1e-15)
    assert np.abs(y_a).max() > 0 and np.abs(y_b).max() > 0


def test_relabelling_experts_leaves_output_unchanged():
    bm = np.array([4, 3, 4, 3, 4, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm)
    x = synth.activations_bf16(w, 4)
    lg = synth.router_logits(w, 4)
    y = L.forward(lay, x, lg)["y"]
    perm = np.array([5, 2, 7, 0, 3, 6, 1, 4])        # new id p holds old expert perm[p]
    bm2 = bm[perm]
    tier, local = L.tier_map(bm, 8)
    tier2, local2 = L.tier_map(bm2, 8)
    lay2 = {**lay, "bit_map": bm2,
            "kept": {k: np.empty_like(v) for k, v in lay["kept"].items()},
            "nf3": {k: np.empty_like(v) for k, v in lay["nf3"].items()}}
    for p in range(8):
        old = perm[p]
        src = lay["kept"] if tier[old] == 0 else lay["nf3"]
        dst = lay2["kept"] if tier2[p] == 0 else lay2["nf3"]
        for key in src:
            dst[key][local2[p]] = src[key][local[old]]
    y2 = L.forward(lay2, x, lg[:, perm])["y"]
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-15)


def test_absent_bit_map_runs_uniform_nvfp4():
    lay, w = _tiny_layer(None, fmt="mxfp4")
    assert lay["kept_format"] == "nvfp4" and lay["kept"]["w13_s"].shape[-1] == 256 // 16
    assert L.kept_format_of(lay) == "nvfp4"


def test_mxfp4_kept_tier_layer_runs():
    bm = np.array([4, 4, 4, 4, 3, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm, fmt="mxfp4")
    assert lay["kept"]["w13_s"].shape[-1] == 256 // 32
    x = synth.activations_bf16(w, 3)
    out = L.forward(lay, x, synth.router_logits(w, 3))
    master13, _ = synth.master_weights(w, 0)
    w13, _ = L.expert_weights(lay, 0)
    # MXFP4 dequant tracks the master weights to within the E2M1 grid step
    assert np.max(np.abs(w13 - master13)) < 0.25 * np.abs(master13).max()
    assert np.all(np.isfinite(out["y"]))


# ---------------------------------------------------------------- load-time demux

def test_demux_places_each_expert_by_brute_force():
    """Tier-local index of expert e = number of experts below e in e's tier; the NF3
    stream of a demuxed expert equals the stream packing of its plane codes."""
    from hmoe_testlib import tiny_packed
    packed, _ = tiny_packed("mxfp4", "prefix", E=8, H=256, I=128, k=2, seed=4)
    E = packed["E"]
    bm = np.array([3, 4, 3, 3, 4, 4, 3, 4], dtype=np.uint8)  # irregular map
    # a layer with this map whose expert e carries data tagged by e
    experts = L.checkpoint_experts(packed)
    kept_src = [e for e in range(E) if packed["bit_map"][e] == 4]
    nf3_src = [e for e in range(E) if packed["bit_map"][e] == 3]
    pool = {4: [experts[e] for e in kept_src], 3: [experts[e] for e in nf3_src]}
    mine = []
    used = {3: 0, 4: 0}
    for e in range(E):
        b = int(bm[e])
        mine.append(pool[b][used[b] % len(pool[b])])
        used[b] += 1
    layer = L.demux(mine, bm, E, packed["H"], packed["I"], packed["top_k"], "mxfp4")
    for e in range(E):
        same = [x for x in range(e) if bm[x] == bm[e]]
        j = len(same)
        if bm[e] == 4:
            assert np.array_equal(layer["kept"]["w13_q"][j], mine[e]["w13_q"])
            assert np.array_equal(layer["kept"]["w2_s"][j], mine[e]["w2_s"])
        else:
            q = F.unpack_nf3_planes(mine[e]["w2_lo"], mine[e]["w2_hi"])
            assert np.array_equal(F.unpack_nf3(layer["nf3"]["w2_q"][j]), q)
            assert np.array_equal(layer["nf3"]["w13_s"][j], mine[e]["w13_s"])
    back = L.checkpoint_experts(layer)
    for e in range(E):
        assert set(back[e]) == set(mine[e]) and all(np.array_equal(back[e][k], mine[e][k]) for k in mine[e])


# ---------------------------------------------------------------- W4A4 (MXFP4 activations)

_E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mx_round_block(vals):
    """One 32-block by the OCP MX v1.0 conversion, written out: shared exponent
    floor(log2(amax)) - 2 (from math.frexp), clamped to [-127, 127]; each element
    divided by 2^shared and set to the nearest E2M1 magnitude (ties to the one with an
    even code index, |t| clipped to 6), sign kept."""
    import math
    amax = max(abs(float(v)) for v in vals)
    if amax == 0.0:
        return [0.0] * len(vals)
    shared = min(max(math.frexp(amax)[1] - 1 - 2, -127), 127)
    out = []
    for v in vals:
        t = math.ldexp(float(v), -shared)
        a = min(abs(t), 6.0)
        best = 0
        for i in range(1, 8):
            d, db = abs(a - _E2M1_MAGS[i]), abs(a - _E2M1_MAGS[best])
            if d < db or (d == db and i % 2 == 0 and best % 2 == 1):
                best = i
        out.append(math.copysign(math.ldexp(_E2M1_MAGS[best], shared), t) if best else 0.0)
    return out


def test_mxfp4_activation_brute_force():
    rng = np.random.default_rng(31)
    a = (rng.standard_normal((6, 128)) * np.exp(rng.standard_normal((6, 1)) * 3)).astype(np.float32)
    a[0, :32] = 0.0                                        # an all-zero block
    a[1, :32] = np.float32(2.0 ** -130)                    # subnormal block: exponent clamp
    a[2, :8] = np.array([4, 1, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5], np.float32)   # ties
    a[2, 8:16] = np.array([3.5, 5, -0.25, -0.75, 6.5, -7, 0.125, 3], np.float32)
    got = L.mxfp4_activation(a)
    ref = np.array([sum((_mx_round_block(row[b:b + 32]) for b in range(0, 128, 32)), [])
                    for row in a.astype(np.float64)], dtype=np.float64)
    assert np.array_equal(got.astype(np.float64), ref)


def test_w4a4_layer_brute_force_loops():
    """The W4A4 forward (MXFP4 kept tier, MXFP4 activations) against explicit loops:
    per-block rounding of x and of h (after fp32 rounding) by the written-out OCP
    conversion, dot products element by element."""
    bm = np.array([4, 4, 4, 4, 3, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm, "mxfp4")
    x = synth.activations_bf16(w, 2)
    lg = synth.router_logits(w, 2)
    lg[0, 1] += 9.0     # token 0 takes a kept-tier expert first
    out = L.forward(lay, x, lg, act_format="mxfp4")
    xs = F.bf16_value(x).astype(np.float64)
    tier, _ = L.tier_map(bm, 8)
    for t in range(2):
        order = sorted(range(8), key=lambda e: (-float(lg[t, e]), e))[:2]
        ex = [np.exp(float(lg[t, e]) - float(lg[t, order[0]])) for e in order]
        y = np.zeros(256)
        for j, e in enumerate(order):
            w13, w2 = L.expert_weights(lay, e)
            kept = tier[e] == L.KEPT
            xv = sum((_mx_round_block(xs[t][b:b + 32]) for b in range(0, 256, 32)), []) if kept else list(xs[t])
            h = np.zeros(128)
            for i in range(128):
                a = sum(float(w13[i][c]) * xv[c] for c in range(256))
                b = sum(float(w13[128 + i][c]) * xv[c] for c in range(256))
                h[i] = a / (1.0 + np.exp(-a)) * b
            if kept:
                h32 = h.astype(np.float32).astype(np.float64)
                h = np.array(sum((_mx_round_block(h32[b:b + 32]) for b in range(0, 128, 32)), []))
            for n in range(256):
                y[n] += ex[j] / sum(ex) * float(np.dot(w2[n].astype(np.float64), h))
        assert np.allclose(out["y"][t], y, rtol=1e-9, atol=1e-12), t
    assert any(tier[e] == L.KEPT for e in out["ids"].ravel())


def test_w4a4_leaves_the_nf3_tier_and_equals_w4a16_there():
    bm = np.array([4, 4, 4, 4, 3, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm, "mxfp4")
    x = synth.activations_bf16(w, 6)
    lg = synth.router_logits(w, 6)
    lg[:, :4] -= 50.0   # every token routed to NF3 experts only
    a = L.forward(lay, x, lg, act_format="mxfp4")
    b = L.forward(lay, x, lg)
    assert np.array_equal(a["y"], b["y"])


def test_w4a4_on_representable_x_matches_w4a16_before_w2():
    """With x exactly representable in MXFP4 the W13 input is unchanged, so W4A4 and
    W4A16 differ only by h's rounding: the W4A4 h equals the MXFP4 rounding of the
    W4A16 h (rounded to fp32 first)."""
    bm = np.array([4, 4, 4, 4, 3, 3, 3, 3], np.uint8)
    lay, w = _tiny_layer(bm, "mxfp4")
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (3, 256)).astype(np.uint8)
    scales = rng.integers(124, 130, (3, 256 // 32)).astype(np.uint8)
    xv = F.mxfp4_dequant(F.pack_fp4(codes), scales)
    x = F.bf16_bits(xv)
    assert np.array_equal(F.bf16_value(x), xv)          # bf16 holds the MX values exactly
    lg = synth.router_logits(w, 3)
    lg[:, 4:] -= 50.0   # kept-tier experts only
    a = L.forward(lay, x, lg, act_format="mxfp4")
    b = L.forward(lay, x, lg)
    for s, h in a["h"].items():
        assert np.array_equal(h, L.mxfp4_activation(b["h"][s].astype(np.float32)).astype(np.float64))
