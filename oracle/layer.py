"""Oracle for the hybrid MoE layer: tier map, routing, grouping, align, expert
MLP and the shared top-k weighted sum.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import this).

Pages (cited by title and section):
* local-inference-lab/vllm PR #92 "quant: nvfp4_nf3_hybrid", "How it works":
  two prepared weight objects per layer (one per tier), both launches share one
  route geometry and one top-k sum, the second accumulates into the first; an
  M <= 8 decode path addressed directly by the top-k result; layers absent from
  the bit map run uniform NVFP4.
* PR #104 description: bit map values 4 = kept tier, 3 = NF3; the kept format
  may switch the kept tier to MXFP4; expert weights are demultiplexed into
  compact tier-local storage.
* vllm-project/vllm PR #42428 "W4A16 NVFP4 fused MoE", "What's in this PR": the
  W4A16 path sits beside W4A4 backends, whose activations are 4-bit as well. The
  W4A4 variant here (act_format "mxfp4") applies to an MXFP4 kept tier: each
  kept-tier matmul input (x before W13, h before W2) is rounded to MXFP4 along K,
  blocks of 32, by the OCP MX v1.0 conversion the weight quantiser uses.
Routing (softmax over the router logits, top-k, renormalised) and SwiGLU
experts are the layer's definition where the pages do not spell them out.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

KEPT, NF3 = 0, 1


# ----------------------------------------------------------------------------
# tier map (global expert id -> tier, tier-local id)
# ----------------------------------------------------------------------------

def tier_map(bit_map, E: int):
    """tier[e] = 0 for the kept tier (bit 4, or no bit map at all), 1 for NF3
    (bit 3); local[e] = number of experts e' < e in the same tier, i.e. the
    position of e in its tier's ascending-id storage."""
    tier = np.zeros(E, dtype=np.int32)
    if bit_map is not None:
        bm = np.asarray(bit_map)
        if bm.shape != (E,) or not np.all((bm == 3) | (bm == 4)):
            raise ValueError("bit map must hold E entries, each 3 or 4")
        tier = np.where(bm == 3, NF3, KEPT).astype(np.int32)
    local = np.zeros(E, dtype=np.int32)
    seen = [0, 0]
    for e in range(E):
        local[e] = seen[tier[e]]
        seen[tier[e]] += 1
    return tier, local


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def route(logits: np.ndarray, top_k: int):
    """Softmax top-k, renormalised. Experts are ranked by logit, descending,
    ties to the lower expert id (a stable sort of the negated logits); the
    weights are the softmax over the selected logits (equal to softmax over all
    experts, then top-k, then renormalise), computed in fp64."""
    L = np.asarray(logits, dtype=np.float32)
    ids = np.argsort(-L, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(L, ids, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


# ----------------------------------------------------------------------------
# decode grouping (M <= 8): distinct experts and their slots
# ----------------------------------------------------------------------------

def decode_groups(ids: np.ndarray, tier: np.ndarray, local: np.ndarray):
    """Distinct experts touched by the top-k result, ordered by (tier, local id),
    each with its slots s = t * k + j in ascending order."""
    flat = np.asarray(ids).reshape(-1)
    experts = sorted(set(int(e) for e in flat), key=lambda e: (int(tier[e]), int(local[e])))
    return [(e, int(tier[e]), int(local[e]), [s for s in range(flat.size) if flat[s] == e])
            for e in experts]


# ----------------------------------------------------------------------------
# align (M > 8): per tier, slots sorted by expert and padded to BM
# ----------------------------------------------------------------------------

def align(ids: np.ndarray, tier: np.ndarray, local: np.ndarray, block_m: int):
    """Per tier: every slot of that tier's experts, grouped by tier-local expert
    in ascending local id, ascending slot order inside an expert, each expert's
    run padded with the sentinel M*k up to a multiple of block_m. Returns, per
    tier, sorted_slots[num_padded], block_expert[num_padded / block_m],
    expert_off[E_tier + 1] and num_padded."""
    flat = np.asarray(ids).reshape(-1)
    sentinel = flat.size
    out = []
    for t in (KEPT, NF3):
        members = [e for e in range(tier.size) if tier[e] == t]   # ascending = local order
        offs = [0]
        sorted_slots = []
        block_expert = []
        for e in members:
            slots = [s for s in range(flat.size) if flat[s] == e]
            n = len(slots)
            padded = -(-n // block_m) * block_m
            sorted_slots += slots + [sentinel] * (padded - n)
            block_expert += [int(local[e])] * (padded // block_m)
            offs.append(offs[-1] + padded)
        out.append({
            "sorted_slots": np.array(sorted_slots, dtype=np.int32),
            "block_expert": np.array(block_expert, dtype=np.int32),
            "expert_off": np.array(offs, dtype=np.int32),
            "num_padded": int(offs[-1]),
        })
    return out


# ----------------------------------------------------------------------------
# dequantised expert weights
# ----------------------------------------------------------------------------

def expert_weights(layer: dict, e: int):
    """fp32 dequantised (W13 [2I, H], W2 [H, I]) of global expert e."""
    tier, local = tier_map(layer["bit_map"], layer["E"])
    j = int(local[e])
    if tier[e] == KEPT:
        k = layer["kept"]
        if layer["kept_format"] == "nvfp4" or layer["bit_map"] is None:
            w13 = F.nvfp4_dequant(k["w13_q"][j], k["w13_s"][j], k["w13_g"][j])
            w2 = F.nvfp4_dequant(k["w2_q"][j], k["w2_s"][j], k["w2_g"][j])
        else:
            w13 = F.mxfp4_dequant(k["w13_q"][j], k["w13_s"][j])
            w2 = F.mxfp4_dequant(k["w2_q"][j], k["w2_s"][j])
    else:
        n = layer["nf3"]
        w13 = F.nf3_dequant(n["w13_q"][j], n["w13_s"][j])
        w2 = F.nf3_dequant(n["w2_q"][j], n["w2_s"][j])
    return w13, w2


def kept_format_of(layer: dict) -> str:
    """A layer with no bit map runs uniform NVFP4 whatever the kept format says."""
    return "nvfp4" if layer["bit_map"] is None else layer["kept_format"]


# ----------------------------------------------------------------------------
# expert MLP and the layer
# ----------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_mlp(x: np.ndarray, w13: np.ndarray, w2: np.ndarray):
    """SwiGLU expert: a = W1 x (gate rows), b = W3 x (up rows), h = silu(a) * b,
    o = W2 h. x is [n, H]; computed in fp64 from the fp32 weights."""
    I = w2.shape[1]
    z = x @ w13.astype(np.float64).T
    h = silu(z[:, :I]) * z[:, I:]
    return h, h @ w2.astype(np.float64).T


def mxfp4_activation(a: np.ndarray) -> np.ndarray:
    """Activations rounded to MXFP4 along their last axis (blocks of 32, the OCP MX
    v1.0 conversion of formats.mxfp4_quantize) and decoded back: the fp32 values a
    W4A4 matmul multiplies."""
    a = np.asarray(a, dtype=np.float32)
    q, s = F.mxfp4_quantize(a.reshape(-1, a.shape[-1]))
    return F.mxfp4_dequant(q, s).reshape(a.shape)


def expert_mlp_w4a4(x: np.ndarray, w13: np.ndarray, w2: np.ndarray):
    """SwiGLU expert with 4-bit activations: x is rounded to MXFP4 before W13; h =
    silu(a) * b is rounded to fp32 (the width it is computed in) and then to MXFP4
    before W2. Products and sums in fp64. Returns (the MXFP4 h that W2 sees, o)."""
    I = w2.shape[1]
    xq = mxfp4_activation(x).astype(np.float64)
    z = xq @ w13.astype(np.float64).T
    h = silu(z[:, :I]) * z[:, I:]
    hq = mxfp4_activation(h.astype(np.float32)).astype(np.float64)
    return hq, hq @ w2.astype(np.float64).T


def forward(layer: dict, x_bits: np.ndarray, logits: np.ndarray, tokens=None, threads: int = 1,
            act_format: str = "bf16"):
    """The layer: route once, run every selected (token, expert) pair through
    the expert's MLP in its own tier, and add the outputs into one top-k
    weighted sum y[t] = sum_j w[t, j] * o[t, j]. `tokens` restricts the
    returned rows to a subset (the routing result is still for every token).
    `threads` > 1 dequantises and runs several experts at once; the outputs are
    still added into y one expert at a time in ascending expert id, so the result
    does not depend on it. act_format "mxfp4" runs the kept tier as W4A4
    (expert_mlp_w4a4; the layer's kept tier must be MXFP4), "bf16" (default) every
    expert as W4A16. Returns ids, weights, per-slot h (only for the computed tokens)
    and y (fp64, one row per computed token)."""
    if act_format not in ("bf16", "mxfp4"):
        raise ValueError("act_format must be 'bf16' or 'mxfp4'")
    if act_format == "mxfp4" and kept_format_of(layer) != "mxfp4":
        raise ValueError("W4A4 needs an MXFP4 kept tier")
    E, k = layer["E"], layer["top_k"]
    ids, w = route(logits, k)
    M = ids.shape[0]
    tokens = list(range(M)) if tokens is None else list(tokens)
    x = F.bf16_value(np.asarray(x_bits)[tokens]).astype(np.float64)
    H, I = layer["H"], layer["I"]
    y = np.zeros((len(tokens), H), dtype=np.float64)
    h_all = {}
    sel = ids[tokens]
    experts = sorted(set(int(v) for v in sel.reshape(-1)))

    tier, _ = tier_map(layer["bit_map"], E)

    def run(e):
        rows, cols = np.nonzero(sel == e)
        w13, w2 = expert_weights(layer, e)
        if act_format == "mxfp4" and tier[e] == KEPT:
            h, o = expert_mlp_w4a4(x[rows], w13, w2)
        else:
            h, o = expert_mlp(x[rows], w13, w2)
        return rows, cols, h, o

    def add(result):
        rows, cols, h, o = result
        y[rows] += w[np.asarray(tokens)[rows], cols][:, None] * o
        for r, c, hh in zip(rows, cols, h):
            h_all[int(tokens[r]) * k + int(c)] = hh

    if threads > 1 and len(experts) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            for result in ex.map(run, experts):   # results come back in submission order
                add(result)
    else:
        for e in experts:
            add(run(e))
    return {"ids": ids, "w": w, "h": h_all, "y": y, "tokens": tokens}


# ----------------------------------------------------------------------------
# quantising a whole layer from master weights (synthetic inputs only)
# ----------------------------------------------------------------------------

def quantize_layer(E: int, H: int, I: int, top_k: int, bit_map, kept_format: str, master):
    """Pack every expert of a layer in its tier with the oracle quantisers.
    `master(e)` returns the fp32 (W13 [2I, H], W2 [H, I]) of expert e."""
    from synth import empty_packed_layer
    layer = empty_packed_layer(E, H, I, top_k, kept_format, bit_map)
    tier, local = tier_map(bit_map, E)
    fmt = "nvfp4" if bit_map is None else kept_format
    for e in range(E):
        w13, w2 = master(e)
        j = int(local[e])
        if tier[e] == KEPT:
            d = layer["kept"]
            if fmt == "nvfp4":
                d["w13_q"][j], d["w13_s"][j], d["w13_g"][j] = F.nvfp4_quantize(w13)
                d["w2_q"][j], d["w2_s"][j], d["w2_g"][j] = F.nvfp4_quantize(w2)
            else:
                d["w13_q"][j], d["w13_s"][j] = F.mxfp4_quantize(w13)
                d["w2_q"][j], d["w2_s"][j] = F.mxfp4_quantize(w2)
                d["w13_g"][j] = d["w2_g"][j] = np.float32(1.0)
        else:
            d = layer["nf3"]
            d["w13_q"][j], d["w13_s"][j] = F.nf3_quantize(w13)
            d["w2_q"][j], d["w2_s"][j] = F.nf3_quantize(w2)
    return layer


# ----------------------------------------------------------------------------
# checkpoint-style per-expert tensors and the load-time demux (tier-local arrays)
# ----------------------------------------------------------------------------

def checkpoint_experts(layer: dict):
    """The layer as a checkpoint keeps it: one dict of tensors per global expert e.
    Kept-tier experts hold their rows as the kept tier does (w13_q, w13_s, w13_g,
    w2_q, w2_s, w2_g); NF3 experts hold two code planes per tensor (w13_lo, w13_hi,
    w2_lo, w2_hi, see formats.pack_nf3_planes) and the fp16 group scales (w13_s, w2_s)."""
    tier, local = tier_map(layer["bit_map"], layer["E"])
    out = []
    for e in range(layer["E"]):
        j = int(local[e])
        if tier[e] == KEPT:
            k = layer["kept"]
            out.append({n: np.array(k[n][j]) for n in ("w13_q", "w13_s", "w13_g", "w2_q", "w2_s", "w2_g")})
        else:
            f = layer["nf3"]
            d = {}
            for t in ("w13", "w2"):
                d[t + "_lo"], d[t + "_hi"] = F.pack_nf3_planes(F.unpack_nf3(f[t + "_q"][j]))
                d[t + "_s"] = np.array(f[t + "_s"][j])
            out.append(d)
    return out


def demux(experts, bit_map, E: int, H: int, I: int, top_k: int, kept_format: str):
    """Tier-local arrays from checkpoint-style experts: each expert goes to its tier at
    its tier-local index (experts below it in the same tier, ascending global id); NF3
    code planes become the 3-bit stream of the kernels. The inverse of
    checkpoint_experts."""
    from synth import empty_packed_layer
    layer = empty_packed_layer(E, H, I, top_k, kept_format, bit_map)
    tier, local = tier_map(bit_map, E)
    for e in range(E):
        j, src = int(local[e]), experts[e]
        if tier[e] == KEPT:
            for n in ("w13_q", "w13_s", "w13_g", "w2_q", "w2_s", "w2_g"):
                layer["kept"][n][j] = src[n]
        else:
            for t in ("w13", "w2"):
                layer["nf3"][t + "_q"][j] = F.pack_nf3(F.unpack_nf3_planes(src[t + "_lo"], src[t + "_hi"]))
                layer["nf3"][t + "_s"][j] = src[t + "_s"]
    return layer
