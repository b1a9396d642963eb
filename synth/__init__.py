"""Seeded synthetic inputs for the hybrid W4A16 MoE layer.

This module only draws random numbers and lays them out in the byte formats the
layer consumes. It contains none of the layer's arithmetic (no decoding,
quantisation, routing or matrix work), so both the CPU oracle and the HIP path
can take their inputs from it without sharing any of the method.

Workloads (shapes from the hybrid NVFP4/NF3 serving pages: a 256-expert
GLM-class layer with a 64-expert kept tier and a 192-expert NF3 tail, and a
smaller 128-expert Qwen3-MoE-shaped layer):

  tiny          E=8,   H=256,  I=128,  k=2,  experts 0-3 kept (NVFP4), 4-7 NF3
  qwen_decode   E=128, H=2048, I=768,  k=8,  32 random experts kept, M in 1..8
  glm           E=256, H=6144, I=2048, k=8,  top-64 experts by a synthetic
                saliency score kept

Every array is drawn from numpy's PCG64 with a SeedSequence key
``[seed, stream, ...]`` so that any expert or token block can be regenerated on
its own, in any order, on any machine.

Packed weight container (a plain dict, the contract between generator, oracle
and the HIP binding):

  {"E", "H", "I", "top_k", "kept_format": "nvfp4" | "mxfp4",
   "bit_map": uint8[E] (4 = kept tier, 3 = NF3 tier) or None (uniform kept),
   "kept": {"w13_q": u8[E4, 2I, H/2], "w13_s": u8[E4, 2I, H/B], "w13_g": f32[E4],
            "w2_q":  u8[E4, H, I/2],  "w2_s":  u8[E4, H, I/B],  "w2_g":  f32[E4]},
   "nf3":  {"w13_q": u8[E3, 2I, 3H/8], "w13_s": u16[E3, 2I, H/64],
            "w2_q":  u8[E3, H, 3I/8],  "w2_s":  u16[E3, H, I/64]}}

B is 16 (E4M3 scales) for NVFP4 and 32 (E8M0 scales) for MXFP4; the "_g"
arrays are all ones for MXFP4 and unused. Tier-local arrays hold the experts of
that tier in ascending global id. W13 rows [0, I) are the gate projection and
rows [I, 2I) the up projection; K is the contiguous last axis everywhere.

Byte layouts: FP4 codes hold element 2j in the low nibble of byte j; NF3 codes
are a little-endian bit stream with element j at bits [3j, 3j+3) of its row;
NF3 scales are IEEE fp16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# stream ids of the SeedSequence keys
_S_MASTER = 1
_S_X = 2
_S_LOGITS = 3
_S_BIAS = 4
_S_BITMAP = 5
_S_PACKED = 6


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int
    H: int
    I: int
    top_k: int
    M: int
    kept_format: str = "nvfp4"
    n_kept: int | None = None      # None -> uniform kept tier (no bit map)
    bitmap_rule: str = "prefix"     # "prefix" | "random" | "saliency" | "none"
    logit_bias: bool = False
    seed: int = 0


def tiny(M: int = 4) -> Workload:
    return Workload("tiny", 8, 256, 128, 2, M, "nvfp4", 4, "prefix")


def qwen_decode(M: int = 8) -> Workload:
    return Workload(f"qwen_decode_m{M}", 128, 2048, 768, 8, M, "nvfp4", 32, "random")


def glm_decode(M: int = 8) -> Workload:
    return Workload(f"glm_decode_m{M}", 256, 6144, 2048, 8, M, "nvfp4", 64, "saliency")


def glm_prefill(M: int = 4096) -> Workload:
    return Workload(f"glm_prefill_m{M}", 256, 6144, 2048, 8, M, "nvfp4", 64, "saliency",
                    logit_bias=True)


def glm_mxfp4(M: int = 512) -> Workload:
    return Workload(f"glm_mxfp4_m{M}", 256, 6144, 2048, 8, M, "mxfp4", 64, "saliency")


def glm_uniform(M: int = 512) -> Workload:
    """Control: the same GLM-class layer with no bit map (uniform NVFP4)."""
    return Workload(f"glm_uniform_m{M}", 256, 6144, 2048, 8, M, "nvfp4", None, "none")


# ----------------------------------------------------------------------------
# tier assignment
# ----------------------------------------------------------------------------

def bit_map(w: Workload) -> np.ndarray | None:
    """uint8[E] of 4 (kept) / 3 (NF3), or None for a uniform kept-tier layer."""
    if w.n_kept is None or w.bitmap_rule == "none":
        return None
    bm = np.full(w.E, 3, dtype=np.uint8)
    if w.bitmap_rule == "prefix":
        bm[: w.n_kept] = 4
    elif w.bitmap_rule == "random":
        bm[_rng(w.seed, _S_BITMAP).permutation(w.E)[: w.n_kept]] = 4
    elif w.bitmap_rule == "saliency":
        sal = _rng(w.seed, _S_BITMAP).standard_normal(w.E)
        bm[np.argsort(-sal, kind="stable")[: w.n_kept]] = 4
    else:
        raise ValueError(w.bitmap_rule)
    return bm


# ----------------------------------------------------------------------------
# activations and router logits
# ----------------------------------------------------------------------------

def activations_f32(w: Workload, M: int | None = None) -> np.ndarray:
    """N(0,1) fp32 draws [M, H]; rows are a prefix of one max-size draw per seed."""
    M = w.M if M is None else M
    return _rng(w.seed, _S_X, w.H).standard_normal((M, w.H), dtype=np.float32)


def activations_bf16(w: Workload, M: int | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16 [M, H]) of the N(0,1) draws, rounded by torch."""
    import torch
    x = torch.from_numpy(activations_f32(w, M))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def router_logits(w: Workload, M: int | None = None) -> np.ndarray:
    """fp32 [M, E] router logits N(0,1), plus a per-expert N(0,1) bias when the
    workload asks for skewed expert load (the bias is added here, in fp32, so the
    layer receives already-biased logits)."""
    M = w.M if M is None else M
    lg = _rng(w.seed, _S_LOGITS, w.E).standard_normal((M, w.E), dtype=np.float32)
    if w.logit_bias:
        b = _rng(w.seed, _S_BIAS, w.E).standard_normal(w.E, dtype=np.float32)
        lg = (lg + b[None, :]).astype(np.float32)
    return lg


def master_weights(w: Workload, e: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 N(0, 0.02) master weights of expert e: W13 [2I, H], W2 [H, I]."""
    r = _rng(w.seed, _S_MASTER, e)
    w13 = (r.standard_normal((2 * w.I, w.H), dtype=np.float32) * np.float32(0.02))
    w2 = (r.standard_normal((w.H, w.I), dtype=np.float32) * np.float32(0.02))
    return w13, w2


# ----------------------------------------------------------------------------
# directly drawn packed weights (no quantiser involved)
# ----------------------------------------------------------------------------
# Code bytes are uniform (every FP4 nibble and every 3-bit NF3 field is a valid
# code, so uniform bytes are uniform codes, including the FP4 negative zero).
# Scale bytes are drawn from the ranges a block-absmax quantiser produces for
# N(0, 0.02) weights, so that dequantised weights have that magnitude:
#   E4M3 block scales: codes 0x70..0x7E (128 .. 448), global scale ~ 4e-5
#   E8M0 block scales: bytes 118..121 (2^-9 .. 2^-6)
#   NF3 group scales:  fp16 values uniform in [0.035, 0.065]
_E4M3_LO, _E4M3_HI = 0x70, 0x7E
_E8M0_LO, _E8M0_HI = 118, 121


def _packed_kept_expert(seed: int, e: int, rows: int, K: int, fmt: str, which: int):
    r = _rng(seed, _S_PACKED, e, which)
    q = r.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    if fmt == "nvfp4":
        s = r.integers(_E4M3_LO, _E4M3_HI + 1, size=(rows, K // 16), dtype=np.uint8)
        g = np.float32(r.uniform(3.0e-5, 5.0e-5))
    else:
        s = r.integers(_E8M0_LO, _E8M0_HI + 1, size=(rows, K // 32), dtype=np.uint8)
        g = np.float32(1.0)
    return q, s, g


def _packed_nf3_expert(seed: int, e: int, rows: int, K: int, which: int):
    r = _rng(seed, _S_PACKED, e, which)
    q = r.integers(0, 256, size=(rows, 3 * K // 8), dtype=np.uint8)
    s = r.uniform(0.035, 0.065, size=(rows, K // 64)).astype(np.float16).view(np.uint16)
    return q, s


def packed_layer(w: Workload, threads: int | None = None) -> dict:
    """Packed tier-local weights drawn directly (see the module docstring)."""
    bm = bit_map(w)
    kept_ids = list(range(w.E)) if bm is None else [e for e in range(w.E) if bm[e] == 4]
    nf3_ids = [] if bm is None else [e for e in range(w.E) if bm[e] == 3]
    E4, E3 = len(kept_ids), len(nf3_ids)
    H, I = w.H, w.I
    fmt = "nvfp4" if bm is None else w.kept_format
    B = 16 if fmt == "nvfp4" else 32
    kept = {
        "w13_q": np.empty((E4, 2 * I, H // 2), np.uint8),
        "w13_s": np.empty((E4, 2 * I, H // B), np.uint8),
        "w13_g": np.empty((E4,), np.float32),
        "w2_q": np.empty((E4, H, I // 2), np.uint8),
        "w2_s": np.empty((E4, H, I // B), np.uint8),
        "w2_g": np.empty((E4,), np.float32),
    }
    nf3 = {
        "w13_q": np.empty((E3, 2 * I, 3 * H // 8), np.uint8),
        "w13_s": np.empty((E3, 2 * I, H // 64), np.uint16),
        "w2_q": np.empty((E3, H, 3 * I // 8), np.uint8),
        "w2_s": np.empty((E3, H, I // 64), np.uint16),
    }

    def fill_kept(j):
        e = kept_ids[j]
        kept["w13_q"][j], kept["w13_s"][j], kept["w13_g"][j] = _packed_kept_expert(
            w.seed, e, 2 * I, H, fmt, 0)
        kept["w2_q"][j], kept["w2_s"][j], kept["w2_g"][j] = _packed_kept_expert(
            w.seed, e, H, I, fmt, 1)

    def fill_nf3(j):
        e = nf3_ids[j]
        nf3["w13_q"][j], nf3["w13_s"][j] = _packed_nf3_expert(w.seed, e, 2 * I, H, 0)
        nf3["w2_q"][j], nf3["w2_s"][j] = _packed_nf3_expert(w.seed, e, H, I, 1)

    nthr = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill_kept, range(E4)))
        list(ex.map(fill_nf3, range(E3)))
    return {"E": w.E, "H": H, "I": I, "top_k": w.top_k, "kept_format": fmt,
            "bit_map": bm, "kept": kept, "nf3": nf3}


def empty_packed_layer(E: int, H: int, I: int, top_k: int, kept_format: str,
                       bm: np.ndarray | None) -> dict:
    """A zero-filled container with the right shapes (filled by a quantiser)."""
    kept_n = E if bm is None else int(np.sum(bm == 4))
    nf3_n = 0 if bm is None else int(np.sum(bm == 3))
    fmt = "nvfp4" if bm is None else kept_format
    B = 16 if fmt == "nvfp4" else 32
    return {
        "E": E, "H": H, "I": I, "top_k": top_k, "kept_format": fmt, "bit_map": bm,
        "kept": {
            "w13_q": np.zeros((kept_n, 2 * I, H // 2), np.uint8),
            "w13_s": np.zeros((kept_n, 2 * I, H // B), np.uint8),
            "w13_g": np.ones((kept_n,), np.float32),
            "w2_q": np.zeros((kept_n, H, I // 2), np.uint8),
            "w2_s": np.zeros((kept_n, H, I // B), np.uint8),
            "w2_g": np.ones((kept_n,), np.float32),
        },
        "nf3": {
            "w13_q": np.zeros((nf3_n, 2 * I, 3 * H // 8), np.uint8),
            "w13_s": np.zeros((nf3_n, 2 * I, H // 64), np.uint16),
            "w2_q": np.zeros((nf3_n, H, 3 * I // 8), np.uint8),
            "w2_s": np.zeros((nf3_n, H, I // 64), np.uint16),
        },
    }


def tier_lists(bm: np.ndarray | None, E: int) -> tuple[list[int], list[int]]:
    """Global ids of the kept and NF3 experts, each ascending (no arithmetic)."""
    if bm is None:
        return list(range(E)), []
    return [e for e in range(E) if bm[e] == 4], [e for e in range(E) if bm[e] == 3]
