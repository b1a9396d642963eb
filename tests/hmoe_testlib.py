"""Helpers shared by the GPU parity tests: device upload, running the HIP path
through the C ABI, and the output tolerance of the layer."""
from __future__ import annotations

import numpy as np

import synth
from oracle import formats as F
from oracle import layer as OL


def torch_mod():
    import torch
    return torch


def fmt_code(packed: dict) -> int:
    import weight_only_quantized_moe_amd as hm
    return hm.KEPT_NVFP4 if OL.kept_format_of(packed) == "nvfp4" else hm.KEPT_MXFP4


def make_layer(packed: dict, max_tokens: int, block_m: int = 0, decode_launch: int = 0,
               act_format: int = 0):
    import weight_only_quantized_moe_amd as hm
    return hm.moe_layer_create(packed["E"], packed["H"], packed["I"], packed["top_k"], max_tokens,
                               fmt_code(packed), packed["bit_map"], block_m, decode_launch,
                               act_format)


def scratch_for(layer):
    import weight_only_quantized_moe_amd as hm
    torch = torch_mod()
    n = hm.moe_scratch_bytes(layer)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def to_dev_bits(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_forward(layer, weights, x_bits: np.ndarray, logits: np.ndarray, scratch=None):
    """Runs hybrid_moe_forward; returns (y bf16 bits as numpy uint16, scratch)."""
    import weight_only_quantized_moe_amd as hm
    torch = torch_mod()
    scratch = scratch_for(layer) if scratch is None else scratch
    x = to_dev_bits(x_bits)
    lg = to_dev(logits.astype(np.float32))
    y = torch.empty(x.shape, dtype=torch.int16, device="cuda")
    hm.hybrid_moe_forward(layer, weights, x, lg, y, scratch)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16), scratch


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers (8 significant bits) at the binade of each value
    of v: the largest error of rounding a real number to nearest into that binade."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(e, -125) - 9)


def check_output(y_bits: np.ndarray, y_ref: np.ndarray, what: str = "") -> dict:
    """The layer-output bar, with RMS = sqrt(mean(y_ref^2)): max err <= 2e-2 RMS and at
    most 1e-3 of the elements with err > 1e-2 RMS, where err is the part of |y - y_ref|
    beyond the half-ulp rounding of y to its bf16 output format. The output format alone
    would exceed the bar wherever |y| is large (at |y| in [16, 32) its rounding is up to
    0.0625), so the bar measures the computation's error before that rounding. The raw
    |y - y_ref| statistics are returned as well."""
    y = F.bf16_value(y_bits).astype(np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    raw = np.abs(y - ref)
    err = np.maximum(raw - bf16_half_ulp(y), 0.0)
    stats = {"rms": rms, "max_err_rel": float(err.max() / rms),
             "frac_gt_1e-2": float(np.mean(err > 1e-2 * rms)),
             "raw_max_err_rel": float(raw.max() / rms),
             "raw_frac_gt_1e-2": float(np.mean(raw > 1e-2 * rms))}
    assert rms > 0, f"{what}: zero reference"
    assert stats["max_err_rel"] <= 2e-2, f"{what}: {stats}"
    assert stats["frac_gt_1e-2"] <= 1e-3, f"{what}: {stats}"
    return stats


def tiny_packed(kept_format="nvfp4", bit_map="prefix", E=8, H=256, I=128, k=2, seed=0):
    """The tiny config, quantised by the oracle quantisers from N(0, 0.02) masters."""
    w = synth.Workload("tiny", E, H, I, k, 4, kept_format, 4 if bit_map == "prefix" else None,
                       bit_map if bit_map else "none", seed=seed)
    bm = synth.bit_map(w)
    return OL.quantize_layer(E, H, I, k, bm, kept_format, lambda e: synth.master_weights(w, e)), w
