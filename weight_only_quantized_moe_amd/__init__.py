"""Python binding of libhmoe, the hybrid-precision W4A16 fused MoE layer for
AMD MI355X (gfx950).

This module only marshals arguments: every step of the layer runs in the HIP
kernels of ``libhmoe.so``, whose C ABI is declared in ``include/hmoe.h``. The
functions carry the C names. Tensors are torch tensors on the GPU (torch is
used for device memory and for the current HIP stream only). Importing works
without a GPU; calling anything that launches kernels needs one. If the shared
library has not been built, every call raises.

Build the library with ``python -m weight_only_quantized_moe_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, byref, c_char_p, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhmoe.so")

KEPT_NVFP4, KEPT_MXFP4 = 0, 1
DECODE_STAGED, DECODE_SINGLE_LAUNCH = 0, 1
ACT_16BIT, ACT_MXFP4 = 0, 1
TIER_KEPT, TIER_NF3 = 0, 1
TENSOR_W13, TENSOR_W2 = 0, 1
STAGE_ROUTE, STAGE_W13, STAGE_W2, STAGE_COMBINE = 0, 1, 2, 3
DECODE_MAX_M = 8

EXPORTED = (
    "moe_layer_create", "moe_layer_destroy", "moe_layer_query", "moe_scratch_bytes",
    "moe_scratch_init",
    "moe_route", "moe_align", "moe_align_view", "moe_decode_view", "moe_topk_view",
    "hybrid_moe_forward", "hybrid_moe_forward_static", "hybrid_moe_forward_stage", "moe_dequant",
    "moe_repack", "moe_quantize_mxfp4",
    "moe_status_string", "moe_last_error",
)


class HmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class LayerDesc(Structure):
    _fields_ = [("num_experts", c_int32), ("hidden", c_int32), ("inter", c_int32),
                ("top_k", c_int32), ("max_tokens", c_int32), ("kept_format", c_int32),
                ("bit_map", c_void_p), ("block_m", c_int32), ("decode_launch", c_int32),
                ("act_format", c_int32)]


class LayerInfo(Structure):
    _fields_ = [(n, c_int32) for n in (
        "num_experts", "hidden", "inter", "top_k", "max_tokens", "kept_format",
        "num_kept", "num_nf3", "block_m", "max_distinct", "cap_kept", "cap_nf3",
        "fused_decode", "single_launch_available", "act_format")]


class Weights(Structure):
    _fields_ = [(n, c_void_p) for n in (
        "kept_w13_q", "kept_w13_s", "kept_w13_g", "kept_w2_q", "kept_w2_s", "kept_w2_g",
        "nf3_w13_q", "nf3_w13_s", "nf3_w2_q", "nf3_w2_s")]


class ExpertSrc(Structure):
    _fields_ = [(n, c_void_p) for n in (
        "w13_q", "w13_hi", "w13_s", "w13_g", "w2_q", "w2_hi", "w2_s", "w2_g")]


class AlignView(Structure):
    _fields_ = [("sorted_slots", c_void_p), ("block_expert", c_void_p), ("expert_off", c_void_p),
                ("num_padded", c_void_p), ("capacity", c_int32), ("num_experts_tier", c_int32)]


class DecodeView(Structure):
    _fields_ = [("counts", c_void_p), ("experts", c_void_p), ("num_slots", c_void_p),
                ("slots", c_void_p), ("expert_tier", c_void_p), ("passes", c_void_p),
                ("max_distinct", c_int32), ("sync_timeouts", c_void_p)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libhmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m weight_only_quantized_moe_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    st = c_int32
    lib.moe_layer_create.argtypes = [POINTER(LayerDesc), POINTER(c_void_p)]
    lib.moe_layer_create.restype = st
    lib.moe_layer_destroy.argtypes = [c_void_p]
    lib.moe_layer_destroy.restype = None
    lib.moe_layer_query.argtypes = [c_void_p, POINTER(LayerInfo)]
    lib.moe_layer_query.restype = st
    lib.moe_scratch_bytes.argtypes = [c_void_p, POINTER(c_size_t)]
    lib.moe_scratch_bytes.restype = st
    lib.moe_scratch_init.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moe_scratch_init.restype = st
    lib.moe_route.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.moe_route.restype = st
    lib.moe_align.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]
    lib.moe_align.restype = st
    lib.moe_align_view.argtypes = [c_void_p, c_void_p, c_int32, POINTER(AlignView)]
    lib.moe_align_view.restype = st
    lib.moe_decode_view.argtypes = [c_void_p, c_void_p, POINTER(DecodeView)]
    lib.moe_decode_view.restype = st
    lib.moe_topk_view.argtypes = [c_void_p, c_void_p, POINTER(c_void_p), POINTER(c_void_p)]
    lib.moe_topk_view.restype = st
    lib.hybrid_moe_forward.argtypes = [c_void_p, POINTER(Weights), c_void_p, c_void_p, c_int32,
                                       c_void_p, c_void_p, c_size_t, c_void_p]
    lib.hybrid_moe_forward.restype = st
    lib.hybrid_moe_forward_static.argtypes = [c_void_p, POINTER(Weights), c_void_p, c_void_p,
                                              c_int32, c_void_p, c_void_p]
    lib.hybrid_moe_forward_static.restype = st
    lib.hybrid_moe_forward_stage.argtypes = [c_void_p, POINTER(Weights), c_void_p, c_void_p, c_int32,
                                             c_void_p, c_void_p, c_size_t, c_int32, c_void_p]
    lib.hybrid_moe_forward_stage.restype = st
    lib.moe_dequant.argtypes = [c_void_p, POINTER(Weights), c_int32, c_int32, c_void_p, c_void_p,
                                c_void_p]
    lib.moe_dequant.restype = st
    lib.moe_repack.argtypes = [c_void_p, POINTER(ExpertSrc), POINTER(Weights), c_void_p]
    lib.moe_repack.restype = st
    lib.moe_quantize_mxfp4.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.moe_quantize_mxfp4.restype = st
    lib.moe_status_string.argtypes = [c_int32]
    lib.moe_status_string.restype = c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise HmoeError(status, f"{lib.moe_status_string(status).decode()}: "
                                f"{lib.moe_last_error().decode()}")


def _stream(stream):
    if stream is not None:
        return c_void_p(stream)
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


class Layer:
    """Owns one hmoe_layer handle (host memory only)."""

    def __init__(self, handle: c_void_p, bit_map):
        self.handle = handle
        self._bit_map = bit_map   # keeps the host bytes alive for the descriptor's lifetime

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.moe_layer_destroy(self.handle)
            self.handle = None


def moe_layer_create(num_experts: int, hidden: int, inter: int, top_k: int, max_tokens: int,
                     kept_format: int = KEPT_NVFP4, bit_map=None, block_m: int = 0,
                     decode_launch: int = DECODE_STAGED, act_format: int = ACT_16BIT) -> Layer:
    lib = load_library()
    bm = None
    if bit_map is not None:
        bm = (ctypes.c_uint8 * num_experts)(*[int(v) for v in bit_map])
    d = LayerDesc(num_experts, hidden, inter, top_k, max_tokens, kept_format,
                  ctypes.cast(bm, c_void_p) if bm is not None else None, block_m, decode_launch,
                  act_format)
    h = c_void_p()
    _check(lib.moe_layer_create(byref(d), byref(h)))
    return Layer(h, bm)


def moe_layer_query(layer: Layer) -> dict:
    info = LayerInfo()
    _check(load_library().moe_layer_query(layer.handle, byref(info)))
    return {n: getattr(info, n) for n, _ in LayerInfo._fields_}


def moe_scratch_bytes(layer: Layer) -> int:
    n = c_size_t()
    _check(load_library().moe_scratch_bytes(layer.handle, byref(n)))
    return n.value


def moe_scratch_init(layer: Layer, scratch, stream=None) -> None:
    """Zero-fills the scratch's decode counters (not needed for a zero-filled buffer)."""
    _check(load_library().moe_scratch_init(layer.handle, _ptr(scratch),
                                           scratch.numel() * scratch.element_size(),
                                           _stream(stream)))


def moe_route(logits, top_k: int, topk_ids, topk_w, stream=None) -> None:
    M, E = logits.shape
    _check(load_library().moe_route(_ptr(logits), M, E, top_k, _ptr(topk_ids), _ptr(topk_w),
                                    _stream(stream)))


def moe_align(layer: Layer, topk_ids, M: int, scratch, stream=None) -> None:
    _check(load_library().moe_align(layer.handle, _ptr(topk_ids), M, _ptr(scratch),
                                    scratch.numel() * scratch.element_size(), _stream(stream)))


def _scratch_view(scratch, ptr: int, count: int, dtype):
    import torch
    off = ptr - scratch.data_ptr()
    esz = torch.empty((), dtype=dtype).element_size()
    return scratch.view(torch.uint8)[off:off + count * esz].view(dtype)


def moe_align_view(layer: Layer, scratch, tier: int) -> dict:
    """Tensors viewing one tier's align arrays inside `scratch` (full capacity)."""
    import torch
    v = AlignView()
    _check(load_library().moe_align_view(layer.handle, _ptr(scratch), tier, byref(v)))
    bm = moe_layer_query(layer)["block_m"]
    return {
        "sorted_slots": _scratch_view(scratch, v.sorted_slots, v.capacity, torch.int32),
        "block_expert": _scratch_view(scratch, v.block_expert, v.capacity // bm, torch.int32),
        "expert_off": _scratch_view(scratch, v.expert_off, v.num_experts_tier + 1, torch.int32),
        "num_padded": _scratch_view(scratch, v.num_padded, 1, torch.int32),
        "capacity": v.capacity,
    }


def moe_decode_view(layer: Layer, scratch) -> dict:
    import torch
    v = DecodeView()
    _check(load_library().moe_decode_view(layer.handle, _ptr(scratch), byref(v)))
    info = moe_layer_query(layer)
    E, k = info["num_experts"], info["top_k"]
    D = v.max_distinct
    n_pass = DECODE_MAX_M * k
    return {
        "counts": _scratch_view(scratch, v.counts, 2, torch.int32),
        "experts": _scratch_view(scratch, v.experts, D, torch.int32),
        "num_slots": _scratch_view(scratch, v.num_slots, D, torch.int32),
        "slots": _scratch_view(scratch, v.slots, D * DECODE_MAX_M, torch.int32).view(D, DECODE_MAX_M),
        "expert_tier": _scratch_view(scratch, v.expert_tier, E, torch.int32),
        # pass records of the first M * k slots of the last decode forward
        "passes": _scratch_view(scratch, v.passes, n_pass * 4, torch.int32).view(n_pass, 4),
        "sync_timeouts": _scratch_view(scratch, v.sync_timeouts, 1, torch.int32),
    }


def moe_topk_view(layer: Layer, scratch, M: int) -> tuple:
    import torch
    ids, w = c_void_p(), c_void_p()
    _check(load_library().moe_topk_view(layer.handle, _ptr(scratch), byref(ids), byref(w)))
    k = moe_layer_query(layer)["top_k"]
    return (_scratch_view(scratch, ids.value, M * k, torch.int32).view(M, k),
            _scratch_view(scratch, w.value, M * k, torch.float32).view(M, k))


def hybrid_moe_forward(layer: Layer, weights: "DeviceWeights", x, router_logits, y, scratch,
                       stream=None) -> None:
    """y[M, H] (bf16) = the hybrid MoE layer applied to x[M, H] (bf16) routed by
    router_logits[M, E] (fp32)."""
    M = x.shape[0]
    _check(load_library().hybrid_moe_forward(
        layer.handle, byref(weights.struct), _ptr(x), _ptr(router_logits), M, _ptr(y),
        _ptr(scratch), scratch.numel() * scratch.element_size(), _stream(stream)))


def hybrid_moe_forward_static(layer: Layer, weights: "DeviceWeights", x, router_logits, y,
                              stream=None) -> None:
    """hybrid_moe_forward with the library's static per-GPU scratch: allocates nothing;
    calls that overlap on one GPU race (see include/hmoe.h)."""
    M = x.shape[0]
    _check(load_library().hybrid_moe_forward_static(
        layer.handle, byref(weights.struct), _ptr(x), _ptr(router_logits), M, _ptr(y),
        _stream(stream)))


def hybrid_moe_forward_stage(layer: Layer, weights: "DeviceWeights", x, router_logits, y, scratch,
                             stage: int, stream=None) -> None:
    """One stage of hybrid_moe_forward (STAGE_ROUTE, _W13, _W2, _COMBINE, in order)."""
    M = x.shape[0]
    _check(load_library().hybrid_moe_forward_stage(
        layer.handle, byref(weights.struct), _ptr(x), _ptr(router_logits), M, _ptr(y),
        _ptr(scratch), scratch.numel() * scratch.element_size(), stage, _stream(stream)))


def moe_dequant(layer: Layer, weights: "DeviceWeights", expert: int, tensor: int,
                out_f32=None, out_bf16=None, stream=None) -> None:
    _check(load_library().moe_dequant(layer.handle, byref(weights.struct), expert, tensor,
                                      _ptr(out_f32), _ptr(out_bf16), _stream(stream)))


def moe_repack(layer: Layer, experts, dst: "DeviceWeights", stream=None) -> None:
    """Load-time demux/repack (include/hmoe.h): `experts` is a list of E dicts of device
    tensors in the checkpoint layout (kept tier: w13_q, w13_s, w13_g, w2_q, w2_s, w2_g;
    NF3 tier: w13_lo, w13_hi, w13_s, w2_lo, w2_hi, w2_s), written into the tier-local
    arrays of `dst`."""
    info = moe_layer_query(layer)
    if len(experts) != info["num_experts"]:
        raise ValueError(f"moe_repack: {len(experts)} experts given, the layer has "
                         f"{info['num_experts']}")
    arr = (ExpertSrc * len(experts))()
    for i, ex in enumerate(experts):
        nf3 = "w13_lo" in ex
        arr[i] = ExpertSrc(
            _ptr(ex["w13_lo"] if nf3 else ex["w13_q"]), _ptr(ex.get("w13_hi")), _ptr(ex["w13_s"]),
            _ptr(ex.get("w13_g")), _ptr(ex["w2_lo"] if nf3 else ex["w2_q"]), _ptr(ex.get("w2_hi")),
            _ptr(ex["w2_s"]), _ptr(ex.get("w2_g")))
    _check(load_library().moe_repack(layer.handle, arr, byref(dst.struct), _stream(stream)))


def moe_quantize_mxfp4(x, codes, scales, stream=None) -> None:
    """x fp32 [rows, K] -> MXFP4 codes u8 [rows, K/2] and E8M0 scales u8 [rows, K/32]."""
    rows, K = x.shape
    _check(load_library().moe_quantize_mxfp4(_ptr(x), rows, K, _ptr(codes), _ptr(scales),
                                             _stream(stream)))


class DeviceWeights:
    """Packed tier weights on the GPU (torch tensors) plus the hmoe_weights struct
    pointing at them. Built from the packed-layer dict layout (see include/hmoe.h)."""

    KEYS = {"kept": ("w13_q", "w13_s", "w13_g", "w2_q", "w2_s", "w2_g"),
            "nf3": ("w13_q", "w13_s", "w2_q", "w2_s")}

    def __init__(self, packed: dict, device="cuda"):
        import numpy as np
        import torch
        self.tensors = {}
        for tier, keys in self.KEYS.items():
            for k in keys:
                arr = packed[tier][k]
                if arr.size == 0:
                    self.tensors[f"{tier}_{k}"] = None
                    continue
                a = np.ascontiguousarray(arr)
                if a.dtype == np.uint16:
                    a = a.view(np.int16)
                self.tensors[f"{tier}_{k}"] = torch.from_numpy(a).to(device)
        self._rebuild()

    def _rebuild(self):
        self.struct = Weights(*[_ptr(self.tensors[n]) for n, _ in Weights._fields_])

    def clone(self) -> "DeviceWeights":
        """A second device copy of the same bytes (for benchmarks that rotate copies)."""
        other = DeviceWeights.__new__(DeviceWeights)
        other.tensors = {k: (None if v is None else v.clone()) for k, v in self.tensors.items()}
        other._rebuild()
        return other

    def nbytes(self) -> int:
        return sum(0 if v is None else v.numel() * v.element_size() for v in self.tensors.values())
