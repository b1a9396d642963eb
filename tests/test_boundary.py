"""The C-ABI library without a GPU: it loads, exports every function that
include/hmoe.h declares, and its host-only paths (layer creation, validation,
the scratch planner, views into scratch, argument errors) behave as the header
documents. Nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import weight_only_quantized_moe_amd as hm

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hmoe.h")

OK, INVALID, UNSUPPORTED, ALIGN, CAPACITY, SCRATCH, HIP = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)) -
                  {"if", "while", "for"})


def test_library_exports_every_declared_function():
    lib = hm.load_library()
    names = _declared_functions()
    assert set(hm.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert hm.moe_status_string(0) == "HMOE_OK"
    assert hm.moe_status_string(5) == "HMOE_ERR_SCRATCH"


def _create_status(**kw):
    d = dict(num_experts=8, hidden=256, inter=128, top_k=2, max_tokens=16)
    d.update(kw)
    try:
        hm.moe_layer_create(**d)
        return OK
    except hm.HmoeError as e:
        return e.status


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"num_experts": 0}, INVALID),
    ({"top_k": 0}, INVALID),
    ({"top_k": 9}, INVALID),
    ({"max_tokens": 0}, INVALID),
    ({"kept_format": 7}, INVALID),
    ({"block_m": 48}, INVALID),
    ({"decode_launch": 2}, INVALID),
    ({"act_format": 2}, INVALID),
    ({"act_format": 1}, INVALID),                                   # no bit map
    ({"act_format": 1, "bit_map": [4] * 4 + [3] * 4}, INVALID),     # NVFP4 kept tier
    ({"act_format": 1, "bit_map": [4] * 4 + [3] * 4, "kept_format": 1, "decode_launch": 1}, INVALID),
    ({"act_format": 1, "bit_map": [4] * 4 + [3] * 4, "kept_format": 1}, OK),
    ({"hidden": 128, "inter": 128, "decode_launch": 1}, UNSUPPORTED),
    ({"bit_map": [4, 3, 5, 3, 3, 3, 3, 3]}, INVALID),
    ({"num_experts": 2048, "top_k": 2}, UNSUPPORTED),
    ({"num_experts": 32, "top_k": 17}, UNSUPPORTED),
    ({"hidden": 200}, UNSUPPORTED),
    ({"inter": 96}, UNSUPPORTED),
])
def test_create_validation(kw, status):
    assert _create_status(**kw) == status


def test_query_and_tiers():
    bm = [4, 4, 3, 3, 3, 4, 3, 3]
    layer = hm.moe_layer_create(8, 256, 128, 2, 64, hm.KEPT_MXFP4, bm, 16)
    q = hm.moe_layer_query(layer)
    assert q["num_kept"] == 3 and q["num_nf3"] == 5 and q["kept_format"] == hm.KEPT_MXFP4
    assert q["block_m"] == 16 and q["max_distinct"] == 8
    # capacity: M*k slots plus (block_m - 1) padding per expert that can own a slot
    assert q["cap_kept"] == -(-(64 * 2 + 3 * 15) // 16) * 16 and q["cap_nf3"] == -(-(128 + 5 * 15) // 16) * 16
    # no bit map: uniform NVFP4 whatever the kept format says
    q2 = hm.moe_layer_query(hm.moe_layer_create(8, 256, 128, 2, 4, hm.KEPT_MXFP4, None))
    assert q2["kept_format"] == hm.KEPT_NVFP4 and q2["num_nf3"] == 0 and q2["block_m"] == 16


@pytest.mark.parametrize("max_tokens,expect", [(1, 16), (127, 16), (128, 32), (767, 32), (768, 128),
                                               (2048, 128), (4096, 128)])
def test_default_block_m(max_tokens, expect):
    # block_m 0: chosen from t = max_tokens * k / E (here E = 256, k = 8: t = max_tokens / 32)
    layer = hm.moe_layer_create(256, 256, 128, 8, max_tokens, hm.KEPT_NVFP4, None, 0)
    assert hm.moe_layer_query(layer)["block_m"] == expect


def test_scratch_planner_covers_every_region():
    E, H, I, k, M = 256, 6144, 2048, 8, 4096
    layer = hm.moe_layer_create(E, H, I, k, M, hm.KEPT_NVFP4, [4] * 64 + [3] * 192, 32)
    q = hm.moe_layer_query(layer)
    n = hm.moe_scratch_bytes(layer)
    needed = ((q["cap_kept"] + q["cap_nf3"]) * I * 2      # prefill h (fp16)
              + M * k * H * 4                              # per-slot outputs (fp32)
              + 8 * k * H * 4 + 8 * k * I * 4              # decode intermediates (fp32)
              + M * H * 2 + M * 4                          # prefill x as scaled fp16
              + (q["cap_kept"] + q["cap_nf3"]) * 4)        # sorted slots
    assert needed <= n < needed + 64 * 1024 + 16 * (q["cap_kept"] + q["cap_nf3"])
    small = hm.moe_layer_create(E, H, I, k, 8, hm.KEPT_NVFP4, [4] * 64 + [3] * 192, 32)
    assert hm.moe_scratch_bytes(small) < 4 * 1024 * 1024     # decode-only layers stay small


def test_views_are_host_arithmetic():
    layer = hm.moe_layer_create(8, 256, 128, 2, 64, hm.KEPT_NVFP4, [4, 4, 4, 4, 3, 3, 3, 3])
    lib = hm.load_library()
    base = 1 << 40
    v = hm.AlignView()
    assert lib.moe_align_view(layer.handle, ctypes.c_void_p(base), 1, ctypes.byref(v)) == OK
    assert v.num_experts_tier == 4 and v.capacity == hm.moe_layer_query(layer)["cap_nf3"]
    n = hm.moe_scratch_bytes(layer)
    for p in (v.sorted_slots, v.block_expert, v.expert_off, v.num_padded):
        assert base <= p < base + n and (p - base) % 256 == 0
    d = hm.DecodeView()
    assert lib.moe_decode_view(layer.handle, ctypes.c_void_p(base), ctypes.byref(d)) == OK
    assert d.max_distinct == 8
    assert lib.moe_align_view(layer.handle, ctypes.c_void_p(base), 2, ctypes.byref(v)) == INVALID


def test_forward_argument_errors_without_launching():
    lib = hm.load_library()
    layer = hm.moe_layer_create(8, 256, 128, 2, 16, hm.KEPT_NVFP4, [4, 4, 4, 4, 3, 3, 3, 3])
    need = hm.moe_scratch_bytes(layer)
    a = 1 << 40   # never dereferenced: every call below fails before any launch
    w = hm.Weights(*([ctypes.c_void_p(a)] * 10))
    def fwd(M, scratch=a, nbytes=need, x=a, weights=w):
        return lib.hybrid_moe_forward(layer.handle, ctypes.byref(weights), ctypes.c_void_p(x),
                                      ctypes.c_void_p(a), M, ctypes.c_void_p(a), ctypes.c_void_p(scratch),
                                      nbytes, None)
    assert fwd(17) == CAPACITY
    assert fwd(-1) == INVALID
    assert fwd(4, nbytes=need - 1) == SCRATCH
    assert fwd(4, scratch=a + 128) == ALIGN
    assert fwd(4, x=a + 2) == ALIGN
    assert fwd(0) == OK                        # M = 0 is a no-op
    w_bad = hm.Weights(*([ctypes.c_void_p(a)] * 6 + [None] * 4))
    assert fwd(4, weights=w_bad) == INVALID    # NF3 tier arrays missing
    assert "NF3" in hm.moe_last_error()
    assert lib.moe_route(ctypes.c_void_p(a), 4, 8, 9, ctypes.c_void_p(a), ctypes.c_void_p(a), None) == INVALID
    assert lib.moe_route(ctypes.c_void_p(a + 4), 4, 8, 2, ctypes.c_void_p(a), ctypes.c_void_p(a), None) == ALIGN
    assert lib.moe_align(layer.handle, ctypes.c_void_p(a), 17, ctypes.c_void_p(a), need, None) == CAPACITY
    assert lib.moe_dequant(layer.handle, ctypes.byref(w), 8, 0, ctypes.c_void_p(a), None, None) == INVALID
    assert lib.moe_dequant(layer.handle, ctypes.byref(w), 0, 2, ctypes.c_void_p(a), None, None) == INVALID
    assert lib.moe_dequant(layer.handle, ctypes.byref(w), 0, 0, None, None, None) == INVALID


def test_repack_argument_errors_without_launching():
    """moe_repack validates on the host before any copy: a NULL expert table or NULL
    destination arrays of a non-empty tier are argument errors."""
    lib = hm.load_library()
    layer = hm.moe_layer_create(8, 256, 128, 2, 16, hm.KEPT_NVFP4,
                                np.array([4, 4, 3, 3, 4, 3, 4, 3], np.uint8), 0)
    w = hm.Weights()
    assert lib.moe_repack(layer.handle, None, ctypes.byref(w), None) == INVALID
    src = (hm.ExpertSrc * 8)()
    assert lib.moe_repack(layer.handle, src, ctypes.byref(w), None) == INVALID
    assert lib.moe_repack(None, src, ctypes.byref(w), None) == INVALID


def test_static_forward_rejects_layers_beyond_its_scratch():
    """hybrid_moe_forward_static checks the layer's scratch plan against its fixed array
    before any device call: a GLM-class prefill layer (hundreds of MiB) is refused."""
    lib = hm.load_library()
    layer = hm.moe_layer_create(256, 6144, 2048, 8, 4096)
    assert hm.moe_scratch_bytes(layer) > (64 << 20)
    w = hm.Weights()
    st = lib.hybrid_moe_forward_static(layer.handle, ctypes.byref(w), None, None, 16, None, None)
    assert st == SCRATCH
    assert "static scratch" in hm.moe_last_error()
