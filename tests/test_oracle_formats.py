"""Pins of the oracle's number formats against things other than itself:
published value tables (tests/golden), library conversions (torch float8 /
bfloat16 casts, numpy float16, scipy's normal quantile), closed forms and
brute force."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- decoders

def test_fp32_subnormals_are_not_flushed():
    # the canonical E8M0 byte 0 (2^-127) and E2M1 * 2^-127 products are fp32
    # subnormals; the oracle's arithmetic must keep them
    a = np.float32(2.0 ** -127)
    assert a != 0 and a * np.float32(0.5) == np.float32(2.0 ** -128)


def test_e2m1_matches_ocp_table():
    rows = _golden("e2m1_ocp_mx_v1.txt")
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows], dtype=np.float32)
    got = F.e2m1_value(codes)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))  # includes -0.0


def test_e4m3_matches_torch_all_codes_and_ocp_edges():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = F.e4m3_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok].view(np.uint32), got[ok].view(np.uint32))
    for code, val in _golden("e4m3_ocp_ofp8_edges.txt"):
        v = F.e4m3_value(int(code, 16))
        if val == "nan":
            assert np.isnan(v)
        else:
            assert np.float32(v).view(np.uint32) == np.float32(float(val)).view(np.uint32)


def test_e8m0_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    got = F.e8m0_value(b)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255].view(np.uint32), got[:255].view(np.uint32))
    assert got[127] == 1.0 and got[0] == np.float32(2.0 ** -127)


def test_fp16_and_bf16_widening():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = F.fp16_value(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(f16[ok].view(np.uint32), ref[ok].view(np.uint32))
    bf = F.bf16_value(bits)
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ok = ~np.isnan(refb)
    assert np.array_equal(bf[ok].view(np.uint32), refb[ok].view(np.uint32))


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(1)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32),
        np.ldexp(r.standard_normal(20000), r.integers(-140, 120, 20000)).astype(np.float32),
        # exact ties between bf16 neighbours, both parities
        ((np.arange(1, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.4e38, -3.4e38, 1e-45], dtype=np.float32),
    ])
    got = F.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- NF codebook

def test_nf4_construction_reproduces_qlora_table():
    want = np.array([float(r[0]) for r in _golden("nf4_qlora.txt")])
    got = F.nf_codebook(4).astype(np.float64)
    # the published table was produced with a different normal-quantile
    # routine and fp32 intermediates; agreement to ~1e-7 pins the recipe
    assert np.max(np.abs(got - want)) < 3e-7
    assert got[0] == -1.0 and got[-1] == 1.0 and got[7] == 0.0


def test_nf3_invariants():
    cb = F.NF3
    assert cb.dtype == np.float32 and cb.size == 8
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[-1] == 1.0
    assert np.sum(cb == 0.0) == 1 and F.NF3_ZERO == 3
    assert np.sum(cb < 0) == 3 and np.sum(cb > 0) == 4


def test_nf3_matches_scipy_quantiles():
    from scipy.stats import norm
    k = 3
    n = 2 ** k
    offset = 1 - 0.5 * (1 / (2 * n) + 1 / (2 * (n - 1)))
    pos = norm.ppf(np.linspace(offset, 0.5, n // 2 + 1)[:-1])
    neg = -norm.ppf(np.linspace(offset, 0.5, n // 2)[:-1])
    v = np.sort(np.concatenate([pos, neg, [0.0]]))
    v = (v / np.abs(v).max()).astype(np.float32)
    assert np.array_equal(v.view(np.uint32), F.NF3.view(np.uint32))
    # the table quoted with the spec of this layer (fp32 bit patterns)
    want = [0xBF800000, 0xBF08F740, 0xBE7CDB98, 0x00000000,
            0x3E3BBCD2, 0x3EC394B6, 0x3F1F7BFE, 0x3F800000]
    assert list(F.NF3.view(np.uint32)) == want


# ---------------------------------------------------------------- rounding

def test_e2m1_round_tie_table_and_saturation():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, code in ties.items():
        assert int(F.e2m1_round(v)) == code, v
        assert int(F.e2m1_round(-v)) == (code | 8 if code else 0), -v
    assert int(F.e2m1_round(7.0)) == 7 and int(F.e2m1_round(-1e9)) == 15
    assert int(F.e2m1_round(-0.0)) == 0 and int(F.e2m1_round(-0.1)) == 0


def test_e2m1_round_is_nearest_by_brute_force():
    r = np.random.default_rng(2)
    t = r.uniform(-7, 7, 100000)
    codes = F.e2m1_round(t)
    vals = F.e2m1_value(codes).astype(np.float64)
    grid = F.e2m1_value(np.arange(16)).astype(np.float64)
    best = np.min(np.abs(np.clip(t, -6, 6)[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(np.clip(t, -6, 6) - vals), best, rtol=0, atol=0)
    assert not np.any(codes == 8)


def test_e4m3_round_matches_torch_cast():
    r = np.random.default_rng(3)
    mids = ((F.e4m3_value(np.arange(0, 0x7E)).astype(np.float64)
             + F.e4m3_value(np.arange(1, 0x7F)).astype(np.float64)) / 2)
    v = np.concatenate([r.uniform(0, 448, 50000), r.uniform(0, 2 ** -5, 50000),
                        mids, -mids, [0.0, 448.0]]).astype(np.float32)
    got = F.e4m3_round(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    with pytest.raises(ValueError):
        F.e4m3_round(np.array([449.0]))


# ---------------------------------------------------------------- packing

def test_fp4_packing_hand_vector_and_roundtrip():
    assert F.pack_fp4(np.array([[1, 2, 15, 0]])).tolist() == [[0x21, 0x0F]]
    r = np.random.default_rng(4)
    c = r.integers(0, 16, (7, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_fp4(F.pack_fp4(c)), c)


def test_nf3_packing_hand_vector_and_roundtrip():
    # element j at bits [3j, 3j+3) of a little-endian stream:
    # 1 | 2<<3 | 3<<6 | 4<<9 | 5<<12 | 6<<15 | 7<<18 | 0<<21 = 0x1F58D1
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 0]])
    assert F.pack_nf3(q).tolist() == [[0xD1, 0x58, 0x1F]]
    one = np.zeros((1, 64), np.int64)
    one[0, 21] = 7          # bits 63..65 straddle bytes 7 and 8
    p = F.pack_nf3(one)
    assert p[0, 7] == 0x80 and p[0, 8] == 0x03 and p.sum() == 0x83
    r = np.random.default_rng(5)
    c = r.integers(0, 8, (5, 128)).astype(np.uint8)
    assert np.array_equal(F.unpack_nf3(F.pack_nf3(c)), c)


# ---------------------------------------------------------------- quantisers

def _blocks(x, n):
    return x.reshape(x.shape[0], -1, n)


def test_nvfp4_quantiser_pins():
    r = np.random.default_rng(6)
    T = (r.standard_normal((32, 256)) * 0.02).astype(np.float32)
    T[3, 16:32] = 0.0                                  # a zero block
    q, s, g = F.nvfp4_quantize(T)
    amax = np.abs(T).max()
    assert g == np.float32(np.float32(amax) / np.float32(2688))
    # the block holding the tensor's absmax gets the largest scale, 448
    i, j = np.unravel_index(np.argmax(np.abs(T)), T.shape)
    assert s[i, j // 16] == 0x7E
    assert np.all(F.unpack_fp4(q)[3, 16:32] == 0)
    # every element is within half a grid step of its decoded value
    w = F.nvfp4_dequant(q, s, g).astype(np.float64)
    unit = np.repeat(F.e4m3_value(s).astype(np.float64) * g, 16, axis=1)
    t = np.abs(T) / np.where(unit > 0, unit, 1)
    half_step = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    assert np.all(np.abs(T - w) <= half_step * unit * (1 + 1e-6) + 1e-12)
    # idempotence: requantising the decoded values with the same scales gives
    # back the same codes
    codes = F.unpack_fp4(q)
    unit32 = np.repeat((F.e4m3_value(s) * g).astype(np.float32), 16, axis=1)
    w32 = w.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t2 = np.where(unit32 > 0, w32 / unit32, np.float32(0))
    live = unit32 > 0
    assert np.array_equal(F.e2m1_round(t2)[live], codes[live])


def test_nvfp4_all_zero_tensor():
    q, s, g = F.nvfp4_quantize(np.zeros((4, 32), np.float32))
    assert g == 1.0 and not q.any() and not s.any()


def test_mxfp4_quantiser_pins():
    r = np.random.default_rng(7)
    T = (r.standard_normal((16, 256)) * 0.02).astype(np.float32)
    T[2, :32] = 0.0
    T[5, 32:64] *= 1e6
    q, s = F.mxfp4_quantize(T)
    for row in range(16):
        for b in range(8):
            blk = T[row, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            if amax == 0:
                assert s[row, b] == 127
            else:
                assert int(s[row, b]) - 127 == math.floor(math.log2(amax)) - 2
    w = F.mxfp4_dequant(q, s).astype(np.float64)
    X = np.repeat(F.e8m0_value(s).astype(np.float64), 32, axis=1)
    t = np.abs(T) / X
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    err = np.abs(T - w)
    sat = t > 6
    assert np.all(err[~sat] <= half[~sat] * X[~sat] * (1 + 1e-12))
    assert np.all(np.abs(w[sat]) == 6 * X[sat])


def test_nf3_quantiser_is_nearest_level():
    r = np.random.default_rng(8)
    T = (r.standard_normal((16, 256)) * 0.02).astype(np.float32)
    T[1, 64:128] = 0.0
    q, s = F.nf3_quantize(T)
    codes = F.unpack_nf3(q).astype(np.int64)
    sd = np.repeat(F.fp16_value(s), 64, axis=1)
    assert np.all(codes[1, 64:128] == F.NF3_ZERO)
    assert np.array_equal(F.fp16_value(s), np.minimum(np.abs(T).reshape(16, 4, 64).max(2), 65504).astype(np.float16).astype(np.float32))
    t = (T / np.where(sd > 0, sd, 1)).astype(np.float32).astype(np.float64)
    d = np.abs(t[..., None] - F.NF3.astype(np.float64)[None, None, :])
    nearest = np.argmin(d, axis=-1)           # ties -> lower index, like the oracle
    ok = sd > 0
    assert np.array_equal(codes[ok], nearest[ok])
    half_gap = np.max(np.diff(F.NF3.astype(np.float64))) / 2
    assert np.all(np.abs(F.nf3_value(codes) - t)[ok] <= half_gap + 1e-7)


def test_dequant_closed_forms():
    # NVFP4: code 7 (6.0) with scale 0x7E (448) and g = 1 -> 2688
    assert F.nvfp4_dequant(np.array([[0x07] + [0] * 7]), np.array([[0x7E]]), 1.0)[0, 0] == 2688.0
    # subnormal E4M3 scale 0x01 (2^-9) times code 1 (0.5) -> 2^-10
    assert F.nvfp4_dequant(np.array([[0x01] + [0] * 7]), np.array([[0x01]]), 1.0)[0, 0] == 2.0 ** -10
    # one rounding by g: 1.5 * 1.125 * g
    g = np.float32(1.0 / 3.0)
    w = F.nvfp4_dequant(np.array([[0x03] + [0] * 7]), np.array([[0x39]]), g)[0, 0]
    assert w == np.float32(np.float64(1.5 * 1.125) * np.float64(g))
    # negative zero survives
    assert np.signbit(F.nvfp4_dequant(np.array([[0x08] + [0] * 7]), np.array([[0x38]]), 1.0)[0, 0])
    # MXFP4 with E8M0 byte 0: 0.5 * 2^-127 = 2^-128 (fp32 subnormal)
    assert F.mxfp4_dequant(np.array([[0x01] + [0] * 15]), np.array([[0]]))[0, 0] == np.float32(2.0 ** -128)
    # NF3: level 7 (1.0) times fp16 scale 0.5
    q = F.pack_nf3(np.array([[7] + [3] * 63]))
    assert F.nf3_dequant(q, np.array([[0x3800]], np.uint16))[0, 0] == 0.5


# ---------------------------------------------------------------- NF3 checkpoint planes

def test_nf3_planes_hand_bit_positions():
    """Element j alone at code c: the low plane holds c & 3 at bits 2 (j mod 4) of byte
    j / 4, the high plane c >> 2 at bit j mod 8 of byte j / 8."""
    K = 64
    for j in (0, 3, 4, 7, 8, 13, 31, 63):
        for c in (1, 2, 3, 4, 5, 7):
            q = np.zeros((1, K), dtype=np.uint8)
            q[0, j] = c
            lo, hi = F.pack_nf3_planes(q)
            exp_lo = np.zeros(K // 4, dtype=np.uint8)
            exp_lo[j // 4] = (c & 3) << (2 * (j % 4))
            exp_hi = np.zeros(K // 8, dtype=np.uint8)
            exp_hi[j // 8] = (c >> 2) << (j % 8)
            assert np.array_equal(lo[0], exp_lo) and np.array_equal(hi[0], exp_hi), (j, c)
            assert np.array_equal(F.unpack_nf3_planes(lo, hi), q)


def test_nf3_planes_round_trip_random():
    q = np.random.default_rng(7).integers(0, 8, (3, 4, 192)).astype(np.uint8)
    assert np.array_equal(F.unpack_nf3_planes(*F.pack_nf3_planes(q)), q)
