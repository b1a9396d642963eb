"""Oracle number formats: value decoding, rounding, quantisers, packing, dequant.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import this).

Every decoder is the bit-field definition of its format written out; every
quantiser follows the block-absmax recipe of its format in the order the
format's documentation gives it. Dequantised values are fp32 and are the
bit-exact targets of the HIP dequantisation routines.
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

# ----------------------------------------------------------------------------
# element and scale decoders
# ----------------------------------------------------------------------------

def e2m1_value(code) -> np.ndarray:
    """FP4 E2M1 (OCP MX v1.0, FP4 element type): bit 3 sign, bits 2..1 exponent
    (bias 1), bit 0 mantissa. Exponent 0 is subnormal: 0.5 * m. No inf/NaN.
    Code 8 decodes to -0.0."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1)))
    return (sign * mag).astype(np.float32)


def e4m3_value(b) -> np.ndarray:
    """FP8 E4M3 "fn" (OCP 8-bit floating point): bit 7 sign, bits 6..3 exponent
    (bias 7), bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); the
    all-ones exponent+mantissa pattern (0x7F / 0xFF) is NaN; no infinities."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    out = sign * mag
    out = np.where((b & 0x7F) == 0x7F, np.nan, out)
    return out.astype(np.float32)


def e8m0_value(b) -> np.ndarray:
    """E8M0 scale (OCP MX v1.0): 2^(b - 127); 0xFF is NaN. Byte 0 is 2^-127,
    an fp32 subnormal."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(np.ones(b.shape), b - 127)
    out = np.where(b == 255, np.nan, out)
    return out.astype(np.float32)


def fp16_value(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> fp32 (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_value(bits) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 (exact widening: the bits become the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """Round fp32 to bfloat16 with round-to-nearest-even; returns the bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = np.where(np.isnan(x), 0x7FC0, rounded)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------
# rounding into the element / scale formats (oracle quantisers only)
# ----------------------------------------------------------------------------

_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(t) -> np.ndarray:
    """Nearest E2M1 code to t, saturating at +-6. A tie between two
    neighbouring magnitudes goes to the one with mantissa bit 0 (the even code
    index), i.e. IEEE round-to-nearest-even on the E2M1 grid. A zero magnitude
    is always emitted as code 0 (never the negative zero code 8)."""
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), 6.0)
    lo = np.searchsorted(_E2M1_MAG, a, side="right") - 1
    hi = np.minimum(lo + 1, 7)
    d_lo = a - _E2M1_MAG[lo]
    d_hi = _E2M1_MAG[hi] - a
    take_hi = (hi != lo) & ((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)))
    mag = np.where(take_hi, hi, lo).astype(np.int64)
    neg = (t < 0) & (mag != 0)
    return (mag | (neg.astype(np.int64) << 3)).astype(np.uint8)


def e4m3_round(v) -> np.ndarray:
    """Round finite |v| <= 448 to the nearest E4M3 "fn" code (RNE). Values are
    counted in quanta of their binade (2^(E-3), with E >= -6 so that the
    subnormal quantum is 2^-9); a carry into the next binade is re-encoded."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448.0) or np.any(~np.isfinite(a)):
        raise ValueError("e4m3_round expects finite |v| <= 448 (clamp first)")
    _, ex = np.frexp(a)
    E = np.maximum(ex - 1, -6)
    n = np.rint(a / np.ldexp(1.0, E - 3))           # quanta, ties to even
    val = n * np.ldexp(1.0, E - 3)
    _, ex2 = np.frexp(val)
    E2 = ex2 - 1
    normal = val >= 2.0 ** -6
    mant = np.where(normal, np.rint(np.ldexp(val, -np.where(normal, E2, 0)) * 8.0 - 8.0), 0)
    code = np.where(normal, ((E2 + 7) << 3) | mant.astype(np.int64),
                    np.rint(val / 2.0 ** -9).astype(np.int64))
    code = np.where(val == 0, 0, code)
    sign = np.signbit(v)          # IEEE: a negative value that rounds to 0 is -0
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


# ----------------------------------------------------------------------------
# NF codebook (QLoRA NormalFloat construction, generalised to k bits)
# ----------------------------------------------------------------------------

def nf_codebook(bits: int) -> np.ndarray:
    """k-bit NormalFloat levels: standard-normal quantiles, asymmetric so that
    zero is exact. Positive half: Phi^-1 of 2^(k-1) evenly spaced probabilities
    from `offset` towards 0.5 (the 0.5 end dropped); negative half: minus Phi^-1
    of 2^(k-1) - 1 such probabilities; plus 0. The offset centres the outermost
    quantile bins, 1 - (1/(2*2^k) + 1/(2*(2^k - 1))) / 2. Levels are sorted,
    divided by the largest magnitude (so the ends are exactly -1 and +1) and
    rounded to fp32."""
    n = 2 ** bits
    offset = 1.0 - 0.5 * (1.0 / (2 * n) + 1.0 / (2 * (n - 1)))
    nd = NormalDist()
    pos_p = np.linspace(offset, 0.5, n // 2 + 1)[:-1]
    neg_p = np.linspace(offset, 0.5, n // 2)[:-1]
    pos = [nd.inv_cdf(float(p)) for p in pos_p]
    neg = [-nd.inv_cdf(float(p)) for p in neg_p]
    levels = np.array(sorted(pos + neg + [0.0]), dtype=np.float64)
    levels = levels / np.max(np.abs(levels))
    return levels.astype(np.float32)


NF3 = nf_codebook(3)
NF3_ZERO = int(np.nonzero(NF3 == 0.0)[0][0])
# decision thresholds between neighbouring levels, computed in fp32
NF3_MID = ((NF3[:-1] + NF3[1:]) * np.float32(0.5)).astype(np.float32)


def nf3_value(q) -> np.ndarray:
    return NF3[np.asarray(q, dtype=np.int64)]


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes 0..15 -> [N, K/2] bytes; element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_nf3(q: np.ndarray) -> np.ndarray:
    """[N, K] codes 0..7 -> [N, 3K/8] bytes: a little-endian bit stream per row
    with element j at bits [3j, 3j+3)."""
    q = np.asarray(q, dtype=np.uint32)
    lead = q.shape[:-1]
    K = q.shape[-1]
    u = q.reshape(lead + (K // 8, 8))
    v = np.zeros(lead + (K // 8,), dtype=np.uint32)
    for i in range(8):
        v |= u[..., i] << (3 * i)
    out = np.stack([(v & 0xFF), (v >> 8) & 0xFF, (v >> 16) & 0xFF], axis=-1)
    return out.reshape(lead + (3 * K // 8,)).astype(np.uint8)


def unpack_nf3(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    nb = p.shape[-1]
    t = p.reshape(lead + (nb // 3, 3)).astype(np.uint32)
    v = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)
    out = np.empty(lead + (nb // 3, 8), dtype=np.uint8)
    for i in range(8):
        out[..., i] = (v >> (3 * i)) & 7
    return out.reshape(lead + (nb // 3 * 8,))


def pack_nf3_planes(q: np.ndarray):
    """[N, K] codes 0..7 -> the two-plane NF3 layout a checkpoint may store (the
    layout the survey of the pages proposed): a 2-bit low plane lo [N, K/4] with element
    j at bits 2 (j mod 4) .. 2 (j mod 4) + 1 of byte j / 4, and a 1-bit high plane hi
    [N, K/8] with element j at bit j mod 8 of byte j / 8; code = lo | hi << 2."""
    q = np.asarray(q, dtype=np.uint32)
    lead, K = q.shape[:-1], q.shape[-1]
    u4 = (q & 3).reshape(lead + (K // 4, 4))
    lo = np.zeros(lead + (K // 4,), dtype=np.uint32)
    for i in range(4):
        lo |= u4[..., i] << (2 * i)
    u8 = (q >> 2).reshape(lead + (K // 8, 8))
    hi = np.zeros(lead + (K // 8,), dtype=np.uint32)
    for i in range(8):
        hi |= (u8[..., i] & 1) << i
    return lo.astype(np.uint8), hi.astype(np.uint8)


def unpack_nf3_planes(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    lo = np.asarray(lo, dtype=np.uint8)
    hi = np.asarray(hi, dtype=np.uint8)
    lead, K = lo.shape[:-1], lo.shape[-1] * 4
    out = np.empty(lead + (K,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (lo >> (2 * j)) & 3
    for j in range(8):
        out[..., j::8] |= ((hi >> j) & 1) << 2
    return out


# ----------------------------------------------------------------------------
# dequantisation (fp32, the canonical values)
# ----------------------------------------------------------------------------

def nvfp4_dequant(q: np.ndarray, s: np.ndarray, g) -> np.ndarray:
    """w = fp32(e2m1(c) * e4m3(s_block)) * g with blocks of 16 along K. The first
    product is exact (at most 6 significant bits); the multiply by the
    per-tensor scale g is the only rounding."""
    v = e2m1_value(unpack_fp4(q))
    sd = np.repeat(e4m3_value(s), 16, axis=-1)
    return ((v * sd).astype(np.float32) * np.float32(g)).astype(np.float32)


def mxfp4_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w = e2m1(c) * 2^(b - 127) with blocks of 32 along K (exact)."""
    v = e2m1_value(unpack_fp4(q))
    sd = np.repeat(e8m0_value(s), 32, axis=-1)
    return (v * sd).astype(np.float32)


def nf3_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w = NF3[q] * fp32(fp16 group scale) with groups of 64 along K; one
    rounding."""
    v = nf3_value(unpack_nf3(q))
    sd = np.repeat(fp16_value(s), 64, axis=-1)
    return (v * sd).astype(np.float32)


# ----------------------------------------------------------------------------
# quantisers (they produce synthetic inputs; the HIP path never quantises)
# ----------------------------------------------------------------------------

def nvfp4_quantize(T: np.ndarray):
    """NVFP4 of one expert weight tensor T [N, K] (fp32).

    g = amax(|T|) / (6 * 448) in fp32 (1 if T is all zero); per 16-block the
    E4M3 scale is RNE(min(amax_block / (6 g), 448)); elements are
    x / fp32(scale * g) rounded to E2M1 (RNE, saturating). A block whose scale
    decodes to 0 gets all-zero codes. Returns (packed codes, scale bytes, g)."""
    T = np.asarray(T, dtype=np.float32)
    N, K = T.shape
    amax = np.float32(np.max(np.abs(T))) if T.size else np.float32(0)
    g = (amax / np.float32(6 * 448)).astype(np.float32) if amax > 0 else np.float32(1.0)
    blocks = T.reshape(N, K // 16, 16)
    bmax = np.max(np.abs(blocks), axis=2)
    six_g = np.float32(np.float32(6.0) * g)
    sval = np.minimum((bmax / six_g).astype(np.float32), np.float32(448.0))
    s = e4m3_round(sval)
    sd = e4m3_value(s)
    denom = (sd * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(denom[..., None] > 0, blocks / denom[..., None], np.float32(0)).astype(np.float32)
    codes = e2m1_round(t)
    codes[sd == 0] = 0
    return pack_fp4(codes.reshape(N, K)), s, np.float32(g)


def mxfp4_quantize(T: np.ndarray):
    """MXFP4 of T [N, K] (OCP MX v1.0 conversion): per 32-block the shared
    exponent is floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), clamped
    to [-127, 127]; elements are x * 2^-exponent rounded to E2M1 (RNE,
    saturating at 6). An all-zero block gets scale byte 127 and zero codes.
    Returns (packed codes, E8M0 scale bytes)."""
    T = np.asarray(T, dtype=np.float32)
    N, K = T.shape
    blocks = T.reshape(N, K // 32, 32).astype(np.float64)
    bmax = np.max(np.abs(blocks), axis=2)
    _, ex = np.frexp(bmax)
    shared = np.clip(ex - 1 - 2, -127, 127)
    b = np.where(bmax > 0, shared + 127, 127).astype(np.int64)
    t = np.ldexp(blocks, -(b - 127)[..., None])
    codes = e2m1_round(t)
    return pack_fp4(codes.reshape(N, K)), b.astype(np.uint8)


def nf3_quantize(T: np.ndarray):
    """NF3 of T [N, K]: per 64-group s = fp16_RNE(min(amax, 65504)); elements
    t = x / fp32(s) map to the level index q = #{j : t > mid_j} with fp32
    midpoints between neighbouring levels (a tie goes to the lower level). A
    group whose scale is 0 gets the zero level. Returns (packed codes, fp16
    scale bits)."""
    T = np.asarray(T, dtype=np.float32)
    N, K = T.shape
    groups = T.reshape(N, K // 64, 64)
    gmax = np.max(np.abs(groups), axis=2)
    s16 = np.minimum(gmax, np.float32(65504.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s32[..., None] > 0, groups / s32[..., None], np.float32(0)).astype(np.float32)
    q = np.zeros(t.shape, dtype=np.int64)
    for m in NF3_MID:
        q += (t > m)
    q[s32 == 0] = NF3_ZERO
    return pack_nf3(q.reshape(N, K)), s16.view(np.uint16)
