// Device primitives shared by the hybrid W4A16 MoE kernels (gfx950 only).
//
// Formats (named by the hybrid NVFP4/NF3 serving pages, local-inference-lab/vllm
// PR #92 "How it works" and PR #104 description; bit layouts from the OCP MX v1.0
// and OCP OFP8 specifications):
//   E2M1  4-bit element: sign, 2 exponent bits (bias 1), 1 mantissa bit.
//   E4M3  8-bit NVFP4 block scale ("fn": no infinities, 0x7F/0xFF NaN).
//   E8M0  8-bit MXFP4 block scale: 2^(b - 127).
//   NF3   3-bit NormalFloat level index with an fp16 group scale.
// gfx950 decodes E2M1 and E4M3 in hardware (v_cvt_scalef32_pk_*_fp4 with a scale
// whose exponent only is applied, and v_cvt_f32_fp8 for OCP E4M3); NF3 goes through
// an LDS-resident table of level pairs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hmoe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// NF3 levels: the 3-bit NormalFloat code book (QLoRA's NormalFloat construction
// carried out at 3 bits: 4 positive and 3 negative standard-normal quantiles plus
// an exact zero, scaled so that the ends are -1 and +1), as fp32 bit patterns in
// ascending level order.
// ---------------------------------------------------------------------------
constexpr uint32_t kNF3Bits[8] = {
    0xBF800000u, 0xBF08F740u, 0xBE7CDB98u, 0x00000000u,
    0x3E3BBCD2u, 0x3EC394B6u, 0x3F1F7BFEu, 0x3F800000u};

// level of code q (a select chain over immediates: an indexed table would be a
// memory load)
__device__ __forceinline__ float nf3_level(uint32_t q) {
  q &= 7u;
  uint32_t b = kNF3Bits[0];
#pragma unroll
  for (uint32_t i = 1; i < 8; ++i) b = (q == i) ? kNF3Bits[i] : b;
  return __uint_as_float(b);
}

// Level tables inside the kernels hold level * c rounded to 16 bits, with c chosen
// so that all eight products are close to representable: the largest relative
// rounding error is 5.5e-4 in bf16 (c = 1.2417735) and 3.5e-5 in fp16 (c =
// 1.1152737), against 3.0e-3 and 2.5e-4 for the plain levels. The kernels take
// the group scale in fp32 and multiply each row result by 1/c.
constexpr float kNF3TableScaleBf16 = 1.2417735f;
constexpr float kNF3TableScaleF16 = 1.1152737f;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair, round to nearest even (a in the low half)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 f = {a, b};
  const bf16x2 v = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, v);
}

// two fp32 -> packed fp16 pair, round to nearest even (a in the low half)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f32x2 f = {a, b};
  const f16x2 v = __builtin_convertvector(f, f16x2);  // v_cvt_pk_f16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 bits -> fp32 (exact)
__device__ __forceinline__ float fp16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// E4M3 byte `sel` of v -> fp32 (exact, hardware decode of OCP E4M3)
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) { return __builtin_amdgcn_cvt_f32_fp8(v, SEL); }

// E8M0 byte -> the fp32 whose exponent field encodes 2^(b - 127); used as the scale
// operand of the scaled FP4 conversions, which apply only that exponent. Byte 0 is
// given a nonzero mantissa so the operand is the fp32 subnormal 2^-127 itself.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t b) {
  return __uint_as_float((b << 23) | (b == 0 ? 0x00400000u : 0u));
}

// exact fp32 value 2^(b - 127) of an E8M0 byte
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : (b << 23));
}

// E2M1 pair in byte SEL of v -> two bf16 (low nibble -> low half) times 2^exp(scale)
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_bf16(uint32_t v, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// E2M1 pair in byte SEL of v -> two fp32 times 2^exp(scale) (exact)
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t v, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, SEL);
}

// E2M1 pair in byte SEL of v -> two fp16 (low nibble -> low half) times 2^exp(scale)
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_f16(uint32_t v, float scale) {
  f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// dot of two fp16 pairs accumulated in fp32
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// dot of two bf16 pairs accumulated in fp32
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// 6-bit NF3 pair field p (elements 2p, 2p+1) of a 32-element unit stored as three
// little-endian dwords (element j at bits [3j, 3j+3) of the 96-bit unit)
template <int P>
__device__ __forceinline__ uint32_t nf3_pair_field(uint32_t d0, uint32_t d1, uint32_t d2) {
  constexpr int bit = 6 * P;
  if constexpr (bit + 6 <= 32) {
    return __builtin_amdgcn_ubfe(d0, bit, 6);
  } else if constexpr (bit < 32) {
    return __builtin_amdgcn_alignbit(d1, d0, bit) & 63u;
  } else if constexpr (bit + 6 <= 64) {
    return __builtin_amdgcn_ubfe(d1, bit - 32, 6);
  } else if constexpr (bit < 64) {
    return __builtin_amdgcn_alignbit(d2, d1, bit - 32) & 63u;
  } else {
    return __builtin_amdgcn_ubfe(d2, bit - 64, 6);
  }
}

// ---------------------------------------------------------------------------
// cross-lane exchange without the LDS crossbar
// ---------------------------------------------------------------------------
// xlane<B>(v) returns v from the partner lane of a butterfly step on lane bit B
// (every lane has a partner, so the DPP moves may zero-fill: that lets the compiler fold
// them into the consuming add or max):
// lane ^ 1, ^ 3, ^ 7, ^ 15 (DPP quad permute, row half-mirror, row mirror) for B <= 8,
// lane ^ 16 and lane ^ 32 (v_permlane16_swap / v_permlane32_swap plus a select). Each
// partner differs from the lane in bit B and only below it, so a sequence of steps over
// B = LR/2 .. 1 visits every lane of an aligned LR-lane segment exactly once.
template <int B>
__device__ __forceinline__ uint32_t xlane_u32(uint32_t v) {
  static_assert(B == 1 || B == 2 || B == 4 || B == 8 || B == 16 || B == 32, "butterfly bit");
  if constexpr (B == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);   // quad [1,0,3,2]
  } else if constexpr (B == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x1B, 0xF, 0xF, true);   // quad [3,2,1,0]
  } else if constexpr (B == 4) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true);  // row half-mirror
  } else if constexpr (B == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true);  // row mirror
  } else if constexpr (B == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

template <int B>
__device__ __forceinline__ float xlane(float v) {
  return __uint_as_float(xlane_u32<B>(__float_as_uint(v)));
}

template <int B>
__device__ __forceinline__ int xlane_i(int v) {
  return (int)xlane_u32<B>((uint32_t)v);
}

template <int B>
__device__ __forceinline__ double xlane_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xlane_u32<B>((uint32_t)u);
  const uint64_t hi = xlane_u32<B>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// a + b across lane halves (B = 32) or rows (B = 16) in two operations: after one
// v_permlane32_swap (v_permlane16_swap) of (a, b), the two results hold, lane by lane,
// the own and the partner lane's values of a for lanes with bit B clear and of b for lanes
// with bit B set; their sum is a[l] + a[l ^ B] (bit B clear) or b[l] + b[l ^ B] (set)
template <int B>
__device__ __forceinline__ float swap_add(float a, float b) {
  static_assert(B == 16 || B == 32, "swap distance");
  if constexpr (B == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// sum / max over aligned WIDTH-lane groups (every lane of the group gets the result)
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (WIDTH >= 64) v = swap_add<32>(v, v);
  if constexpr (WIDTH >= 32) v = swap_add<16>(v, v);
  if constexpr (WIDTH >= 16) v += xlane<8>(v);
  if constexpr (WIDTH >= 8) v += xlane<4>(v);
  if constexpr (WIDTH >= 4) v += xlane<2>(v);
  if constexpr (WIDTH >= 2) v += xlane<1>(v);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (WIDTH >= 64) v = fmaxf(v, xlane<32>(v));
  if constexpr (WIDTH >= 32) v = fmaxf(v, xlane<16>(v));
  if constexpr (WIDTH >= 16) v = fmaxf(v, xlane<8>(v));
  if constexpr (WIDTH >= 8) v = fmaxf(v, xlane<4>(v));
  if constexpr (WIDTH >= 4) v = fmaxf(v, xlane<2>(v));
  if constexpr (WIDTH >= 2) v = fmaxf(v, xlane<1>(v));
  return v;
}

// z * sigmoid(z) with the hardware reciprocal (1 ulp) in place of an IEEE division:
// exp(-z) = inf for z < -88 gives rcp = 0 and -0, the limit
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace hmoe
