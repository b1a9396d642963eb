// Dequantisation test hook: writes one expert tensor's canonical fp32 values (and
// their bf16 rounding). It shares the format primitives of device_common.h with the
// forward kernels (the hardware E2M1 / E4M3 conversions, the E8M0 scale and the NF3
// level bit patterns) but not their decode paths: the forward kernels fold scales
// into 16-bit operands, scaled level tables and fp32 partials, which only the layer
// output tolerance covers.
// Canonical values: NVFP4 fp32(e2m1 * e4m3) * g (the first product is exact, the
// per-tensor multiply is the one rounding), MXFP4 e2m1 * 2^(b - 127) (exact), NF3
// level[q] * fp16 scale (one rounding).
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

struct DequantArgs {
  const uint8_t* q;   // codes of this expert tensor [rows, K/2] or [rows, 3K/8]
  const uint8_t* s8;  // FP4 scales
  const uint16_t* s16;  // NF3 scales
  const float* gp;  // NVFP4 per-tensor scale of this expert tensor
  int fmt;  // 0 NVFP4, 1 MXFP4, 2 NF3
  int rows, K;
  float* out_f32;
  uint16_t* out_bf16;
};

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const size_t units = (size_t)a.rows * (a.K / 32);
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const size_t row = u / (a.K / 32);
  const int ku = (int)(u - row * (a.K / 32));
  float v[32];
  if (a.fmt == 2) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(a.q + row * (3 * a.K / 8) + 12 * ku);
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
    const float s = fp16_to_f32(a.s16[row * (a.K / 64) + (ku >> 1)]);
    uint32_t f[16];
    f[0] = nf3_pair_field<0>(d0, d1, d2); f[1] = nf3_pair_field<1>(d0, d1, d2);
    f[2] = nf3_pair_field<2>(d0, d1, d2); f[3] = nf3_pair_field<3>(d0, d1, d2);
    f[4] = nf3_pair_field<4>(d0, d1, d2); f[5] = nf3_pair_field<5>(d0, d1, d2);
    f[6] = nf3_pair_field<6>(d0, d1, d2); f[7] = nf3_pair_field<7>(d0, d1, d2);
    f[8] = nf3_pair_field<8>(d0, d1, d2); f[9] = nf3_pair_field<9>(d0, d1, d2);
    f[10] = nf3_pair_field<10>(d0, d1, d2); f[11] = nf3_pair_field<11>(d0, d1, d2);
    f[12] = nf3_pair_field<12>(d0, d1, d2); f[13] = nf3_pair_field<13>(d0, d1, d2);
    f[14] = nf3_pair_field<14>(d0, d1, d2); f[15] = nf3_pair_field<15>(d0, d1, d2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[2 * i] = nf3_level(f[i] & 7u) * s;
      v[2 * i + 1] = nf3_level(f[i] >> 3) * s;
    }
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(a.q + row * (a.K / 2) + 16 * ku);
    const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
    if (a.fmt == 0) {
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(a.s8 + row * (a.K / 16) + 2 * ku);
      const float s0 = e4m3_to_f32<0>(sc);
      const float s1 = e4m3_to_f32<1>(sc);
      const float g = *a.gp;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float s = w < 2 ? s0 : s1;
        const f32x2 p0 = e2m1x2_f32<0>(qq[w], 1.0f);
        const f32x2 p1 = e2m1x2_f32<1>(qq[w], 1.0f);
        const f32x2 p2 = e2m1x2_f32<2>(qq[w], 1.0f);
        const f32x2 p3 = e2m1x2_f32<3>(qq[w], 1.0f);
        const float e[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float exact = e[i] * s;  // at most 6 significant bits: exact
          v[8 * w + i] = exact * g;
        }
      }
    } else {
      const float so = e8m0_scale_operand(a.s8[row * (a.K / 32) + ku]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 p0 = e2m1x2_f32<0>(qq[w], so);
        const f32x2 p1 = e2m1x2_f32<1>(qq[w], so);
        const f32x2 p2 = e2m1x2_f32<2>(qq[w], so);
        const f32x2 p3 = e2m1x2_f32<3>(qq[w], so);
        v[8 * w + 0] = p0[0]; v[8 * w + 1] = p0[1];
        v[8 * w + 2] = p1[0]; v[8 * w + 3] = p1[1];
        v[8 * w + 4] = p2[0]; v[8 * w + 5] = p2[1];
        v[8 * w + 6] = p3[0]; v[8 * w + 7] = p3[1];
      }
    }
  }
  const size_t off = row * a.K + 32 * ku;
  if (a.out_f32) {
    float4* o = reinterpret_cast<float4*>(a.out_f32 + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
  if (a.out_bf16) {
    uint4* o = reinterpret_cast<uint4*>(a.out_bf16 + off);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = make_uint4(pack_bf16(v[8 * i], v[8 * i + 1]), pack_bf16(v[8 * i + 2], v[8 * i + 3]),
                        pack_bf16(v[8 * i + 4], v[8 * i + 5]), pack_bf16(v[8 * i + 6], v[8 * i + 7]));
  }
}

hipError_t launch_dequant(const Layer& L, const hmoe_weights& W, int expert, int tensor,
                          float* out_f32, uint16_t* out_bf16, hipStream_t s) {
  const bool nf3 = L.has_map && L.bit_map[expert] == 3;
  int loc = 0;
  for (int e = 0; e < expert; ++e)
    loc += ((L.has_map && L.bit_map[e] == 3) == nf3) ? 1 : 0;
  DequantArgs a{};
  const bool w13 = tensor == HMOE_TENSOR_W13;
  a.rows = w13 ? 2 * L.I : L.H;
  a.K = w13 ? L.H : L.I;
  a.out_f32 = out_f32;
  a.out_bf16 = out_bf16;
  const size_t n = (size_t)a.rows * a.K;
  if (nf3) {
    a.fmt = 2;
    a.q = (w13 ? W.nf3_w13_q : W.nf3_w2_q) + (size_t)loc * n * 3 / 8;
    a.s16 = (w13 ? W.nf3_w13_s : W.nf3_w2_s) + (size_t)loc * (n / 64);
  } else {
    a.fmt = L.kept_format;
    a.q = (w13 ? W.kept_w13_q : W.kept_w2_q) + (size_t)loc * n / 2;
    const int B = L.kept_format == HMOE_KEPT_NVFP4 ? 16 : 32;
    a.s8 = (w13 ? W.kept_w13_s : W.kept_w2_s) + (size_t)loc * (n / B);
    if (L.kept_format == HMOE_KEPT_NVFP4) a.gp = (w13 ? W.kept_w13_g : W.kept_w2_g) + loc;
  }
  const size_t units = n / 32;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hmoe
