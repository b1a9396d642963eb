// Prefill path (M > 8): route, per-tier align, grouped GEMM over W13 with a fused
// SwiGLU, grouped GEMM over W2 with the top-k weight applied per slot, and a
// fixed-order combine of each token's k slot outputs. Both tiers run in the same
// launches over their concatenated block lists (local-inference-lab/vllm PR #92,
// "How it works": both tiers share one routing result and one top-k sum).
//
// GEMM tile: block_m rows (slots of one expert) x 64 output columns, K in steps of
// 64 (one NF3 group). The weight tile is decoded once per step into LDS as 16-bit
// values, the activation tile is gathered into LDS, and each wave runs 16x16x32
// MFMAs over its 16 output columns.
//   W13: bf16 MFMA. x is bf16. NVFP4 e2m1 * E4M3 and MXFP4 e2m1 * 2^(b-127) are exact
//        in bf16; NF3 tiles hold scaled levels (kNF3TableScaleBf16) and each step's
//        fp32 partial is multiplied by the group scale before accumulation. The
//        epilogue applies the per-tensor factor, SwiGLU, and stores h as fp16
//        (saturated at +-65504: 11 significant bits for the W2 input).
//   W2:  fp16 MFMA. NVFP4 e2m1 * E4M3 is exact in fp16 (2^-10 .. 2688); MXFP4 rows are
//        stored as e2m1 * 2^(b - bref) with bref the row's largest block exponent, and
//        2^(bref - 127) returns in the epilogue; NF3 as in W13 with the fp16 table. The
//        epilogue multiplies by the routing weight and stores fp32 per-slot outputs.
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kPfThreads = 256;
constexpr int kBK = 64;
constexpr int kLds = kBK + 8;  // 16-bit elements per LDS row (16-byte pad)
constexpr int kBN = 64;        // output columns per block

struct PrefillArgs {
  const uint8_t* kq;
  const uint8_t* ks;
  const float* kg;
  const uint8_t* nq;
  const uint16_t* ns;
  int kept_fmt;
  int rows_w;  // rows of the weight tensor per expert
  int K;
  const uint16_t* act;   // W13: x bf16 [M, H]; W2: h fp16 [cap0 + cap1, I]
  int k, nslot;
  const int32_t* slots[2];
  const int32_t* bexp[2];
  const int32_t* npad[2];
  int nblk0;   // block count of tier 0 in this launch (tier 1 blocks follow)
  int nblk1;
  int E4, E3;
  int hrow1;   // h row of tier 1's first block
  int I, H;
  uint16_t* h_out;     // W13: fp16 [cap0 + cap1, I]
  float* o_out;        // W2: fp32 [nslot, H]
  const float* topk_w;
};

template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (F16) return pack_f16(a, b);
  else return pack_bf16(a, b);
}

template <int BM, bool W13>
__global__ __launch_bounds__(kPfThreads) void grouped_gemm_kernel(PrefillArgs a) {
  constexpr bool F16 = !W13;                   // W2 runs on fp16
  constexpr int BROWS = W13 ? 2 * kBN : kBN;   // weight rows per tile
  constexpr int NT = W13 ? 2 : 1;              // MFMA column tiles per wave
  constexpr int MT = BM / 16;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BROWS][kLds];
  __shared__ uint32_t lutp[64];     // scaled NF3 level pairs (16-bit each)
  __shared__ float sS[BROWS];       // NF3 group scale of each tile row, this step
  __shared__ int sRef[BROWS];       // MXFP4 (W2): row reference exponent
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;

  const int by = blockIdx.x;
  const int tier = by < a.nblk0 ? 0 : 1;
  const int b = tier ? by - a.nblk0 : by;
  // npad and the block table come from the align stage; clamp to this launch's grid
  // and the tier's expert count so stale scratch cannot index out of range
  if (b * BM >= a.npad[tier][0] || b >= (tier ? a.nblk1 : a.nblk0)) return;
  const int loc = a.bexp[tier][b];
  if ((unsigned)loc >= (unsigned)(tier ? a.E3 : a.E4)) return;
  const bool nf3 = tier == HMOE_TIER_NF3;
  const bool mx = !nf3 && a.kept_fmt == HMOE_KEPT_MXFP4;
  const int n0 = blockIdx.y * kBN;
  const int32_t* bslots = a.slots[tier] + (size_t)b * BM;
  const size_t hbase = (size_t)(tier ? a.hrow1 : 0) + (size_t)b * BM;

  if (tid < 64) {
    const float c = F16 ? kNF3TableScaleF16 : kNF3TableScaleBf16;
    lutp[tid] = pack16<F16>(nf3_level(tid & 7) * c, nf3_level(tid >> 3) * c);
  }
  if (F16 && mx) {
    // largest E8M0 byte of each of the tile's rows (over the whole K)
    for (int r = wave; r < BROWS; r += kPfThreads / kWave) {
      const uint8_t* srow = a.ks + ((size_t)loc * a.rows_w + n0 + r) * (a.K / 32);
      int m = 0;
      for (int i = lane; i < a.K / 32; i += kWave) m = max(m, (int)srow[i]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
      if (lane == 0) sRef[r] = m;
    }
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < a.K; k0 += kBK) {
    __syncthreads();
    // activation tile: BM rows x 64 16-bit values, 16-byte chunks
    for (int c = tid; c < BM * (kBK / 8); c += kPfThreads) {
      const int m = c / (kBK / 8);
      const int ch = c - m * (kBK / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (W13) {
        const int slot = bslots[m];
        if ((unsigned)slot < (unsigned)a.nslot)
          v = *reinterpret_cast<const uint4*>(a.act + (size_t)(slot / a.k) * a.K + k0 + 8 * ch);
      } else {
        v = *reinterpret_cast<const uint4*>(a.act + (hbase + m) * a.K + k0 + 8 * ch);
      }
      *reinterpret_cast<uint4*>(&As[m][8 * ch]) = v;
    }
    // weight tile: BROWS rows x 2 units of 32
    for (int u = tid; u < BROWS * 2; u += kPfThreads) {
      const int r = u >> 1;
      const int uu = u & 1;
      int row;
      if (W13) row = r < kBN ? n0 + r : a.I + n0 + (r - kBN);
      else row = n0 + r;
      const size_t grow = (size_t)loc * a.rows_w + row;
      const int ku = k0 / 32 + uu;
      uint32_t w[16];
      if (nf3) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(a.nq + grow * (3 * a.K / 8) + 12 * ku);
        const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
        w[0] = lutp[nf3_pair_field<0>(d0, d1, d2)]; w[1] = lutp[nf3_pair_field<1>(d0, d1, d2)];
        w[2] = lutp[nf3_pair_field<2>(d0, d1, d2)]; w[3] = lutp[nf3_pair_field<3>(d0, d1, d2)];
        w[4] = lutp[nf3_pair_field<4>(d0, d1, d2)]; w[5] = lutp[nf3_pair_field<5>(d0, d1, d2)];
        w[6] = lutp[nf3_pair_field<6>(d0, d1, d2)]; w[7] = lutp[nf3_pair_field<7>(d0, d1, d2)];
        w[8] = lutp[nf3_pair_field<8>(d0, d1, d2)]; w[9] = lutp[nf3_pair_field<9>(d0, d1, d2)];
        w[10] = lutp[nf3_pair_field<10>(d0, d1, d2)]; w[11] = lutp[nf3_pair_field<11>(d0, d1, d2)];
        w[12] = lutp[nf3_pair_field<12>(d0, d1, d2)]; w[13] = lutp[nf3_pair_field<13>(d0, d1, d2)];
        w[14] = lutp[nf3_pair_field<14>(d0, d1, d2)]; w[15] = lutp[nf3_pair_field<15>(d0, d1, d2)];
        if (uu == 0) sS[r] = fp16_to_f32(a.ns[grow * (a.K / 64) + k0 / 64]);
      } else {
        const uint4 q = *reinterpret_cast<const uint4*>(a.kq + grow * (a.K / 2) + 16 * ku);
        const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
        if (!mx) {
          const uint32_t sc = *reinterpret_cast<const uint16_t*>(a.ks + grow * (a.K / 16) + 2 * ku);
          const float s0 = e4m3_to_f32<0>(sc);
          const float s1 = e4m3_to_f32<1>(sc);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float s = v < 2 ? s0 : s1;
            const f32x2 p0 = e2m1x2_f32<0>(qq[v], 1.0f);
            const f32x2 p1 = e2m1x2_f32<1>(qq[v], 1.0f);
            const f32x2 p2 = e2m1x2_f32<2>(qq[v], 1.0f);
            const f32x2 p3 = e2m1x2_f32<3>(qq[v], 1.0f);
            w[4 * v + 0] = pack16<F16>(p0[0] * s, p0[1] * s);
            w[4 * v + 1] = pack16<F16>(p1[0] * s, p1[1] * s);
            w[4 * v + 2] = pack16<F16>(p2[0] * s, p2[1] * s);
            w[4 * v + 3] = pack16<F16>(p3[0] * s, p3[1] * s);
          }
        } else if (!F16) {
          const float so = e8m0_scale_operand(a.ks[grow * (a.K / 32) + ku]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            w[4 * v + 0] = e2m1x2_bf16<0>(qq[v], so);
            w[4 * v + 1] = e2m1x2_bf16<1>(qq[v], so);
            w[4 * v + 2] = e2m1x2_bf16<2>(qq[v], so);
            w[4 * v + 3] = e2m1x2_bf16<3>(qq[v], so);
          }
        } else {
          const int be = (int)a.ks[grow * (a.K / 32) + ku] - sRef[r];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const f32x2 p0 = e2m1x2_f32<0>(qq[v], 1.0f);
            const f32x2 p1 = e2m1x2_f32<1>(qq[v], 1.0f);
            const f32x2 p2 = e2m1x2_f32<2>(qq[v], 1.0f);
            const f32x2 p3 = e2m1x2_f32<3>(qq[v], 1.0f);
            w[4 * v + 0] = pack_f16(__builtin_ldexpf(p0[0], be), __builtin_ldexpf(p0[1], be));
            w[4 * v + 1] = pack_f16(__builtin_ldexpf(p1[0], be), __builtin_ldexpf(p1[1], be));
            w[4 * v + 2] = pack_f16(__builtin_ldexpf(p2[0], be), __builtin_ldexpf(p2[1], be));
            w[4 * v + 3] = pack_f16(__builtin_ldexpf(p3[0], be), __builtin_ldexpf(p3[1], be));
          }
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[r][32 * uu]);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      dst[2] = make_uint4(w[8], w[9], w[10], w[11]);
      dst[3] = make_uint4(w[12], w[13], w[14], w[15]);
    }
    __syncthreads();
    f32x4 part[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) part[mt][nt] = nf3 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt][nt];
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      uint4 bq[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bq[nt] = *reinterpret_cast<const uint4*>(&Bs[nt * kBN + 16 * wave + (lane & 15)][kk]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 aq = *reinterpret_cast<const uint4*>(&As[mt * 16 + (lane & 15)][kk]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (F16)
            part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, aq), __builtin_bit_cast(f16x8, bq[nt]), part[mt][nt], 0, 0, 0);
          else
            part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, aq), __builtin_bit_cast(bf16x8, bq[nt]), part[mt][nt], 0, 0, 0);
        }
      }
    }
    if (nf3) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float s = sS[nt * kBN + 16 * wave + (lane & 15)];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf(s, part[mt][nt][r], acc[mt][nt][r]);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = part[mt][nt];
    }
  }
  // epilogue: lane holds rows 4*(lane/16)+r of each 16-row tile, column lane%16
  const int col = 16 * wave + (lane & 15);
  const int n = n0 + col;
  float g;
  if (nf3) g = 1.0f / (F16 ? kNF3TableScaleF16 : kNF3TableScaleBf16);
  else if (!mx) g = a.kg[loc];
  else g = F16 ? e8m0_to_f32((uint32_t)sRef[col]) : 1.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + 4 * (lane >> 4) + r;
      if (W13) {
        const float gate = acc[mt][0][r] * g;
        const float up = acc[mt][NT - 1][r] * g;
        const float h = fminf(fmaxf(silu(gate) * up, -65504.0f), 65504.0f);
        a.h_out[(hbase + m) * a.I + n] = (uint16_t)(pack_f16(h, 0.0f) & 0xFFFFu);
      } else {
        const int slot = bslots[m];
        if ((unsigned)slot < (unsigned)a.nslot) a.o_out[(size_t)slot * a.H + n] = acc[mt][0][r] * g * a.topk_w[slot];
      }
    }
  }
}

// y[t, n] = sum_j o[t*k + j, n] in fixed j order (the routing weight is already in o)
__global__ __launch_bounds__(256) void prefill_combine_kernel(const float* __restrict__ o, int M,
                                                              int k, int H,
                                                              uint16_t* __restrict__ y) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)M * H) return;
  const size_t t = idx / H;
  const size_t n = idx - t * H;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc += o[(t * k + j) * H + n];
  y[idx] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
}

typedef void (*GemmFn)(PrefillArgs);

template <bool W13>
static GemmFn pick_gemm(int bm) {
  switch (bm) {
    case 16: return grouped_gemm_kernel<16, W13>;
    case 32: return grouped_gemm_kernel<32, W13>;
    case 64: return grouped_gemm_kernel<64, W13>;
    case 128: return grouped_gemm_kernel<128, W13>;
  }
  return nullptr;
}

hipError_t launch_prefill(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                          uint16_t* y, void* scratch, int stage, hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  float* w = reinterpret_cast<float*>(base + P.topk_w);
  PrefillArgs a{};
  a.kept_fmt = L.kept_format;
  a.k = L.k;
  a.nslot = M * L.k;
  a.E4 = L.E4;
  a.E3 = L.E3;
  for (int t = 0; t < 2; ++t) {
    a.slots[t] = reinterpret_cast<const int32_t*>(base + P.a_slots[t]);
    a.bexp[t] = reinterpret_cast<const int32_t*>(base + P.a_bexp[t]);
    a.npad[t] = reinterpret_cast<const int32_t*>(base + P.a_npad[t]);
  }
  // grid sized from the capacity at this M (an upper bound, not data)
  const int bm = L.block_m;
  const int ns = M * L.k;
  const int cap0 = ns + (L.E4 < ns ? L.E4 : ns) * (bm - 1);
  const int cap1 = ns + (L.E3 < ns ? L.E3 : ns) * (bm - 1);
  a.nblk0 = L.E4 > 0 ? (cap0 + bm - 1) / bm : 0;
  a.nblk1 = L.E3 > 0 ? (cap1 + bm - 1) / bm : 0;
  a.hrow1 = L.cap[0];
  a.I = L.I;
  a.H = L.H;
  uint16_t* h = reinterpret_cast<uint16_t*>(base + P.h_pre);
  float* o = reinterpret_cast<float*>(base + P.o_pre);
  const int nblk = a.nblk0 + a.nblk1;
  if (stage == HMOE_STAGE_W13) {
    PrefillArgs b = a;
    b.kq = W.kept_w13_q; b.ks = W.kept_w13_s; b.kg = W.kept_w13_g;
    b.nq = W.nf3_w13_q; b.ns = W.nf3_w13_s;
    b.rows_w = 2 * L.I;
    b.K = L.H;
    b.act = x;
    b.h_out = h;
    GemmFn fn = pick_gemm<true>(bm);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(nblk, L.I / kBN), dim3(kPfThreads), 0, s, b);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_W2) {
    PrefillArgs c = a;
    c.kq = W.kept_w2_q; c.ks = W.kept_w2_s; c.kg = W.kept_w2_g;
    c.nq = W.nf3_w2_q; c.ns = W.nf3_w2_s;
    c.rows_w = L.H;
    c.K = L.I;
    c.act = h;
    c.o_out = o;
    c.topk_w = w;
    GemmFn fn = pick_gemm<false>(bm);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(nblk, L.H / kBN), dim3(kPfThreads), 0, s, c);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_COMBINE) {
    const size_t n = (size_t)M * L.H;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       o, M, L.k, L.H, y);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace hmoe
