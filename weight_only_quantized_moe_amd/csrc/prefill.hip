// Prefill path (M > 8): route, per-tier align, then grouped GEMMs over each tier's
// padded expert blocks: W13 with a fused SwiGLU, W2 with the top-k weight applied per
// slot, and a fixed-order combine of each token's k slot outputs. Both tiers run in
// the same launches over their concatenated block lists (local-inference-lab/vllm PR
// #92, "How it works": both tiers share one routing result and one top-k sum).
//
// GEMM: a block computes BM slots x 128 weight rows (W13: 64 gate rows and the
// matching 64 up rows; W2: 128 output columns) over K in steps of 64 (one NF3 group),
// BM being the smallest of 16, 32, 64 and block_m rows that holds the real slots of
// its block_m-row align block (so an expert's last, partly padded block costs less),
// with fp16 16x16x32 MFMAs. Four waves split the tile 2 x 2 (1 x 4 for BM = 16). LDS
// holds two stages of the activation and the decoded weight tile: while one stage
// feeds the MFMAs, the next step's raw weights and activations are already in
// registers and are decoded into the other stage afterwards, one barrier per step.
//
// Precision. The MFMAs run on fp16 operands with fp32 accumulation.
//   x:  bf16 tokens are converted once per token to fp16 times 2^-e, e chosen so the
//       token's largest |x| lands in [2^14, 2^15) (exact for every element within 2^29
//       of it); 2^e returns in the W13 epilogue.
//   h:  W13's SwiGLU output is stored as fp16 times 2^-he, he = 2 (e + 14) with e
//       the token's x exponent above (clamped to [-100, 100]): gate and up grow
//       with the token's largest |x|, so h / max|x|^2 stays within the product of
//       the gate and up rows' L1 norms whatever the activations' scale. The stored
//       value saturates at +-65504 only beyond that; 2^he returns in the W2 epilogue.
//   NVFP4: e2m1 * E4M3 has at most 6 significant bits and lies in [2^-10, 2688]: the
//       conversion applies the scale's power of two, a packed fp16 multiply its 1.m
//       factor, both exact. The per-tensor fp32 scale returns in the epilogue.
//   MXFP4: e2m1 * 2^(b - bref) with bref the row's largest E8M0 byte (exact unless a
//       block is 2^24 below the row's largest); 2^(bref - 127) returns in the epilogue.
//   NF3: the 64-entry table holds level pairs times kNF3TableScaleF16 in fp16 (within
//       3.5e-5 relative of the exact products); a unit's pairs are multiplied (packed
//       fp16) by its group scale times 2^(15 - ref), ref the largest fp16 exponent
//       field among the row's group scales, so each weight takes one fp16 rounding of
//       level times scale; 2^(ref - 15) and 1 / kNF3TableScaleF16 return in the
//       epilogue.
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "hmoe_internal.h"
#include "mx_gemm.h"

namespace hmoe {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kPfThreads = 256;
constexpr int kBK = 64;         // K per step (one NF3 group)
constexpr int kBN = 128;        // weight rows per tile
constexpr int kActAhead = 2;    // steps between an activation load and its LDS store
constexpr int kPipeGroup = 8;   // unrolled steps (a multiple of both distances, 2 and 8)
constexpr int kXcdGroup = 1;    // expert blocks per XCD assignment unit

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<0>) ... f(integral_constant<N - 1>), in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS tiles hold rows of 64 16-bit values (eight 16-byte chunks, one row spanning all
// 32 four-byte banks) with chunk c of row r stored at chunk c ^ (r & 7) ^ (2 * bit 4
// of r). The low term spreads the 16-byte MFMA operand reads of 16 consecutive rows
// over all banks (a 16-byte access is served eight lanes at a time); the high term
// separates rows r and r + 16, which the decoding threads of one eight-lane group
// write in the same step (without it those stores conflict two ways).
__device__ __forceinline__ int swz_lo(int r) { return r & 7; }
__device__ __forceinline__ int swz_hi(int r) { return (r >> 3) & 2; }
__device__ __forceinline__ int swz(int r, int c) { return 8 * (c ^ swz_lo(r) ^ swz_hi(r)); }

struct PrefillArgs {
  const uint8_t* kq;
  const uint8_t* ks;
  const float* kg;
  const uint8_t* nq;
  const uint16_t* ns;
  int kept_fmt;
  int rows_w;  // rows of the weight tensor per expert
  int K;
  const uint16_t* act;   // W13: x fp16 [M, H] (scaled per token); W2: h fp16 [cap0 + cap1, I]
  const int32_t* xe;     // per-token exponent of the x scaling (W2: gives h's scaling)
  int k, nslot;
  const int32_t* slots[2];
  const int32_t* bexp[2];
  const int32_t* npad[2];
  int nblk0;   // block count of tier 0 in this launch (tier 1 blocks follow)
  int nblk1;
  int ntile;   // column tiles per expert block
  int vec_scales;  // weight scale rows hold whole 16-byte vectors of 8 steps (K % 512 == 0)
  int E4, E3;
  int hrow1;   // h row of tier 1's first block
  int I, H;
  uint16_t* h_out;     // W13: fp16 [cap0 + cap1, I]
  float* o_out;        // W2: fp32 [nslot, H]
  const float* topk_w; // W13: [nslot] routing weights
  float* row_fac;      // [cap0 + cap1]: the W2 output factor of each h row (routing weight
                       // times 2^he, 0 for padding), written by W13's first column tile
};

enum : int { kPfNvfp4 = 0, kPfMxfp4 = 1, kPfNf3 = 2 };

// exponent he of a token's h scaling from its x exponent e (see the header)
__device__ __forceinline__ int h_exponent(int e) { return min(max(2 * (e + 14), -100), 100); }

__device__ __forceinline__ uint32_t mul_f16x2(uint32_t v, f16x2 m) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v) * m);
}

template <int BM, bool W13>
struct GemmShape {
  static constexpr int WAVES_M = BM >= 32 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int MT = BM / WAVES_M / 16;     // 16-row MFMA tiles per wave
  static constexpr int NT = kBN / WAVES_N / 16;    // 16-column MFMA tiles per wave
  static constexpr int A_CHUNKS = BM * (kBK / 8);  // 16-byte pieces of an activation tile
  static constexpr int A_PER = (A_CHUNKS + kPfThreads - 1) / kPfThreads;
};

// Weight row (within the 128-row tile) of MFMA column tile nt of wave wn. W13 pairs
// gate tile nt with up tile nt + NT/2 (same h columns, same lane).
template <int BM, bool W13>
__device__ __forceinline__ int tile_row(int wn, int nt) {
  using S = GemmShape<BM, W13>;
  if constexpr (W13) {
    constexpr int HALF = S::NT / 2;
    const int base = wn * (kBN / 2 / S::WAVES_N);
    return nt < HALF ? base + 16 * nt : kBN / 2 + base + 16 * (nt - HALF);
  } else {
    return wn * (kBN / S::WAVES_N) + 16 * nt;
  }
}

// LDS of one GEMM block: two stages of the activation and the decoded weight tile,
// the NF3 pair table and the per-row reference exponents.
template <int BM>
struct GemmSmem {
  __attribute__((aligned(16))) uint16_t As[2][BM][kBK];
  __attribute__((aligned(16))) uint16_t Bs[2][kBN][kBK];
  uint32_t lut[64 * 32];  // NF3: fp16 pairs of scaled levels, [pair field][lane % 32]
  int sRef[kBN];          // MXFP4: largest E8M0 byte; NF3: largest fp16 scale exponent
  int rowSlot[BM];        // the epilogue's per-row data, loaded at the block's start:
  int rowE[BM];           //   slot, W13: the token's x exponent,
  float rowF[BM];         //   W2: the row's output factor
};

// NVFP4 16-element block (two code words) -> 8 fp16 pairs, exact (see the header).
__device__ __forceinline__ void nvfp4_block_f16(uint32_t q0, uint32_t q1, uint32_t sbyte,
                                                uint32_t* w) {
  const float s = __builtin_amdgcn_cvt_f32_fp8(sbyte, 0);
  // +-1.m of the scale: the conversion applies the scale's exponent only, so its sign
  // rides on this factor
  const float mu32 = __uint_as_float((__float_as_uint(s) & 0x807FFFFFu) | 0x3F800000u);
  const _Float16 mu = (s == 0.0f) ? (_Float16)0.0f : (s != s ? (_Float16)s : (_Float16)mu32);
  const f16x2 m = {mu, mu};
  w[0] = mul_f16x2(e2m1x2_f16<0>(q0, s), m);
  w[1] = mul_f16x2(e2m1x2_f16<1>(q0, s), m);
  w[2] = mul_f16x2(e2m1x2_f16<2>(q0, s), m);
  w[3] = mul_f16x2(e2m1x2_f16<3>(q0, s), m);
  w[4] = mul_f16x2(e2m1x2_f16<0>(q1, s), m);
  w[5] = mul_f16x2(e2m1x2_f16<1>(q1, s), m);
  w[6] = mul_f16x2(e2m1x2_f16<2>(q1, s), m);
  w[7] = mul_f16x2(e2m1x2_f16<3>(q1, s), m);
}

// VS: the weight scales of 8 consecutive steps of a row are one aligned 16-byte vector
// (two for NVFP4) and are loaded 8 steps at a time; otherwise one load per step.
template <int BM, bool W13, int FMT, bool VS>
__device__ __forceinline__ void gemm_tile(const PrefillArgs& a, int tier, int r0, int loc, int tile,
                                          GemmSmem<BM>& sm) {
  using S = GemmShape<BM, W13>;
  constexpr int MT = S::MT, NT = S::NT;
  auto& As = sm.As;
  auto& Bs = sm.Bs;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;
  const int j = lane & 15, g = lane >> 4;
  const int n0 = tile * (W13 ? kBN / 2 : kBN);
  const int32_t* bslots = a.slots[tier] + r0;
  const size_t hbase = (size_t)(tier ? a.hrow1 : 0) + r0;
  const int steps = a.K / kBK;

  // ---- weight units. Thread (wave w, lane l) owns tile rows rA = 32 w + (l >> 2) and
  // rB = rA + 16 and, of every pair of steps, quarter p = l & 3 of each row's two-step
  // code segment (a quarter is one step's half row: step 2k + (p >> 1), half p & 1).
  // It loads quarter p of rA and quarter p ^ 2 of rB, so one load instruction reads 16
  // whole 64-byte (NF3: 48-byte) segments instead of 32 half-used ones, and the thread
  // ends up with one unit of each step: for step parity e the unit of row rowE[e], from
  // the rA load when (p >> 1) == e. Both rows have the same XOR swizzle (rA = rB mod 8).
  const int q4 = lane >> 2, p4 = lane & 3;
  const int hp = p4 >> 1, uu = p4 & 1;
  const int rA = 32 * wave + q4, rB = rA + 16;
  const int rowE[2] = {hp == 0 ? rA : rB, hp == 1 ? rA : rB};
  auto wrow_of = [&](int tr) {
    return W13 ? (tr < kBN / 2 ? n0 + tr : a.I + n0 + (tr - kBN / 2)) : n0 + tr;
  };
  const int RB = FMT == kPfNf3 ? 3 * a.K / 8 : a.K / 2;  // code bytes per row
  const int CB = FMT == kPfNf3 ? 24 : 32;                 // code bytes per row per step
  const int HB = CB / 2;                                  // code bytes of a half row step
  const uint8_t* qbase = FMT == kPfNf3 ? a.nq : a.kq;
  const size_t row0 = (size_t)loc * a.rows_w;
  const uint8_t* qA = qbase + (row0 + wrow_of(rA)) * RB + HB * p4;
  const uint8_t* qB = qbase + (row0 + wrow_of(rB)) * RB + HB * (p4 ^ 2);
  const int SRB = FMT == kPfNf3 ? a.K / 32 : a.K / (FMT == kPfNvfp4 ? 16 : 32);  // scale bytes per row
  const uint8_t* sE[2] = {a.ks, a.ks};
  if (FMT == kPfNf3) {
    sE[0] = reinterpret_cast<const uint8_t*>(a.ns) + (row0 + wrow_of(rowE[0])) * SRB;
    sE[1] = reinterpret_cast<const uint8_t*>(a.ns) + (row0 + wrow_of(rowE[1])) * SRB;
  } else {
    sE[0] = a.ks + (row0 + wrow_of(rowE[0])) * SRB;
    sE[1] = a.ks + (row0 + wrow_of(rowE[1])) * SRB;
  }
  // raw units of one pair of steps: x from row rA, y from row rB (scale words only
  // without VS; with VS they come from the per-parity scale vectors)
  struct PairRaw {
    uint4 qx, qy;
    uint32_t sx, sy;
  };
  // scale word of row rowE[e], step st, this thread's half (one load)
  auto load_s = [&](int e, int st) -> uint32_t {
    if constexpr (FMT == kPfNf3) return reinterpret_cast<const uint16_t*>(sE[e])[st];
    else if constexpr (FMT == kPfNvfp4) return *reinterpret_cast<const uint16_t*>(sE[e] + 4 * st + 2 * uu);
    else return sE[e][2 * st + uu];
  };
  auto load_pair = [&](int k, PairRaw& w) {
    if constexpr (FMT == kPfNf3) {
      const uint3 x = *reinterpret_cast<const uint3*>(qA + 2 * k * CB);
      const uint3 y = *reinterpret_cast<const uint3*>(qB + 2 * k * CB);
      w.qx = make_uint4(x.x, x.y, x.z, 0u);
      w.qy = make_uint4(y.x, y.y, y.z, 0u);
    } else {
      w.qx = *reinterpret_cast<const uint4*>(qA + 2 * k * CB);
      w.qy = *reinterpret_cast<const uint4*>(qB + 2 * k * CB);
    }
    if constexpr (!VS) {
      // the x unit is step 2k + hp of rA = rowE[hp]; the y unit the other step of rB
      w.sx = load_s(hp, 2 * k + hp);
      w.sy = load_s(hp ^ 1, 2 * k + (hp ^ 1));
    }
  };
  constexpr int SG = 8;                         // steps per scale vector
  constexpr int SW = FMT == kPfNvfp4 ? 8 : 4;   // dwords per scale vector
  typedef uint32_t SVec[SW];
  // scale vector of row rowE[e], steps SG grp .. SG grp + SG - 1
  auto load_sv = [&](int e, int grp, SVec& v) {
    const uint4* p = reinterpret_cast<const uint4*>(sE[e] + (FMT == kPfNvfp4 ? 4 : 2) * SG * grp);
    const uint4 v0 = p[0];
    v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
    if constexpr (FMT == kPfNvfp4) {
      const uint4 v1 = p[1];
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
  };
  // scale word of step SI (0..7) of a vector, for this thread's half of the row
  auto scale_of = [&](const SVec& v, auto si) -> uint32_t {
    constexpr int t = decltype(si)::value;
    if constexpr (FMT == kPfNvfp4) return __builtin_amdgcn_ubfe(v[t], 16 * uu, 16);
    else if constexpr (FMT == kPfMxfp4) return __builtin_amdgcn_ubfe(v[t >> 1], 16 * (t & 1) + 8 * uu, 8);
    else return __builtin_amdgcn_ubfe(v[t >> 1], 16 * (t & 1), 16);
  };

  // ---- per-row reference exponent (MXFP4: largest E8M0 byte; NF3: largest fp16
  // exponent field of the row's group scales) of rows rowE[0] and rowE[1], the four
  // lanes of a quad splitting each row's scales (lanes p and p ^ 2 hold the same two
  // rows, swapped); the loads of a lane's share are independent and issued together
  int refE[2] = {0, 0};
  if constexpr (FMT != kPfNvfp4) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      int ref = 0;
      if constexpr (VS) {
        const uint4* pv = reinterpret_cast<const uint4*>(sE[e]);
        const int nv = steps / SG;  // 16-byte vectors per row
#pragma unroll 4
        for (int c = uu; c < nv; c += 2) {
          const uint4 v = pv[c];
          const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (FMT == kPfMxfp4) {
              ref = max(ref, (int)__builtin_amdgcn_ubfe(d[i], 0, 8));
              ref = max(ref, (int)__builtin_amdgcn_ubfe(d[i], 8, 8));
              ref = max(ref, (int)__builtin_amdgcn_ubfe(d[i], 16, 8));
              ref = max(ref, (int)(d[i] >> 24));
            } else {
              ref = max(ref, (int)__builtin_amdgcn_ubfe(d[i], 10, 5));
              ref = max(ref, (int)__builtin_amdgcn_ubfe(d[i], 26, 5));
            }
          }
        }
      } else if constexpr (FMT == kPfMxfp4) {
#pragma unroll 8
        for (int i = uu; i < a.K / 32; i += 2) ref = max(ref, (int)sE[e][i]);
      } else {
        const uint16_t* s16 = reinterpret_cast<const uint16_t*>(sE[e]);
#pragma unroll 8
        for (int i = uu; i < a.K / 64; i += 2) ref = max(ref, (int)((s16[i] >> 10) & 0x1F));
      }
      refE[e] = max(ref, xlane_i<1>(ref));  // lanes p and p ^ 1 share row rowE[e]
    }
    if (uu == 0) {
      sm.sRef[rowE[0]] = refE[0];
      sm.sRef[rowE[1]] = refE[1];
    }
  }
  if (FMT == kPfNf3) {
    // thread t writes fields (t >> 5) + 8 i of column t & 31: low code t >> 5, high i
    const float lo = nf3_level(tid >> 5) * kNF3TableScaleF16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sm.lut[((tid >> 5) + 8 * i) * 32 + (tid & 31)] =
          pack_f16(lo, __uint_as_float(kNF3Bits[i]) * kNF3TableScaleF16);
  }
  const uint32_t* lut = sm.lut + (lane & 31);

  // decodes the unit of step parity e (codes q, scale word sw) into the B stage: 16 fp16
  // pairs, four 16-byte chunks of row rowE[e]
  auto store_w = [&](int buf, int e, const uint4& q, uint32_t sw) {
    const int r = rowE[e];
    const int ref = refE[e];
    uint32_t v[16];
    if constexpr (FMT == kPfNvfp4) {
      nvfp4_block_f16(q.x, q.y, sw & 0xFFu, v);
      nvfp4_block_f16(q.z, q.w, (sw >> 8) & 0xFFu, v + 8);
    } else if constexpr (FMT == kPfMxfp4) {
      const float so = e8m0_scale_operand((uint32_t)max((int)sw - ref + 127, 0));
      const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[4 * i + 0] = e2m1x2_f16<0>(qq[i], so);
        v[4 * i + 1] = e2m1x2_f16<1>(qq[i], so);
        v[4 * i + 2] = e2m1x2_f16<2>(qq[i], so);
        v[4 * i + 3] = e2m1x2_f16<3>(qq[i], so);
      }
    } else {
      const uint32_t d0 = q.x, d1 = q.y, d2 = q.z;
      const _Float16 mu = (_Float16)__builtin_ldexpf(fp16_to_f32(sw), 15 - ref);
      const f16x2 m = {mu, mu};
      v[0] = mul_f16x2(lut[nf3_pair_field<0>(d0, d1, d2) << 5], m);
      v[1] = mul_f16x2(lut[nf3_pair_field<1>(d0, d1, d2) << 5], m);
      v[2] = mul_f16x2(lut[nf3_pair_field<2>(d0, d1, d2) << 5], m);
      v[3] = mul_f16x2(lut[nf3_pair_field<3>(d0, d1, d2) << 5], m);
      v[4] = mul_f16x2(lut[nf3_pair_field<4>(d0, d1, d2) << 5], m);
      v[5] = mul_f16x2(lut[nf3_pair_field<5>(d0, d1, d2) << 5], m);
      v[6] = mul_f16x2(lut[nf3_pair_field<6>(d0, d1, d2) << 5], m);
      v[7] = mul_f16x2(lut[nf3_pair_field<7>(d0, d1, d2) << 5], m);
      v[8] = mul_f16x2(lut[nf3_pair_field<8>(d0, d1, d2) << 5], m);
      v[9] = mul_f16x2(lut[nf3_pair_field<9>(d0, d1, d2) << 5], m);
      v[10] = mul_f16x2(lut[nf3_pair_field<10>(d0, d1, d2) << 5], m);
      v[11] = mul_f16x2(lut[nf3_pair_field<11>(d0, d1, d2) << 5], m);
      v[12] = mul_f16x2(lut[nf3_pair_field<12>(d0, d1, d2) << 5], m);
      v[13] = mul_f16x2(lut[nf3_pair_field<13>(d0, d1, d2) << 5], m);
      v[14] = mul_f16x2(lut[nf3_pair_field<14>(d0, d1, d2) << 5], m);
      v[15] = mul_f16x2(lut[nf3_pair_field<15>(d0, d1, d2) << 5], m);
    }
    *reinterpret_cast<uint4*>(&Bs[buf][r][swz(r, 4 * uu + 0)]) = make_uint4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<uint4*>(&Bs[buf][r][swz(r, 4 * uu + 1)]) = make_uint4(v[4], v[5], v[6], v[7]);
    *reinterpret_cast<uint4*>(&Bs[buf][r][swz(r, 4 * uu + 2)]) = make_uint4(v[8], v[9], v[10], v[11]);
    *reinterpret_cast<uint4*>(&Bs[buf][r][swz(r, 4 * uu + 3)]) = make_uint4(v[12], v[13], v[14], v[15]);
  };

  // ---- activation rows of this thread (16-byte piece pc of row m), fixed over K.
  // Padding rows (no slot) read row 0: a GEMM never mixes rows, their outputs are
  // never used (W13's h rows of padding only feed W2's padding rows, whose outputs
  // the epilogue drops), and unconditional loads let the compiler count outstanding
  // loads exactly across the pipeline.
  uint32_t aoff[S::A_PER];
#pragma unroll
  for (int i = 0; i < S::A_PER; ++i) {
    const int c = tid + kPfThreads * i;
    const int m = c / (kBK / 8);
    const int pc = c - m * (kBK / 8);
    aoff[i] = 0;
    if (c < S::A_CHUNKS) {
      if (W13) {
        const int slot = bslots[m];
        if ((unsigned)slot < (unsigned)a.nslot) aoff[i] = (uint32_t)(slot / a.k) * a.K + 8 * pc;
      } else {
        aoff[i] = (uint32_t)((hbase + m) * a.K) + 8 * pc;
      }
    }
  }
  auto load_a = [&](int st, uint4 (&v)[S::A_PER]) {
#pragma unroll
    for (int i = 0; i < S::A_PER; ++i)
      v[i] = *reinterpret_cast<const uint4*>(a.act + aoff[i] + st * kBK);
  };
  auto store_a = [&](int buf, const uint4 (&v)[S::A_PER]) {
#pragma unroll
    for (int i = 0; i < S::A_PER; ++i) {
      const int c = tid + kPfThreads * i;
      if (S::A_CHUNKS % kPfThreads == 0 || c < S::A_CHUNKS) {
        const int m = c / (kBK / 8);
        // per-component copy: a whole-vector copy out of the register set makes the
        // compiler keep the sets in private memory
        *reinterpret_cast<uint4*>(&As[buf][m][swz(m, c - m * (kBK / 8))]) =
            make_uint4(v[i].x, v[i].y, v[i].z, v[i].w);
      }
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      // row bases are multiples of 16: the low swizzle term comes from j, the high
      // one from the base
      const int kk = 8 * ((4 * ks + g) ^ swz_lo(j));
      uint4 bq[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tr = tile_row<BM, W13>(wn, nt);
        bq[nt] = *reinterpret_cast<const uint4*>(&Bs[buf][tr + j][kk ^ (8 * swz_hi(tr))]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int ar = (wm * MT + mt) * 16;
        const uint4 aq = *reinterpret_cast<const uint4*>(&As[buf][ar + j][kk ^ (8 * swz_hi(ar))]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, aq), __builtin_bit_cast(f16x8, bq[nt]), acc[mt][nt], 0, 0, 0);
      }
    }
  };

  // ---- pipeline. The raw units of step pair k are loaded at step 2k - 3 into pair
  // slot k % 2 (a slot is free once its pair's second step has been decoded, at step
  // 2k - 4) and decoded into the free LDS stage one step ahead; activations are loaded
  // AD steps ahead into AD register sets. A group of U steps (a multiple of 2 pairs,
  // AD, the two LDS stages and a scale vector) names every slot at compile time. Each
  // step issues its loads in the order they are consumed (vector memory completes in
  // order), and the stores of the next stage stay behind the MFMAs. Whole groups run
  // unguarded; the last steps run guarded (steps is even: K is a multiple of 128).
  constexpr int AD = kActAhead, U = kPipeGroup;
  static_assert(U % 4 == 0 && U % AD == 0 && U % SG == 0, "pipeline group");
  PairRaw pr[2];
  uint4 av[AD][S::A_PER];
  // VS: per-parity scale vectors of the current and the next group of SG steps
  SVec scur[2] = {}, snext[2] = {};
  if constexpr (VS) {
    load_sv(0, 0, scur[0]);
    load_sv(1, 0, scur[1]);
  }
  static_for<AD>([&](auto i) {
    if (i.value < steps) load_a(i.value, av[i.value]);
  });
  load_pair(0, pr[0]);
  if (2 < steps) load_pair(1, pr[1]);
  // unit of step t (parity E) from pair slot (t / 2) % 2; VC: the current scale
  // vectors hold step t (else the next ones do)
  auto unit_store = [&](int buf, auto E, auto TS, auto VC, const PairRaw& w) {
    constexpr int e = decltype(E)::value;
    const bool from_x = hp == e;
    const uint4 q = from_x ? w.qx : w.qy;
    uint32_t sw;
    if constexpr (VS) sw = scale_of(VC.value ? scur[e] : snext[e], TS);
    else sw = from_x ? w.sx : w.sy;
    store_w(buf, e, q, sw);
  };
  // the epilogue's per-row data, requested behind the first loads so that its latency
  // overlaps theirs instead of adding to the block's end (W13's first column tile also
  // writes the rows' W2 output factors)
  if (tid < BM) {
    const int slot = bslots[tid];
    sm.rowSlot[tid] = slot;
    if constexpr (W13) {
      const bool real = (unsigned)slot < (unsigned)a.nslot;
      const int e = real ? a.xe[slot / a.k] : 0;
      sm.rowE[tid] = e;
      if (tile == 0)
        a.row_fac[hbase + tid] = real ? __builtin_ldexpf(a.topk_w[slot], h_exponent(e)) : 0.0f;
    } else {
      sm.rowF[tid] = a.row_fac[hbase + tid];
    }
  }
  __syncthreads();  // table, reference exponents, row data
  store_a(0, av[0]);
  unit_store(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
             std::true_type{}, pr[0]);
  __syncthreads();
  // step st = group base + i: MFMAs on stage i & 1; stage (i + 1) & 1 takes the
  // activations and the raw unit of step st + 1; loads fill the activation set of
  // st + AD and, at odd steps, pair slot of pair (st + 3) / 2; a scale vector pair is
  // requested at the group's first step for the next group
  auto step = [&](int st0, auto I, bool guarded) {
    constexpr int i = I.value;
    const int s = st0 + i;
    if constexpr (VS && i % SG == 0) {
      if (!guarded || s + SG < steps) {
        load_sv(0, (s + SG) / SG, snext[0]);
        load_sv(1, (s + SG) / SG, snext[1]);
      }
    }
    if (!guarded || s + AD < steps) load_a(s + AD, av[(i + AD) % AD]);
    if constexpr (i % 2 == 1) {
      if (!guarded || s + 3 < steps) load_pair((s + 3) / 2, pr[((i + 3) / 2) % 2]);
    }
    compute(i & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (!guarded || s + 1 < steps) {
      store_a((i + 1) & 1, av[(i + 1) % AD]);
      constexpr int t = i + 1;  // step decoded now, relative to the group base
      unit_store((i + 1) & 1, std::integral_constant<int, t & 1>{},
                 std::integral_constant<int, t % SG>{},
                 std::integral_constant<bool, (t < SG)>{}, pr[(t / 2) % 2]);
    }
    __syncthreads();
    if constexpr (VS && i % SG == SG - 1) {
#pragma unroll
      for (int e = 0; e < SW; ++e) {
        scur[0][e] = snext[0][e];
        scur[1][e] = snext[1][e];
      }
    }
  };
  int st = 0;
  for (; st + U + 3 <= steps; st += U) {
    static_for<U>([&](auto I) { step(st, I, false); });
  }
  for (; st < steps; st += U) {
    static_for<U>([&](auto I) {
      if (st + I.value < steps) step(st, I, true);
    });
  }

  // ---- epilogue: lane holds rows 4 * g + q of each 16-row tile, column j
  auto col_factor = [&](int trow) {
    if (FMT == kPfNf3) return __builtin_ldexpf(1.0f / kNF3TableScaleF16, sm.sRef[trow] - 15);
    if (FMT == kPfNvfp4) return a.kg[loc];
    return e8m0_to_f32((uint32_t)sm.sRef[trow]);
  };
#pragma unroll
  for (int nt = 0; nt < (W13 ? NT / 2 : NT); ++nt) {
    const int tr = tile_row<BM, W13>(wn, nt) + j;
    const int n = n0 + tr;
    const float gf = col_factor(tr);
    const float uf = W13 ? col_factor(tile_row<BM, W13>(wn, nt + NT / 2) + j) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = (wm * MT + mt) * 16 + 4 * g + q;
        const int slot = sm.rowSlot[m];
        if (W13) {
          // x was scaled by 2^-e, h is stored times 2^-he
          const bool real = (unsigned)slot < (unsigned)a.nslot;
          const int e = sm.rowE[m];
          const float xs = real ? __builtin_ldexpf(1.0f, e) : 0.0f;
          const float gate = acc[mt][nt][q] * gf * xs;
          const float up = acc[mt][nt + NT / 2][q] * uf * xs;
          const float hv = __builtin_ldexpf(silu(gate) * up, -h_exponent(e));
          const float h = fminf(fmaxf(hv, -65504.0f), 65504.0f);
          a.h_out[(hbase + m) * a.I + n] = (uint16_t)(pack_f16(h, 0.0f) & 0xFFFFu);
        } else {
          // factor = w * 2^he exactly, so this is the rounded (acc * gf * w) scaled by 2^he
          if ((unsigned)slot < (unsigned)a.nslot)
            a.o_out[(size_t)slot * a.H + n] = acc[mt][nt][q] * gf * sm.rowF[m];
        }
      }
    }
  }
}

// One tile of BMC slot rows at row r0 (BMC <= BMAX), in the format of its tier and the
// layer's scale layout.
template <int BMC, int BMAX, bool W13>
__device__ __forceinline__ void gemm_tile_any(const PrefillArgs& a, int tier, int r0, int loc, int tile,
                                              unsigned char* smem) {
  static_assert(sizeof(GemmSmem<BMC>) <= sizeof(GemmSmem<BMAX>), "tile class larger than its block");
  GemmSmem<BMC>& sm = *reinterpret_cast<GemmSmem<BMC>*>(smem);
  if (a.vec_scales) {
    if (tier == HMOE_TIER_NF3) gemm_tile<BMC, W13, kPfNf3, true>(a, tier, r0, loc, tile, sm);
    else if (a.kept_fmt == HMOE_KEPT_NVFP4) gemm_tile<BMC, W13, kPfNvfp4, true>(a, tier, r0, loc, tile, sm);
    else gemm_tile<BMC, W13, kPfMxfp4, true>(a, tier, r0, loc, tile, sm);
  } else {
    if (tier == HMOE_TIER_NF3) gemm_tile<BMC, W13, kPfNf3, false>(a, tier, r0, loc, tile, sm);
    else if (a.kept_fmt == HMOE_KEPT_NVFP4) gemm_tile<BMC, W13, kPfNvfp4, false>(a, tier, r0, loc, tile, sm);
    else gemm_tile<BMC, W13, kPfMxfp4, false>(a, tier, r0, loc, tile, sm);
  }
}

// Grid blocks cover the align stage's BMAX-row blocks. An expert's last block holds its
// remaining slots followed by sentinel padding, so the block runs the smallest tile
// class (16, 32, 64 or BMAX rows) that reaches its first sentinel: padding rows past
// that class are neither multiplied nor written, by this launch or the W2 launch (the
// same slots give it the same class).
template <int BMAX, bool W13>
__device__ __forceinline__ void grouped_gemm_block(const PrefillArgs& a, int L) {
  // A 1-D grid. The dispatcher hands consecutive block ids to the eight XCDs in
  // turn (id L runs on XCD L % 8), so id L is given a group of kXcdGroup expert blocks
  // owned by XCD L % 8, and the ids of one XCD walk a group's column tiles with its
  // blocks innermost: an expert block's activation rows and the weight tile its
  // group's blocks share stay in that XCD's L2.
  const int idx = L >> 3;
  const int per_group = a.ntile * kXcdGroup;
  const int grp = idx / per_group;
  const int rem = idx - grp * per_group;
  const int tile = rem / kXcdGroup;
  const int by = (grp * 8 + (L & 7)) * kXcdGroup + (rem - tile * kXcdGroup);
  if (by >= a.nblk0 + a.nblk1) return;
  const int tier = by < a.nblk0 ? 0 : 1;
  const int b = tier ? by - a.nblk0 : by;
  // npad and the block table come from the align stage; clamp to this launch's grid
  // and the tier's expert count so stale scratch cannot index out of range
  if (b * BMAX >= a.npad[tier][0] || b >= (tier ? a.nblk1 : a.nblk0)) return;
  const int loc = a.bexp[tier][b];
  if ((unsigned)loc >= (unsigned)(tier ? a.E3 : a.E4)) return;
  const int r0 = b * BMAX;
  // real rows r of this block: slots [r0, r0 + r) are real, the rest sentinels (>= nslot)
  const int32_t* sl = a.slots[tier] + r0;
  int cls = BMAX;
  if constexpr (BMAX >= 128) if (sl[64] >= a.nslot) cls = 64;
  if constexpr (BMAX >= 64) if (sl[32] >= a.nslot) cls = 32;
  if constexpr (BMAX >= 32) if (sl[16] >= a.nslot) cls = 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[sizeof(GemmSmem<BMAX>)];
  if constexpr (BMAX >= 32) {
    if (cls == 16) return gemm_tile_any<16, BMAX, W13>(a, tier, r0, loc, tile, smem);
  }
  if constexpr (BMAX >= 64) {
    if (cls == 32) return gemm_tile_any<32, BMAX, W13>(a, tier, r0, loc, tile, smem);
  }
  if constexpr (BMAX >= 128) {
    if (cls == 64) return gemm_tile_any<64, BMAX, W13>(a, tier, r0, loc, tile, smem);
  }
  gemm_tile_any<BMAX, BMAX, W13>(a, tier, r0, loc, tile, smem);
}

template <int BMAX, bool W13>
__global__ __launch_bounds__(kPfThreads, 2) void grouped_gemm_kernel(PrefillArgs a) {
  grouped_gemm_block<BMAX, W13>(a, blockIdx.x);
}

// The W4A4 layer's GEMM launch: the NF3 tier's W4A16 blocks (ids below nf3_grid, the
// grouped_gemm_kernel grid) and then the kept tier's MX blocks (column tiles fastest), so
// both tiers run in one launch and overlap on the GPU.
template <int BMAX, bool W13>
__global__ __launch_bounds__(kPfThreads, 2) void grouped_gemm_w4a4_kernel(PrefillArgs a, MxArgs m,
                                                                          int nf3_grid, int mx_tiles) {
  const int L = blockIdx.x;
  if (L < nf3_grid) {
    grouped_gemm_block<BMAX, W13>(a, L);
  } else {
    const int i = L - nf3_grid;
    mx_gemm_tile<BMAX, W13>(m, i / mx_tiles, i - (i / mx_tiles) * mx_tiles);
  }
}

// x16[t] = fp16(x[t] * 2^-e[t]), e[t] putting the token's largest |x| in [2^14, 2^15);
// eight elements per thread and step (16-byte loads and stores; H is a multiple of 128)
__global__ __launch_bounds__(256) void prefill_x16_kernel(const uint16_t* __restrict__ x, int H,
                                                          uint16_t* __restrict__ x16,
                                                          int32_t* __restrict__ xe) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4* out = reinterpret_cast<uint4*>(x16 + (size_t)t * H);
  const int n8 = H / 8;
  float mx = 0.0f;
  for (int i = threadIdx.x; i < n8; i += 256) {
    const uint4 v = row[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(w[c])), fabsf(bf16_hi(w[c]))));
  }
  mx = group_max<kWave>(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int ef = (int)((__float_as_uint(mx) >> 23) & 0xFF);
  const int e = mx > 0.0f ? (ef == 0 ? -126 : ef - 127) - 14 : 0;
  for (int i = threadIdx.x; i < n8; i += 256) {
    const uint4 v = row[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = pack_f16(__builtin_ldexpf(bf16_lo(w[c]), -e), __builtin_ldexpf(bf16_hi(w[c]), -e));
    out[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (threadIdx.x == 0) xe[t] = e;
}

// y[t, n..n+3] = sum_j o[t*k + j, n..n+3] in fixed j order (the routing weight is
// already in o); four columns per thread, 16-byte loads (H is a multiple of 128)
__global__ __launch_bounds__(256) void prefill_combine_kernel(const float* __restrict__ o, int M,
                                                              int k, int H,
                                                              uint16_t* __restrict__ y) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // index of a 4-column group
  const size_t nq = (size_t)M * (H / 4);
  if (q >= nq) return;
  const size_t t = q / (H / 4);
  const size_t n = (q - t * (H / 4)) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(o + (t * k + j) * H + n);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *reinterpret_cast<uint2*>(y + t * H + n) = make_uint2(pack_bf16(acc.x, acc.y), pack_bf16(acc.z, acc.w));
}

typedef void (*GemmFn)(PrefillArgs);
typedef void (*GemmW4a4Fn)(PrefillArgs, MxArgs, int, int);

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

template <bool W13>
static GemmW4a4Fn pick_gemm_w4a4(int bm) {
  switch (bm) {
    case 16: return grouped_gemm_w4a4_kernel<16, W13>;
    case 32: return grouped_gemm_w4a4_kernel<32, W13>;
    case 64: return grouped_gemm_w4a4_kernel<64, W13>;
    case 128: return grouped_gemm_w4a4_kernel<128, W13>;
  }
  return nullptr;
}

// one GEMM launch: the grouped GEMM alone, or (W4A4 layers) with the kept tier's MX
// blocks after the NF3 tier's
template <bool W13>
static hipError_t launch_gemm(const Layer& L, const hmoe_weights& W, int M, void* scratch,
                              const PrefillArgs& b, unsigned grid, bool w4a4, hipStream_t s) {
  if (!w4a4) {
    GemmFn fn = pick_gemm<W13>(L.block_m);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kPfThreads), 0, s, b);
    return hipGetLastError();
  }
  GemmW4a4Fn fn = pick_gemm_w4a4<W13>(L.block_m);
  if (!fn) return hipErrorInvalidValue;
  const MxArgs m = mx_args(L, W, M, scratch, W13 ? HMOE_STAGE_W13 : HMOE_STAGE_W2);
  const int tiles = mx_tiles(L, W13);
  const unsigned total = grid + (unsigned)(m.nblk * tiles);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(total), dim3(kPfThreads), 0, s, b, m, (int)grid, tiles);
  return hipGetLastError();
}

// scale rows of whole, aligned 16-byte vectors of 8 K steps (512 K values), both tiers
static int vec_scales_ok(const PrefillArgs& a) {
  const bool rows = a.K % (8 * kBK) == 0;
  const bool al = (reinterpret_cast<uintptr_t>(a.ks) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.ns) % 16 == 0);
  return rows && al ? 1 : 0;
}

// blocks of the 1-D GEMM grid: whole XCD groups of expert blocks times column tiles
static unsigned gemm_grid(int nblk, int ntile) {
  const int unit = 8 * kXcdGroup;
  return (unsigned)((nblk + unit - 1) / unit * unit) * (unsigned)ntile;
}

hipError_t launch_prefill_x16(const Layer& L, const uint16_t* x, int M, void* scratch,
                              hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  hipLaunchKernelGGL(prefill_x16_kernel, dim3(M), dim3(256), 0, s, x, L.H,
                     reinterpret_cast<uint16_t*>(base + L.plan.x16_pre),
                     reinterpret_cast<int32_t*>(base + L.plan.xe_pre));
  return hipGetLastError();
}

hipError_t launch_prefill(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                          uint16_t* y, void* scratch, int stage, hipStream_t s, bool nf3_only) {
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
  a.nblk0 = (L.E4 > 0 && !nf3_only) ? (cap0 + bm - 1) / bm : 0;
  a.nblk1 = L.E3 > 0 ? (cap1 + bm - 1) / bm : 0;
  a.hrow1 = L.cap[0];
  a.I = L.I;
  a.H = L.H;
  uint16_t* h = reinterpret_cast<uint16_t*>(base + P.h_pre);
  float* o = reinterpret_cast<float*>(base + P.o_pre);
  a.row_fac = reinterpret_cast<float*>(base + P.pf_fac);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base + P.x16_pre);
  int32_t* xe = reinterpret_cast<int32_t*>(base + P.xe_pre);
  const int nblk = a.nblk0 + a.nblk1;
  if (stage == HMOE_STAGE_W13) {
    PrefillArgs b = a;
    b.kq = W.kept_w13_q; b.ks = W.kept_w13_s; b.kg = W.kept_w13_g;
    b.nq = W.nf3_w13_q; b.ns = W.nf3_w13_s;
    b.rows_w = 2 * L.I;
    b.K = L.H;
    b.act = x16;
    b.xe = xe;
    b.h_out = h;
    b.topk_w = w;
    b.ntile = L.I / (kBN / 2);
    b.vec_scales = vec_scales_ok(b);
    return launch_gemm<true>(L, W, M, scratch, b, nblk > 0 ? gemm_grid(nblk, b.ntile) : 0u, nf3_only, s);
  }
  if (stage == HMOE_STAGE_W2) {
    PrefillArgs c = a;
    c.kq = W.kept_w2_q; c.ks = W.kept_w2_s; c.kg = W.kept_w2_g;
    c.nq = W.nf3_w2_q; c.ns = W.nf3_w2_s;
    c.rows_w = L.H;
    c.K = L.I;
    c.act = h;
    c.xe = xe;
    c.o_out = o;
    c.topk_w = w;
    c.ntile = L.H / kBN;
    c.vec_scales = vec_scales_ok(c);
    return launch_gemm<false>(L, W, M, scratch, c, nblk > 0 ? gemm_grid(nblk, c.ntile) : 0u, nf3_only, s);
  }
  if (stage == HMOE_STAGE_COMBINE) {
    const size_t n = (size_t)M * (L.H / 4);
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       o, M, L.k, L.H, y);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace hmoe
