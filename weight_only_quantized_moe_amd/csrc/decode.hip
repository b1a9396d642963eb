// Decode path (M <= 8): route + grouping, then for every distinct touched expert a
// GEMV over its packed W13 with a fused SwiGLU, a GEMV over its packed W2, and the
// deterministic top-k weighted combine into y. Both tiers run in the same launches
// from one routing result (local-inference-lab/vllm PR #92, "How it works": launches
// sharing one route geometry and one top-k sum; M <= 8 addressed directly by the
// top-k result).
//
// GEMV mapping: a task is (distinct expert d, tile of rows). The 4 waves of a block
// split K into WK parts and the task's rows into 4/WK groups. Inside a wave, LR lanes
// share a row and each lane owns KU units of 32 K-elements (unit u = c + LR*j), so a
// wave instruction reads LR consecutive 16-byte (FP4) or 12-byte (NF3) units of P =
// 64/LR rows. The lane keeps the matching activations of up to two tokens in
// registers as 16-bit pairs and meets the decoded weight pairs in v_dot2_f32_*.
//
// Precision: W13 runs on bf16 pairs (x is bf16; E2M1 values are exact in bf16; the
// NVFP4 E4M3 block scale multiplies the fp32 partial of its 16-block; MXFP4's
// power-of-two scale is folded into the conversion; NF3 levels come from a scaled
// table, see kNF3TableScaleBf16, with the fp16 group scale on the fp32 partial). h
// leaves W13 in fp32. W2 runs on fp16 pairs: each slot's h row is scaled by a power
// of two so its largest magnitude lands in [2^14, 2^15), which keeps 11 significant
// bits for every element that matters; E2M1 is exact in fp16 and every block or
// group scale again multiplies an fp32 partial.
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

constexpr int kGemvThreads = 256;
constexpr int kMaxTaskRows = 256;

struct GemvArgs {
  const uint8_t* kq;   // kept codes [E4, rows, K/2]
  const uint8_t* ks;   // kept scales [E4, rows, K/16] (E4M3) or [E4, rows, K/32] (E8M0)
  const float* kg;     // kept per-tensor scale [E4] (NVFP4)
  const uint8_t* nq;   // NF3 codes [E3, rows, 3K/8]
  const uint16_t* ns;  // NF3 scales [E3, rows, K/64]
  int kept_fmt;
  int rows, K;
  const uint16_t* act_bf16;  // W13: x bf16 [M, K]
  const float* act_f32;      // W2: h fp32 [slots, K]
  int act_row_div;           // activation row of slot s is s / act_row_div
  const int32_t* counts;
  const int32_t* experts;
  const int32_t* nslots;
  const int32_t* slots;
  const int32_t* expert_tier;
  int tile_rows;  // output rows per task (W13: gate rows; each also brings its up row)
  int tiles;      // tasks per expert
  int I;          // W13: row offset of the up projection
  float* h_out;   // W13: fp32 [slots, I]
  float* o_out;   // W2: fp32 [slots, rows]
};

// Partial dot products of one lane for one row over its KU units. F16 selects the
// fp16 pair path (W2) over the bf16 one (W13).
template <int LR, int KU, int NT, bool F16>
struct RowDot {
  static __device__ __forceinline__ float dot(uint32_t w, uint32_t x, float c) {
    if constexpr (F16) return dot2_f16(w, x, c);
    else return dot2(w, x, c);
  }
  template <int SEL>
  static __device__ __forceinline__ uint32_t fp4(uint32_t v, float s) {
    if constexpr (F16) return e2m1x2_f16<SEL>(v, s);
    else return e2m1x2_bf16<SEL>(v, s);
  }
  static __device__ __forceinline__ void fp4x16(const uint4& q, float s, uint32_t (&w)[16]) {
    w[0] = fp4<0>(q.x, s); w[1] = fp4<1>(q.x, s); w[2] = fp4<2>(q.x, s); w[3] = fp4<3>(q.x, s);
    w[4] = fp4<0>(q.y, s); w[5] = fp4<1>(q.y, s); w[6] = fp4<2>(q.y, s); w[7] = fp4<3>(q.y, s);
    w[8] = fp4<0>(q.z, s); w[9] = fp4<1>(q.z, s); w[10] = fp4<2>(q.z, s); w[11] = fp4<3>(q.z, s);
    w[12] = fp4<0>(q.w, s); w[13] = fp4<1>(q.w, s); w[14] = fp4<2>(q.w, s); w[15] = fp4<3>(q.w, s);
  }
  // NVFP4: E2M1 exact, E4M3 scale on each 16-block's fp32 partial
  static __device__ __forceinline__ void nvfp4(const uint8_t* __restrict__ qrow,
                                               const uint8_t* __restrict__ srow, int c,
                                               const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      const uint4 q = *reinterpret_cast<const uint4*>(qrow + 16 * u);
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(srow + 2 * u);
      const float s0 = e4m3_to_f32<0>(sc);
      const float s1 = e4m3_to_f32<1>(sc);
      uint32_t w[16];
      fp4x16(q, 1.0f, w);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p0 = dot(w[i], x[t][j][i], p0);
#pragma unroll
        for (int i = 8; i < 16; ++i) p1 = dot(w[i], x[t][j][i], p1);
        acc[t] = __builtin_fmaf(s0, p0, acc[t]);
        acc[t] = __builtin_fmaf(s1, p1, acc[t]);
      }
    }
  }
  // MXFP4: bf16 folds the E8M0 exponent into the conversion (exact); fp16 cannot
  // hold that range, so there the exact fp32 2^(b - 127) scales the partial
  static __device__ __forceinline__ void mxfp4(const uint8_t* __restrict__ qrow,
                                               const uint8_t* __restrict__ srow, int c,
                                               const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      const uint4 q = *reinterpret_cast<const uint4*>(qrow + 16 * u);
      const uint32_t b = srow[u];
      uint32_t w[16];
      if constexpr (F16) {
        fp4x16(q, 1.0f, w);
        const float sc = e8m0_to_f32(b);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float p = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) p = dot(w[i], x[t][j][i], p);
          acc[t] = __builtin_fmaf(sc, p, acc[t]);
        }
      } else {
        fp4x16(q, e8m0_scale_operand(b), w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[t] = dot(w[i], x[t][j][i], acc[t]);
        }
      }
    }
  }
  // NF3: level pairs from the per-lane LDS table, fp16 group scale per 64
  static __device__ __forceinline__ void nf3(const uint8_t* __restrict__ qrow,
                                             const uint16_t* __restrict__ srow, int c,
                                             const uint32_t* __restrict__ lut_lane,
                                             const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      const uint32_t* p = reinterpret_cast<const uint32_t*>(qrow + 12 * u);
      const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
      const float s = fp16_to_f32(srow[u >> 1]);
      uint32_t w[16];
      w[0] = lut_lane[nf3_pair_field<0>(d0, d1, d2) << 6];
      w[1] = lut_lane[nf3_pair_field<1>(d0, d1, d2) << 6];
      w[2] = lut_lane[nf3_pair_field<2>(d0, d1, d2) << 6];
      w[3] = lut_lane[nf3_pair_field<3>(d0, d1, d2) << 6];
      w[4] = lut_lane[nf3_pair_field<4>(d0, d1, d2) << 6];
      w[5] = lut_lane[nf3_pair_field<5>(d0, d1, d2) << 6];
      w[6] = lut_lane[nf3_pair_field<6>(d0, d1, d2) << 6];
      w[7] = lut_lane[nf3_pair_field<7>(d0, d1, d2) << 6];
      w[8] = lut_lane[nf3_pair_field<8>(d0, d1, d2) << 6];
      w[9] = lut_lane[nf3_pair_field<9>(d0, d1, d2) << 6];
      w[10] = lut_lane[nf3_pair_field<10>(d0, d1, d2) << 6];
      w[11] = lut_lane[nf3_pair_field<11>(d0, d1, d2) << 6];
      w[12] = lut_lane[nf3_pair_field<12>(d0, d1, d2) << 6];
      w[13] = lut_lane[nf3_pair_field<13>(d0, d1, d2) << 6];
      w[14] = lut_lane[nf3_pair_field<14>(d0, d1, d2) << 6];
      w[15] = lut_lane[nf3_pair_field<15>(d0, d1, d2) << 6];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float pp = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) pp = dot(w[i], x[t][j][i], pp);
        acc[t] = __builtin_fmaf(s, pp, acc[t]);
      }
    }
  }
};

// One pass over the task's rows for NT (1 or 2) tokens; writes per-K-part row
// results into res[kpart][row][t].
template <int LR, int KU, int WK, int RI, int NT, bool W13>
__device__ __forceinline__ void gemv_pass(const GemvArgs& a, bool nf3, int loc, int tile,
                                          const uint32_t (&x)[NT][KU][16],
                                          const uint32_t* __restrict__ lut_lane,
                                          float (*res)[kMaxTaskRows][2]) {
  constexpr bool F16 = !W13;
  constexpr int P = kWave / LR;
  constexpr int RG = 4 / WK;  // row groups
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int kpart = wave % WK;
  const int rgroup = wave / WK;
  const int c = lane % LR;
  const int rw = lane / LR;
  const int task_rows = W13 ? 2 * a.tile_rows : a.tile_rows;
  const int Kp = a.K / WK;  // K-elements of this part
  for (int r0 = rgroup * P * RI; r0 < task_rows; r0 += RG * P * RI) {
    float acc[RI][NT];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[ri][t] = 0.0f;
      const int rr = r0 + ri * P + rw;
      const int row = W13 ? (rr < a.tile_rows ? tile * a.tile_rows + rr
                                             : a.I + tile * a.tile_rows + (rr - a.tile_rows))
                          : tile * a.tile_rows + rr;
      const size_t grow = (size_t)loc * a.rows + row;
      if (nf3) {
        const uint8_t* qrow = a.nq + grow * (3 * a.K / 8) + (size_t)kpart * (3 * Kp / 8);
        const uint16_t* srow = a.ns + grow * (a.K / 64) + kpart * (Kp / 64);
        RowDot<LR, KU, NT, F16>::nf3(qrow, srow, c, lut_lane, x, acc[ri]);
      } else if (a.kept_fmt == HMOE_KEPT_NVFP4) {
        const uint8_t* qrow = a.kq + grow * (a.K / 2) + (size_t)kpart * (Kp / 2);
        const uint8_t* srow = a.ks + grow * (a.K / 16) + kpart * (Kp / 16);
        RowDot<LR, KU, NT, F16>::nvfp4(qrow, srow, c, x, acc[ri]);
      } else {
        const uint8_t* qrow = a.kq + grow * (a.K / 2) + (size_t)kpart * (Kp / 2);
        const uint8_t* srow = a.ks + grow * (a.K / 32) + kpart * (Kp / 32);
        RowDot<LR, KU, NT, F16>::mxfp4(qrow, srow, c, x, acc[ri]);
      }
    }
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      const int rr = r0 + ri * P + rw;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = group_sum<LR>(acc[ri][t]);
        if (c == 0) res[kpart][rr][t] = v;
      }
    }
  }
}

// W13 activations: the lane's x units of up to two tokens as bf16 pairs.
template <int LR, int KU, int WK, int NT>
__device__ __forceinline__ void load_act_bf16(const GemvArgs& a, int s0, int s1,
                                              uint32_t (&x)[NT][KU][16]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kpart = (threadIdx.x >> 6) % WK;
  const int c = lane % LR;
  const int Kp = a.K / WK;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int s = t == 0 ? s0 : s1;
    const uint16_t* row = a.act_bf16 + (size_t)(s / a.act_row_div) * a.K + (size_t)kpart * Kp;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const uint4* p = reinterpret_cast<const uint4*>(row + 32 * (c + LR * j));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 q = p[v];
        x[t][j][4 * v + 0] = q.x;
        x[t][j][4 * v + 1] = q.y;
        x[t][j][4 * v + 2] = q.z;
        x[t][j][4 * v + 3] = q.w;
      }
    }
  }
}

// W2 activations: the lane's h units (fp32) of up to two slots, scaled by 2^-e[t]
// with e[t] chosen from the slot's largest |h| (over the whole row, reduced across
// the block) and rounded to fp16 pairs. The row is read twice (max, then convert);
// it is a few KB and cache-resident. Every thread of the block must call this.
template <int LR, int KU, int WK, int NT>
__device__ __forceinline__ void load_act_f16(const GemvArgs& a, int s0, int s1,
                                             uint32_t (&x)[NT][KU][16], int (&e)[NT],
                                             float (*s_max)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int kpart = wave % WK;
  const int c = lane % LR;
  const int Kp = a.K / WK;
  const float* rows[NT];
  float mx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int s = t == 0 ? s0 : s1;
    rows[t] = a.act_f32 + (size_t)(s / a.act_row_div) * a.K + (size_t)kpart * Kp;
    mx[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const float4* p = reinterpret_cast<const float4*>(rows[t] + 32 * (c + LR * j));
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 q = p[v];
        mx[t] = fmaxf(mx[t], fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) s_max[wave][t] = mx[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float m = fmaxf(fmaxf(s_max[0][t], s_max[1][t]), fmaxf(s_max[2][t], s_max[3][t]));
    // scale so that max * 2^-e lands in [2^14, 2^15), inside fp16's range
    const int ef = (int)((__float_as_uint(m) >> 23) & 0xFF);
    e[t] = m > 0.0f ? (ef == 0 ? -126 : ef - 127) - 14 : 0;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const float4* p = reinterpret_cast<const float4*>(rows[t] + 32 * (c + LR * j));
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 q = p[v];
        x[t][j][2 * v] = pack_f16(__builtin_ldexpf(q.x, -e[t]), __builtin_ldexpf(q.y, -e[t]));
        x[t][j][2 * v + 1] = pack_f16(__builtin_ldexpf(q.z, -e[t]), __builtin_ldexpf(q.w, -e[t]));
      }
    }
  }
  __syncthreads();
}

template <int LR, int KU, int WK, int RI, bool W13>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  __shared__ uint32_t lut[64 * kWave];  // [pair field][lane]: 16-bit pair of scaled NF3 levels
  __shared__ float res[WK][kMaxTaskRows][2];
  __shared__ float s_max[4][2];
  for (int i = threadIdx.x; i < 64 * kWave; i += kGemvThreads) {
    const int f = i / kWave;
    if (W13)
      lut[i] = pack_bf16(nf3_level(f & 7) * kNF3TableScaleBf16, nf3_level(f >> 3) * kNF3TableScaleBf16);
    else
      lut[i] = pack_f16(nf3_level(f & 7) * kNF3TableScaleF16, nf3_level(f >> 3) * kNF3TableScaleF16);
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t* lut_lane = lut + lane;
  const int ntask = a.counts[0] * a.tiles;
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int d = task / a.tiles;
    const int tile = task - d * a.tiles;
    const int e = a.experts[d];
    const int tc = a.expert_tier[e];
    const bool nf3 = (tc >> 16) != 0;
    const int loc = tc & 0xFFFF;
    const int n = a.nslots[d];
    // per-row factor: NVFP4 per-tensor scale, or 1/c of the scaled NF3 table
    float g = 1.0f;
    if (nf3) g = 1.0f / (W13 ? kNF3TableScaleBf16 : kNF3TableScaleF16);
    else if (a.kept_fmt == HMOE_KEPT_NVFP4) g = a.kg[loc];
    for (int p0 = 0; p0 < n; p0 += 2) {
      const int nt = n - p0 >= 2 ? 2 : 1;
      const int s0 = a.slots[d * kDecodeMaxM + p0];
      const int s1 = nt == 2 ? a.slots[d * kDecodeMaxM + p0 + 1] : s0;
      int ex[2] = {0, 0};
      if (nt == 2) {
        uint32_t x[2][KU][16];
        if constexpr (W13) {
          load_act_bf16<LR, KU, WK, 2>(a, s0, s1, x);
        } else {
          int e2[2];
          load_act_f16<LR, KU, WK, 2>(a, s0, s1, x, e2, s_max);
          ex[0] = e2[0];
          ex[1] = e2[1];
        }
        gemv_pass<LR, KU, WK, RI, 2, W13>(a, nf3, loc, tile, x, lut_lane, res);
      } else {
        uint32_t x[1][KU][16];
        if constexpr (W13) {
          load_act_bf16<LR, KU, WK, 1>(a, s0, s1, x);
        } else {
          int e1[1];
          load_act_f16<LR, KU, WK, 1>(a, s0, s1, x, e1, s_max);
          ex[0] = e1[0];
        }
        gemv_pass<LR, KU, WK, RI, 1, W13>(a, nf3, loc, tile, x, lut_lane, res);
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < a.tile_rows * nt; idx += kGemvThreads) {
        const int t = idx / a.tile_rows;
        const int i = idx - t * a.tile_rows;
        const int slot = t == 0 ? s0 : s1;
        if (W13) {
          float gate = 0.0f, up = 0.0f;
#pragma unroll
          for (int kp = 0; kp < WK; ++kp) {
            gate += res[kp][i][t];
            up += res[kp][a.tile_rows + i][t];
          }
          gate *= g;
          up *= g;
          a.h_out[(size_t)slot * a.I + tile * a.tile_rows + i] = silu(gate) * up;
        } else {
          float o = 0.0f;
#pragma unroll
          for (int kp = 0; kp < WK; ++kp) o += res[kp][i][t];
          a.o_out[(size_t)slot * a.rows + tile * a.tile_rows + i] = __builtin_ldexpf(o * g, ex[t]);
        }
      }
      __syncthreads();
    }
  }
}

// y[t, n] = sum_j w[t, j] * o[t*k + j, n], in fixed j order, rounded to bf16.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ o,
                                                             const float* __restrict__ w, int M,
                                                             int k, int H,
                                                             uint16_t* __restrict__ y) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * H) return;
  const int t = idx / H;
  const int n = idx - t * H;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc = __builtin_fmaf(w[t * k + j], o[(size_t)(t * k + j) * H + n], acc);
  y[idx] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

typedef void (*GemvFn)(GemvArgs);

template <bool W13>
static GemvFn pick_gemv(const GemvTiling& t, int wk) {
#define HMOE_GEMV_CASE(LR_, KU_, WK_)                                         \
  if (t.lr == LR_ && t.ku == KU_ && wk == WK_)                               \
    return gemv_kernel<LR_, KU_, WK_, (KU_ == 1 ? 4 : 2), W13>;
#define HMOE_GEMV_LR(LR_, WK_) \
  HMOE_GEMV_CASE(LR_, 1, WK_) HMOE_GEMV_CASE(LR_, 2, WK_) HMOE_GEMV_CASE(LR_, 3, WK_)
  HMOE_GEMV_LR(64, 1) HMOE_GEMV_LR(32, 1) HMOE_GEMV_LR(16, 1) HMOE_GEMV_LR(8, 1) HMOE_GEMV_LR(4, 1)
  HMOE_GEMV_LR(64, 4) HMOE_GEMV_LR(32, 4) HMOE_GEMV_LR(16, 4) HMOE_GEMV_LR(8, 4) HMOE_GEMV_LR(4, 4)
#undef HMOE_GEMV_LR
#undef HMOE_GEMV_CASE
  return nullptr;
}

// WK for a GEMV over K: split K across the 4 waves when each part still gives a
// wave at least 16 units of 32 elements and holds whole NF3 groups of 64.
static int gemv_wk(int K) {
  const int U = K / 32;
  return (U % 8 == 0 && U / 4 >= 16) ? 4 : 1;
}

hipError_t launch_decode(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                         uint16_t* y, void* scratch, hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  GemvArgs a{};
  a.kept_fmt = L.kept_format;
  a.counts = reinterpret_cast<const int32_t*>(base + P.d_counts);
  a.experts = reinterpret_cast<const int32_t*>(base + P.d_experts);
  a.nslots = reinterpret_cast<const int32_t*>(base + P.d_nslots);
  a.slots = reinterpret_cast<const int32_t*>(base + P.d_slots);
  a.expert_tier = reinterpret_cast<const int32_t*>(base + P.expert_tier);
  a.I = L.I;
  float* h = reinterpret_cast<float*>(base + P.h_dec);
  float* o = reinterpret_cast<float*>(base + P.o_dec);
  const int bound = (M * L.k < L.E) ? M * L.k : L.E;  // distinct experts at most

  // W13 + SwiGLU
  {
    GemvArgs b = a;
    b.kq = W.kept_w13_q; b.ks = W.kept_w13_s; b.kg = W.kept_w13_g;
    b.nq = W.nf3_w13_q; b.ns = W.nf3_w13_s;
    b.rows = 2 * L.I; b.K = L.H;
    b.act_bf16 = x; b.act_row_div = L.k;
    b.tile_rows = L.w13.rows_per_task;
    b.tiles = L.I / b.tile_rows;
    b.h_out = h;
    GemvFn fn = pick_gemv<true>(L.w13, gemv_wk(L.H));
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(b.tiles * bound), dim3(kGemvThreads), 0, s, b);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // W2
  {
    GemvArgs b = a;
    b.kq = W.kept_w2_q; b.ks = W.kept_w2_s; b.kg = W.kept_w2_g;
    b.nq = W.nf3_w2_q; b.ns = W.nf3_w2_s;
    b.rows = L.H; b.K = L.I;
    b.act_f32 = h; b.act_row_div = 1;
    b.tile_rows = L.w2.rows_per_task;
    b.tiles = L.H / b.tile_rows;
    b.o_out = o;
    GemvFn fn = pick_gemv<false>(L.w2, gemv_wk(L.I));
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(b.tiles * bound), dim3(kGemvThreads), 0, s, b);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int n = M * L.H;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, o,
                     reinterpret_cast<const float*>(base + P.topk_w), M, L.k, L.H, y);
  return hipGetLastError();
}

// Decode tiling of a GEMV over K with `out_rows` output rows per expert: lanes per
// row and units per lane, and the rows per task (a multiple of what one block
// iteration covers, dividing `out_rows`, at least `min_rows`).
bool plan_gemv(int K, int out_rows, bool w13, int min_rows, GemvTiling* t) {
  const int wk = gemv_wk(K);
  const int U = K / 32 / wk;
  int lr = 1;
  while (lr < 64 && U % (2 * lr) == 0) lr *= 2;
  const int ku = U / lr;
  if (lr < 4 || ku < 1 || ku > 3) return false;
  const int P = 64 / lr;
  const int ri = ku == 1 ? 4 : 2;
  const int per_iter = (4 / wk) * P * ri;  // task rows covered per block iteration
  // W13 tasks hold tile_rows gate rows plus tile_rows up rows
  const int step = w13 ? (per_iter % 2 == 0 ? per_iter / 2 : per_iter) : per_iter;
  int rows = step;
  while (rows < min_rows || out_rows % rows != 0) {
    rows += step;
    if (rows > out_rows || (w13 ? 2 * rows : rows) > kMaxTaskRows) return false;
  }
  if ((w13 ? 2 * rows : rows) > kMaxTaskRows) return false;
  t->lr = lr;
  t->ku = ku;
  t->rows_per_task = rows;
  return true;
}

}  // namespace hmoe
