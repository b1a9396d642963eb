// Decode path (M <= 8): after routing and grouping, a GEMV over the packed W13 of
// every touched expert with a fused SwiGLU, a GEMV over their packed W2, and the
// deterministic top-k weighted combine into y. Both tiers run in the same launches
// from one routing result (local-inference-lab/vllm PR #92, "How it works":
// launches sharing one route geometry and one top-k sum; M <= 8 addressed directly
// by the top-k result).
//
// Work split: every (token, top-k) slot is one pass over its expert's rows (W13:
// pairs of a gate row i and its up row I + i; W2: rows n). The routing kernel lists
// the passes in slot order (token-major); two tokens that share an expert stream its
// rows in separate passes, the later one mostly from cache. Passes are cut into chunks of
// P * RI rows (or pairs); the M * k * chunks-per-pass units form one flat range and
// every wave of a persistent grid takes an equal contiguous run of it, so the work
// is balanced whatever the expert multiplicities are, and a wave's first load (its
// pass record) depends on nothing but its position. Inside a wave, LR lanes share a
// row and each lane owns KU units of 32 K-elements (unit u = c + LR*j), so one load
// instruction reads LR consecutive 16-byte (FP4) or 12-byte (NF3) units of each of
// P = 64/LR rows. The lane's activations sit in registers as 16-bit pairs and meet
// the decoded weights in v_dot2_f32_*; per-row sums are finished by a transposing
// reduction across the LR lanes. The next chunk's weights are in flight while the
// current one is computed.
//
// Precision: W13 runs on bf16 pairs (x is bf16; E2M1 is exact in bf16; the NVFP4
// E4M3 block scale multiplies each 16-block's fp32 partial; MXFP4's power-of-two
// scale is folded into the conversion; NF3 levels come from a scaled table, see
// kNF3TableScaleBf16, with the fp16 group scale on the fp32 partial). h leaves W13
// in fp32. W2 runs on fp16 pairs: each pass stages its slot's h row in LDS scaled by
// a power of two that puts the row's largest magnitude in [2^14, 2^15); E2M1 is
// exact in fp16 and every block or group scale multiplies an fp32 partial.
#include <type_traits>

#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

struct GemvArgs {
  const uint8_t* kq;   // kept codes [E4, rows, K/2]
  const uint8_t* ks;   // kept scales [E4, rows, K/16] (E4M3) or [E4, rows, K/32] (E8M0)
  const float* kg;     // kept per-tensor scale [E4] (NVFP4)
  const uint8_t* nq;   // NF3 codes [E3, rows, 3K/8]
  const uint16_t* ns;  // NF3 scales [E3, rows, K/64]
  int kept_fmt;
  int rows, K;       // rows of the weight tensor per expert, reduction length
  int out_units;     // W13: I (row pairs per expert); W2: H (rows per expert)
  const uint16_t* act_bf16;  // W13: x bf16 [M, K]
  const float* act_f32;      // W2: h fp32 [slots, K]
  const int4* pass;          // pass records [npass]: slot, tier code, token, expert
  int npass;                 // M * k
  int M, E, E4, E3;          // range checks of the records left in scratch
  int I;
  float* h_out;  // W13: fp32 [slots, I]
  float* o_out;  // W2: fp32 [slots, H]
};

// Transposing reduction of V values per lane over aligned LR-lane segments (V <= LR,
// both powers of two): each step keeps one half of the values and adds the partner
// lane's other half (partners from xlane), so V sums cost V - 1 + log2(LR / V)
// exchanges instead of V * log2(LR). The lane ends with the sum of value index
// seg_index<V, LR>(lane).
template <int V, int LR>
__device__ __forceinline__ float seg_reduce(const float (&v)[V]) {
  if constexpr (V == 1) {
    return group_sum<LR>(v[0]);
  } else {
    constexpr int H = V / 2;
    constexpr int off = LR / 2;
    float nv[H];
    if constexpr (off == 32 || off == 16) {
#pragma unroll
      for (int j = 0; j < H; ++j) nv[j] = swap_add<off>(v[j], v[j + H]);
    } else {
      const bool hi = (threadIdx.x & off) != 0;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float keep = hi ? v[j + H] : v[j];
        const float send = hi ? v[j] : v[j + H];
        nv[j] = keep + xlane<off>(send);
      }
    }
    return seg_reduce<H, LR / 2>(nv);
  }
}

template <int V, int LR>
__device__ __forceinline__ int seg_index(int lane) {
  int o = 0;
#pragma unroll
  for (int v = V, lr = LR; v > 1;) {
    lr >>= 1;
    v >>= 1;
    if (lane & lr) o += v;
  }
  return o;
}

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
  static __device__ __forceinline__ void nvfp4(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                               const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const float s0 = e4m3_to_f32<0>(sc[j]);
      const float s1 = e4m3_to_f32<1>(sc[j]);
      uint32_t w[16];
      fp4x16(q[j], 1.0f, w);
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
  static __device__ __forceinline__ void mxfp4(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                               const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      uint32_t w[16];
      if constexpr (F16) {
        fp4x16(q[j], 1.0f, w);
        const float s = e8m0_to_f32(sc[j]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float p = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) p = dot(w[i], x[t][j][i], p);
          acc[t] = __builtin_fmaf(s, p, acc[t]);
        }
      } else {
        fp4x16(q[j], e8m0_scale_operand(sc[j]), w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[t] = dot(w[i], x[t][j][i], acc[t]);
        }
      }
    }
  }
  // NF3: level pairs from the per-lane LDS table, fp16 group scale per 64
  static __device__ __forceinline__ void nf3(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                             const uint32_t* __restrict__ lut_lane,
                                             const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const uint32_t d0 = q[j].x, d1 = q[j].y, d2 = q[j].z;
      const float s = fp16_to_f32(sc[j]);
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

// One pass: the slot it serves, the x row (token) it reads and its expert's tier
// and tier-local index; ok is false for a record that is out of range (stale
// scratch), which the pass then skips.
struct PassInfo {
  bool ok;
  bool nf3;
  int loc;
  int slot;
  int token;
};

__device__ __forceinline__ PassInfo pass_info(const GemvArgs& a, int4 r) {
  PassInfo p;
  p.slot = r.x;
  p.nf3 = (r.y >> 16) != 0;
  p.loc = r.y & 0xFFFF;
  p.token = r.z;
  p.ok = (unsigned)r.x < (unsigned)a.npass && (unsigned)r.z < (unsigned)a.M &&
         (unsigned)r.w < (unsigned)a.E && p.loc < (p.nf3 ? a.E3 : a.E4);
  return p;
}

// Weight formats of one segment; the dispatch happens once per expert segment so
// every load and decode below is straight-line code.
enum : int { kFmtNvfp4 = 0, kFmtMxfp4 = 1, kFmtNf3 = 2 };

// Loads one row's KU units (codes + scale word) for this lane.
template <int LR, int KU, int FMT>
__device__ __forceinline__ void load_row(const GemvArgs& a, size_t grow, int c, uint4 (&q)[KU],
                                         uint32_t (&sc)[KU]) {
  if constexpr (FMT == kFmtNf3) {
    const uint8_t* qrow = a.nq + grow * (3 * a.K / 8);
    const uint16_t* srow = a.ns + grow * (a.K / 64);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      const uint3 v = *reinterpret_cast<const uint3*>(qrow + 12 * u);
      q[j] = make_uint4(v.x, v.y, v.z, 0u);
      sc[j] = srow[u >> 1];
    }
  } else if constexpr (FMT == kFmtNvfp4) {
    const uint8_t* qrow = a.kq + grow * (a.K / 2);
    const uint8_t* srow = a.ks + grow * (a.K / 16);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      q[j] = *reinterpret_cast<const uint4*>(qrow + 16 * u);
      sc[j] = *reinterpret_cast<const uint16_t*>(srow + 2 * u);
    }
  } else {
    const uint8_t* qrow = a.kq + grow * (a.K / 2);
    const uint8_t* srow = a.ks + grow * (a.K / 32);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = c + LR * j;
      q[j] = *reinterpret_cast<const uint4*>(qrow + 16 * u);
      sc[j] = srow[u];
    }
  }
}

template <int LR, int KU, int NT, bool F16, int FMT>
__device__ __forceinline__ void row_dot(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                        const uint32_t* lut_lane,
                                        const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  if constexpr (FMT == kFmtNf3) RowDot<LR, KU, NT, F16>::nf3(q, sc, lut_lane, x, acc);
  else if constexpr (FMT == kFmtNvfp4) RowDot<LR, KU, NT, F16>::nvfp4(q, sc, x, acc);
  else RowDot<LR, KU, NT, F16>::mxfp4(q, sc, x, acc);
}

// Calls f with the pass's weight format as a compile-time constant.
template <typename F>
__device__ __forceinline__ void with_format(const GemvArgs& a, const PassInfo& pi, F&& f) {
  if (pi.nf3) f(std::integral_constant<int, kFmtNf3>{});
  else if (a.kept_fmt == HMOE_KEPT_NVFP4) f(std::integral_constant<int, kFmtNvfp4>{});
  else f(std::integral_constant<int, kFmtMxfp4>{});
}

// Position of this wave's run in the flat range of npass * per units.
struct WaveRange {
  int begin, end;
};

// WAVE_MAJOR numbers the runs wave index first, so the waves of one block (one CU)
// take runs spread over the pass list and share each SIMD between both tiers' costs.
template <bool WAVE_MAJOR>
__device__ __forceinline__ WaveRange wave_range(int total) {
  const int nw = gridDim.x * kGemvWaves;
  // wave-uniform (scalar) from here on: the range, the pass, its tier and slot
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = WAVE_MAJOR ? wv * gridDim.x + blockIdx.x : blockIdx.x * kGemvWaves + wv;
  return {(int)((long)gw * total / nw), (int)((long)(gw + 1) * total / nw)};
}

// Builds the per-lane NF3 pair table [64 pair fields][64 lanes]: entry f holds the
// 16-bit pair (level(f & 7) * c, level(f >> 3) * c), bf16 or fp16. Thread t of the
// 256 writes fields (t >> 6) + 4m, m = 0..15, of lane t & 63: its low code takes two
// values and its high code is m >> 1, a constant once the loop is unrolled.
template <bool F16>
__device__ __forceinline__ void build_nf3_lut(uint32_t* lut, float c) {
  static_assert(kGemvThreads == 256, "four waves build the table");
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const float lo0 = nf3_level(w) * c, lo1 = nf3_level(w + 4) * c;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float hi = __uint_as_float(kNF3Bits[m >> 1]) * c;
    const float lo = (m & 1) ? lo1 : lo0;
    lut[(w + 4 * m) * kWave + lane] = F16 ? pack_f16(lo, hi) : pack_bf16(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU
// ---------------------------------------------------------------------------

// x units of one token (bf16 pairs) for this lane
template <int LR, int KU>
__device__ __forceinline__ void load_x(const GemvArgs& a, int token, int c,
                                       uint32_t (&x)[1][KU][16]) {
  const uint16_t* row = a.act_bf16 + (size_t)token * a.K;
#pragma unroll
  for (int j = 0; j < KU; ++j) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 32 * (c + LR * j));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 qv = p[v];
      x[0][j][4 * v + 0] = qv.x;
      x[0][j][4 * v + 1] = qv.y;
      x[0][j][4 * v + 2] = qv.z;
      x[0][j][4 * v + 3] = qv.w;
    }
  }
}

// Weights of one W13 chunk (P * RI row pairs) for this lane: gate and up rows.
template <int KU, int RI>
struct W13Buf {
  uint4 qg[RI][KU], qu[RI][KU];
  uint32_t sg[RI][KU], su[RI][KU];
};

// Buffer resources of one expert's codes and scales: a load then takes the chunk's row
// offset in a scalar register and the lane's fixed offset in a vector register, so no
// vector instruction computes addresses inside the loop.
struct ExpertRsrc {
  __amdgpu_buffer_rsrc_t q, s;
};

template <int FMT>
__device__ __forceinline__ ExpertRsrc expert_rsrc(const GemvArgs& a, int loc) {
  const int RB = FMT == kFmtNf3 ? 3 * a.K / 8 : a.K / 2;
  const int SB = FMT == kFmtNvfp4 ? a.K / 16 : a.K / 32;
  const uint8_t* q = (FMT == kFmtNf3 ? a.nq : a.kq) + (size_t)loc * a.rows * RB;
  const uint8_t* s = (FMT == kFmtNf3 ? reinterpret_cast<const uint8_t*>(a.ns) : a.ks) +
                     (size_t)loc * a.rows * SB;
  return {__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(q), 0, a.rows * RB, 0x00020000),
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(s), 0, a.rows * SB, 0x00020000)};
}

// one row's KU units (codes + scale word) for this lane: row = uniform row of the
// expert, rw = this lane's row within the load
template <int LR, int KU, int FMT>
__device__ __forceinline__ void load_row_rsrc(const ExpertRsrc& r, int K, int row, int rw, int c,
                                              uint4 (&q)[KU], uint32_t (&sc)[KU]) {
  const int RB = FMT == kFmtNf3 ? 3 * K / 8 : K / 2;
  const int SB = FMT == kFmtNvfp4 ? K / 16 : K / 32;
#pragma unroll
  for (int j = 0; j < KU; ++j) {
    const int u = c + LR * j;
    if constexpr (FMT == kFmtNf3) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(r.q, rw * RB + 12 * u, row * RB, 0);
      q[j] = make_uint4(v[0], v[1], v[2], 0u);
      sc[j] = __builtin_amdgcn_raw_buffer_load_b16(r.s, rw * SB + 2 * (u >> 1), row * SB, 0);
    } else if constexpr (FMT == kFmtNvfp4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r.q, rw * RB + 16 * u, row * RB, 0);
      q[j] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[j] = __builtin_amdgcn_raw_buffer_load_b16(r.s, rw * SB + 2 * u, row * SB, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r.q, rw * RB + 16 * u, row * RB, 0);
      q[j] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[j] = __builtin_amdgcn_raw_buffer_load_b8(r.s, rw * SB + u, row * SB, 0);
    }
  }
}

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_load(const GemvArgs& a, int loc, int i0, W13Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  const ExpertRsrc r = expert_rsrc<FMT>(a, loc);
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int i = i0 + ri * P;
    load_row_rsrc<LR, KU, FMT>(r, a.K, i, rw, c, b.qg[ri], b.sg[ri]);
    load_row_rsrc<LR, KU, FMT>(r, a.K, a.I + i, rw, c, b.qu[ri], b.su[ri]);
  }
}

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_compute(const GemvArgs& a, int i0, int slot, float g,
                                            const uint32_t (&x)[1][KU][16],
                                            const uint32_t* lut_lane, const W13Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  float vg[RI], vu[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    float ag[1], au[1];
    row_dot<LR, KU, 1, false, FMT>(b.qg[ri], b.sg[ri], lut_lane, x, ag);
    row_dot<LR, KU, 1, false, FMT>(b.qu[ri], b.su[ri], lut_lane, x, au);
    vg[ri] = ag[0];
    vu[ri] = au[0];
  }
  const float gate = seg_reduce<RI, LR>(vg) * g;
  const float up = seg_reduce<RI, LR>(vu) * g;
  const int ri = seg_index<RI, LR>(c);
  if ((c & (LR / RI - 1)) == 0)
    a.h_out[(size_t)slot * a.I + i0 + ri * P + rw] = silu(gate) * up;
}

// Chunks [c0, end) of one pass (chunk `first` is the expert's pair 0). A holds
// chunk c0 on entry when a_loaded.
template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_pass(const GemvArgs& a, const PassInfo& pi, int c0, int end,
                                         int first, float g, const uint32_t* lut_lane,
                                         W13Buf<KU, RI>& A, W13Buf<KU, RI>& B, bool a_loaded) {
  constexpr int CH = (kWave / LR) * RI;
  const int c = (threadIdx.x & (kWave - 1)) % LR;
  int cc = c0;
  if (!a_loaded) w13_load<LR, KU, RI, FMT>(a, pi.loc, (cc - first) * CH, A);
  uint32_t x[1][KU][16];
  load_x<LR, KU>(a, pi.token, c, x);
  // the next chunk's loads are issued unconditionally (the last chunk repeats itself)
  // so that the wait counts before each compute are the same on every path
  while (cc < end) {
    w13_load<LR, KU, RI, FMT>(a, pi.loc, (min(cc + 1, end - 1) - first) * CH, B);
    w13_compute<LR, KU, RI, FMT>(a, (cc - first) * CH, pi.slot, g, x, lut_lane, A);
    if (++cc >= end) break;
    w13_load<LR, KU, RI, FMT>(a, pi.loc, (min(cc + 1, end - 1) - first) * CH, A);
    w13_compute<LR, KU, RI, FMT>(a, (cc - first) * CH, pi.slot, g, x, lut_lane, B);
    ++cc;
  }
}

template <int LR, int KU, int RI>
__global__ __launch_bounds__(kGemvThreads) void w13_gemv_kernel(GemvArgs a) {
  __shared__ uint32_t lut[64 * kWave];  // [pair field][lane]: bf16 pair of scaled NF3 levels
  constexpr int CH = (kWave / LR) * RI;  // pairs per chunk
  const uint32_t* lut_lane = lut + (threadIdx.x & (kWave - 1));
  const int per = a.out_units / CH;      // chunks per pass
  const WaveRange wr = wave_range<false>(a.npass * per);
  // the first chunk's weights are requested before the table is built
  W13Buf<KU, RI> A, B;
  PassInfo pi{};
  int4 r_first{}, r_next{};
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    r_first = a.pass[p];
    if (p + 1 < a.npass) r_next = a.pass[p + 1];
  }
  build_nf3_lut<false>(lut, kNF3TableScaleBf16);
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    pi = pass_info(a, r_first);
    if (pi.ok)
      with_format(a, pi, [&](auto f) {
        w13_load<LR, KU, RI, decltype(f)::value>(a, pi.loc, (wr.begin - p * per) * CH, A);
      });
  }
  __syncthreads();
  bool first = true;
  for (int ch = wr.begin; ch < wr.end;) {
    const int p = ch / per;
    const int p_end = min(wr.end, (p + 1) * per);
    if (!first) {
      pi = pass_info(a, r_next);
      if (p + 1 < a.npass) r_next = a.pass[p + 1];
    }
    if (pi.ok) {
      const float g = pi.nf3 ? 1.0f / kNF3TableScaleBf16
                             : (a.kept_fmt == HMOE_KEPT_NVFP4 ? a.kg[pi.loc] : 1.0f);
      with_format(a, pi, [&](auto f) {
        w13_pass<LR, KU, RI, decltype(f)::value>(a, pi, ch, p_end, p * per, g, lut_lane, A, B,
                                                 first);
      });
    }
    first = false;
    ch = p_end;
  }
}

// ---------------------------------------------------------------------------
// W2
// ---------------------------------------------------------------------------

// Stages the slot's h row in this wave's LDS region as fp16 pairs scaled by 2^-e (e
// from the row's largest |h|, so the largest lands in [2^14, 2^15)), then reads this
// lane's KU units into x. Returns e.
template <int LR, int KU>
__device__ __forceinline__ int stage_h(const GemvArgs& a, int slot, uint32_t* hs, int c,
                                       uint32_t (&x)[1][KU][16]) {
  constexpr int NF4 = 8 * LR * KU;          // float4s per row (K = 32 * LR * KU)
  constexpr int PER = (NF4 + kWave - 1) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const float4* row = reinterpret_cast<const float4*>(a.act_f32 + (size_t)slot * a.K);
  float4 v[PER];
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = lane + kWave * i;
    v[i] = (NF4 % kWave == 0 || f < NF4) ? row[f] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
  mx = group_max<kWave>(mx);
  const int ef = (int)((__float_as_uint(mx) >> 23) & 0xFF);
  const int e = mx > 0.0f ? (ef == 0 ? -126 : ef - 127) - 14 : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = lane + kWave * i;
    if (NF4 % kWave == 0 || f < NF4) {
      uint2 w;
      w.x = pack_f16(__builtin_ldexpf(v[i].x, -e), __builtin_ldexpf(v[i].y, -e));
      w.y = pack_f16(__builtin_ldexpf(v[i].z, -e), __builtin_ldexpf(v[i].w, -e));
      *reinterpret_cast<uint2*>(hs + 2 * f) = w;
    }
  }
  // LDS operations of one wave complete in order: the reads below see the writes
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < KU; ++j) {
    const uint4* p = reinterpret_cast<const uint4*>(hs + 16 * (c + LR * j));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = p[q];
      x[0][j][4 * q + 0] = t.x;
      x[0][j][4 * q + 1] = t.y;
      x[0][j][4 * q + 2] = t.z;
      x[0][j][4 * q + 3] = t.w;
    }
  }
  __builtin_amdgcn_wave_barrier();
  return e;
}

template <int KU, int RI>
struct W2Buf {
  uint4 q[RI][KU];
  uint32_t sc[RI][KU];
};

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w2_load(const GemvArgs& a, int loc, int n0, W2Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  // flat loads here: buffer loads made the W2 GEMV slower on the GLM-class layer
#pragma unroll
  for (int ri = 0; ri < RI; ++ri)
    load_row<LR, KU, FMT>(a, (size_t)loc * a.rows + n0 + ri * P + rw, c, b.q[ri], b.sc[ri]);
}

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w2_compute(const GemvArgs& a, int n0, int slot, float g,
                                           const uint32_t (&x)[1][KU][16],
                                           const uint32_t* lut_lane, const W2Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  float v[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    float acc[1];
    row_dot<LR, KU, 1, true, FMT>(b.q[ri], b.sc[ri], lut_lane, x, acc);
    v[ri] = acc[0];
  }
  const float sum = seg_reduce<RI, LR>(v);
  const int ri = seg_index<RI, LR>(c);
  if ((c & (LR / RI - 1)) == 0) a.o_out[(size_t)slot * a.rows + n0 + ri * P + rw] = sum * g;
}

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w2_pass(const GemvArgs& a, const PassInfo& pi, int c0, int end,
                                        int first, float gt, const uint32_t* lut_lane,
                                        uint32_t* hs, W2Buf<KU, RI>& A, W2Buf<KU, RI>& B,
                                        bool a_loaded) {
  constexpr int CH = (kWave / LR) * RI;
  const int c = (threadIdx.x & (kWave - 1)) % LR;
  int cc = c0;
  if (!a_loaded) w2_load<LR, KU, RI, FMT>(a, pi.loc, (cc - first) * CH, A);
  uint32_t x[1][KU][16];
  const float g = __builtin_ldexpf(gt, stage_h<LR, KU>(a, pi.slot, hs, c, x));
  while (cc < end) {
    if (cc + 1 < end) w2_load<LR, KU, RI, FMT>(a, pi.loc, (cc + 1 - first) * CH, B);
    w2_compute<LR, KU, RI, FMT>(a, (cc - first) * CH, pi.slot, g, x, lut_lane, A);
    if (++cc >= end) break;
    if (cc + 1 < end) w2_load<LR, KU, RI, FMT>(a, pi.loc, (cc + 1 - first) * CH, A);
    w2_compute<LR, KU, RI, FMT>(a, (cc - first) * CH, pi.slot, g, x, lut_lane, B);
    ++cc;
  }
}

// dynamic LDS: one staged h row (K fp16) per wave
template <int LR, int KU, int RI>
__global__ __launch_bounds__(kGemvThreads) void w2_gemv_kernel(GemvArgs a) {
  __shared__ uint32_t lut[64 * kWave];  // [pair field][lane]: fp16 pair of scaled NF3 levels
  extern __shared__ uint32_t h_stage[];
  constexpr int CH = (kWave / LR) * RI;  // rows per chunk
  constexpr int KD = 16 * LR * KU;        // dwords per staged row (K / 2)
  const uint32_t* lut_lane = lut + (threadIdx.x & (kWave - 1));
  uint32_t* hs = h_stage + KD * (threadIdx.x >> 6);
  const int per = a.out_units / CH;
  const WaveRange wr = wave_range<true>(a.npass * per);
  W2Buf<KU, RI> A, B;
  PassInfo pi{};
  int4 r_first{}, r_next{};
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    r_first = a.pass[p];
    if (p + 1 < a.npass) r_next = a.pass[p + 1];
  }
  build_nf3_lut<true>(lut, kNF3TableScaleF16);
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    pi = pass_info(a, r_first);
    if (pi.ok)
      with_format(a, pi, [&](auto f) {
        w2_load<LR, KU, RI, decltype(f)::value>(a, pi.loc, (wr.begin - p * per) * CH, A);
      });
  }
  __syncthreads();
  bool first = true;
  for (int ch = wr.begin; ch < wr.end;) {
    const int p = ch / per;
    const int p_end = min(wr.end, (p + 1) * per);
    if (!first) {
      pi = pass_info(a, r_next);
      if (p + 1 < a.npass) r_next = a.pass[p + 1];
    }
    if (pi.ok) {
      const float gt = pi.nf3 ? 1.0f / kNF3TableScaleF16
                              : (a.kept_fmt == HMOE_KEPT_NVFP4 ? a.kg[pi.loc] : 1.0f);
      with_format(a, pi, [&](auto f) {
        w2_pass<LR, KU, RI, decltype(f)::value>(a, pi, ch, p_end, p * per, gt, lut_lane, hs, A,
                                                B, first);
      });
    }
    first = false;
    ch = p_end;
  }
}

// Decode grouping (M <= 8), kept for inspection (moe_decode_view): the distinct experts
// the M * k slots touch, in tier order (kept tier by local index, then NF3), each with
// its slots in ascending order, and the two counts.
struct GroupSmem {
  int32_t ids[kDecodeMaxM * kMaxTopK];
  uint32_t mask[kMaxExperts][4];  // slot bit masks (M * k <= 128 slots)
  int32_t order[kMaxExperts];     // (tier, local) position -> expert or -1
  int32_t pos[kMaxExperts];       // expert -> (tier, local) position
  int32_t d[kMaxExperts];         // expert -> group index
};

struct GroupArgs {
  const int32_t* ids;  // [M * k] top-k ids
  int M, E, k, E4;
  int32_t* counts;     // [2]: distinct experts, distinct kept-tier experts
  int32_t* experts;    // [max_distinct]
  int32_t* nslots;     // [max_distinct]
  int32_t* slots;      // [max_distinct, 8]
};

// built by one block of 256 threads
__device__ __forceinline__ void decode_grouping(const GroupArgs& a, const TierMask& tm,
                                                GroupSmem& sm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int nslot = a.M * a.k;
  for (int s = threadIdx.x; s < nslot; s += blockDim.x) sm.ids[s] = a.ids[s];
  // tier positions: one wave per 64-expert chunk, ranks by ballot
  for (int chunk = wave; chunk * kWave < a.E; chunk += nwaves) {
    const int e = chunk * kWave + lane;
    const bool in = e < a.E;
    const bool nf3 = in && ((tm.w[e >> 5] >> (e & 31)) & 1u);
    const uint64_t b = __ballot(nf3);
    int below = 0;
    for (int i = 0; i < 2 * chunk; ++i) below += __popc(tm.w[i]);
    below += __popcll(b & lt);
    if (in) {
      sm.pos[e] = nf3 ? a.E4 + below : e - below;
      sm.mask[e][0] = sm.mask[e][1] = sm.mask[e][2] = sm.mask[e][3] = 0u;
    }
  }
  __syncthreads();
  for (int s = threadIdx.x; s < nslot; s += blockDim.x) {
    const int e = sm.ids[s];
    if ((unsigned)e < (unsigned)a.E) atomicOr(&sm.mask[e][s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    const bool touched = (sm.mask[e][0] | sm.mask[e][1] | sm.mask[e][2] | sm.mask[e][3]) != 0u;
    sm.order[sm.pos[e]] = touched ? e : -1;
  }
  __syncthreads();
  if (wave == 0) {
    int running = 0, kept_distinct = 0;
    for (int base = 0; base < a.E; base += kWave) {
      const int p = base + lane;
      const int e = (p < a.E) ? sm.order[p] : -1;
      const bool f = e >= 0;
      const uint64_t b = __ballot(f);
      if (f) {
        const int d = running + __popcll(b & lt);
        const int n = __popc(sm.mask[e][0]) + __popc(sm.mask[e][1]) + __popc(sm.mask[e][2]) +
                      __popc(sm.mask[e][3]);
        sm.d[e] = d;
        a.experts[d] = e;
        a.nslots[d] = n < kDecodeMaxM ? n : kDecodeMaxM;
      }
      const int cnt = __popcll(b);
      if (base + kWave <= a.E4) kept_distinct += cnt;
      else if (base < a.E4) kept_distinct += __popcll(b & ((1ull << (a.E4 - base)) - 1ull));
      running += cnt;
    }
    if (lane == 0) {
      a.counts[0] = running;
      a.counts[1] = kept_distinct;
    }
  }
  __syncthreads();
  // each slot at its rank among its expert's slots
  for (int s = threadIdx.x; s < nslot; s += blockDim.x) {
    const int e = sm.ids[s];
    if ((unsigned)e >= (unsigned)a.E) continue;
    int rank = 0;
    for (int wd = 0; wd < (s >> 5); ++wd) rank += __popc(sm.mask[e][wd]);
    rank += __popc(sm.mask[e][s >> 5] & ((1u << (s & 31)) - 1u));
    if (rank < kDecodeMaxM) a.slots[sm.d[e] * kDecodeMaxM + rank] = s;
  }
}

// y[t, n] = sum_j w[t, j] * o[t*k + j, n], in fixed j order, rounded to bf16. The last
// block builds the decode grouping instead.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ o,
                                                             const float* __restrict__ w, int M,
                                                             int k, int H,
                                                             uint16_t* __restrict__ y,
                                                             GroupArgs ga, TierMask tm) {
  if (blockIdx.x == gridDim.x - 1) {
    __shared__ GroupSmem sm;
    decode_grouping(ga, tm, sm);
    return;
  }
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * H) return;
  const int t = idx / H;
  const int n = idx - t * H;
  float ov[kMaxTopK], wv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {   // all loads first, then the fixed-order sum
    ov[j] = j < k ? o[(size_t)(t * k + j) * H + n] : 0.0f;
    wv[j] = j < k ? w[t * k + j] : 0.0f;
  }
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) acc = __builtin_fmaf(wv[j], ov[j], acc);
  y[idx] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

typedef void (*GemvFn)(GemvArgs);

template <bool W13>
static GemvFn pick_gemv(const GemvTiling& t) {
#define HMOE_GEMV_CASE(LR_, KU_, RI_)                                            \
  if (t.lr == LR_ && t.ku == KU_ && t.ri == RI_) {                              \
    if constexpr (W13) return w13_gemv_kernel<LR_, KU_, RI_>;                   \
    else return w2_gemv_kernel<LR_, KU_, RI_>;                                  \
  }
  HMOE_GEMV_CASE(64, 1, 2) HMOE_GEMV_CASE(64, 2, 2) HMOE_GEMV_CASE(64, 3, 1) HMOE_GEMV_CASE(64, 4, 1)
  HMOE_GEMV_CASE(32, 1, 2) HMOE_GEMV_CASE(32, 2, 2) HMOE_GEMV_CASE(32, 3, 1) HMOE_GEMV_CASE(32, 4, 1)
  HMOE_GEMV_CASE(16, 1, 2) HMOE_GEMV_CASE(16, 2, 2) HMOE_GEMV_CASE(16, 3, 1) HMOE_GEMV_CASE(16, 4, 1)
  HMOE_GEMV_CASE(8, 1, 2) HMOE_GEMV_CASE(8, 2, 2) HMOE_GEMV_CASE(8, 3, 1) HMOE_GEMV_CASE(8, 4, 1)
  HMOE_GEMV_CASE(4, 1, 2) HMOE_GEMV_CASE(4, 2, 2) HMOE_GEMV_CASE(4, 3, 1) HMOE_GEMV_CASE(4, 4, 1)
#undef HMOE_GEMV_CASE
  return nullptr;
}

// Decode GEMV tiling over reduction length K: LR = the largest power of two up to 64
// dividing the K/32 units, KU = units per lane, RI = rows (or row pairs) per lane per
// chunk, at most half the lanes of an LR-lane segment (the transposing reduction
// hands each row's sum to LR / RI lanes).
bool plan_gemv(int K, GemvTiling* t) {
  const int U = K / 32;
  int lr = 1;
  while (lr < 64 && U % (2 * lr) == 0) lr *= 2;
  const int ku = U / lr;
  if (lr < 4 || ku < 1 || ku > 4) return false;
  int ri = ku <= 2 ? 2 : 1;  // two row (pair) groups at most: three waves per SIMD fit
  while (ri * 2 > lr) ri /= 2;
  if (ri < 1) return false;
  t->lr = lr;
  t->ku = ku;
  t->ri = ri;
  return true;
}

// blocks of one GEMV kernel resident per CU at the given dynamic LDS size (occupancy
// query, cached)
static int resident_blocks(GemvFn fn, size_t smem) {
  struct Entry {
    GemvFn fn;
    size_t smem;
    int n;
  };
  static Entry cache[32] = {};
  for (int i = 0; i < 32; ++i) {
    if (cache[i].fn == fn && cache[i].smem == smem) return cache[i].n;
    if (cache[i].fn == nullptr) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn),
                                                       kGemvThreads, smem) != hipSuccess || n < 1)
        n = 1;
      cache[i] = {fn, smem, n};
      return n;
    }
  }
  return 1;
}

static int cu_count() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
  }
  return cached;
}

hipError_t launch_decode(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                         uint16_t* y, void* scratch, int stage, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  GemvArgs a{};
  a.kept_fmt = L.kept_format;
  a.pass = reinterpret_cast<const int4*>(base + P.d_pass);
  a.npass = M * L.k;
  a.M = M;
  a.E = L.E;
  a.E4 = L.E4;
  a.E3 = L.E3;
  a.I = L.I;
  float* h = reinterpret_cast<float*>(base + P.h_dec);
  float* o = reinterpret_cast<float*>(base + P.o_dec);
  // a persistent grid: as many blocks as fit on the GPU at once, never more waves
  // than chunks
  auto grid_for = [&](GemvFn fn, const GemvTiling& t, int out_units, size_t smem) {
    const long chunks = (long)a.npass * (out_units / ((64 / t.lr) * t.ri));
    const long blocks = (chunks + kGemvWaves - 1) / kGemvWaves;
    const long cap = (long)resident_blocks(fn, smem) * cu_count();
    return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
  };
  if (stage == HMOE_STAGE_W13) {
    GemvArgs b = a;
    b.kq = W.kept_w13_q; b.ks = W.kept_w13_s; b.kg = W.kept_w13_g;
    b.nq = W.nf3_w13_q; b.ns = W.nf3_w13_s;
    b.rows = 2 * L.I; b.K = L.H; b.out_units = L.I;
    b.act_bf16 = x;
    b.h_out = h;
    GemvFn fn = pick_gemv<true>(L.w13);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid_for(fn, L.w13, L.I, 0)), dim3(kGemvThreads), 0, s, b);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_W2) {
    GemvArgs b = a;
    b.kq = W.kept_w2_q; b.ks = W.kept_w2_s; b.kg = W.kept_w2_g;
    b.nq = W.nf3_w2_q; b.ns = W.nf3_w2_s;
    b.rows = L.H; b.K = L.I; b.out_units = L.H;
    b.act_f32 = h;
    b.o_out = o;
    GemvFn fn = pick_gemv<false>(L.w2);
    if (!fn) return hipErrorInvalidValue;
    const size_t smem = (size_t)kGemvWaves * L.I * 2;  // one fp16 h row per wave
    hipLaunchKernelGGL(fn, dim3(grid_for(fn, L.w2, L.H, smem)), dim3(kGemvThreads), smem, s, b);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_COMBINE) {
    const int n = M * L.H;
    GroupArgs ga;
    ga.ids = reinterpret_cast<const int32_t*>(base + P.topk_ids);
    ga.M = M;
    ga.E = L.E;
    ga.k = L.k;
    ga.E4 = L.E4;
    ga.counts = reinterpret_cast<int32_t*>(base + P.d_counts);
    ga.experts = reinterpret_cast<int32_t*>(base + P.d_experts);
    ga.nslots = reinterpret_cast<int32_t*>(base + P.d_nslots);
    ga.slots = reinterpret_cast<int32_t*>(base + P.d_slots);
    // one more block than the sum needs: it builds the grouping
    hipLaunchKernelGGL(decode_combine_kernel, dim3((n + 255) / 256 + 1), dim3(256), 0, s, o,
                       reinterpret_cast<const float*>(base + P.topk_w), M, L.k, L.H, y, ga,
                       make_tier_mask(L));
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace hmoe
