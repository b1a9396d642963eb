// Decode path (M <= 8): after routing and grouping, a GEMV over the packed W13 of
// every touched expert with a fused SwiGLU, a GEMV over their packed W2, and the
// deterministic top-k weighted combine into y. Both tiers run in the same launches
// from one routing result (local-inference-lab/vllm PR #92, "How it works":
// launches sharing one route geometry and one top-k sum; M <= 8 addressed directly
// by the top-k result).
//
// Work split: every (token, top-k) slot is one pass over its expert's rows (W13:
// pairs of a gate row i and its up row I + i; W2: rows n). The routing kernel lists
// the passes grouped by expert, so a token pair sharing an expert streams the same
// rows back to back (the second time from cache). Passes are cut into chunks of
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
    const bool hi = (threadIdx.x & off) != 0;
    float nv[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float keep = hi ? v[j + H] : v[j];
      const float send = hi ? v[j] : v[j + H];
      nv[j] = keep + xlane<off>(send);
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

template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_load(const GemvArgs& a, int loc, int i0, W13Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  const size_t base = (size_t)loc * a.rows;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int i = i0 + ri * P + rw;
    load_row<LR, KU, FMT>(a, base + i, c, b.qg[ri], b.sg[ri]);
    load_row<LR, KU, FMT>(a, base + a.I + i, c, b.qu[ri], b.su[ri]);
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

// decode W13 kernel: 0 = register double-buffered GEMV, 1 = LDS-staged GEMV,
// 2 = matrix cores (falls back to 0 where its LDS plan does not fit)
#ifndef HMOE_W13_IMPL
#define HMOE_W13_IMPL 0
#endif
constexpr int kW13Impl = HMOE_W13_IMPL;
constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kLdsBytes = 160 * 1024;
// s_waitcnt vmcnt(0) with the other counters left alone (expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0F70;

// ---------------------------------------------------------------------------
// W13 + SwiGLU, LDS-staged
// ---------------------------------------------------------------------------
// One block serves a contiguous run of one pass's chunks; its waves take the run's
// chunks round-robin. Each wave streams its chunks' packed codes and scales into a
// ring of S stages of its own in LDS with direct global-to-LDS loads (no registers
// hold data in flight), S - 1 chunks ahead of the one it computes, and waits for a
// stage by the count of loads issued after it. Outputs collect in LDS and leave in
// one coalesced store per block at the end, so the only vector memory operations in
// flight during the loop are the staged loads themselves.
//
// LDS per block: the NF3 pair table (16 KB), the x row (bf16, arranged so that lane
// c's 16-byte pieces of unit j sit side by side), the block's h outputs, and WPB * S
// stages of codes (one 1 KB load per row segment) and scales (one flat run of dwords).

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// direct loads into LDS: lane l's bytes land at lds + 16 l (12- and 16-byte forms) or
// lds + 4 l (4-byte form); the LDS address goes through M0
__device__ __forceinline__ void lds_load_b128(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load_b96(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load_b32(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vm<R * D> for a run-time R in [0, S)
template <int D, int S>
__device__ __forceinline__ void wait_stages(int r) {
  static_assert(S >= 2 && S <= 4, "stages");
  if (S > 3 && r >= 3) wait_vm<(S > 3 ? 3 * D : 0)>();
  else if (S > 2 && r >= 2) wait_vm<(S > 2 ? 2 * D : 0)>();
  else if (r >= 1) wait_vm<D>();
  else wait_vm<0>();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// LDS layout of one streaming block (byte offsets; host and device agree)
struct StreamLayout {
  int lut, x, h, stages;  // region offsets
  int stage_bytes;        // one stage: codes, then scales
  int nstage;             // S
  int runs;               // runs (blocks) per pass
  int total;              // bytes
};

// Per-lane table of scaled NF3 level pairs for any block size (256 threads per step).
template <bool F16>
__device__ __forceinline__ void build_nf3_lut_any(uint32_t* lut, float c) {
  for (int t = threadIdx.x; t < 64 * kWave; t += blockDim.x) {
    const int f = t >> 6, lane = t & (kWave - 1);
    const float lo = nf3_level(f & 7) * c, hi = nf3_level(f >> 3) * c;
    lut[f * kWave + lane] = F16 ? pack_f16(lo, hi) : pack_bf16(lo, hi);
  }
}

template <int LR, int KU, int RI, int FMT>
struct W13Stream {
  static constexpr int P = kWave / LR;
  static constexpr int CH = P * RI;                        // row pairs per chunk
  static constexpr int K = 32 * LR * KU;                   // reduction length
  static constexpr int UB = FMT == kFmtNf3 ? 12 : 16;      // code bytes per 32-unit
  static constexpr int RB = UB * LR * KU;                  // code bytes per row
  static constexpr int SB = FMT == kFmtNvfp4 ? 2 * LR * KU : LR * KU;  // scale bytes per row
  static constexpr int NCODE = 2 * RI * KU;                // code loads per chunk
  static constexpr int SDW = 2 * RI * P * SB / 4;          // scale dwords per chunk
  static constexpr int NSC = (SDW + kWave - 1) / kWave;    // scale loads per chunk
  static constexpr int D = NCODE + NSC;                    // loads per chunk
  static constexpr int CODE_BYTES = NCODE * 1024;
  static_assert(SB % 4 == 0, "scale rows hold whole dwords");
};

// issue chunk ch's loads (row pairs ch * CH ...) into the stage at LDS address sb
template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_issue(const uint8_t* codes, const uint8_t* scales, int I,
                                          int ch, uint32_t sb) {
  using T = W13Stream<LR, KU, RI, FMT>;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR, rw = lane / LR;
  const int i0 = ch * T::CH;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu) {
      const uint8_t* row = codes + (size_t)(gu * I + i0 + ri * T::P + rw) * T::RB;
#pragma unroll
      for (int j = 0; j < KU; ++j) {
        const uint32_t dst = sb + ((ri * 2 + gu) * KU + j) * 1024;
        if constexpr (FMT == kFmtNf3) lds_load_b96(row + 12 * (c + LR * j), dst);
        else lds_load_b128(row + 16 * (c + LR * j), dst);
      }
    }
#pragma unroll
  for (int t = 0; t < T::NSC; ++t) {
    int f = t * kWave + lane;
    f = f < T::SDW ? f : T::SDW - 1;  // a spare lane repeats the last dword
    const int r = f / (T::SB / 4), dw = f % (T::SB / 4);
    const int srw = r % T::P, rg = r / T::P;
    const int row = (rg & 1) * I + i0 + (rg >> 1) * T::P + srw;
    lds_load_b32(scales + (size_t)row * T::SB + 4 * dw, sb + T::CODE_BYTES + t * 256);
  }
}

// compute chunk ch (local index lc in the block's run) from the stage at sbp
template <int LR, int KU, int RI, int FMT>
__device__ __forceinline__ void w13_stage_compute(const uint8_t* sbp, const uint32_t (&x)[1][KU][16],
                                                  const uint32_t* lut_lane, float g, int lc,
                                                  float* hbuf) {
  using T = W13Stream<LR, KU, RI, FMT>;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR, rw = lane / LR;
  W13Buf<KU, RI> b;
  const uint8_t* scp = sbp + T::CODE_BYTES;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri)
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      b.qg[ri][j] = *reinterpret_cast<const uint4*>(sbp + ((ri * 2) * KU + j) * 1024 + 16 * lane);
      b.qu[ri][j] = *reinterpret_cast<const uint4*>(sbp + ((ri * 2 + 1) * KU + j) * 1024 + 16 * lane);
      const int u = c + LR * j;
      const int off = FMT == kFmtNvfp4 ? 2 * u : (FMT == kFmtMxfp4 ? u : 2 * (u >> 1));
      const uint8_t* sg = scp + ((ri * 2) * T::P + rw) * T::SB + off;
      const uint8_t* su = scp + ((ri * 2 + 1) * T::P + rw) * T::SB + off;
      if constexpr (FMT == kFmtMxfp4) {
        b.sg[ri][j] = *sg;
        b.su[ri][j] = *su;
      } else {
        b.sg[ri][j] = *reinterpret_cast<const uint16_t*>(sg);
        b.su[ri][j] = *reinterpret_cast<const uint16_t*>(su);
      }
    }
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
  if ((c & (LR / RI - 1)) == 0) hbuf[lc * T::CH + ri * T::P + rw] = silu(gate) * up;
}

template <int LR, int KU, int RI, int WPB, int S, int FMT>
__device__ __forceinline__ void w13_stream_run(const GemvArgs& a, const StreamLayout& sl,
                                               uint8_t* smem, uint32_t* lut_s, const PassInfo& pi,
                                               int cb, int ce, float g) {
  using T = W13Stream<LR, KU, RI, FMT>;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const size_t erows = (size_t)pi.loc * a.rows;
  const uint8_t* codes = (FMT == kFmtNf3 ? a.nq : a.kq) + erows * T::RB;
  const uint8_t* scales =
      (FMT == kFmtNf3 ? reinterpret_cast<const uint8_t*>(a.ns) : a.ks) + erows * T::SB;
  const int cnt = ce - cb;
  const int n = cnt > wave ? (cnt - wave + WPB - 1) / WPB : 0;  // this wave's chunks
  const uint32_t base = lds_addr(smem);
  const uint32_t ring = base + sl.stages + wave * S * sl.stage_bytes;
  uint32_t* lut = lut_s;
  float* hbuf = reinterpret_cast<float*>(smem + sl.h);
  // x row of the pass's token: piece f = (j * 4 + v) * LR + c holds x units' 16-byte
  // piece v of unit c + LR * j; the block's waves share the loads
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(a.act_bf16 + (size_t)pi.token * a.K);
  constexpr int XPIECES = T::K / 8;
  constexpr int XLOADS = (XPIECES + kWave - 1) / kWave;
  for (int t = wave; t < XLOADS; t += WPB) {
    int f = t * kWave + lane;
    f = f < XPIECES ? f : XPIECES - 1;
    const int xc = f % LR, jv = f / LR;
    lds_load_b128(xrow + ((xc + LR * (jv >> 2)) * 4 + (jv & 3)) * 16, base + sl.x + t * 1024);
  }
  // the first S - 1 chunks
#pragma unroll
  for (int m = 0; m < S - 1; ++m)
    if (m < n)
      w13_issue<LR, KU, RI, FMT>(codes, scales, a.I, cb + wave + WPB * m,
                                 ring + m * sl.stage_bytes);
  build_nf3_lut_any<false>(lut, kNF3TableScaleBf16);
  // every load of the prologue has landed (the builtin form lets the compiler know
  // that its own earlier loads are complete too)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  uint32_t x[1][KU][16];
#pragma unroll
  for (int j = 0; j < KU; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 q = *reinterpret_cast<const uint4*>(smem + sl.x + (((j * 4 + v) * LR + c) * 16));
      x[0][j][4 * v + 0] = q.x;
      x[0][j][4 * v + 1] = q.y;
      x[0][j][4 * v + 2] = q.z;
      x[0][j][4 * v + 3] = q.w;
    }
  const uint32_t* lut_lane = lut + lane;
  for (int m = 0; m < n; ++m) {
    if (m + S - 1 < n)
      w13_issue<LR, KU, RI, FMT>(codes, scales, a.I, cb + wave + WPB * (m + S - 1),
                                 ring + ((m + S - 1) % S) * sl.stage_bytes);
    const int rem = min(n - 1 - m, S - 1);  // chunks issued after chunk m
    wait_stages<T::D, S>(rem);
    w13_stage_compute<LR, KU, RI, FMT>(smem + sl.stages + (wave * S + m % S) * sl.stage_bytes,
                                       x, lut_lane, g, wave + WPB * m, hbuf);
  }
  __syncthreads();
  // the run's outputs: h[slot, cb * CH ...], coalesced
  float* hout = a.h_out + (size_t)pi.slot * a.I + (size_t)cb * T::CH;
  for (int i = threadIdx.x; i < cnt * T::CH; i += WPB * kWave) hout[i] = hbuf[i];
}

template <int LR, int KU, int RI, int S>
__global__ __launch_bounds__(kStreamThreads) void w13_stream_kernel(GemvArgs a, StreamLayout sl) {
  // the pair table at a fixed LDS address (16 KB aligned) lets one and-or form its
  // per-lane addresses
  __shared__ __attribute__((aligned(16384))) uint32_t lut_s[64 * kWave];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int CH = (kWave / LR) * RI;
  const int p = blockIdx.x / sl.runs, r = blockIdx.x % sl.runs;
  const int per = a.out_units / CH;
  const int cb = (int)((long)r * per / sl.runs), ce = (int)((long)(r + 1) * per / sl.runs);
  if (p >= a.npass || cb >= ce) return;
  const PassInfo pi = pass_info(a, a.pass[p]);
  if (!pi.ok) return;  // the same for every wave of the block
  const float g = pi.nf3 ? 1.0f / kNF3TableScaleBf16
                         : (a.kept_fmt == HMOE_KEPT_NVFP4 ? a.kg[pi.loc] : 1.0f);
  with_format(a, pi, [&](auto f) {
    w13_stream_run<LR, KU, RI, kStreamWaves, S, decltype(f)::value>(a, sl, smem, lut_s, pi, cb, ce, g);
  });
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU on matrix cores (decode)
// ---------------------------------------------------------------------------
// The touched experts are served once each, for all of their tokens: a block finds
// the distinct experts of the M * k slots (ordered by first slot), takes one expert
// and a run of its 16-row-pair tiles, and computes, for every token routed to it, the
// gate and up rows of each tile with v_mfma_f32_32x32x16_bf16: the A operand holds the
// tokens' x (row m = token, rows past the expert's token count read zeros), the B
// operand 16 gate and the 16 matching up rows decoded to bf16. Each MFMA step covers
// 16 K-elements that share one scale: NVFP4 the two 8-element halves of one 16-block
// (the lane pair of a row reads the same 16-byte unit), MXFP4 half a 32-block, NF3 8
// elements of each of the two 32-element units of one 64-group (lane half g owns unit
// 2G + g and feeds 8 of its elements per step, so its pair fields sit at fixed bit
// positions). Block scales multiply the token rows of the fp32 step result.
//
// Codes and scales stream into a per-wave ring of LDS stages (32 rows x 256 K) by
// direct global-to-LDS loads, S - 1 stages ahead; the tokens' x rows (bf16, padded
// rows) are loaded into LDS once per block; outputs collect in LDS and leave at the
// end. The only vector memory operations in flight inside the loop are the staged
// loads.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMfWaves = 8;
constexpr int kMfThreads = kMfWaves * kWave;
constexpr int kMfStageCode = 32 * 128;      // 32 rows x 256 K of codes (16-byte unit slots)
constexpr int kMfTok = kDecodeMaxM;         // token rows of the x tile

struct MfLayout {
  int fs;         // first-slot table [E] int32
  int x;          // x tile [kMfTok][K + 8] bf16
  int xstride;    // bytes per x row
  int stages;     // WPB * S stages
  int stage_bytes;
  int nstage;     // S
  int nblocks;    // grid size
  int total;      // dynamic bytes
};

struct MfArgs {
  GemvArgs a;
  const int32_t* ids;  // top-k ids [M * k]
  int k;
  MfLayout lay;
  TierMask tm;
};

template <int FMT>
struct MfFmt {
  static constexpr int UB = FMT == kFmtNf3 ? 12 : 16;            // code bytes per 32-unit
  static constexpr int SBSEG = FMT == kFmtNvfp4 ? 16 : 8;        // scale bytes per row per 256 K
  static constexpr int NSC = 32 * SBSEG / 256;                   // scale loads per stage
  static constexpr int D = 4 + NSC;                              // loads per stage
};

// Unit slots of a stage row are permuted by the row (slot = unit ^ mf_swz(row)) so that
// the 32 rows of one MFMA operand read from different LDS banks.
__device__ __forceinline__ int mf_swz(int rr) { return (rr >> 1) & 7; }

// issue the loads of stage (tile t, K segment ks) into LDS address sb
template <int FMT>
__device__ __forceinline__ void mf_issue(const uint8_t* codes, const uint8_t* scales, int I, int K,
                                         int t, int ks, uint32_t sb) {
  using F = MfFmt<FMT>;
  const int lane = threadIdx.x & (kWave - 1);
  const int RB = F::UB * (K / 32);
  const int SB = FMT == kFmtNvfp4 ? K / 16 : K / 32;  // scale bytes per row
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // LDS slot lane & 7 of stage row rr holds unit (lane & 7) ^ mf_swz(rr)
    const int rr = 8 * j + (lane >> 3), c = (lane & 7) ^ mf_swz(rr);
    const int row = (rr < 16 ? 0 : I - 16) + 16 * t + rr;
    const uint8_t* src = codes + (size_t)row * RB + (size_t)(8 * ks + c) * F::UB;
    if constexpr (FMT == kFmtNf3) lds_load_b96(src, sb + j * 1024);
    else lds_load_b128(src, sb + j * 1024);
  }
#pragma unroll
  for (int u = 0; u < F::NSC; ++u) {
    const int f = u * kWave + lane;                     // flat dword of the stage's scales
    const int rr = f / (F::SBSEG / 4), dw = f % (F::SBSEG / 4);
    const int row = (rr < 16 ? 0 : I - 16) + 16 * t + rr;
    lds_load_b32(scales + (size_t)row * SB + (size_t)ks * F::SBSEG + 4 * dw,
                 sb + kMfStageCode + u * 256);
  }
}

// eight bf16 of E2M1 codes (one dword, element 2j in the low nibble of byte j)
__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t v) {
  uint32_t w[4];
  w[0] = e2m1x2_bf16<0>(v, 1.0f);
  w[1] = e2m1x2_bf16<1>(v, 1.0f);
  w[2] = e2m1x2_bf16<2>(v, 1.0f);
  w[3] = e2m1x2_bf16<3>(v, 1.0f);
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint8_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// one stage: acc[r] (token row 4 g + r of this lane's row) += scale * partial
template <int FMT, int NTF>
__device__ __forceinline__ void mf_compute(const uint8_t* stg, const uint8_t* xa, int kbase,
                                           const uint32_t* lut_lane, float (&acc)[4]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 31, g = lane >> 5;
  const uint8_t* crow = stg + n * 128;
  const int swz = mf_swz(n);
  const f32x16_t zero = {};
  if constexpr (FMT == kFmtNf3) {
    const uint8_t* srow = stg + kMfStageCode + n * 8;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const uint4 q = *reinterpret_cast<const uint4*>(crow + ((2 * G + g) ^ swz) * 16);
      const float s = fp16_to_f32(*reinterpret_cast<const uint16_t*>(srow + 2 * G));
      f32x16_t c = zero;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t w[4];
#define HMOE_F(P) lut_lane[nf3_pair_field<P>(q.x, q.y, q.z) << 6]
        if (st == 0) { w[0] = HMOE_F(0); w[1] = HMOE_F(1); w[2] = HMOE_F(2); w[3] = HMOE_F(3); }
        if (st == 1) { w[0] = HMOE_F(4); w[1] = HMOE_F(5); w[2] = HMOE_F(6); w[3] = HMOE_F(7); }
        if (st == 2) { w[0] = HMOE_F(8); w[1] = HMOE_F(9); w[2] = HMOE_F(10); w[3] = HMOE_F(11); }
        if (st == 3) { w[0] = HMOE_F(12); w[1] = HMOE_F(13); w[2] = HMOE_F(14); w[3] = HMOE_F(15); }
#undef HMOE_F
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, w);
        const bf16x8_t xv = lds_bf16x8(xa + 2 * (kbase + 64 * G + 32 * g + 8 * st));
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, b, c, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < NTF; ++r) acc[r] = __builtin_fmaf(s, c[r], acc[r]);
    }
  } else {
    const uint8_t* srow = stg + kMfStageCode + n * MfFmt<FMT>::SBSEG;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // dwords g and 2 + g of the unit: elements [8 g, 8 g + 8) of both 16-blocks
      const uint8_t* cu = crow + (u ^ swz) * 16 + 4 * g;
      const uint32_t d0 = *reinterpret_cast<const uint32_t*>(cu);
      const uint32_t d1 = *reinterpret_cast<const uint32_t*>(cu + 8);
      const bf16x8_t x0 = lds_bf16x8(xa + 2 * (kbase + 32 * u + 8 * g));
      const bf16x8_t x1 = lds_bf16x8(xa + 2 * (kbase + 32 * u + 16 + 8 * g));
      if constexpr (FMT == kFmtNvfp4) {
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(srow + 2 * u);
        const float s0 = e4m3_to_f32<0>(sc), s1 = e4m3_to_f32<1>(sc);
        const f32x16_t c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, fp4x8_bf16(d0), zero, 0, 0, 0);
        const f32x16_t c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, fp4x8_bf16(d1), zero, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < NTF; ++r) acc[r] = __builtin_fmaf(s1, c1[r], __builtin_fmaf(s0, c0[r], acc[r]));
      } else {
        const float s = e8m0_to_f32(srow[u]);
        f32x16_t c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, fp4x8_bf16(d0), zero, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, fp4x8_bf16(d1), c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < NTF; ++r) acc[r] = __builtin_fmaf(s, c[r], acc[r]);
      }
    }
  }
}


// j-th slot (ascending) among the slots whose bit is set in (lo, hi): every lane gets it
__device__ __forceinline__ int nth_slot(uint64_t lo, uint64_t hi, int j) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lt = (1ull << lane) - 1ull;
  const int nlo = __popcll(lo);
  const bool in_lo = ((lo >> lane) & 1ull) && __popcll(lo & lt) == j;
  const bool in_hi = ((hi >> lane) & 1ull) && nlo + __popcll(hi & lt) == j;
  const uint64_t blo = __ballot(in_lo), bhi = __ballot(in_hi);
  return blo ? __builtin_ctzll(blo) : (bhi ? 64 + __builtin_ctzll(bhi) : -1);
}

template <int S, int FMT, int NTF>
__device__ __forceinline__ void mf_run(const MfArgs& A, uint8_t* smem, const uint32_t* lut, int loc,
                                       int nt, uint64_t mlo, uint64_t mhi, int tb, int te,
                                       float g) {
  using F = MfFmt<FMT>;
  const GemvArgs& a = A.a;
  const MfLayout& L = A.lay;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int K = a.K, KS = K / 256;
  const size_t erows = (size_t)loc * a.rows;
  const uint8_t* codes = (FMT == kFmtNf3 ? a.nq : a.kq) + erows * (size_t)(F::UB * (K / 32));
  const uint8_t* scales = (FMT == kFmtNf3 ? reinterpret_cast<const uint8_t*>(a.ns) : a.ks) +
                          erows * (size_t)(FMT == kFmtNvfp4 ? K / 16 : K / 32);
  const int cnt = te - tb;
  const int ntile = cnt > wave ? (cnt - wave + kMfWaves - 1) / kMfWaves : 0;
  const int nst = ntile * KS;  // this wave's stages
  const uint32_t ring = lds_addr(smem) + L.stages + wave * S * L.stage_bytes;
#pragma unroll
  for (int m = 0; m < S - 1; ++m)
    if (m < nst)
      mf_issue<FMT>(codes, scales, a.I, K, tb + wave + kMfWaves * (m / KS), m % KS,
                    ring + m * L.stage_bytes);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();  // x tile and pair table are in place
  const int n = lane & 31, gl = lane >> 5;
  // A-operand token row of this lane; rows past the expert's tokens only feed output
  // rows that are never read, so they repeat row 0 (the same LDS words: a broadcast)
  const uint8_t* xa = smem + L.x + (n < nt ? n : 0) * L.xstride;
  const uint32_t* lut_lane = lut + lane;
  // output rows of this lane: token rows 4 gl + r
  int oslot[NTF];
#pragma unroll
  for (int r = 0; r < NTF; ++r) {
    const int lo = nth_slot(mlo, mhi, r), hi = nth_slot(mlo, mhi, 4 + r);  // wave-uniform ranks
    oslot[r] = gl ? hi : lo;
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int st = 0; st < nst; ++st) {
    if (st + S - 1 < nst) {
      const int sn = st + S - 1;
      mf_issue<FMT>(codes, scales, a.I, K, tb + wave + kMfWaves * (sn / KS), sn % KS,
                    ring + (sn % S) * L.stage_bytes);
    }
    wait_stages<F::D, S>(min(nst - 1 - st, S - 1));
    const int ks = st % KS;
    const uint8_t* stg = smem + L.stages + (wave * S + st % S) * L.stage_bytes;
    mf_compute<FMT, NTF>(stg, xa, 256 * ks, lut_lane, acc);
    if (ks == KS - 1) {
      // gate (lanes n < 16) and up (n >= 16) of row pair 16 t + (n & 15)
      const int t = tb + wave + kMfWaves * (st / KS);
#pragma unroll
      for (int r = 0; r < NTF; ++r) {
        const float up = xlane<16>(acc[r]);
        if (n < 16 && 4 * gl + r < nt)
          a.h_out[(size_t)oslot[r] * a.I + 16 * t + n] = silu(acc[r] * g) * (up * g);
        acc[r] = 0.0f;
      }
    }
  }
}

template <int S>
__global__ __launch_bounds__(kMfThreads) void w13_mfma_kernel(MfArgs A) {
  // the pair table at a fixed, 16 KB aligned LDS address (one and-or per address)
  __shared__ __attribute__((aligned(16384))) uint32_t lut_s[64 * kWave];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const GemvArgs& a = A.a;
  const MfLayout& L = A.lay;
  const int nslot = a.M * A.k;  // <= 128
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int* fs = reinterpret_cast<int*>(smem + L.fs);
  for (int e = threadIdx.x; e < a.E; e += kMfThreads) fs[e] = 0x7FFFFFFF;
  __syncthreads();
  for (int s = threadIdx.x; s < nslot; s += kMfThreads) {
    const int e = A.ids[s];
    if ((unsigned)e < (unsigned)a.E) atomicMin(&fs[e], s);
  }
  __syncthreads();
  // every wave: the distinct experts in order of their first slot; this block's
  // expert is number gi, and the block is run r of that expert's runs
  int e0 = -1, e1 = -1;
  if (lane < nslot) e0 = A.ids[lane];
  if (lane + kWave < nslot) e1 = A.ids[lane + kWave];
  const bool f0 = (unsigned)e0 < (unsigned)a.E && fs[e0] == lane;
  const bool f1 = (unsigned)e1 < (unsigned)a.E && fs[e1] == lane + kWave;
  const uint64_t b0 = __ballot(f0), b1 = __ballot(f1);
  const int G = __popcll(b0) + __popcll(b1);
  if (G == 0) return;  // the same in every wave
  const int NB = gridDim.x;
  const int gi = (int)((long)blockIdx.x * G / NB);
  const int blo = (int)(((long)gi * NB + G - 1) / G);
  const int bhi = (int)(((long)(gi + 1) * NB + G - 1) / G);
  const int runs = bhi - blo, r = blockIdx.x - blo;
  const int fslot = nth_slot(b0, b1, gi);
  const int e = __builtin_amdgcn_readfirstlane(
      fslot < kWave ? __shfl(e0, fslot) : __shfl(e1, fslot - kWave));
  const uint64_t mlo = __ballot(e0 == e), mhi = __ballot(e1 == e);
  int nt = __popcll(mlo) + __popcll(mhi);
  nt = nt < kMfTok ? nt : kMfTok;
  const bool nf3 = (A.tm.w[e >> 5] >> (e & 31)) & 1u;
  int below = 0;  // experts of the same tier below e
  for (int i = 0; i < (e >> 5); ++i) below += __popc(A.tm.w[i]);
  below += __popc(A.tm.w[e >> 5] & ((1u << (e & 31)) - 1u));
  const int loc = nf3 ? below : e - below;
  if (loc >= (nf3 ? a.E3 : a.E4)) return;
  const int per = a.I / 16;
  const int tb = (int)((long)r * per / runs), te = (int)((long)(r + 1) * per / runs);
  // x rows of the expert's tokens (bf16, 1 KB per load)
  const int rowloads = a.K / 512;
  for (int q = wave; q < nt * rowloads; q += kMfWaves) {
    const int j = q / rowloads, c = q % rowloads;
    const int tok = nth_slot(mlo, mhi, j) / A.k;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.act_bf16 + (size_t)tok * a.K);
    lds_load_b128(src + c * 1024 + lane * 16, lds_addr(smem) + L.x + j * L.xstride + c * 1024);
  }
  const float g = nf3 ? 1.0f / kNF3TableScaleBf16
                      : (a.kept_fmt == HMOE_KEPT_NVFP4 ? a.kg[loc] : 1.0f);
  build_nf3_lut_any<false>(lut_s, kNF3TableScaleBf16);
  auto go = [&](auto fmt) {
    constexpr int FMT = decltype(fmt)::value;
    if (nt <= 1) mf_run<S, FMT, 1>(A, smem, lut_s, loc, nt, mlo, mhi, tb, te, g);
    else if (nt <= 2) mf_run<S, FMT, 2>(A, smem, lut_s, loc, nt, mlo, mhi, tb, te, g);
    else mf_run<S, FMT, 4>(A, smem, lut_s, loc, nt, mlo, mhi, tb, te, g);
  };
  if (nf3) go(std::integral_constant<int, kFmtNf3>{});
  else if (a.kept_fmt == HMOE_KEPT_NVFP4) go(std::integral_constant<int, kFmtNvfp4>{});
  else go(std::integral_constant<int, kFmtMxfp4>{});
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

typedef void (*StreamFn)(GemvArgs, StreamLayout);

template <int S>
static StreamFn pick_w13_stream_s(const GemvTiling& t) {
#define HMOE_STREAM_CASE(LR_, KU_, RI_) \
  if (t.lr == LR_ && t.ku == KU_ && t.ri == RI_) return w13_stream_kernel<LR_, KU_, RI_, S>;
  HMOE_STREAM_CASE(64, 1, 2) HMOE_STREAM_CASE(64, 2, 2) HMOE_STREAM_CASE(64, 3, 1) HMOE_STREAM_CASE(64, 4, 1)
  HMOE_STREAM_CASE(32, 1, 2) HMOE_STREAM_CASE(32, 2, 2) HMOE_STREAM_CASE(32, 3, 1) HMOE_STREAM_CASE(32, 4, 1)
  HMOE_STREAM_CASE(16, 1, 2) HMOE_STREAM_CASE(16, 2, 2) HMOE_STREAM_CASE(16, 3, 1) HMOE_STREAM_CASE(16, 4, 1)
  HMOE_STREAM_CASE(8, 1, 2) HMOE_STREAM_CASE(8, 2, 2) HMOE_STREAM_CASE(8, 3, 1) HMOE_STREAM_CASE(8, 4, 1)
  HMOE_STREAM_CASE(4, 1, 2) HMOE_STREAM_CASE(4, 2, 2) HMOE_STREAM_CASE(4, 3, 1) HMOE_STREAM_CASE(4, 4, 1)
#undef HMOE_STREAM_CASE
  return nullptr;
}

static StreamFn pick_w13_stream(const GemvTiling& t, int S) {
  if (S >= 4) return pick_w13_stream_s<4>(t);
  if (S == 3) return pick_w13_stream_s<3>(t);
  if (S == 2) return pick_w13_stream_s<2>(t);
  return nullptr;
}

// Decode GEMV tiling over reduction length K: LR = the largest power of two up to 64
// dividing the K/32 units, KU = units per lane, RI = rows (or row pairs) per lane per
// chunk, at most half the lanes of an LR-lane segment (the transposing reduction
// hands each row's sum to LR / RI lanes).
#ifndef HMOE_GEMV_LR_CAP
#define HMOE_GEMV_LR_CAP 64
#endif
#ifndef HMOE_GEMV_RI_CAP
#define HMOE_GEMV_RI_CAP 2
#endif
bool plan_gemv(int K, GemvTiling* t) {
  const int U = K / 32;
  int lr = 1;
  while (lr < HMOE_GEMV_LR_CAP && U % (2 * lr) == 0) lr *= 2;
  if (U / lr > 4) while (lr < 64 && U % (2 * lr) == 0) lr *= 2;
  const int ku = U / lr;
  if (lr < 4 || ku < 1 || ku > 4) return false;
  int ri = ku <= 2 ? HMOE_GEMV_RI_CAP : 1;  // two row (pair) groups at most: three waves per SIMD fit
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

// LDS layout of the matrix-core W13 kernel: the first-slot table, the x tile (M
// bf16 rows of K + 8), WPB * S stages of 32 rows x 256 K; one block per CU (at least
// one per distinct expert)
static bool plan_w13_mfma(const Layer& L, int M, MfLayout* ml) {
  if (M < 1 || M > kMfTok || L.H % 512 != 0 || L.I % 16 != 0) return false;
  const int gmax = M * L.k < L.E ? M * L.k : L.E;
  ml->fs = 0;
  ml->x = ((L.E * 4 + 15) / 16) * 16;
  ml->xstride = 2 * L.H + 16;
  ml->stages = ml->x + M * ml->xstride;
  ml->stage_bytes = kMfStageCode + 512;  // NVFP4 scales: the most
  int S = (kLdsBytes - 64 * kWave * 4 - ml->stages) / (kMfWaves * ml->stage_bytes);
  if (S > 3) S = 3;
  if (S < 2) return false;
  ml->nstage = S;
  ml->nblocks = cu_count() > gmax ? cu_count() : gmax;
  ml->total = ml->stages + kMfWaves * S * ml->stage_bytes;
  return true;
}

// LDS layout and run split of the staged W13 kernel: one block per run of a pass's
// chunks, about one block per CU over all passes; as many stages as fit in LDS (2-4).
static bool plan_w13_stream(const Layer& L, int npass, StreamLayout* sl) {
  const GemvTiling& t = L.w13;
  const int P = kWave / t.lr, CH = P * t.ri;
  const int per = L.I / CH;
  if (per < 1 || npass < 1) return false;
  int runs = cu_count() / npass;
  runs = runs < 1 ? 1 : (runs > per ? per : runs);
  const int run_max = (per + runs - 1) / runs;
  const int ncode = 2 * t.ri * t.ku;
  const int sdw = 2 * t.ri * P * (2 * t.lr * t.ku) / 4;  // NVFP4 scales: the most
  const int stage = ncode * 1024 + ((sdw + kWave - 1) / kWave) * 256;
  const int xbytes = ((L.H / 8 + kWave - 1) / kWave) * 1024;
  const int hbytes = ((run_max * CH * 4 + 255) / 256) * 256;
  sl->lut = 0;  // static
  sl->x = 0;
  sl->h = sl->x + xbytes;
  sl->stages = sl->h + hbytes;
  sl->stage_bytes = stage;
  int S = (kLdsBytes - 64 * kWave * 4 - sl->stages) / (kStreamWaves * stage);
  if (S > 4) S = 4;
  if (S < 2) return false;
  sl->nstage = S;
  sl->runs = runs;
  sl->total = sl->stages + kStreamWaves * S * stage;
  return true;
}

// raises a kernel's dynamic LDS limit to `bytes` (once per kernel and size)
static bool allow_lds(const void* fn, int bytes) {
  struct Entry {
    const void* fn;
    int bytes;
  };
  static Entry done[64] = {};
  for (int i = 0; i < 64; ++i) {
    if (done[i].fn == fn && done[i].bytes >= bytes) return true;
    if (done[i].fn == nullptr || done[i].fn == fn) {
      if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
        return false;
      done[i] = {fn, bytes};
      return true;
    }
  }
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
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
    MfArgs ma;
    if (kW13Impl == 2 && plan_w13_mfma(L, M, &ma.lay)) {
      ma.a = b;
      ma.ids = reinterpret_cast<const int32_t*>(base + P.topk_ids);
      ma.k = L.k;
      ma.tm = make_tier_mask(L);
      void (*mfn)(MfArgs) = ma.lay.nstage >= 3 ? w13_mfma_kernel<3> : w13_mfma_kernel<2>;
      if (!allow_lds(reinterpret_cast<const void*>(mfn), ma.lay.total)) return hipErrorInvalidValue;
      hipLaunchKernelGGL(mfn, dim3(ma.lay.nblocks), dim3(kMfThreads), ma.lay.total, s, ma);
      return hipGetLastError();
    }
    StreamLayout sl;
    if (kW13Impl == 1 && plan_w13_stream(L, a.npass, &sl)) {
      StreamFn sfn = pick_w13_stream(L.w13, sl.nstage);
      if (!sfn) return hipErrorInvalidValue;
      if (!allow_lds(reinterpret_cast<const void*>(sfn), sl.total)) return hipErrorInvalidValue;
      hipLaunchKernelGGL(sfn, dim3(a.npass * sl.runs), dim3(kStreamThreads), sl.total, s, b, sl);
      return hipGetLastError();
    }
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
