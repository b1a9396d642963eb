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
#include "route_common.h"

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

// Agent-coherent (write-through) store and load of one fp32 value: the single-launch
// decode hands h and the per-slot outputs from one workgroup to another, possibly on
// another XCD, without cache-wide fences (see decode_fused_kernel).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Byte offset (field * 8) of the NF3 quad table entry for 12-bit field Q (elements 4Q ..
// 4Q + 3, bits [12 Q, 12 Q + 12) of the 96-bit unit d0 d1 d2): the field shifted to bit 3
// and masked, one shift (or funnel shift) and one mask.
template <int Q>
__device__ __forceinline__ uint32_t nf3_quad_offset(uint32_t d0, uint32_t d1, uint32_t d2) {
  constexpr uint32_t kMask = 0xFFFu << 3;
  if constexpr (Q == 0) return (d0 << 3) & kMask;
  else if constexpr (Q == 1) return (d0 >> 9) & kMask;
  else if constexpr (Q == 2) return __builtin_amdgcn_alignbit(d1, d0, 21) & kMask;
  else if constexpr (Q == 3) return (d1 >> 1) & kMask;
  else if constexpr (Q == 4) return (d1 >> 13) & kMask;
  else if constexpr (Q == 5) return __builtin_amdgcn_alignbit(d2, d1, 25) & kMask;
  else if constexpr (Q == 6) return (d2 >> 5) & kMask;
  else return (d2 >> 17) & kMask;
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
  // NF3 from the per-lane pair table [64 pair fields][64 lanes] (the smaller table, for
  // kernels whose occupancy the quad table's LDS would limit): fp16 group scale per 64.
  // Both tables hold the same values and the dot products run in the same order, so the
  // results are the same bits.
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
  // NF3: level quads from the LDS table, fp16 group scale per 64. Each 12-bit field (four
  // codes) gives its entry's byte offset in a shift and a mask; the entry holds the
  // quad's two level pairs.
  static __device__ __forceinline__ void nf3(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                             const uint2* __restrict__ qlut,
                                             const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
    const char* base = reinterpret_cast<const char*>(qlut);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const uint32_t d0 = q[j].x, d1 = q[j].y, d2 = q[j].z;
      const float s = fp16_to_f32(sc[j]);
      uint32_t w[16];
      auto quad = [&](auto Q) {
        constexpr int qi = decltype(Q)::value;
        const uint2 v = *reinterpret_cast<const uint2*>(base + nf3_quad_offset<qi>(d0, d1, d2));
        w[2 * qi] = v.x;
        w[2 * qi + 1] = v.y;
      };
      quad(std::integral_constant<int, 0>{});
      quad(std::integral_constant<int, 1>{});
      quad(std::integral_constant<int, 2>{});
      quad(std::integral_constant<int, 3>{});
      quad(std::integral_constant<int, 4>{});
      quad(std::integral_constant<int, 5>{});
      quad(std::integral_constant<int, 6>{});
      quad(std::integral_constant<int, 7>{});
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

template <int LR, int KU, int NT, bool F16, int FMT, typename TAB>
__device__ __forceinline__ void row_dot(const uint4 (&q)[KU], const uint32_t (&sc)[KU],
                                        const TAB* qlut,
                                        const uint32_t (&x)[NT][KU][16], float (&acc)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  if constexpr (FMT == kFmtNf3) RowDot<LR, KU, NT, F16>::nf3(q, sc, qlut, x, acc);
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
__device__ __forceinline__ void build_nf3_pair_lut(uint32_t* lut, float c) {
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

// Builds the NF3 quad table [4096 quad fields]: entry f holds the 16-bit level pairs of
// its four codes, (level(f & 7) c, level((f >> 3) & 7) c) and (level((f >> 6) & 7) c,
// level(f >> 9) c), bf16 or fp16 (the low half holds the lower element). Thread t of the
// 256 writes entries t + 256 i, i = 0..15: their first pair is that of field t & 63, their
// second pair that of field w + 4 i, w = t >> 6 (the same for the whole wave). Each lane
// computes one pair (field = lane) and puts it in its wave's list at (lane & 3) * 16 +
// (lane >> 2), so the sixteen second pairs of wave w are the list's w-th 64 bytes, read
// back as four broadcast 16-byte loads: the level selects run once per lane instead of
// once per entry, which matters at kernel start, where every wave of a CU builds a copy.
template <bool F16>
__device__ __forceinline__ void build_nf3_lut(uint2* lut, float c) {
  static_assert(kGemvThreads == 256, "four waves build the table");
  __shared__ uint32_t pairs_t[kGemvWaves][kWave];
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const float lo = nf3_level((uint32_t)lane & 7u) * c, hi = nf3_level((uint32_t)lane >> 3) * c;
  const uint32_t mine = F16 ? pack_f16(lo, hi) : pack_bf16(lo, hi);
  pairs_t[w][(lane & 3) * 16 + (lane >> 2)] = mine;
  // LDS operations of one wave complete in order: the reads below see the writes
  __builtin_amdgcn_wave_barrier();
  const uint4* src = reinterpret_cast<const uint4*>(&pairs_t[w][16 * w]);
  uint32_t p[16];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 q = src[v];
    p[4 * v] = q.x;
    p[4 * v + 1] = q.y;
    p[4 * v + 2] = q.z;
    p[4 * v + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) lut[t + 256 * i] = make_uint2(mine, p[i]);
}

// The routing of every token, shared by a block's waves through LDS: slot s = t * k + j
// routes to expert ids[s] with weight w[s]; the tier map's words and, for each word, the
// NF3 experts below it (so a pass's tier code is two LDS reads, not a loop over the
// kernel argument's words).
struct BlockRoute {
  int32_t ids[kDecodeMaxM * kMaxTopK];
  float w[kDecodeMaxM * kMaxTopK];
  uint32_t tier_w[kMaxExperts / 32];
  int32_t tier_below[kMaxExperts / 32];
};

// tier_code (bit 16: NF3 tier; low bits: index within the tier) from the block's copy
__device__ __forceinline__ int block_tier_code(const BlockRoute& br, int e) {
  const uint32_t w = br.tier_w[e >> 5];
  const int below = br.tier_below[e >> 5] + __popc(w & ((1u << (e & 31)) - 1u));
  return ((w >> (e & 31)) & 1u) ? ((1 << 16) | below) : (e - below);
}

// calls f with NV (logits per lane for E experts) as a compile-time constant
template <typename F>
__device__ __forceinline__ void with_nv(int E, F&& f) {
  if (E <= 64) f(std::integral_constant<int, 1>{});
  else if (E <= 128) f(std::integral_constant<int, 2>{});
  else if (E <= 256) f(std::integral_constant<int, 4>{});
  else if (E <= 512) f(std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{});
}

// Pass p (slot p: token p / k) from the block's routing: the same record the routing
// launch writes to scratch (pass_info), taken from LDS.
__device__ __forceinline__ PassInfo block_pass(const GemvArgs& a, int k, int p,
                                               const BlockRoute& br) {
  const int e = __builtin_amdgcn_readfirstlane(br.ids[p]);
  const int code = (unsigned)e < (unsigned)a.E ? block_tier_code(br, e) : 0;
  PassInfo pi;
  pi.slot = p;
  pi.token = p / k;
  pi.nf3 = (code >> 16) != 0;
  pi.loc = code & 0xFFFF;
  pi.ok = (unsigned)e < (unsigned)a.E && pi.loc < (pi.nf3 ? a.E3 : a.E4);
  return pi;
}

// Every token's routing into the block's LDS (wave w: tokens w and w + 4), the logits
// rows requested before `between` runs (the level table build), and the tier map's copy.
template <typename F>
__device__ __forceinline__ void block_route(const float* __restrict__ logits, int M, int E, int k,
                                            const TierMask& tm, BlockRoute& br, F&& between) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    int below = 0;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 32; ++i) {
      br.tier_w[i] = tm.w[i];
      br.tier_below[i] = below;
      below += __popc(tm.w[i]);
    }
  }
  with_nv(E, [&](auto nvc) {
    constexpr int NV = decltype(nvc)::value;
    const int ta = wv, tb = wv + kGemvWaves;
    if (tb < M) {
      // two tokens, their routing steps interleaved
      float x[2][NV];
      route_fetch<NV>(logits + (size_t)ta * E, E, lane, x[0]);
      route_fetch<NV>(logits + (size_t)tb * E, E, lane, x[1]);
      between();
      int e[2];
      float wl[2];
      route_rank_n<NV, 2>(x, E, k, lane, e, wl);
      if (lane < k) {
        br.ids[ta * k + lane] = e[0];
        br.w[ta * k + lane] = wl[0];
        br.ids[tb * k + lane] = e[1];
        br.w[tb * k + lane] = wl[1];
      }
    } else {
      float x[NV];
      if (ta < M) route_fetch<NV>(logits + (size_t)ta * E, E, lane, x);
      between();
      if (ta < M) {
        float wl;
        const int e = route_rank<NV>(x, E, k, lane, &wl);
        if (lane < k) {
          br.ids[ta * k + lane] = e;
          br.w[ta * k + lane] = wl;
        }
      }
    }
  });
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

template <int LR, int KU, int RI, int FMT, bool COH = false, typename TAB>
__device__ __forceinline__ void w13_compute(const GemvArgs& a, int i0, int slot, float g,
                                            const uint32_t (&x)[1][KU][16],
                                            const TAB* qlut, const W13Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  float vg[RI], vu[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    float ag[1], au[1];
    row_dot<LR, KU, 1, false, FMT>(b.qg[ri], b.sg[ri], qlut, x, ag);
    row_dot<LR, KU, 1, false, FMT>(b.qu[ri], b.su[ri], qlut, x, au);
    vg[ri] = ag[0];
    vu[ri] = au[0];
  }
  const float gate = seg_reduce<RI, LR>(vg) * g;
  const float up = seg_reduce<RI, LR>(vu) * g;
  const int ri = seg_index<RI, LR>(c);
  if ((c & (LR / RI - 1)) == 0) {
    float* out = a.h_out + (size_t)slot * a.I + i0 + ri * P + rw;
    if constexpr (COH) store_coherent(out, silu(gate) * up);
    else *out = silu(gate) * up;
  }
}

// Chunks [c0, end) of one pass (chunk `first` is the expert's pair 0). A holds
// chunk c0 on entry when a_loaded.
template <int LR, int KU, int RI, int FMT, bool COH = false, typename TAB>
__device__ __forceinline__ void w13_pass(const GemvArgs& a, const PassInfo& pi, int c0, int end,
                                         int first, float g, const TAB* qlut,
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
    w13_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, A);
    if (++cc >= end) break;
    w13_load<LR, KU, RI, FMT>(a, pi.loc, (min(cc + 1, end - 1) - first) * CH, A);
    w13_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, B);
    ++cc;
  }
}

template <int LR, int KU, int RI>
__global__ __launch_bounds__(kGemvThreads) void w13_gemv_kernel(GemvArgs a) {
  __shared__ uint2 lut[4096];  // [quad field]: bf16 pairs of scaled NF3 levels
  constexpr int CH = (kWave / LR) * RI;  // pairs per chunk
  const uint2* qlut = lut;
  const int per = a.out_units / CH;      // chunks per pass
  const WaveRange wr = wave_range<false>(a.npass * per);
  // the first chunk's weights are requested before the table is built
  W13Buf<KU, RI> A, B;
  PassInfo pi{};
  int4 r_next{};
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    const int4 r_first = a.pass[p];
    if (p + 1 < a.npass) r_next = a.pass[p + 1];
    pi = pass_info(a, r_first);
    if (pi.ok)
      with_format(a, pi, [&](auto f) {
        w13_load<LR, KU, RI, decltype(f)::value>(a, pi.loc, (wr.begin - p * per) * CH, A);
      });
  }
  build_nf3_lut<false>(lut, kNF3TableScaleBf16);
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
        w13_pass<LR, KU, RI, decltype(f)::value>(a, pi, ch, p_end, p * per, g, qlut, A, B,
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
template <int LR, int KU, bool COH = false>
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
    if constexpr (COH) {
      const float* r = reinterpret_cast<const float*>(row + f);
      v[i] = (NF4 % kWave == 0 || f < NF4)
                 ? make_float4(load_coherent(r), load_coherent(r + 1), load_coherent(r + 2),
                               load_coherent(r + 3))
                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      v[i] = (NF4 % kWave == 0 || f < NF4) ? row[f] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
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

// BUF: buffer loads (the chunk's row offset in a scalar register, the lane's offset
// fixed); otherwise flat loads (the single-launch decode, where they measured faster)
template <int LR, int KU, int RI, int FMT, bool BUF = true>
__device__ __forceinline__ void w2_load(const GemvArgs& a, int loc, int n0, W2Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  if constexpr (BUF) {
    const ExpertRsrc r = expert_rsrc<FMT>(a, loc);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
      load_row_rsrc<LR, KU, FMT>(r, a.K, n0 + ri * P, rw, c, b.q[ri], b.sc[ri]);
  } else {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
      load_row<LR, KU, FMT>(a, (size_t)loc * a.rows + n0 + ri * P + rw, c, b.q[ri], b.sc[ri]);
  }
}

template <int LR, int KU, int RI, int FMT, bool COH = false, typename TAB>
__device__ __forceinline__ void w2_compute(const GemvArgs& a, int n0, int slot, float g,
                                           const uint32_t (&x)[1][KU][16],
                                           const TAB* qlut, const W2Buf<KU, RI>& b) {
  constexpr int P = kWave / LR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LR;
  const int rw = lane / LR;
  float v[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    float acc[1];
    row_dot<LR, KU, 1, true, FMT>(b.q[ri], b.sc[ri], qlut, x, acc);
    v[ri] = acc[0];
  }
  const float sum = seg_reduce<RI, LR>(v);
  const int ri = seg_index<RI, LR>(c);
  if ((c & (LR / RI - 1)) == 0) {
    float* out = a.o_out + (size_t)slot * a.rows + n0 + ri * P + rw;
    if constexpr (COH) store_coherent(out, sum * g);
    else *out = sum * g;
  }
}

template <int LR, int KU, int RI, int FMT, bool COH = false, typename TAB>
__device__ __forceinline__ void w2_pass(const GemvArgs& a, const PassInfo& pi, int c0, int end,
                                        int first, float gt, const TAB* qlut,
                                        uint32_t* hs, W2Buf<KU, RI>& A, W2Buf<KU, RI>& B,
                                        bool a_loaded) {
  constexpr int CH = (kWave / LR) * RI;
  const int c = (threadIdx.x & (kWave - 1)) % LR;
  int cc = c0;
  if (!a_loaded) w2_load<LR, KU, RI, FMT, !COH>(a, pi.loc, (cc - first) * CH, A);
  uint32_t x[1][KU][16];
  const float g = __builtin_ldexpf(gt, stage_h<LR, KU, COH>(a, pi.slot, hs, c, x));
  if constexpr (COH) {
    // the single-launch decode: the next chunk is loaded only when there is one
    while (cc < end) {
      if (cc + 1 < end) w2_load<LR, KU, RI, FMT, false>(a, pi.loc, (cc + 1 - first) * CH, B);
      w2_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, A);
      if (++cc >= end) break;
      if (cc + 1 < end) w2_load<LR, KU, RI, FMT, false>(a, pi.loc, (cc + 1 - first) * CH, A);
      w2_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, B);
      ++cc;
    }
  } else {
    // as in the W13 pass: the next chunk's loads are issued on every path (the last
    // chunk repeats itself) and the compiler may not move the current chunk's wait above
    // them, so each compute waits only for its own chunk
    while (cc < end) {
      w2_load<LR, KU, RI, FMT>(a, pi.loc, (min(cc + 1, end - 1) - first) * CH, B);
      __builtin_amdgcn_sched_barrier(0);
      w2_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, A);
      if (++cc >= end) break;
      w2_load<LR, KU, RI, FMT>(a, pi.loc, (min(cc + 1, end - 1) - first) * CH, A);
      __builtin_amdgcn_sched_barrier(0);
      w2_compute<LR, KU, RI, FMT, COH>(a, (cc - first) * CH, pi.slot, g, x, qlut, B);
      ++cc;
    }
  }
}

// dynamic LDS: one staged h row (K fp16) per wave
template <int LR, int KU, int RI>
__global__ __launch_bounds__(kGemvThreads) void w2_gemv_kernel(GemvArgs a) {
  __shared__ uint2 lut[4096];  // [quad field]: fp16 pairs of scaled NF3 levels
  extern __shared__ uint32_t h_stage[];
  constexpr int CH = (kWave / LR) * RI;  // rows per chunk
  constexpr int KD = 16 * LR * KU;        // dwords per staged row (K / 2)
  const uint2* qlut = lut;
  uint32_t* hs = h_stage + KD * (threadIdx.x >> 6);
  const int per = a.out_units / CH;
  const WaveRange wr = wave_range<true>(a.npass * per);
  // the first chunk's weights are requested before the table is built
  W2Buf<KU, RI> A, B;
  PassInfo pi{};
  int4 r_next{};
  if (wr.begin < wr.end) {
    const int p = wr.begin / per;
    const int4 r_first = a.pass[p];
    if (p + 1 < a.npass) r_next = a.pass[p + 1];
    pi = pass_info(a, r_first);
    if (pi.ok)
      with_format(a, pi, [&](auto f) {
        w2_load<LR, KU, RI, decltype(f)::value>(a, pi.loc, (wr.begin - p * per) * CH, A);
      });
  }
  build_nf3_lut<true>(lut, kNF3TableScaleF16);
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
        w2_pass<LR, KU, RI, decltype(f)::value>(a, pi, ch, p_end, p * per, gt, qlut, hs, A,
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
// Single-launch decode (M <= 8)
// ---------------------------------------------------------------------------
//
// decode_fused_kernel runs the whole decode forward in one launch: routing, W13 +
// SwiGLU, W2 and the weighted top-k combine (local-inference-lab/vllm PR #92, "How it
// works": the M <= 8 path is addressed directly by the top-k result, and both tiers
// share one routing and one top-k sum). The grid is persistent (as many blocks as are
// resident at once). Blocks 0 .. G-2 are work blocks: each of their waves takes a
// contiguous run of the flat W13 range (npass * per13 chunks), then one of the W2 range,
// with the same chunk code as the four-launch path, so h, the per-slot outputs and y are
// bit-identical to it. Every block routes all M tokens itself (one wave per token, the
// rows requested before its level tables are built) and shares the result in LDS, so no
// block waits for routing done elsewhere. The last block
// routes every token once more and writes the inspection outputs (top-k ids and weights,
// pass records, tier map, decode grouping) off the critical path.
//
// Hand-offs between workgroups go through counters in scratch, one 64-byte line each:
//   h_cnt[s]      W13 chunks of slot s finished; the wave whose increment completes it
//                 sets slot s's ready flag in all kReadyCopies copies;
//   ready[s][c]   a W2 run of slot s first requests its weights, then polls copy
//                 blockIdx % kReadyCopies of the flag (many waiters on one line slow
//                 down every access to that memory channel, so they are spread out);
//   comb[t][g]    W2 chunks of token t's 64-row output group g finished over all k slots;
//                 the wave whose increment completes it sums the k slot rows in fixed slot
//                 order and writes those 64 outputs of y;
//   exit          blocks finished; the last one clears every counter, so each launch
//                 starts from zeros (the scratch's sync region must be zero before the
//                 first decode forward: moe_scratch_init, or a zero-filled allocation).
// h and the per-slot outputs are written with agent-coherent (write-through) stores and
// read with agent-coherent loads; before a counter increment the wave waits for all its
// memory operations to complete, so the data it signals is visible on every XCD. This
// avoids cache-wide release/acquire fences, which measured about 70 ns each, serialised
// per XCD, on MI355X. Waits are bounded (kSpinLimit polls): a wait that gives up, which
// only a grid that is not fully resident can cause, is counted in the sync region
// (moe_decode_view's sync_timeouts) and the launch still ends.

constexpr int kSyncLine = 16;                  // sync words per counter (one 64-byte line)
constexpr int kSyncExit = 0;                   // blocks finished
constexpr int kSyncTimeouts = kSyncLine;       // bounded waits that gave up (never cleared)
constexpr int kSyncH = 2 * kSyncLine;          // h_cnt[s] at kSyncH + s * kSyncLine
constexpr int kReadyCopies = 16;               // copies of each slot's ready flag
constexpr int kCombRows = 64;                  // rows of y per combine group
constexpr int kSpinLimit = 1 << 16;
// gfx9 s_waitcnt operand: vmcnt 0 (every vector memory operation of the wave, its
// coherent stores and atomics included, has completed), expcnt 7 and lgkmcnt 15 free
constexpr int kWaitVmem = 0x0F70;

struct FusedArgs {
  GemvArgs a13, a2;
  const float* logits;
  int M, E, k;
  int per13, per2;   // chunks per pass of each GEMV
  int nwork;         // work waves (four per work block)
  int nwork_blocks;
  int G;             // combine groups per token: H / 64
  int ready_base;    // word offset of ready[0][0]
  int comb_base;     // word offset of comb[0][0]
  uint32_t* sync;
  const float* o;    // per-slot outputs (a2.o_out)
  uint16_t* y;
  int32_t* ids;      // inspection outputs, written by the last block
  float* w;
  int32_t* expert_tier;
  int32_t* pass;
  GroupArgs ga;
};

__device__ __forceinline__ uint32_t sync_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sync_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// all of this wave's memory operations complete before anything after it is issued
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ PassInfo fused_pass(const FusedArgs& f, const TierMask& tm, int p,
                                               const BlockRoute& br) {
  return block_pass(f.a13, f.k, p, br);
}

// this wave's run [b, e) of a flat range of n chunks: runs numbered block-major (the
// waves of a block take consecutive runs) or wave-major (consecutive blocks do)
template <bool WAVE_MAJOR>
__device__ __forceinline__ void wave_run(const FusedArgs& f, int n, int* b, int* e) {
  const int wv = threadIdx.x >> 6;
  const int gw = WAVE_MAJOR ? wv * f.nwork_blocks + (int)blockIdx.x : (int)blockIdx.x * kGemvWaves + wv;
  *b = (int)((long)gw * n / f.nwork);
  *e = (int)((long)(gw + 1) * n / f.nwork);
}

// waits until all W13 chunks of slot p are done (bounded), polling this block's copy of
// the slot's ready flag
__device__ __forceinline__ void wait_h(const FusedArgs& f, int p) {
  const uint32_t* c =
      f.sync + f.ready_base + (p * kReadyCopies + (int)(blockIdx.x % kReadyCopies)) * kSyncLine;
  for (int it = 0;; ++it) {
    if (sync_load(c) != 0u) break;
    if (it == kSpinLimit) {
      if ((threadIdx.x & (kWave - 1)) == 0) sync_add(f.sync + kSyncTimeouts, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// y[t, 64 g + lane] = sum_j w[t, j] * o[t*k + j, 64 g + lane] in fixed j order (the
// order of decode_combine_kernel), eight slot rows requested at a time
__device__ __forceinline__ void fused_combine(const FusedArgs& f, int t, int g, const BlockRoute& br) {
  const int lane = threadIdx.x & (kWave - 1);
  const int H = f.a2.rows;
  const int n = g * kCombRows + lane;
  float acc = 0.0f;
#pragma unroll
  for (int j0 = 0; j0 < kMaxTopK; j0 += 8) {
    float ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ov[j] = j0 + j < f.k ? load_coherent(f.o + (size_t)(t * f.k + j0 + j) * H + n) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc = __builtin_fmaf(j0 + j < f.k ? br.w[t * f.k + j0 + j] : 0.0f, ov[j], acc);
  }
  f.y[(size_t)t * H + n] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
}

// QUAD: NF3 through the quad tables (two 32 KB tables); otherwise the per-lane pair tables
// (two 16 KB tables), for tilings whose register use leaves room for a third block per
// CU that the larger tables would take away. Same values, same bits either way.
template <int LR13, int KU13, int RI13, int LR2, int KU2, int RI2, bool QUAD>
__global__ __launch_bounds__(kGemvThreads) void decode_fused_kernel(FusedArgs f, TierMask tm) {
  constexpr int CH13 = (kWave / LR13) * RI13;
  constexpr int CH2 = (kWave / LR2) * RI2;
  constexpr int KD2 = 16 * LR2 * KU2;          // dwords of one staged h row
  static_assert(kCombRows % CH2 == 0, "combine groups hold whole W2 chunks");
  struct QuadLuts {
    uint2 w13[4096];   // [quad field]: bf16 pairs of scaled NF3 levels
    uint2 w2[4096];    // the same in fp16
  };
  struct PairLuts {
    uint32_t w13[64 * kWave];   // [pair field][lane]: bf16 pairs of scaled NF3 levels
    uint32_t w2[64 * kWave];    // the same in fp16
  };
  using Luts = std::conditional_t<QUAD, QuadLuts, PairLuts>;
  union Big {
    Luts luts;
    GroupSmem group;
  };
  __shared__ Big big;
  __shared__ BlockRoute br;
  __shared__ int last_block;
  extern __shared__ uint32_t h_stage[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;

  if (blockIdx.x == gridDim.x - 1) {
    // inspection outputs: routing of every token, pass records, tier map, grouping
    for (int t = wv; t < f.M; t += kGemvWaves) {
      float wl;
      const int e = route_select_any(f.logits + (size_t)t * f.E, f.E, f.k, lane, &wl);
      if (lane < f.k) {
        const int s = t * f.k + lane;
        f.ids[s] = e;
        f.w[s] = wl;
        reinterpret_cast<int4*>(f.pass)[s] = make_int4(s, tier_code(tm, e), t, e);
      }
    }
    for (int e = threadIdx.x; e < f.E; e += kGemvThreads) f.expert_tier[e] = tier_code(tm, e);
    __syncthreads();
    decode_grouping(f.ga, tm, big.group);
  } else {
    // every token's routing, its logits rows requested before the level tables are built
    block_route(f.logits, f.M, f.E, f.k, tm, br, [&] {
      if constexpr (QUAD) {
        build_nf3_lut<false>(big.luts.w13, kNF3TableScaleBf16);
        build_nf3_lut<true>(big.luts.w2, kNF3TableScaleF16);
      } else {
        build_nf3_pair_lut<false>(big.luts.w13, kNF3TableScaleBf16);
        build_nf3_pair_lut<true>(big.luts.w2, kNF3TableScaleF16);
      }
    });
    __syncthreads();
    const auto* lut13 = QUAD ? big.luts.w13 : big.luts.w13 + lane;
    const auto* lut2 = QUAD ? big.luts.w2 : big.luts.w2 + lane;
    const int npass = f.M * f.k;

    // ---- W13 + SwiGLU: run gw of the flat range (blocks first)
    {
      int b, e;
      wave_run<false>(f, npass * f.per13, &b, &e);
      W13Buf<KU13, RI13> A, B;
      for (int ch = b; ch < e;) {
        const int p = __builtin_amdgcn_readfirstlane(ch / f.per13);
        const int p_end = min(e, (p + 1) * f.per13);
        const PassInfo pi = fused_pass(f, tm, p, br);
        if (pi.ok) {
          const float g = pi.nf3 ? 1.0f / kNF3TableScaleBf16
                                 : (f.a13.kept_fmt == HMOE_KEPT_NVFP4 ? f.a13.kg[pi.loc] : 1.0f);
          with_format(f.a13, pi, [&](auto fm) {
            w13_pass<LR13, KU13, RI13, decltype(fm)::value, true>(f.a13, pi, ch, p_end, p * f.per13, g,
                                                                  lut13, A, B, false);
          });
        }
        wait_vmem();
        const uint32_t inc = (uint32_t)(p_end - ch);
        uint32_t old = 0;
        if (lane == 0) old = sync_add(f.sync + kSyncH + p * kSyncLine, inc);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old + inc == (uint32_t)f.per13 && lane < kReadyCopies)
          sync_store(f.sync + f.ready_base + (p * kReadyCopies + lane) * kSyncLine, 1u);
        ch = p_end;
      }
    }

    // ---- W2 and the combine: run gw of the flat range (waves first)
    {
      int b, e;
      wave_run<true>(f, npass * f.per2, &b, &e);
      uint32_t* hs = h_stage + KD2 * wv;
      constexpr int CPG = kCombRows / CH2;   // W2 chunks per combine group
      W2Buf<KU2, RI2> A, B;
      for (int ch = b; ch < e;) {
        const int p = __builtin_amdgcn_readfirstlane(ch / f.per2);
        const int p_end = min(e, (p + 1) * f.per2);
        const int t = p / f.k;
        const PassInfo pi = fused_pass(f, tm, p, br);
        // the first chunk's weights are requested before the wait for h
        if (pi.ok)
          with_format(f.a2, pi, [&](auto fm) {
            w2_load<LR2, KU2, RI2, decltype(fm)::value, false>(f.a2, pi.loc, (ch - p * f.per2) * CH2, A);
          });
        wait_h(f, p);
        if (pi.ok) {
          const float gt = pi.nf3 ? 1.0f / kNF3TableScaleF16
                                  : (f.a2.kept_fmt == HMOE_KEPT_NVFP4 ? f.a2.kg[pi.loc] : 1.0f);
          with_format(f.a2, pi, [&](auto fm) {
            w2_pass<LR2, KU2, RI2, decltype(fm)::value, true>(f.a2, pi, ch, p_end, p * f.per2, gt, lut2,
                                                              hs, A, B, true);
          });
        }
        wait_vmem();
        for (int c = ch; c < p_end;) {
          const int grp = (c - p * f.per2) / CPG;
          const int gend = min(p_end, p * f.per2 + (grp + 1) * CPG);
          const uint32_t inc = (uint32_t)(gend - c);
          uint32_t old = 0;
          if (lane == 0) old = sync_add(f.sync + f.comb_base + (t * f.G + grp) * kSyncLine, inc);
          old = __builtin_amdgcn_readfirstlane(old);
          if (old + inc == (uint32_t)(f.k * CPG)) fused_combine(f, t, grp, br);
          c = gend;
        }
        ch = p_end;
      }
    }
  }

  // ---- exit: the last block clears the counters for the next launch
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) last_block = sync_add(f.sync + kSyncExit, 1u) + 1u == gridDim.x;
  __syncthreads();
  if (last_block) {
    const int nh = f.M * f.k, nc = f.M * f.G;
    for (int i = threadIdx.x; i < nh; i += kGemvThreads) sync_store(f.sync + kSyncH + i * kSyncLine, 0u);
    for (int i = threadIdx.x; i < nh * kReadyCopies; i += kGemvThreads)
      sync_store(f.sync + f.ready_base + i * kSyncLine, 0u);
    for (int i = threadIdx.x; i < nc; i += kGemvThreads) sync_store(f.sync + f.comb_base + i * kSyncLine, 0u);
    if (threadIdx.x == 0) sync_store(f.sync + kSyncExit, 0u);
  }
}

// zero-fills n words of the sync region (moe_scratch_init; no memset, so it is safe
// under graph capture)
__global__ __launch_bounds__(256) void sync_clear_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
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

// GEMV arguments of one decode stage (W13 or W2) over the scratch regions
static GemvArgs gemv_args(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                          void* scratch, bool w13) {
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
  if (w13) {
    a.kq = W.kept_w13_q; a.ks = W.kept_w13_s; a.kg = W.kept_w13_g;
    a.nq = W.nf3_w13_q; a.ns = W.nf3_w13_s;
    a.rows = 2 * L.I; a.K = L.H; a.out_units = L.I;
    a.act_bf16 = x;
    a.h_out = h;
  } else {
    a.kq = W.kept_w2_q; a.ks = W.kept_w2_s; a.kg = W.kept_w2_g;
    a.nq = W.nf3_w2_q; a.ns = W.nf3_w2_s;
    a.rows = L.H; a.K = L.I; a.out_units = L.H;
    a.act_f32 = h;
    a.o_out = o;
  }
  return a;
}

static GroupArgs group_args(const Layer& L, int M, void* scratch) {
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
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
  return ga;
}

hipError_t launch_decode(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                         uint16_t* y, void* scratch, int stage, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  const GemvArgs a = gemv_args(L, W, x, M, scratch, true);
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
    const GemvArgs b = a;
    GemvFn fn = pick_gemv<true>(L.w13);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid_for(fn, L.w13, L.I, 0)), dim3(kGemvThreads), 0, s, b);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_W2) {
    const GemvArgs b = gemv_args(L, W, x, M, scratch, false);
    GemvFn fn = pick_gemv<false>(L.w2);
    if (!fn) return hipErrorInvalidValue;
    const size_t smem = (size_t)kGemvWaves * L.I * 2;  // one fp16 h row per wave
    hipLaunchKernelGGL(fn, dim3(grid_for(fn, L.w2, L.H, smem)), dim3(kGemvThreads), smem, s, b);
    return hipGetLastError();
  }
  if (stage == HMOE_STAGE_COMBINE) {
    const int n = M * L.H;
    const GroupArgs ga = group_args(L, M, scratch);
    // one more block than the sum needs: it builds the grouping
    hipLaunchKernelGGL(decode_combine_kernel, dim3((n + 255) / 256 + 1), dim3(256), 0, s, o,
                       reinterpret_cast<const float*>(base + P.topk_w), M, L.k, L.H, y, ga,
                       make_tier_mask(L));
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// ---- single-launch decode: the tiling pairs (W13 over K = H, W2 over K = I) it is
// instantiated for; other layer shapes run the four-launch path
typedef void (*FusedFn)(FusedArgs, TierMask);

// QUAD (last field): the tiling's registers already hold it to two blocks per CU, which
// the quad tables' LDS allows; the others keep the pair tables and their third block
static FusedFn pick_fused(const GemvTiling& a, const GemvTiling& b) {
#define HMOE_FUSED_CASE(L1, K1, R1, L2, K2, R2, Q)                                     \
  if (a.lr == L1 && a.ku == K1 && a.ri == R1 && b.lr == L2 && b.ku == K2 && b.ri == R2) \
    return decode_fused_kernel<L1, K1, R1, L2, K2, R2, Q>;
  HMOE_FUSED_CASE(8, 1, 2, 4, 1, 2, false)     // H = 256, I = 128
  HMOE_FUSED_CASE(4, 3, 1, 8, 1, 2, false)     // H = 384, I = 256
  HMOE_FUSED_CASE(16, 1, 2, 8, 1, 2, false)    // H = 512, I = 256
  HMOE_FUSED_CASE(32, 1, 2, 16, 1, 2, false)   // H = 1024, I = 512
  HMOE_FUSED_CASE(64, 1, 2, 8, 3, 1, true)     // H = 2048, I = 768 (Qwen3-MoE-shaped)
  HMOE_FUSED_CASE(64, 3, 1, 64, 1, 2, false)   // H = 6144, I = 2048 (GLM-class)
  HMOE_FUSED_CASE(64, 2, 2, 32, 3, 1, true)    // H = 4096, I = 1536
  HMOE_FUSED_CASE(64, 2, 2, 64, 1, 2, false)   // H = 4096, I = 2048
  HMOE_FUSED_CASE(64, 1, 2, 16, 3, 1, true)    // H = 2048, I = 1536
#undef HMOE_FUSED_CASE
  return nullptr;
}

bool fused_decode_available(const Layer& L) { return pick_fused(L.w13, L.w2) != nullptr; }

// words of the single-launch decode's sync region: exit, timeouts, h_cnt per slot
// (8k slots), kReadyCopies ready flags per slot, comb per token and 64-row group (8
// tokens), one 64-byte line each
size_t fused_sync_words(int k, int H) {
  return (size_t)(2 + kDecodeMaxM * k * (1 + kReadyCopies) + kDecodeMaxM * (H / kCombRows)) *
         kSyncLine;
}

static int fused_resident_blocks(FusedFn fn, size_t smem) {
  static FusedFn cfn[8] = {};
  static size_t csmem[8] = {};
  static int cn[8] = {};
  for (int i = 0; i < 8; ++i) {
    if (cfn[i] == fn && csmem[i] == smem) return cn[i];
    if (cfn[i] == nullptr) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn),
                                                       kGemvThreads, smem) != hipSuccess || n < 1)
        n = 1;
      cfn[i] = fn;
      csmem[i] = smem;
      cn[i] = n;
      return n;
    }
  }
  return 1;
}

hipError_t launch_decode_fused(const Layer& L, const hmoe_weights& W, const uint16_t* x,
                               const float* logits, int M, uint16_t* y, void* scratch,
                               hipStream_t s) {
  if (M <= 0) return hipSuccess;
  FusedFn fn = pick_fused(L.w13, L.w2);
  if (!fn) return hipErrorInvalidValue;
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  FusedArgs f{};
  f.a13 = gemv_args(L, W, x, M, scratch, true);
  f.a2 = gemv_args(L, W, x, M, scratch, false);
  f.logits = logits;
  f.M = M;
  f.E = L.E;
  f.k = L.k;
  f.per13 = L.I / ((64 / L.w13.lr) * L.w13.ri);
  f.per2 = L.H / ((64 / L.w2.lr) * L.w2.ri);
  f.G = L.H / kCombRows;
  f.ready_base = kSyncH + kDecodeMaxM * L.k * kSyncLine;
  f.comb_base = f.ready_base + kDecodeMaxM * L.k * kReadyCopies * kSyncLine;
  f.sync = reinterpret_cast<uint32_t*>(base + P.d_sync);
  f.o = f.a2.o_out;
  f.y = y;
  f.ids = reinterpret_cast<int32_t*>(base + P.topk_ids);
  f.w = reinterpret_cast<float*>(base + P.topk_w);
  f.expert_tier = reinterpret_cast<int32_t*>(base + P.expert_tier);
  f.pass = reinterpret_cast<int32_t*>(base + P.d_pass);
  f.ga = group_args(L, M, scratch);
  // a persistent grid that is resident at once: the work blocks, never more waves than
  // W13 chunks, plus the block that writes the inspection outputs
  const size_t smem = (size_t)kGemvWaves * L.I * 2;   // one fp16 h row per wave
  const long cap = (long)fused_resident_blocks(fn, smem) * cu_count() - 1;
  const long n13 = (long)M * L.k * f.per13;
  long work = (n13 + kGemvWaves - 1) / kGemvWaves;
  if (work > cap) work = cap;
  if (work < 1) work = 1;
  f.nwork_blocks = (int)work;
  f.nwork = (int)work * kGemvWaves;
  hipLaunchKernelGGL(fn, dim3((unsigned)work + 1), dim3(kGemvThreads), smem, s, f, make_tier_mask(L));
  return hipGetLastError();
}

hipError_t launch_sync_clear(const Layer& L, void* scratch, hipStream_t s) {
  const int n = (int)fused_sync_words(L.k, L.H);
  uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<char*>(scratch) + L.plan.d_sync);
  hipLaunchKernelGGL(sync_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace hmoe
