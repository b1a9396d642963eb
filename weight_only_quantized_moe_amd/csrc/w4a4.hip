// W4A4 kept tier (an MXFP4 kept tier with MXFP4 activations): the activation quantiser
// and the grouped GEMM on gfx950's MX-scaled matrix cores. vllm-project/vllm PR #42428,
// "What's in this PR", places the W4A16 path beside W4A4 backends, whose activations are
// 4-bit too; here each kept-tier matmul input (x before W13, h before W2) is rounded to
// MXFP4 along K in blocks of 32 (OCP MX v1.0 conversion: shared exponent floor(log2
// amax) - 2, elements rounded to E2M1 nearest-even, saturating at 6), and both operands
// go to v_mfma_scale_f32_16x16x128_f8f6f4 as they are stored: 16-byte fragments of 32
// E2M1 codes plus one E8M0 byte per lane, no decode, no LDS.
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMxThreads = 256;
constexpr int kMxBN = 128;   // weight rows per block tile (W13: 64 gate + the 64 matching up rows)
constexpr int kMxBK = 128;   // K per MFMA step: four 32-blocks

// E2M1 code of t (|t| < 8 after scaling): nearest magnitude of {0, .5, 1, 1.5, 2, 3, 4,
// 6}, ties to the even code index, saturating at 6; a zero magnitude is code 0
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fminf(fabsf(t), 6.0f);
  uint32_t m;
  if (a <= 0.25f) m = 0;
  else if (a < 0.75f) m = 1;
  else if (a <= 1.25f) m = 2;
  else if (a < 1.75f) m = 3;
  else if (a <= 2.5f) m = 4;
  else if (a < 3.5f) m = 5;
  else if (a <= 5.0f) m = 6;
  else m = 7;
  return (m != 0 && t < 0.0f) ? (m | 8u) : m;
}

// One 32-element block of a row to MXFP4: 16 code bytes (element 2j in the low nibble of
// byte j) and its E8M0 byte (127 for an all-zero block).
__device__ __forceinline__ void mx_block(const float (&v)[32], uint4* codes, uint8_t* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int shared = 0;
  if (amax > 0.0f) {
    int E;
    (void)frexpf(amax, &E);                       // amax = m 2^E, m in [0.5, 1)
    shared = min(max(E - 1 - 2, -127), 127);
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i)
    w[i >> 3] |= e2m1_code(__builtin_ldexpf(v[i], -shared)) << (4 * (i & 7));
  *codes = make_uint4(w[0], w[1], w[2], w[3]);
  *scale = (uint8_t)(shared + 127);
}

// rows x (K / 32) blocks, one thread each; BF16 input (x) or fp32 (h); rows at or past
// *nrows (when given) are skipped
template <bool BF16>
__global__ __launch_bounds__(kMxThreads) void mx_quant_kernel(const void* __restrict__ in, int rows,
                                                              int K, const int32_t* __restrict__ nrows,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const long i = (long)blockIdx.x * kMxThreads + threadIdx.x;
  const int nb = K / 32;
  if (i >= (long)rows * nb) return;
  const int r = (int)(i / nb), c = (int)(i - (long)r * nb);
  if (nrows && r >= nrows[0]) return;
  float v[32];
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + (size_t)r * K + 32 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = p[q];
      const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = bf16_lo(d[e]);
        v[8 * q + 2 * e + 1] = bf16_hi(d[e]);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + (size_t)r * K + 32 * c);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 t = p[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  }
  mx_block(v, reinterpret_cast<uint4*>(codes + (size_t)r * (K / 2) + 16 * c), scales + (size_t)r * nb + c);
}

struct MxArgs {
  const uint8_t* wq;    // kept-tier codes [E4, rows_w, K/2]
  const uint8_t* ws;    // E8M0 scales [E4, rows_w, K/32]
  int rows_w, K;
  const uint8_t* aq;    // activation codes [arows, K/2]: W13 x per token, W2 h per align row
  const uint8_t* as;    // [arows, K/32]
  int k, nslot;
  const int32_t* slots; // kept-tier align: sorted slots, block -> expert, num_padded
  const int32_t* bexp;
  const int32_t* npad;
  int nblk;             // align blocks this launch covers
  int E4, I, H;
  float* h_out;         // W13: fp32 [cap_kept, I]
  float* o_out;         // W2: fp32 [nslot, H]
  const float* topk_w;
};

// Block: BM slot rows of one kept-tier align block x kMxBN weight rows (W13: 64 gate
// rows and the matching 64 up rows, so the block makes 64 h columns; W2: 128 output
// columns). Four waves split it 2 x 2 (1 x 4 for BM = 16); each wave keeps MT x NT
// 16x16 tiles in registers and loads, per 128-K step, one 16-byte fragment and one scale
// byte per tile row and per tile column, the next step's already in flight.
template <int BM, bool W13>
__global__ __launch_bounds__(kMxThreads) void mx_gemm_kernel(MxArgs a) {
  constexpr int WAVES_M = BM >= 32 ? 2 : 1;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int MT = BM / WAVES_M / 16;
  constexpr int NT = kMxBN / WAVES_N / 16;
  const int blk = blockIdx.y, tile = blockIdx.x;
  if (blk >= a.nblk || blk * BM >= a.npad[0]) return;
  const int loc = a.bexp[blk];
  if ((unsigned)loc >= (unsigned)a.E4) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int j = lane & 15, g = lane >> 4;
  const int r0 = blk * BM;
  const int n0 = tile * (W13 ? kMxBN / 2 : kMxBN);
  const int KB = a.K / 2, SB = a.K / 32;   // code and scale bytes per row

  // tile row (within the block's weight rows) of column tile nt; W13 pairs gate tile nt
  // with up tile nt + NT / 2 in the same lanes
  auto wrow = [&](int nt) {
    if constexpr (W13) {
      constexpr int HALF = NT / 2;
      const int base = wn * (kMxBN / 2 / WAVES_N);
      return nt < HALF ? n0 + base + 16 * nt : a.I + n0 + base + 16 * (nt - HALF);
    } else {
      return n0 + wn * (kMxBN / WAVES_N) + 16 * nt;
    }
  };
  const uint8_t* bq[NT];
  const uint8_t* bs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const size_t row = (size_t)loc * a.rows_w + wrow(nt) + j;
    bq[nt] = a.wq + row * KB + 16 * g;
    bs[nt] = a.ws + row * SB + g;
  }
  // activation rows: W13 the token of the slot (padding rows read row 0; a GEMM never
  // mixes rows and padding outputs are dropped), W2 the align row
  const uint8_t* aqp[MT];
  const uint8_t* asp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = (wm * MT + mt) * 16 + j;
    size_t row;
    if constexpr (W13) {
      const int slot = a.slots[r0 + m];
      row = (unsigned)slot < (unsigned)a.nslot ? (size_t)(slot / a.k) : 0;
    } else {
      row = (size_t)(r0 + m);
    }
    aqp[mt] = a.aq + row * KB + 16 * g;
    asp[mt] = a.as + row * SB + g;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Frag {
    uint4 aq[MT], bq[NT];
    uint32_t as[MT], bs[NT];
  };
  auto load = [&](int st, Frag& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.aq[mt] = *reinterpret_cast<const uint4*>(aqp[mt] + st * (kMxBK / 2));
      f.as[mt] = asp[mt][st * (kMxBK / 32)];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f.bq[nt] = *reinterpret_cast<const uint4*>(bq[nt] + st * (kMxBK / 2));
      f.bs[nt] = bs[nt][st * (kMxBK / 32)];
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const i32x8 av = {(int)f.aq[mt].x, (int)f.aq[mt].y, (int)f.aq[mt].z, (int)f.aq[mt].w, 0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const i32x8 bv = {(int)f.bq[nt].x, (int)f.bq[nt].y, (int)f.bq[nt].z, (int)f.bq[nt].w, 0, 0, 0, 0};
        // operand formats 4 = FP4 (E2M1); scales: E8M0 in byte 0 of each lane's word
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bv, acc[mt][nt], 4, 4, 0, (int)f.as[mt], 0, (int)f.bs[nt]);
      }
    }
  };
  const int steps = a.K / kMxBK;
  Frag f0, f1;
  load(0, f0);
  int st = 0;
  for (; st + 2 <= steps; st += 2) {
    load(st + 1, f1);
    mma(f0);
    if (st + 2 < steps) load(st + 2, f0);
    mma(f1);
  }
  if (st < steps) mma(f0);

  // epilogue: lane holds rows 4 g + q of each 16-row tile, column j
#pragma unroll
  for (int nt = 0; nt < (W13 ? NT / 2 : NT); ++nt) {
    const int n = wrow(nt) + j;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = (wm * MT + mt) * 16 + 4 * g + q;
        if constexpr (W13) {
          const float gate = acc[mt][nt][q], up = acc[mt][nt + NT / 2][q];
          a.h_out[(size_t)(r0 + m) * a.I + n] = silu(gate) * up;
        } else {
          const int slot = a.slots[r0 + m];
          if ((unsigned)slot < (unsigned)a.nslot)
            a.o_out[(size_t)slot * a.H + n] = acc[mt][nt][q] * a.topk_w[slot];
        }
      }
    }
  }
}

typedef void (*MxGemmFn)(MxArgs);

template <bool W13>
static MxGemmFn pick_mx(int bm) {
  switch (bm) {
    case 16: return mx_gemm_kernel<16, W13>;
    case 32: return mx_gemm_kernel<32, W13>;
    case 64: return mx_gemm_kernel<64, W13>;
    case 128: return mx_gemm_kernel<128, W13>;
  }
  return nullptr;
}

hipError_t launch_mx_quant(const void* in, bool bf16, int rows, int K, const int32_t* nrows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long n = (long)rows * (K / 32);
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kMxThreads - 1) / kMxThreads);
  if (bf16) hipLaunchKernelGGL(mx_quant_kernel<true>, dim3(grid), dim3(kMxThreads), 0, s, in, rows, K, nrows, codes, scales);
  else hipLaunchKernelGGL(mx_quant_kernel<false>, dim3(grid), dim3(kMxThreads), 0, s, in, rows, K, nrows, codes, scales);
  return hipGetLastError();
}

// The kept tier's W4A4 work of one forward stage: HMOE_STAGE_ROUTE quantises x,
// HMOE_STAGE_W13 runs the W13 GEMM and quantises h, HMOE_STAGE_W2 runs the W2 GEMM.
hipError_t launch_w4a4(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                       void* scratch, int stage, hipStream_t s) {
  if (L.E4 == 0 || M <= 0) return hipSuccess;
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + P.mx_xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + P.mx_xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(base + P.mx_hq);
  uint8_t* hs = reinterpret_cast<uint8_t*>(base + P.mx_hs);
  float* h32 = reinterpret_cast<float*>(base + P.mx_h32);
  const int32_t* npad = reinterpret_cast<const int32_t*>(base + P.a_npad[0]);
  if (stage == HMOE_STAGE_ROUTE) return launch_mx_quant(x, true, M, L.H, nullptr, xq, xs, s);
  const int bm = L.block_m;
  const int ns = M * L.k;
  const int cap = ns + (L.E4 < ns ? L.E4 : ns) * (bm - 1);
  MxArgs a{};
  a.k = L.k;
  a.nslot = ns;
  a.slots = reinterpret_cast<const int32_t*>(base + P.a_slots[0]);
  a.bexp = reinterpret_cast<const int32_t*>(base + P.a_bexp[0]);
  a.npad = npad;
  a.nblk = (cap + bm - 1) / bm;
  a.E4 = L.E4;
  a.I = L.I;
  a.H = L.H;
  if (stage == HMOE_STAGE_W13) {
    a.wq = W.kept_w13_q; a.ws = W.kept_w13_s;
    a.rows_w = 2 * L.I; a.K = L.H;
    a.aq = xq; a.as = xs;
    a.h_out = h32;
    MxGemmFn fn = pick_mx<true>(bm);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(L.I / (kMxBN / 2), a.nblk), dim3(kMxThreads), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_mx_quant(h32, false, L.cap[0], L.I, npad, hq, hs, s);
  }
  if (stage == HMOE_STAGE_W2) {
    a.wq = W.kept_w2_q; a.ws = W.kept_w2_s;
    a.rows_w = L.H; a.K = L.I;
    a.aq = hq; a.as = hs;
    a.o_out = reinterpret_cast<float*>(base + P.o_pre);
    a.topk_w = reinterpret_cast<const float*>(base + P.topk_w);
    MxGemmFn fn = pick_mx<false>(bm);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(L.H / kMxBN, a.nblk), dim3(kMxThreads), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace hmoe
