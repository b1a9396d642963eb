// W4A4 kept tier (an MXFP4 kept tier with MXFP4 activations): the activation quantiser
// and the grouped GEMM on gfx950's MX-scaled matrix cores. vllm-project/vllm PR #42428,
// "What's in this PR", places the W4A16 path beside W4A4 backends, whose activations are
// 4-bit too; here each kept-tier matmul input (x before W13, h before W2) is rounded to
// MXFP4 along K in blocks of 32 (OCP MX v1.0 conversion: shared exponent floor(log2
// amax) - 2, elements rounded to E2M1 nearest-even, saturating at 6), and both operands
// go to v_mfma_scale_f32_16x16x128_f8f6f4 as they are stored: 16-byte fragments of 32
// E2M1 codes plus one E8M0 byte per lane, no decode, no LDS.
#include "mx_gemm.h"

namespace hmoe {

constexpr int kMxQuantThreads = 256;

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
__global__ __launch_bounds__(kMxQuantThreads) void mx_quant_kernel(const void* __restrict__ in, int rows,
                                                              int K, const int32_t* __restrict__ nrows,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const long i = (long)blockIdx.x * kMxQuantThreads + threadIdx.x;
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

hipError_t launch_mx_quant(const void* in, bool bf16, int rows, int K, const int32_t* nrows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long n = (long)rows * (K / 32);
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kMxQuantThreads - 1) / kMxQuantThreads);
  if (bf16) hipLaunchKernelGGL(mx_quant_kernel<true>, dim3(grid), dim3(kMxQuantThreads), 0, s, in, rows, K, nrows, codes, scales);
  else hipLaunchKernelGGL(mx_quant_kernel<false>, dim3(grid), dim3(kMxQuantThreads), 0, s, in, rows, K, nrows, codes, scales);
  return hipGetLastError();
}

MxArgs mx_args(const Layer& L, const hmoe_weights& W, int M, void* scratch, int stage) {
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  const int bm = L.block_m;
  const int ns = M * L.k;
  const int cap = ns + (L.E4 < ns ? L.E4 : ns) * (bm - 1);
  MxArgs a{};
  a.k = L.k;
  a.nslot = ns;
  a.slots = reinterpret_cast<const int32_t*>(base + P.a_slots[0]);
  a.bexp = reinterpret_cast<const int32_t*>(base + P.a_bexp[0]);
  a.npad = reinterpret_cast<const int32_t*>(base + P.a_npad[0]);
  a.nblk = L.E4 > 0 ? (cap + bm - 1) / bm : 0;
  a.E4 = L.E4;
  a.I = L.I;
  a.H = L.H;
  a.topk_w = reinterpret_cast<const float*>(base + P.topk_w);
  a.row_fac = reinterpret_cast<float*>(base + P.pf_fac);  // the kept tier's rows [0, cap0)
  if (stage == HMOE_STAGE_W13) {
    a.wq = W.kept_w13_q; a.ws = W.kept_w13_s;
    a.rows_w = 2 * L.I; a.K = L.H;
    a.aq = reinterpret_cast<const uint8_t*>(base + P.mx_xq);
    a.as = reinterpret_cast<const uint8_t*>(base + P.mx_xs);
    a.h_out = reinterpret_cast<float*>(base + P.mx_h32);
  } else {
    a.wq = W.kept_w2_q; a.ws = W.kept_w2_s;
    a.rows_w = L.H; a.K = L.I;
    a.aq = reinterpret_cast<const uint8_t*>(base + P.mx_hq);
    a.as = reinterpret_cast<const uint8_t*>(base + P.mx_hs);
    a.o_out = reinterpret_cast<float*>(base + P.o_pre);
  }
  return a;
}

// The kept tier's W4A4 work around the shared GEMM launches: HMOE_STAGE_ROUTE rounds x to
// MXFP4, HMOE_STAGE_W13 rounds h (after the W13 GEMM) to MXFP4.
hipError_t launch_w4a4(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                       void* scratch, int stage, hipStream_t s) {
  (void)W;
  if (L.E4 == 0 || M <= 0) return hipSuccess;
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  if (stage == HMOE_STAGE_ROUTE)
    return launch_mx_quant(x, true, M, L.H, nullptr, reinterpret_cast<uint8_t*>(base + P.mx_xq),
                           reinterpret_cast<uint8_t*>(base + P.mx_xs), s);
  if (stage == HMOE_STAGE_W13)
    return launch_mx_quant(base + P.mx_h32, false, L.cap[0], L.I,
                           reinterpret_cast<const int32_t*>(base + P.a_npad[0]),
                           reinterpret_cast<uint8_t*>(base + P.mx_hq),
                           reinterpret_cast<uint8_t*>(base + P.mx_hs), s);
  return hipSuccess;
}

}  // namespace hmoe
