// Routing kernels: softmax top-k renormalised (one 64-lane wave per token), and the
// decode variant that also writes each (token, top-k) slot's pass record and the
// expert tier map (the direct top-k addressing of the decode path,
// local-inference-lab/vllm PR #92, "How it works").
#include <math.h>

#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

constexpr int kRouteWaves = 4;  // tokens per block of the general route kernel

// Per-wave LDS of the top-k: the k selected (key, id, logit) in id order, then in rank
// order.
struct TopkLds {
  __attribute__((aligned(16))) uint32_t key[kMaxTopK];
  __attribute__((aligned(16))) int32_t id[kMaxTopK];
  float v[kMaxTopK];
  int32_t rid[kMaxTopK];
  float rv[kMaxTopK];
};

// order-preserving unsigned image of a float (NaN excluded): larger float, larger key
__device__ __forceinline__ uint32_t order_key(float t) {
  const uint32_t b = __float_as_uint(t);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Top-k of one token's logits row by one wave; each lane holds NV >= E / 64 logits
// (expert lane + 64 i). Experts rank by logit, descending, ties to the lower id; NaN
// ranks below -inf and -0 ties with +0. The k-th largest logit comes from a bitwise search over
// its order-preserving 32-bit key (one ballot count per bit); the keys above it and,
// by ascending id, as many of those equal to it as needed make the selection, which is
// ranked by pairwise comparison in LDS. Lane j < k ends with the j-th selection in
// (sel_v, sel_id). Weights: softmax over the selected logits, in fp64, rounded once to
// fp32.
template <int NV>
__device__ __forceinline__ int route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, TopkLds& tl) {
  float v[NV];
  uint32_t u[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    float t = (e < E) ? row[e] : -INFINITY;
    const bool nan = t != t;
    t = nan ? -INFINITY : t;       // a NaN logit weighs as -inf in the softmax
    t = (t == 0.0f) ? 0.0f : t;    // -0 ties with +0
    v[i] = t;
    // keys: -inf is 0x007FFFFF, NaN 1 (below every number), padding 0 (last)
    u[i] = (e < E) ? (nan ? 1u : order_key(t)) : 0u;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  // tau = the largest key with at least k keys >= tau (the k-th largest key), two bits
  // per step: the counts at the three candidate digits are independent
  uint32_t tau = 0;
#pragma unroll
  for (int bit = 30; bit >= 0; bit -= 2) {
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      n1 += __popcll(__ballot(u[i] >= (tau | (1u << bit))));
      n2 += __popcll(__ballot(u[i] >= (tau | (2u << bit))));
      n3 += __popcll(__ballot(u[i] >= (tau | (3u << bit))));
    }
    tau |= (uint32_t)((n1 >= k) + (n2 >= k) + (n3 >= k)) << bit;
  }
  int above = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) above += __popcll(__ballot(u[i] > tau));
  const int need = k - above;  // ties taken, lowest ids first
  int ties_before = 0, placed = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint64_t tie = __ballot(u[i] == tau);
    const bool sel = u[i] > tau || (u[i] == tau && ties_before + (int)__popcll(tie & lt) < need);
    const uint64_t sb = __ballot(sel);
    if (sel) {
      const int pos = placed + __popcll(sb & lt);
      tl.key[pos] = u[i];
      tl.id[pos] = lane + kWave * i;
      tl.v[pos] = v[i];
    }
    placed += __popcll(sb);
    ties_before += __popcll(tie);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    const uint32_t uj = tl.key[lane];
    const int ej = tl.id[lane];
    const float vj = tl.v[lane];
    // the whole list at once (same address in every lane: broadcast reads)
    uint32_t km[kMaxTopK];
    int32_t im[kMaxTopK];
#pragma unroll
    for (int q = 0; q < kMaxTopK / 4; ++q) {
      const uint4 kk = reinterpret_cast<const uint4*>(tl.key)[q];
      const int4 ii = reinterpret_cast<const int4*>(tl.id)[q];
      km[4 * q] = kk.x; km[4 * q + 1] = kk.y; km[4 * q + 2] = kk.z; km[4 * q + 3] = kk.w;
      im[4 * q] = ii.x; im[4 * q + 1] = ii.y; im[4 * q + 2] = ii.z; im[4 * q + 3] = ii.w;
    }
    int rank = 0;
#pragma unroll
    for (int m = 0; m < kMaxTopK; ++m)
      rank += (m < k && (km[m] > uj || (km[m] == uj && im[m] < ej))) ? 1 : 0;
    tl.rid[rank] = ej;
    tl.rv[rank] = vj;
  }
  __builtin_amdgcn_wave_barrier();
  const float sel_v = lane < k ? tl.rv[lane] : 0.0f;
  const int sel_id = lane < k ? tl.rid[lane] : 0;
  const float v0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(sel_v), 0));
  const double ex = (lane < k) ? exp((double)sel_v - (double)v0) : 0.0;
  double sum = ex;
  sum += xlane_d<32>(sum);
  sum += xlane_d<16>(sum);
  sum += xlane_d<8>(sum);
  sum += xlane_d<4>(sum);
  sum += xlane_d<2>(sum);
  sum += xlane_d<1>(sum);
  if (lane < k) {
    ids_out[lane] = sel_id;
    w_out[lane] = (float)(ex / sum);
  }
  return sel_id;
}

// route_token with NV = the smallest power of two covering E / 64 logits per lane; returns
// lane j's selection (j < k)
__device__ __forceinline__ int route_token_any(const float* __restrict__ row, int E, int k,
                                               int lane, int32_t* __restrict__ ids_out,
                                               float* __restrict__ w_out, TopkLds& tl) {
  if (E <= 64) return route_token<1>(row, E, k, lane, ids_out, w_out, tl);
  if (E <= 128) return route_token<2>(row, E, k, lane, ids_out, w_out, tl);
  if (E <= 256) return route_token<4>(row, E, k, lane, ids_out, w_out, tl);
  if (E <= 512) return route_token<8>(row, E, k, lane, ids_out, w_out, tl);
  return route_token<16>(row, E, k, lane, ids_out, w_out, tl);
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w) {
  __shared__ TopkLds tl[kRouteWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  route_token_any(logits + (size_t)t * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k,
                  tl[threadIdx.x >> 6]);
}

// Tier code of expert e (bit 16: NF3 tier; low 16 bits: index within its tier).
__device__ __forceinline__ int tier_code(const TierMask& m, int e) {
  int below = 0;
  for (int i = 0; i < (e >> 5); ++i) below += __popc(m.w[i]);
  const uint32_t w = m.w[e >> 5];
  below += __popc(w & ((1u << (e & 31)) - 1u));
  return ((w >> (e & 31)) & 1u) ? ((1 << 16) | below) : (e - below);
}

struct RouteDecodeArgs {
  const float* logits;
  int M, E, k;
  int32_t* ids;
  float* w;
  int32_t* expert_tier;
  int32_t* pass;  // [M * k, 4]: slot, tier code, token, e (slot order)
};

constexpr int kGroupThreads = kDecodeMaxM * kWave;  // one wave per decode token
constexpr int kGroupWaves = kDecodeMaxM;

// Decode routing (M <= 8): one wave per token; each slot's pass record (the direct
// top-k addressing of the decode GEMVs) and the expert tier map. No block-wide step:
// the distinct-expert grouping is built later, off the critical path, by the combine.
__global__ __launch_bounds__(kGroupThreads) void route_decode_kernel(RouteDecodeArgs a, TierMask tm) {
  __shared__ TopkLds s_topk[kGroupWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  if (wave < a.M) {
    const int e = route_token_any(a.logits + (size_t)wave * a.E, a.E, a.k, lane,
                                  a.ids + wave * a.k, a.w + wave * a.k, s_topk[wave]);
    if (lane < a.k) {
      const int s = wave * a.k + lane;
      reinterpret_cast<int4*>(a.pass)[s] = make_int4(s, tier_code(tm, e), wave, e);
    }
  }
  for (int e = threadIdx.x; e < a.E; e += kGroupThreads) a.expert_tier[e] = tier_code(tm, e);
}

hipError_t launch_route(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int blocks = (M + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kRouteWaves * kWave), 0, s, logits, M, E,
                     k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_group(const Layer& L, const float* logits, int M, void* scratch,
                              hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  RouteDecodeArgs a;
  a.logits = logits;
  a.M = M;
  a.E = L.E;
  a.k = L.k;
  a.ids = reinterpret_cast<int32_t*>(base + L.plan.topk_ids);
  a.w = reinterpret_cast<float*>(base + L.plan.topk_w);
  a.expert_tier = reinterpret_cast<int32_t*>(base + L.plan.expert_tier);
  a.pass = reinterpret_cast<int32_t*>(base + L.plan.d_pass);
  hipLaunchKernelGGL(route_decode_kernel, dim3(1), dim3(kGroupThreads), 0, s, a, make_tier_mask(L));
  return hipGetLastError();
}

TierMask make_tier_mask(const Layer& L) {
  TierMask m;
  for (int i = 0; i < kMaxExperts / 32; ++i) m.w[i] = L.nf3_mask[i];
  return m;
}

}  // namespace hmoe
