// Routing kernels: softmax top-k renormalised (one 64-lane wave per token), and the
// decode variant that also writes each (token, top-k) slot's pass record and the
// expert tier map (the direct top-k addressing of the decode path,
// local-inference-lab/vllm PR #92, "How it works").
#include "route_common.h"

namespace hmoe {

constexpr int kRouteWaves = 4;  // tokens per block of the general route kernel

// route_select of one token, writing its k ids and weights
__device__ __forceinline__ int route_token_any(const float* __restrict__ row, int E, int k,
                                               int lane, int32_t* __restrict__ ids_out,
                                               float* __restrict__ w_out) {
  float w;
  const int id = route_select_any(row, E, k, lane, &w);
  if (lane < k) {
    ids_out[lane] = id;
    w_out[lane] = w;
  }
  return id;
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  route_token_any(logits + (size_t)t * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k);
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
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  if (wave < a.M) {
    const int e = route_token_any(a.logits + (size_t)wave * a.E, a.E, a.k, lane,
                                  a.ids + wave * a.k, a.w + wave * a.k);
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
