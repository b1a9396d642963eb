// Routing kernels: softmax top-k renormalised (one 64-lane wave per token), and the
// decode variant that also writes the expert tier map and groups the M <= 8 tokens'
// slots by distinct touched expert (the direct top-k addressing of the decode path,
// local-inference-lab/vllm PR #92, "How it works").
#include <math.h>

#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

constexpr int kRouteWaves = 4;  // tokens per block of the general route kernel

// Top-k of one token's logits row by one wave. Experts rank by logit, descending,
// ties to the lower id. Lane j < k ends with the j-th selection in (sel_v, sel_id).
// Weights: softmax over the selected logits, in fp64, rounded once to fp32.
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, int32_t* lds_ids) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? row[e] : -INFINITY;
    if (v[i] != v[i]) v[i] = -INFINITY;  // NaN ranks below every number: a total order
  }
  uint32_t taken = 0;
  float sel_v = 0.0f;
  int sel_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + kWave * i;
      const bool ok = (e < E) && !((taken >> i) & 1u);
      // ids grow with i inside a lane, so a strict > keeps the lowest id on ties
      if (ok && (v[i] > bv || bi == 0x7FFFFFFF)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      sel_v = bv;
      sel_id = bi;
    }
  }
  const float v0 = __shfl(sel_v, 0);
  const double ex = (lane < k) ? exp((double)sel_v - (double)v0) : 0.0;
  double sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids_out[lane] = sel_id;
    w_out[lane] = (float)(ex / sum);
    if (lds_ids) lds_ids[lane] = sel_id;
  }
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  route_token(logits + (size_t)t * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k, nullptr);
}

// Tier of expert e and its position in its tier's ascending-id storage.
__device__ __forceinline__ int32_t tier_code(const TierMask& m, int e) {
  int below = 0;
  const int wd = e >> 5;
  for (int i = 0; i < wd; ++i) below += __popc(m.w[i]);
  below += __popc(m.w[wd] & ((1u << (e & 31)) - 1u));
  const bool nf3 = (m.w[wd] >> (e & 31)) & 1u;
  return nf3 ? ((1 << 16) | below) : (e - below);
}

struct RouteGroupArgs {
  const float* logits;
  int M, E, k, E4;
  int32_t* ids;
  float* w;
  int32_t* expert_tier;
  int32_t* counts;     // [2]
  int32_t* experts;    // [max_distinct]
  int32_t* nslots;     // [max_distinct]
  int32_t* slots;      // [max_distinct, 8]
};

constexpr int kGroupThreads = kDecodeMaxM * kWave;  // one wave per decode token

__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(RouteGroupArgs a, TierMask tm) {
  __shared__ int32_t s_ids[kDecodeMaxM * kMaxTopK];
  __shared__ uint32_t s_mask[kMaxExperts][4];   // slot bit masks (M * k <= 128 slots)
  __shared__ int32_t s_order[kMaxExperts];      // (tier, local) position -> expert or -1
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  if (wave < a.M)
    route_token(a.logits + (size_t)wave * a.E, a.E, a.k, lane, a.ids + wave * a.k,
                a.w + wave * a.k, s_ids + wave * a.k);
  for (int e = threadIdx.x; e < a.E; e += kGroupThreads) {
    a.expert_tier[e] = tier_code(tm, e);
    s_mask[e][0] = s_mask[e][1] = s_mask[e][2] = s_mask[e][3] = 0u;
  }
  __syncthreads();
  const int nslot = a.M * a.k;
  for (int s = threadIdx.x; s < nslot; s += kGroupThreads) {
    const int e = s_ids[s];
    if ((unsigned)e < (unsigned)a.E) atomicOr(&s_mask[e][s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kGroupThreads) {
    const int32_t tc = tier_code(tm, e);
    const int pos = (tc >> 16) ? a.E4 + (tc & 0xFFFF) : tc;
    const bool touched = (s_mask[e][0] | s_mask[e][1] | s_mask[e][2] | s_mask[e][3]) != 0u;
    s_order[pos] = touched ? e : -1;
  }
  __syncthreads();
  if (wave == 0) {
    int running = 0;
    int kept_distinct = 0;
    for (int base = 0; base < a.E; base += kWave) {
      const int pos = base + lane;
      const int e = (pos < a.E) ? s_order[pos] : -1;
      const bool f = e >= 0;
      const uint64_t b = __ballot(f);
      const int d = running + __popcll(b & ((1ull << lane) - 1ull));
      if (f) {
        a.experts[d] = e;
        int n = 0;
        for (int wd = 0; wd < 4; ++wd) {
          uint32_t m = s_mask[e][wd];
          while (m) {
            const int bit = __ffs(m) - 1;
            m &= m - 1u;
            if (n < kDecodeMaxM) a.slots[d * kDecodeMaxM + n] = wd * 32 + bit;
            ++n;
          }
        }
        a.nslots[d] = n < kDecodeMaxM ? n : kDecodeMaxM;
      }
      const int cnt = __popcll(b);
      if (base + kWave <= a.E4) {
        kept_distinct += cnt;
      } else if (base < a.E4) {
        kept_distinct += __popcll(b & ((1ull << (a.E4 - base)) - 1ull));
      }
      running += cnt;
    }
    if (lane == 0) {
      a.counts[0] = running;
      a.counts[1] = kept_distinct;
    }
  }
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
  RouteGroupArgs a;
  a.logits = logits;
  a.M = M;
  a.E = L.E;
  a.k = L.k;
  a.E4 = L.E4;
  a.ids = reinterpret_cast<int32_t*>(base + L.plan.topk_ids);
  a.w = reinterpret_cast<float*>(base + L.plan.topk_w);
  a.expert_tier = reinterpret_cast<int32_t*>(base + L.plan.expert_tier);
  a.counts = reinterpret_cast<int32_t*>(base + L.plan.d_counts);
  a.experts = reinterpret_cast<int32_t*>(base + L.plan.d_experts);
  a.nslots = reinterpret_cast<int32_t*>(base + L.plan.d_nslots);
  a.slots = reinterpret_cast<int32_t*>(base + L.plan.d_slots);
  hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, a, make_tier_mask(L));
  return hipGetLastError();
}

TierMask make_tier_mask(const Layer& L) {
  TierMask m;
  for (int i = 0; i < kMaxExperts / 32; ++i) m.w[i] = L.nf3_mask[i];
  return m;
}

}  // namespace hmoe
