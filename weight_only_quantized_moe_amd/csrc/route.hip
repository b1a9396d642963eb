// Routing kernels: softmax top-k renormalised (one 64-lane wave per token), and the
// decode variant that also writes the expert tier map and groups the M <= 8 tokens'
// slots by distinct touched expert (the direct top-k addressing of the decode path,
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
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, int32_t* lds_ids,
                                            TopkLds& tl) {
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
    const bool sel = u[i] > tau || (u[i] == tau && ties_before + __popcll(tie & lt) < need);
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
    if (lds_ids) lds_ids[lane] = sel_id;
  }
}

// route_token with NV = the smallest power of two covering E / 64 logits per lane
__device__ __forceinline__ void route_token_any(const float* __restrict__ row, int E, int k,
                                                int lane, int32_t* __restrict__ ids_out,
                                                float* __restrict__ w_out, int32_t* lds_ids,
                                                TopkLds& tl) {
  if (E <= 64) route_token<1>(row, E, k, lane, ids_out, w_out, lds_ids, tl);
  else if (E <= 128) route_token<2>(row, E, k, lane, ids_out, w_out, lds_ids, tl);
  else if (E <= 256) route_token<4>(row, E, k, lane, ids_out, w_out, lds_ids, tl);
  else if (E <= 512) route_token<8>(row, E, k, lane, ids_out, w_out, lds_ids, tl);
  else route_token<16>(row, E, k, lane, ids_out, w_out, lds_ids, tl);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then each row's total carried into the rows above (DPP row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w) {
  __shared__ TopkLds tl[kRouteWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  route_token_any(logits + (size_t)t * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k,
                  nullptr, tl[threadIdx.x >> 6]);
}

// Number of NF3-tier experts with id below 64 * chunk (the mask holds one bit per
// expert, two words per 64-expert chunk).
__device__ __forceinline__ int nf3_below_chunk(const TierMask& m, int chunk) {
  int below = 0;
  for (int i = 0; i < 2 * chunk; ++i) below += __popc(m.w[i]);
  return below;
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
  int32_t* recs;       // [max_distinct, 16]: e, tier code, n, 0, slots[8], 0 x 4
  int32_t* pass;       // [M * k, 4]: slot, tier code, token, e (grouped by expert)
};

constexpr int kGroupThreads = kDecodeMaxM * kWave;  // one wave per decode token
constexpr int kGroupWaves = kDecodeMaxM;

__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(RouteGroupArgs a, TierMask tm) {
  __shared__ int32_t s_ids[kDecodeMaxM * kMaxTopK];
  __shared__ TopkLds s_topk[kGroupWaves];
  __shared__ uint32_t s_mask[kMaxExperts][4];   // slot bit masks (M * k <= 128 slots)
  __shared__ int32_t s_order[kMaxExperts];      // (tier, local) position -> expert or -1
  __shared__ int32_t s_pos[kMaxExperts];        // expert -> (tier, local) position
  __shared__ int32_t s_d[kMaxExperts];          // expert -> group index
  __shared__ int32_t s_tc[kMaxExperts];         // expert -> tier code
  __shared__ int32_t s_poff[kMaxExperts];       // expert -> first pass record
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  if (wave < a.M)
    route_token_any(a.logits + (size_t)wave * a.E, a.E, a.k, lane, a.ids + wave * a.k,
                    a.w + wave * a.k, s_ids + wave * a.k, s_topk[wave]);
  // tier map: one wave per 64-expert chunk, ranks by ballot
  for (int chunk = wave; chunk * kWave < a.E; chunk += kGroupWaves) {
    const int e = chunk * kWave + lane;
    const bool in = e < a.E;
    const bool nf3 = in && ((tm.w[e >> 5] >> (e & 31)) & 1u);
    const uint64_t b = __ballot(nf3);
    const int nf3_below = nf3_below_chunk(tm, chunk) + __popcll(b & lt);
    if (in) {
      const int32_t tc = nf3 ? ((1 << 16) | nf3_below) : (e - nf3_below);
      a.expert_tier[e] = tc;
      s_tc[e] = tc;
      s_pos[e] = nf3 ? a.E4 + nf3_below : e - nf3_below;
      s_mask[e][0] = s_mask[e][1] = s_mask[e][2] = s_mask[e][3] = 0u;
    }
  }
  __syncthreads();
  const int nslot = a.M * a.k;
  for (int s = threadIdx.x; s < nslot; s += kGroupThreads) {
    const int e = s_ids[s];
    if ((unsigned)e < (unsigned)a.E) atomicOr(&s_mask[e][s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kGroupThreads) {
    const bool touched = (s_mask[e][0] | s_mask[e][1] | s_mask[e][2] | s_mask[e][3]) != 0u;
    s_order[s_pos[e]] = touched ? e : -1;
  }
  __syncthreads();
  if (wave == 0) {
    int running = 0, running_slots = 0;
    int kept_distinct = 0;
    for (int base = 0; base < a.E; base += kWave) {
      const int pos = base + lane;
      const int e = (pos < a.E) ? s_order[pos] : -1;
      const bool f = e >= 0;
      const uint64_t b = __ballot(f);
      const int n = f ? __popc(s_mask[e][0]) + __popc(s_mask[e][1]) + __popc(s_mask[e][2]) +
                            __popc(s_mask[e][3])
                      : 0;
      // inclusive scan of the slot counts over the wave: first pass record of each
      const int incl = wave_incl_scan(n);
      if (f) {
        const int d = running + __popcll(b & lt);
        s_d[e] = d;
        s_poff[e] = running_slots + incl - n;
        a.experts[d] = e;
        a.nslots[d] = n < kDecodeMaxM ? n : kDecodeMaxM;
        int4* rec = reinterpret_cast<int4*>(a.recs + d * kGroupRec);
        rec[0] = make_int4(e, s_tc[e], n < kDecodeMaxM ? n : kDecodeMaxM, 0);
        rec[3] = make_int4(0, 0, 0, 0);
      }
      const int cnt = __popcll(b);
      if (base + kWave <= a.E4) kept_distinct += cnt;
      else if (base < a.E4) kept_distinct += __popcll(b & ((1ull << (a.E4 - base)) - 1ull));
      running += cnt;
      running_slots += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) {
      a.counts[0] = running;
      a.counts[1] = kept_distinct;
    }
  }
  __syncthreads();
  // each slot lands at its rank among its expert's slots (ascending slot order)
  for (int s = threadIdx.x; s < nslot; s += kGroupThreads) {
    const int e = s_ids[s];
    if ((unsigned)e >= (unsigned)a.E) continue;
    int rank = 0;
    for (int wd = 0; wd < (s >> 5); ++wd) rank += __popc(s_mask[e][wd]);
    rank += __popc(s_mask[e][s >> 5] & ((1u << (s & 31)) - 1u));
    if (rank < kDecodeMaxM) {
      a.slots[s_d[e] * kDecodeMaxM + rank] = s;
      a.recs[s_d[e] * kGroupRec + 4 + rank] = s;
    }
    const int p = s_poff[e] + rank;
    if (p < nslot)
      reinterpret_cast<int4*>(a.pass)[p] = make_int4(s, s_tc[e], s / a.k, e);
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
  a.recs = reinterpret_cast<int32_t*>(base + L.plan.d_recs);
  a.pass = reinterpret_cast<int32_t*>(base + L.plan.d_pass);
  hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, a, make_tier_mask(L));
  return hipGetLastError();
}

TierMask make_tier_mask(const Layer& L) {
  TierMask m;
  for (int i = 0; i < kMaxExperts / 32; ++i) m.w[i] = L.nf3_mask[i];
  return m;
}

}  // namespace hmoe
