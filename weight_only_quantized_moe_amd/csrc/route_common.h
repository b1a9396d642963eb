// Softmax top-k routing of one token by one 64-lane wave, shared by the routing
// kernels and the single-launch decode kernel (local-inference-lab/vllm PR #92, "How it
// works": the M <= 8 path is addressed directly by the top-k result).
#pragma once

#include <math.h>

#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

// order-preserving unsigned image of a float (NaN excluded): larger float, larger key
__device__ __forceinline__ uint32_t order_key(float t) {
  const uint32_t b = __float_as_uint(t);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// the float of a key (the inverse of order_key); the NaN key 1 and padding 0 give -inf
__device__ __forceinline__ float key_value(uint32_t key) {
  if (key <= 1u) return -INFINITY;
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// the lane's share of one token's logits row: expert lane + 64 i in slot i (slots past
// E are not loaded). Split from route_rank so that a kernel can request the row early.
template <int NV>
__device__ __forceinline__ void route_fetch(const float* __restrict__ row, int E, int lane,
                                            float (&x)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    x[i] = e < E ? row[e] : 0.0f;
  }
}

// Top-k of T tokens' logits by one wave (each lane holds NV >= E / 64 of each row, from
// route_fetch), the tokens' steps interleaved so that their dependency chains overlap.
// Experts rank by logit, descending, ties to the lower id; NaN ranks below -inf and -0
// ties with +0. Each of the k rounds takes the wave's largest order-preserving 32-bit key
// (lane maxima, then a butterfly max), the lowest expert id holding it (one ballot per
// slot), and clears that key, so round r yields rank r. Lane j < k gets the j-th
// selection of token t in sel[t] and its weight in w[t] (lanes >= k: 0). Weights: softmax
// over the selected logits, in fp64, rounded once to fp32. Every token takes the same
// operations whatever T is, so the results do not depend on T.
template <int NV, int T>
__device__ __forceinline__ void route_rank_n(const float (&x)[T][NV], int E, int k, int lane,
                                             int (&sel)[T], float (&w)[T]) {
  uint32_t u[T][NV];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      float v = x[t][i];
      const bool nan = v != v;
      v = (v == 0.0f) ? 0.0f : v;    // -0 ties with +0
      // keys: -inf is 0x007FFFFF, NaN 1 (below every number), padding 0 (never chosen: k <= E)
      u[t][i] = (e < E) ? (nan ? 1u : order_key(v)) : 0u;
    }
  uint32_t sel_key[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    sel[t] = 0;
    sel_key[t] = 0u;
  }
  for (int r = 0; r < k; ++r) {
    uint32_t m[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      m[t] = u[t][0];
#pragma unroll
      for (int i = 1; i < NV; ++i) m[t] = max(m[t], u[t][i]);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<32>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<16>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<8>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<4>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<2>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) m[t] = max(m[t], xlane_u32<1>(m[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) {
      m[t] = __builtin_amdgcn_readfirstlane(m[t]);
      // the lowest id with key m: slots hold ids 64 i .. 64 i + 63, so the first slot
      // with a match and its lowest matching lane
      int id = -1;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const uint64_t b = __ballot(u[t][i] == m[t]);
        if (id < 0 && b != 0ull) id = kWave * i + (int)__builtin_ctzll(b);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (id == kWave * i + lane) u[t][i] = 0u;
      if (lane == r) {
        sel[t] = id;
        sel_key[t] = m[t];
      }
    }
  }
  double ex[T], sum[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float sel_v = key_value(sel_key[t]);
    const float v0 =
        __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(sel_v), 0));
    ex[t] = (lane < k) ? exp((double)sel_v - (double)v0) : 0.0;
    sum[t] = ex[t];
  }
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<32>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<16>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<8>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<4>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<2>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) sum[t] += xlane_d<1>(sum[t]);
#pragma unroll
  for (int t = 0; t < T; ++t) w[t] = lane < k ? (float)(ex[t] / sum[t]) : 0.0f;
}

// route_rank_n of one token: lane j < k returns the j-th selection and writes its weight
// to *w_lane
template <int NV>
__device__ __forceinline__ int route_rank(const float (&x)[NV], int E, int k, int lane,
                                          float* w_lane) {
  const float (&x1)[1][NV] = *reinterpret_cast<const float (*)[1][NV]>(&x);
  int sel[1];
  float w[1];
  route_rank_n<NV, 1>(x1, E, k, lane, sel, w);
  *w_lane = w[0];
  return sel[0];
}

template <int NV>
__device__ __forceinline__ int route_select(const float* __restrict__ row, int E, int k, int lane,
                                             float* w_lane) {
  float x[NV];
  route_fetch<NV>(row, E, lane, x);
  return route_rank<NV>(x, E, k, lane, w_lane);
}

// route_select with NV = the smallest power of two covering E / 64 logits per lane
__device__ __forceinline__ int route_select_any(const float* __restrict__ row, int E, int k,
                                                int lane, float* w_lane) {
  if (E <= 64) return route_select<1>(row, E, k, lane, w_lane);
  if (E <= 128) return route_select<2>(row, E, k, lane, w_lane);
  if (E <= 256) return route_select<4>(row, E, k, lane, w_lane);
  if (E <= 512) return route_select<8>(row, E, k, lane, w_lane);
  return route_select<16>(row, E, k, lane, w_lane);
}

// Tier code of expert e (bit 16: NF3 tier; low 16 bits: index within its tier).
__device__ __forceinline__ int tier_code(const TierMask& m, int e) {
  int below = 0;
  for (int i = 0; i < (e >> 5); ++i) below += __popc(m.w[i]);
  const uint32_t w = m.w[e >> 5];
  below += __popc(w & ((1u << (e & 31)) - 1u));
  return ((w >> (e & 31)) & 1u) ? ((1 << 16) | below) : (e - below);
}

}  // namespace hmoe
