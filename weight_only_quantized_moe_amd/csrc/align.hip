// Per-tier align for the prefill path: the slots of each tier's experts grouped by
// tier-local expert (ascending local id = ascending global id inside the tier,
// local-inference-lab/vllm PR #104: compact tier-local storage), ascending slot order
// inside an expert, each expert's run padded with the sentinel M*k to a multiple of
// block_m, plus the block -> expert table and the padded offsets. One block of 1024
// threads: each of its 16 waves places one contiguous chunk of the slots, starting
// from per-wave, per-expert offsets, so the result is the stable order of a serial
// counting sort. Deterministic; no host read-back.
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
// slot ids each lane requests at once (16 steps of 64 slots): the counting and placing
// loops wait for one load latency per 16 steps, not per step
constexpr int kAlignBatch = 16;
// s_waitcnt operand waiting for LDS only (gfx9 fields: vmcnt 63, expcnt 7, lgkmcnt 0):
// the placement loop orders its position reads and counter updates in LDS but leaves
// its global stores of slot ids in flight
constexpr int kWaitLdsOnly = 0xC07F;

struct AlignArgs {
  const int32_t* ids;
  int nslot, E, bm;
  int32_t* expert_tier;
  int32_t* slots[2];
  int32_t* bexp[2];
  int32_t* eoff[2];
  int32_t* npad[2];
};

__device__ __forceinline__ int32_t tier_code_a(const TierMask& m, int e) {
  int below = 0;
  const int wd = e >> 5;
  for (int i = 0; i < wd; ++i) below += __popc(m.w[i]);
  below += __popc(m.w[wd] & ((1u << (e & 31)) - 1u));
  const bool nf3 = (m.w[wd] >> (e & 31)) & 1u;
  return nf3 ? ((1 << 16) | below) : (e - below);
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(AlignArgs a, TierMask tm) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts];
  __shared__ int32_t s_tc[kMaxExperts];
  __shared__ int32_t s_w[kAlignWaves][kMaxExperts];  // per-wave counts, then positions
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  // wave w places slots [w * chunk, (w + 1) * chunk), chunk a multiple of 64
  const int chunk = ((a.nslot + kAlignWaves * kWave - 1) / (kAlignWaves * kWave)) * kWave;
  const int c0 = min(wave * chunk, a.nslot), c1 = min(c0 + chunk, a.nslot);
  for (int e = tid; e < a.E; e += kAlignThreads) {
    const int32_t tc = tier_code_a(tm, e);
    s_tc[e] = tc;
    s_cnt[e] = 0;
    a.expert_tier[e] = tc;
  }
  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&s_w[0][0])[i] = 0;
  __syncthreads();
  for (int b0 = c0; b0 < c1; b0 += kAlignBatch * kWave) {
    int ev[kAlignBatch];
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      const int s = b0 + i * kWave + lane;
      ev[i] = s < c1 ? a.ids[s] : -1;
    }
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      const int e = ev[i];
      if ((unsigned)e < (unsigned)a.E) {  // ids outside [0, E) are dropped
        atomicAdd(&s_cnt[e], 1);
        atomicAdd(&s_w[wave][e], 1);
      }
    }
  }
  __syncthreads();
  // padded exclusive offsets, one wave per tier, experts in ascending id
  if (wave < 2) {
    int running = 0, n_in_tier = 0;
    for (int base = 0; base < a.E; base += kWave) {
      const int e = base + lane;
      const bool in = e < a.E && (s_tc[e] >> 16) == wave;
      n_in_tier += __popcll(__ballot(in));
      const int padded = in ? (s_cnt[e] + a.bm - 1) / a.bm * a.bm : 0;
      int incl = padded;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int excl = running + incl - padded;
      if (in) {
        s_off[e] = excl;
        a.eoff[wave][s_tc[e] & 0xFFFF] = excl;
      }
      running += __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
      // E_tier entries precede the terminal offset
      a.eoff[wave][n_in_tier] = running;
      a.npad[wave][0] = running;
    }
  }
  __syncthreads();
  // block -> expert table and sentinel padding, one thread per expert; the per-wave
  // counts become each wave's first position for that expert
  for (int e = tid; e < a.E; e += kAlignThreads) {
    const int t = s_tc[e] >> 16;
    const int loc = s_tc[e] & 0xFFFF;
    const int n = s_cnt[e];
    const int padded = (n + a.bm - 1) / a.bm * a.bm;
    const int off = s_off[e];
    for (int b = off / a.bm; b < (off + padded) / a.bm; ++b) a.bexp[t][b] = loc;
    for (int p = off + n; p < off + padded; ++p) a.slots[t][p] = a.nslot;
    int run = off;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = s_w[w][e];
      s_w[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  // real slots in ascending order inside each wave's chunk: 64 at a time, ranking
  // equal experts inside the step with ballots over the id bits
  int idbits = 1;
  while ((1 << idbits) < a.E) ++idbits;
  for (int b0 = c0; b0 < c1; b0 += kAlignBatch * kWave) {
    int ev[kAlignBatch];
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      const int s = b0 + i * kWave + lane;
      ev[i] = s < c1 ? a.ids[s] : -1;
    }
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      const int base = b0 + i * kWave;
      if (base >= c1) break;
      const int s = base + lane;
      const int e0 = ev[i];
      const bool valid = (unsigned)e0 < (unsigned)a.E;
      const int e = valid ? e0 : 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < idbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      const int cnt = __popcll(m);
      int pos = 0;
      if (valid) pos = s_w[wave][e] + rank;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
      if (valid) {
        a.slots[s_tc[e] >> 16][pos] = s;
        if (rank == cnt - 1) s_w[wave][e] += cnt;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
    }
  }
}

hipError_t launch_align(const Layer& L, const int32_t* ids, int M, void* scratch, hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  const ScratchPlan& P = L.plan;
  AlignArgs a;
  a.ids = ids;
  a.nslot = M * L.k;
  a.E = L.E;
  a.bm = L.block_m;
  a.expert_tier = reinterpret_cast<int32_t*>(base + P.expert_tier);
  for (int t = 0; t < 2; ++t) {
    a.slots[t] = reinterpret_cast<int32_t*>(base + P.a_slots[t]);
    a.bexp[t] = reinterpret_cast<int32_t*>(base + P.a_bexp[t]);
    a.eoff[t] = reinterpret_cast<int32_t*>(base + P.a_eoff[t]);
    a.npad[t] = reinterpret_cast<int32_t*>(base + P.a_npad[t]);
  }
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, a, make_tier_mask(L));
  return hipGetLastError();
}

}  // namespace hmoe
