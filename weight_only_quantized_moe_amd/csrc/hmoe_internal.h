// Internal declarations of libhmoe: the layer object, the scratch plan and the
// kernel launchers each kernel file provides. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "hmoe.h"

namespace hmoe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kDecodeMaxM = HMOE_DECODE_MAX_M;
// decode pass record (int4), one per (token, top-k) slot, in slot order: slot, tier
// code, token, expert id (written by the routing stage, read by the GEMVs)
constexpr int kPassRec = 4;

// Byte offsets of every scratch region (each 256-byte aligned).
struct ScratchPlan {
  size_t topk_ids = 0, topk_w = 0, expert_tier = 0;
  size_t d_counts = 0, d_experts = 0, d_nslots = 0, d_slots = 0, d_pass = 0;
  size_t h_dec = 0, o_dec = 0;
  size_t d_sync = 0;                       // single-launch decode counters (zero between calls)
  size_t a_counts = 0;                     // int32 [E] slot counts per expert
  size_t a_slots[2] = {0, 0}, a_bexp[2] = {0, 0}, a_eoff[2] = {0, 0}, a_npad[2] = {0, 0};
  size_t h_pre = 0, o_pre = 0, x16_pre = 0, xe_pre = 0;
  size_t pf_fac = 0;                       // fp32 [cap0 + cap1]: W2 output factor per h row
  size_t mx_xq = 0, mx_xs = 0, mx_h32 = 0, mx_hq = 0, mx_hs = 0;   // W4A4 kept tier
  size_t total = 0;
};

// GEMV tiling of one weight tensor on the decode path: lanes per row (LR), units of
// 32 K-elements per lane (KU), rows (or row pairs) per lane per chunk (RI).
struct GemvTiling {
  int lr = 0, ku = 0, ri = 0;
};

struct Layer {
  int E = 0, H = 0, I = 0, k = 0, max_tokens = 0;
  int kept_format = HMOE_KEPT_NVFP4;  // effective
  int act_format = HMOE_ACT_16BIT;    // HMOE_ACT_MXFP4: the kept tier runs W4A4
  int block_m = 32;
  bool has_map = false;
  std::vector<uint8_t> bit_map;
  int E4 = 0, E3 = 0;
  uint32_t nf3_mask[kMaxExperts / 32] = {};  // bit e set: expert e is in the NF3 tier
  int max_distinct = 0;                        // min(8k, E)
  int cap[2] = {0, 0};                         // align capacity per tier
  GemvTiling w13, w2;
  bool fused_decode = false;                   // the forward runs decode as one launch
  bool single_available = false;               // a single-launch decode exists for H, I
  ScratchPlan plan;
};

// Expert-tier bit mask passed by value to the kernels that need the tier map.
struct TierMask {
  uint32_t w[kMaxExperts / 32];
};

// ---- launchers (each returns hipGetLastError() of its launch) -------------------

// route.hip
hipError_t launch_route(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);
hipError_t launch_route_group(const Layer& L, const float* logits, int M, void* scratch,
                              hipStream_t s);

// align.hip
hipError_t launch_align(const Layer& L, const int32_t* ids, int M, void* scratch, hipStream_t s);

// decode.hip: one stage (HMOE_STAGE_W13 / _W2 / _COMBINE) of the decode path
hipError_t launch_decode(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                         uint16_t* y, void* scratch, int stage, hipStream_t s);

// decode.hip: the whole decode forward in one launch (only for the layer shapes
// fused_decode_available accepts), the size of its sync region, and its zero fill
bool fused_decode_available(const Layer& L);
size_t fused_sync_words(int k, int H);
hipError_t launch_decode_fused(const Layer& L, const hmoe_weights& W, const uint16_t* x,
                               const float* logits, int M, uint16_t* y, void* scratch,
                               hipStream_t s);
hipError_t launch_sync_clear(const Layer& L, void* scratch, hipStream_t s);

// prefill.hip: one stage (HMOE_STAGE_W13 / _W2 / _COMBINE) of the prefill path;
// nf3_only (W4A4 layers): the W4A16 GEMM covers the NF3 tier and the same launch runs
// the kept tier on MX matrix cores
hipError_t launch_prefill(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                          uint16_t* y, void* scratch, int stage, hipStream_t s,
                          bool nf3_only = false);

// w4a4.hip: the W4A4 kept tier's quantisation around the GEMM launches (ROUTE: x to
// MXFP4; W13: h to MXFP4), and the MXFP4 activation quantiser (rows x K, bf16 or fp32
// input; rows at or past *nrows skipped when nrows is given)
hipError_t launch_w4a4(const Layer& L, const hmoe_weights& W, const uint16_t* x, int M,
                       void* scratch, int stage, hipStream_t s);
hipError_t launch_mx_quant(const void* in, bool bf16, int rows, int K, const int32_t* nrows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);

// prefill.hip: tokens to fp16 with a per-token power-of-two scale (prefill input)
hipError_t launch_prefill_x16(const Layer& L, const uint16_t* x, int M, void* scratch,
                              hipStream_t s);

// dequant.hip
hipError_t launch_dequant(const Layer& L, const hmoe_weights& W, int expert, int tensor,
                          float* out_f32, uint16_t* out_bf16, hipStream_t s);

// repack.hip: a batch of copy jobs (n bytes) and NF3 plane-to-stream jobs (n units of
// 32 elements: src = low plane, src_hi = high plane, dst = stream), one launch
constexpr int kRepackThreads = 256;
constexpr int kRepackJobs = 24;
enum : int { kRepackCopy = 0, kRepackNf3 = 1 };
struct RepackJob {
  const void* src;
  const void* src_hi;
  void* dst;
  long n;
  int kind;
  int blocks;
};
struct RepackBatch {
  RepackJob job[kRepackJobs];
  int first_block[kRepackJobs];
  int njobs;
};
hipError_t launch_repack(RepackBatch& b, hipStream_t s);

TierMask make_tier_mask(const Layer& L);

// noalloc.hip: this device's file-scope scratch array (address looked up once per
// device) and its size
hipError_t static_scratch(void** out);
size_t static_scratch_bytes();

bool plan_gemv(int K, GemvTiling* t);

}  // namespace hmoe
