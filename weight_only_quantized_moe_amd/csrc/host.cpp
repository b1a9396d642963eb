// C ABI of libhmoe: layer creation and validation, the scratch planner, views into
// scratch, and dispatch of the route / align / forward / dequant kernels.
// Nothing here allocates, frees or synchronises device memory.
#include <string.h>

#include <algorithm>
#include <new>
#include <string>

#include "hmoe_internal.h"

struct hmoe_layer {
  hmoe::Layer L;
};

namespace {

thread_local std::string g_last_error;

hmoe_status fail(hmoe_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

hmoe_status hip_fail(hipError_t err, const char* what) {
  return fail(HMOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Align capacity of one tier: M*k slots plus, for every expert that can own a slot,
// up to block_m - 1 padding entries.
int tier_capacity(int tokens, int k, int experts_in_tier, int bm) {
  if (experts_in_tier == 0) return 0;
  const long ns = (long)tokens * k;
  const long touched = std::min<long>(experts_in_tier, ns);
  const long cap = ns + touched * (bm - 1);
  return (int)((cap + bm - 1) / bm * bm);
}

void plan_scratch(hmoe::Layer& L) {
  hmoe::ScratchPlan& P = L.plan;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + std::max<size_t>(bytes, 4));
    return at;
  };
  const size_t mk = (size_t)L.max_tokens * L.k;
  const size_t dec_slots = (size_t)hmoe::kDecodeMaxM * L.k;
  P.topk_ids = take(std::max(mk, dec_slots) * 4);
  P.topk_w = take(std::max(mk, dec_slots) * 4);
  P.expert_tier = take((size_t)L.E * 4);
  P.d_counts = take(2 * 4);
  P.d_experts = take((size_t)L.max_distinct * 4);
  P.d_nslots = take((size_t)L.max_distinct * 4);
  P.d_slots = take((size_t)L.max_distinct * hmoe::kDecodeMaxM * 4);
  P.d_pass = take(dec_slots * hmoe::kPassRec * 4);
  P.h_dec = take(dec_slots * L.I * 4);
  P.o_dec = take(dec_slots * L.H * 4);
  P.d_sync = take(hmoe::fused_sync_words(L.k, L.H) * 4);
  for (int t = 0; t < 2; ++t) {
    const int cap = L.cap[t];
    const int ne = t == 0 ? L.E4 : L.E3;
    P.a_slots[t] = take((size_t)cap * 4);
    P.a_bexp[t] = take((size_t)(cap / L.block_m) * 4);
    P.a_eoff[t] = take((size_t)(ne + 1) * 4);
    P.a_npad[t] = take(4);
  }
  if (L.max_tokens > hmoe::kDecodeMaxM || L.act_format == HMOE_ACT_MXFP4) {
    P.h_pre = take((size_t)(L.cap[0] + L.cap[1]) * L.I * 2);
    P.o_pre = take(mk * L.H * 4);
    P.x16_pre = take((size_t)L.max_tokens * L.H * 2);
    P.xe_pre = take((size_t)L.max_tokens * 4);
    P.pf_fac = take((size_t)(L.cap[0] + L.cap[1]) * 4);
  } else {
    P.h_pre = take(0);
    P.o_pre = take(0);
    P.x16_pre = take(0);
    P.xe_pre = take(0);
    P.pf_fac = take(0);
  }
  if (L.act_format == HMOE_ACT_MXFP4) {
    P.mx_xq = take((size_t)L.max_tokens * L.H / 2);
    P.mx_xs = take((size_t)L.max_tokens * L.H / 32);
    P.mx_h32 = take((size_t)L.cap[0] * L.I * 4);
    P.mx_hq = take((size_t)L.cap[0] * L.I / 2);
    P.mx_hs = take((size_t)L.cap[0] * L.I / 32);
  }
  P.total = off;
}

hmoe_status check_layer(const hmoe_layer* layer) {
  if (!layer) return fail(HMOE_ERR_INVALID_ARG, "layer is NULL");
  return HMOE_OK;
}

hmoe_status check_scratch(const hmoe::Layer& L, void* scratch, size_t bytes) {
  if (!scratch) return fail(HMOE_ERR_ALIGN, "scratch is NULL");
  if (!aligned(scratch, 256)) return fail(HMOE_ERR_ALIGN, "scratch must be 256-byte aligned");
  if (bytes < L.plan.total)
    return fail(HMOE_ERR_SCRATCH, "scratch has " + std::to_string(bytes) + " bytes, needs " +
                                      std::to_string(L.plan.total));
  return HMOE_OK;
}

hmoe_status check_weights(const hmoe::Layer& L, const hmoe_weights* w) {
  if (!w) return fail(HMOE_ERR_INVALID_ARG, "weights is NULL");
  if (L.E4 > 0) {
    if (!w->kept_w13_q || !w->kept_w13_s || !w->kept_w2_q || !w->kept_w2_s)
      return fail(HMOE_ERR_INVALID_ARG, "kept-tier weight or scale array is NULL");
    if (L.kept_format == HMOE_KEPT_NVFP4 && (!w->kept_w13_g || !w->kept_w2_g))
      return fail(HMOE_ERR_INVALID_ARG, "NVFP4 per-tensor scale array is NULL");
    if (!aligned(w->kept_w13_q, 16) || !aligned(w->kept_w2_q, 16) || !aligned(w->kept_w13_s, 4) ||
        !aligned(w->kept_w2_s, 4) || (w->kept_w13_g && !aligned(w->kept_w13_g, 4)) ||
        (w->kept_w2_g && !aligned(w->kept_w2_g, 4)))
      return fail(HMOE_ERR_ALIGN, "kept-tier arrays: codes need 16-byte and scales 4-byte alignment");
  }
  if (L.E3 > 0) {
    if (!w->nf3_w13_q || !w->nf3_w13_s || !w->nf3_w2_q || !w->nf3_w2_s)
      return fail(HMOE_ERR_INVALID_ARG, "NF3-tier weight or scale array is NULL");
    if (!aligned(w->nf3_w13_q, 16) || !aligned(w->nf3_w2_q, 16) || !aligned(w->nf3_w13_s, 4) ||
        !aligned(w->nf3_w2_s, 4))
      return fail(HMOE_ERR_ALIGN, "NF3-tier arrays: codes need 16-byte and scales 4-byte alignment");
  }
  return HMOE_OK;
}

}  // namespace

extern "C" {

// Prefill rows per expert block when the caller leaves it to the library: from the mean
// number of slots per expert at max_tokens, t = max_tokens * k / E. The GEMM runs an
// expert's last, partly padded block as a 16-, 32- or 64-row tile, so a large block_m
// costs little for small experts; but its LDS stage allows two blocks per CU where a
// 32-row block_m allows three. Measured on the GLM-class layer on MI355X, skewed and
// unskewed routing: 16 rows are fastest below t = 4, 32 below t = 24 and 128 above.
static int auto_block_m(long max_tokens, long k, long E) {
  const long t = max_tokens * k;
  if (t < 4 * E) return 16;
  if (t < 24 * E) return 32;
  return 128;
}

hmoe_status moe_layer_create(const hmoe_layer_desc* d, hmoe_layer** out) {
  if (!d || !out) return fail(HMOE_ERR_INVALID_ARG, "desc and out must not be NULL");
  *out = nullptr;
  if (d->num_experts < 1) return fail(HMOE_ERR_INVALID_ARG, "num_experts must be >= 1");
  if (d->top_k < 1 || d->top_k > d->num_experts)
    return fail(HMOE_ERR_INVALID_ARG, "top_k must be in [1, num_experts]");
  if (d->max_tokens < 1) return fail(HMOE_ERR_INVALID_ARG, "max_tokens must be >= 1");
  if (d->hidden < 1 || d->inter < 1) return fail(HMOE_ERR_INVALID_ARG, "hidden and inter must be >= 1");
  if (d->kept_format != HMOE_KEPT_NVFP4 && d->kept_format != HMOE_KEPT_MXFP4)
    return fail(HMOE_ERR_INVALID_ARG, "unknown kept_format");
  if (d->block_m != 0 && d->block_m != 16 && d->block_m != 32 && d->block_m != 64 && d->block_m != 128)
    return fail(HMOE_ERR_INVALID_ARG, "block_m must be 0, 16, 32, 64 or 128");
  if (d->decode_launch != HMOE_DECODE_STAGED && d->decode_launch != HMOE_DECODE_SINGLE_LAUNCH)
    return fail(HMOE_ERR_INVALID_ARG, "unknown decode_launch");
  if (d->act_format != HMOE_ACT_16BIT && d->act_format != HMOE_ACT_MXFP4)
    return fail(HMOE_ERR_INVALID_ARG, "unknown act_format");
  if (d->act_format == HMOE_ACT_MXFP4 && (!d->bit_map || d->kept_format != HMOE_KEPT_MXFP4))
    return fail(HMOE_ERR_INVALID_ARG, "W4A4 needs a bit map and an MXFP4 kept tier");
  if (d->act_format == HMOE_ACT_MXFP4 && d->decode_launch != HMOE_DECODE_STAGED)
    return fail(HMOE_ERR_INVALID_ARG, "the single-launch decode runs W4A16 only");
  if (d->num_experts > hmoe::kMaxExperts) return fail(HMOE_ERR_UNSUPPORTED, "num_experts > 1024");
  if (d->top_k > hmoe::kMaxTopK) return fail(HMOE_ERR_UNSUPPORTED, "top_k > 16");
  if (d->hidden % 128 || d->inter % 128)
    return fail(HMOE_ERR_UNSUPPORTED, "hidden and inter must be multiples of 128");
  if ((long)d->max_tokens * d->top_k > (1L << 24))
    return fail(HMOE_ERR_UNSUPPORTED, "max_tokens * top_k > 2^24");
  if (d->bit_map) {
    for (int e = 0; e < d->num_experts; ++e)
      if (d->bit_map[e] != 3 && d->bit_map[e] != 4)
        return fail(HMOE_ERR_INVALID_ARG, "bit_map[" + std::to_string(e) + "] = " +
                                              std::to_string(d->bit_map[e]) + ", expected 3 or 4");
  }
  hmoe_layer* h = new (std::nothrow) hmoe_layer;
  if (!h) return fail(HMOE_ERR_INVALID_ARG, "out of host memory");
  hmoe::Layer& L = h->L;
  L.E = d->num_experts;
  L.H = d->hidden;
  L.I = d->inter;
  L.k = d->top_k;
  L.max_tokens = d->max_tokens;
  L.has_map = d->bit_map != nullptr;
  L.kept_format = L.has_map ? d->kept_format : HMOE_KEPT_NVFP4;
  L.block_m = d->block_m ? d->block_m : auto_block_m(d->max_tokens, d->top_k, d->num_experts);
  L.act_format = d->act_format;
  L.bit_map.assign(L.E, 4);
  if (L.has_map) memcpy(L.bit_map.data(), d->bit_map, L.E);
  for (int e = 0; e < L.E; ++e) {
    if (L.bit_map[e] == 3) {
      ++L.E3;
      L.nf3_mask[e >> 5] |= 1u << (e & 31);
    } else {
      ++L.E4;
    }
  }
  L.max_distinct = std::min(hmoe::kDecodeMaxM * L.k, L.E);
  L.cap[0] = tier_capacity(L.max_tokens, L.k, L.E4, L.block_m);
  L.cap[1] = tier_capacity(L.max_tokens, L.k, L.E3, L.block_m);
  // the prefill GEMMs address activation rows with 32-bit element offsets
  if ((long)L.max_tokens * L.H >= (1L << 31) || (long)(L.cap[0] + L.cap[1]) * L.I >= (1L << 31)) {
    delete h;
    return fail(HMOE_ERR_UNSUPPORTED, "max_tokens too large for this layer's prefill buffers");
  }
  // the prefill GEMMs run (expert blocks of both tiers, rounded up to 64) x (column
  // tiles) blocks on a 1-D grid
  if (((long)(L.cap[0] + L.cap[1]) / L.block_m + 64) * std::max(L.I / 64, L.H / 128) >=
      (1L << 31)) {
    delete h;
    return fail(HMOE_ERR_UNSUPPORTED, "max_tokens * top_k / block_m too large for the prefill "
                                      "grid: use a larger block_m");
  }
  const bool tiled = hmoe::plan_gemv(L.H, &L.w13) && hmoe::plan_gemv(L.I, &L.w2) &&
                     L.I % ((64 / L.w13.lr) * L.w13.ri) == 0 && L.H % ((64 / L.w2.lr) * L.w2.ri) == 0;
  if (!tiled) {
    delete h;
    return fail(HMOE_ERR_UNSUPPORTED, "no decode GEMV tiling for H=" + std::to_string(d->hidden) +
                                          ", I=" + std::to_string(d->inter));
  }
  L.single_available = hmoe::fused_decode_available(L);
  if (d->decode_launch == HMOE_DECODE_SINGLE_LAUNCH && !L.single_available) {
    delete h;
    return fail(HMOE_ERR_UNSUPPORTED, "no single-launch decode for H=" + std::to_string(d->hidden) +
                                          ", I=" + std::to_string(d->inter));
  }
  L.fused_decode = d->decode_launch == HMOE_DECODE_SINGLE_LAUNCH;
  plan_scratch(L);
  *out = h;
  return HMOE_OK;
}

void moe_layer_destroy(hmoe_layer* layer) { delete layer; }

hmoe_status moe_layer_query(const hmoe_layer* layer, hmoe_layer_info* out) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (!out) return fail(HMOE_ERR_INVALID_ARG, "out is NULL");
  const hmoe::Layer& L = layer->L;
  out->num_experts = L.E;
  out->hidden = L.H;
  out->inter = L.I;
  out->top_k = L.k;
  out->max_tokens = L.max_tokens;
  out->kept_format = L.kept_format;
  out->num_kept = L.E4;
  out->num_nf3 = L.E3;
  out->block_m = L.block_m;
  out->max_distinct = L.max_distinct;
  out->cap_kept = L.cap[0];
  out->cap_nf3 = L.cap[1];
  out->fused_decode = L.fused_decode ? 1 : 0;
  out->single_launch_available = L.single_available ? 1 : 0;
  out->act_format = L.act_format;
  return HMOE_OK;
}

hmoe_status moe_scratch_bytes(const hmoe_layer* layer, size_t* bytes) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (!bytes) return fail(HMOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layer->L.plan.total;
  return HMOE_OK;
}

hmoe_status moe_route(const float* logits, int32_t M, int32_t E, int32_t k, int32_t* topk_ids,
                      float* topk_w, hipStream_t stream) {
  if (M < 0) return fail(HMOE_ERR_INVALID_ARG, "M < 0");
  if (E < 1 || E > hmoe::kMaxExperts) return fail(HMOE_ERR_INVALID_ARG, "E must be in [1, 1024]");
  if (k < 1 || k > std::min(hmoe::kMaxTopK, (int)E))
    return fail(HMOE_ERR_INVALID_ARG, "k must be in [1, min(16, E)]");
  if (M == 0) return HMOE_OK;
  if (!logits || !topk_ids || !topk_w || !aligned(logits, 16) || !aligned(topk_ids, 16) ||
      !aligned(topk_w, 16))
    return fail(HMOE_ERR_ALIGN, "logits, topk_ids and topk_w must be non-NULL and 16-byte aligned");
  hipError_t err = hmoe::launch_route(logits, M, E, k, topk_ids, topk_w, stream);
  if (err != hipSuccess) return hip_fail(err, "route launch");
  return HMOE_OK;
}

hmoe_status moe_align(const hmoe_layer* layer, const int32_t* topk_ids, int32_t M, void* scratch,
                      size_t scratch_bytes, hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  const hmoe::Layer& L = layer->L;
  if (M < 0) return fail(HMOE_ERR_INVALID_ARG, "M < 0");
  if (M > L.max_tokens) return fail(HMOE_ERR_CAPACITY, "M exceeds max_tokens");
  if (hmoe_status st = check_scratch(L, scratch, scratch_bytes)) return st;
  if (!topk_ids || !aligned(topk_ids, 16))
    return fail(HMOE_ERR_ALIGN, "topk_ids must be non-NULL and 16-byte aligned");
  hipError_t err = hmoe::launch_align(L, topk_ids, M, scratch, stream);
  if (err != hipSuccess) return hip_fail(err, "align launch");
  return HMOE_OK;
}

hmoe_status moe_align_view(const hmoe_layer* layer, void* scratch, int32_t tier,
                           hmoe_align_view* out) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (!scratch || !out || (tier != 0 && tier != 1))
    return fail(HMOE_ERR_INVALID_ARG, "scratch/out NULL or tier not 0/1");
  const hmoe::Layer& L = layer->L;
  char* b = static_cast<char*>(scratch);
  out->sorted_slots = reinterpret_cast<int32_t*>(b + L.plan.a_slots[tier]);
  out->block_expert = reinterpret_cast<int32_t*>(b + L.plan.a_bexp[tier]);
  out->expert_off = reinterpret_cast<int32_t*>(b + L.plan.a_eoff[tier]);
  out->num_padded = reinterpret_cast<int32_t*>(b + L.plan.a_npad[tier]);
  out->capacity = L.cap[tier];
  out->num_experts_tier = tier == 0 ? L.E4 : L.E3;
  return HMOE_OK;
}

hmoe_status moe_decode_view(const hmoe_layer* layer, void* scratch, hmoe_decode_view* out) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (!scratch || !out) return fail(HMOE_ERR_INVALID_ARG, "scratch/out NULL");
  const hmoe::Layer& L = layer->L;
  char* b = static_cast<char*>(scratch);
  out->counts = reinterpret_cast<int32_t*>(b + L.plan.d_counts);
  out->experts = reinterpret_cast<int32_t*>(b + L.plan.d_experts);
  out->num_slots = reinterpret_cast<int32_t*>(b + L.plan.d_nslots);
  out->slots = reinterpret_cast<int32_t*>(b + L.plan.d_slots);
  out->expert_tier = reinterpret_cast<int32_t*>(b + L.plan.expert_tier);
  out->passes = reinterpret_cast<int32_t*>(b + L.plan.d_pass);
  out->max_distinct = L.max_distinct;
  out->sync_timeouts = reinterpret_cast<int32_t*>(b + L.plan.d_sync) + 16;
  return HMOE_OK;
}

hmoe_status moe_topk_view(const hmoe_layer* layer, void* scratch, int32_t** topk_ids, float** topk_w) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (!scratch || !topk_ids || !topk_w) return fail(HMOE_ERR_INVALID_ARG, "NULL argument");
  char* b = static_cast<char*>(scratch);
  *topk_ids = reinterpret_cast<int32_t*>(b + layer->L.plan.topk_ids);
  *topk_w = reinterpret_cast<float*>(b + layer->L.plan.topk_w);
  return HMOE_OK;
}

hmoe_status hybrid_moe_forward_stage(const hmoe_layer* layer, const hmoe_weights* weights,
                                     const uint16_t* x, const float* router_logits, int32_t M,
                                     uint16_t* y, void* scratch, size_t scratch_bytes,
                                     int32_t stage, hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  const hmoe::Layer& L = layer->L;
  if (stage < HMOE_STAGE_ROUTE || stage > HMOE_STAGE_COMBINE)
    return fail(HMOE_ERR_INVALID_ARG, "unknown stage");
  if (M < 0) return fail(HMOE_ERR_INVALID_ARG, "M < 0");
  if (M > L.max_tokens) return fail(HMOE_ERR_CAPACITY, "M exceeds max_tokens");
  if (hmoe_status st = check_weights(L, weights)) return st;
  if (M == 0) return HMOE_OK;
  if (hmoe_status st = check_scratch(L, scratch, scratch_bytes)) return st;
  if (!x || !router_logits || !y || !aligned(x, 16) || !aligned(router_logits, 16) || !aligned(y, 16))
    return fail(HMOE_ERR_ALIGN, "x, router_logits and y must be non-NULL and 16-byte aligned");
  const bool w4a4 = L.act_format == HMOE_ACT_MXFP4;
  const bool decode = M <= hmoe::kDecodeMaxM && !w4a4;
  hipError_t err;
  if (stage == HMOE_STAGE_ROUTE) {
    if (decode) {
      err = hmoe::launch_route_group(L, router_logits, M, scratch, stream);
    } else {
      char* b = static_cast<char*>(scratch);
      int32_t* ids = reinterpret_cast<int32_t*>(b + L.plan.topk_ids);
      err = hmoe::launch_route(router_logits, M, L.E, L.k, ids,
                               reinterpret_cast<float*>(b + L.plan.topk_w), stream);
      if (err == hipSuccess) err = hmoe::launch_align(L, ids, M, scratch, stream);
      if (err == hipSuccess) err = hmoe::launch_prefill_x16(L, x, M, scratch, stream);
      if (err == hipSuccess && w4a4) err = hmoe::launch_w4a4(L, *weights, x, M, scratch, stage, stream);
    }
  } else if (decode) {
    err = hmoe::launch_decode(L, *weights, x, M, y, scratch, stage, stream);
  } else {
    // W4A4: the GEMM launches run both tiers (kept tier on MX matrix cores); the W13
    // stage then rounds the kept tier's h to MXFP4
    err = hmoe::launch_prefill(L, *weights, x, M, y, scratch, stage, stream, w4a4);
    if (err == hipSuccess && w4a4 && stage == HMOE_STAGE_W13)
      err = hmoe::launch_w4a4(L, *weights, x, M, scratch, stage, stream);
  }
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return HMOE_OK;
}

hmoe_status hybrid_moe_forward(const hmoe_layer* layer, const hmoe_weights* weights,
                               const uint16_t* x, const float* router_logits, int32_t M,
                               uint16_t* y, void* scratch, size_t scratch_bytes,
                               hipStream_t stream) {
  if (layer && layer->L.fused_decode && M > 0 && M <= hmoe::kDecodeMaxM) {
    const hmoe::Layer& L = layer->L;
    if (M > L.max_tokens) return fail(HMOE_ERR_CAPACITY, "M exceeds max_tokens");
    if (hmoe_status st = check_weights(L, weights)) return st;
    if (hmoe_status st = check_scratch(L, scratch, scratch_bytes)) return st;
    if (!x || !router_logits || !y || !aligned(x, 16) || !aligned(router_logits, 16) ||
        !aligned(y, 16))
      return fail(HMOE_ERR_ALIGN, "x, router_logits and y must be non-NULL and 16-byte aligned");
    hipError_t err = hmoe::launch_decode_fused(L, *weights, x, router_logits, M, y, scratch, stream);
    if (err != hipSuccess) return hip_fail(err, "decode launch");
    return HMOE_OK;
  }
  for (int32_t stage = HMOE_STAGE_ROUTE; stage <= HMOE_STAGE_COMBINE; ++stage) {
    const hmoe_status st = hybrid_moe_forward_stage(layer, weights, x, router_logits, M, y, scratch,
                                                    scratch_bytes, stage, stream);
    if (st != HMOE_OK) return st;
  }
  return HMOE_OK;
}

hmoe_status hybrid_moe_forward_static(const hmoe_layer* layer, const hmoe_weights* weights,
                                      const uint16_t* x, const float* router_logits, int32_t M,
                                      uint16_t* y, hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  const size_t need = layer->L.plan.total, have = hmoe::static_scratch_bytes();
  if (need > have)
    return fail(HMOE_ERR_SCRATCH, "the layer needs " + std::to_string(need) +
                                      " bytes of scratch, the static scratch holds " +
                                      std::to_string(have) + ": use hybrid_moe_forward");
  void* scratch = nullptr;
  hipError_t err = hmoe::static_scratch(&scratch);
  if (err != hipSuccess) return hip_fail(err, "static scratch address");
  // every layer on this GPU shares the array, so the single-launch decode's counters may
  // hold another call's data: they are cleared first (a fill kernel, capturable)
  const hmoe::Layer& L = layer->L;
  if (L.fused_decode && M > 0 && M <= hmoe::kDecodeMaxM && M <= L.max_tokens) {
    err = hmoe::launch_sync_clear(L, scratch, stream);
    if (err != hipSuccess) return hip_fail(err, "static scratch counter clear");
  }
  return hybrid_moe_forward(layer, weights, x, router_logits, M, y, scratch, have, stream);
}

hmoe_status moe_scratch_init(const hmoe_layer* layer, void* scratch, size_t scratch_bytes,
                             hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  if (hmoe_status st = check_scratch(layer->L, scratch, scratch_bytes)) return st;
  hipError_t err = hmoe::launch_sync_clear(layer->L, scratch, stream);
  if (err != hipSuccess) return hip_fail(err, "scratch init launch");
  return HMOE_OK;
}

hmoe_status moe_dequant(const hmoe_layer* layer, const hmoe_weights* weights, int32_t expert,
                        int32_t tensor, float* out_f32, uint16_t* out_bf16, hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  const hmoe::Layer& L = layer->L;
  if (expert < 0 || expert >= L.E) return fail(HMOE_ERR_INVALID_ARG, "expert out of range");
  if (tensor != HMOE_TENSOR_W13 && tensor != HMOE_TENSOR_W2)
    return fail(HMOE_ERR_INVALID_ARG, "tensor must be HMOE_TENSOR_W13 or HMOE_TENSOR_W2");
  if (!out_f32 && !out_bf16) return fail(HMOE_ERR_INVALID_ARG, "both outputs are NULL");
  if ((out_f32 && !aligned(out_f32, 16)) || (out_bf16 && !aligned(out_bf16, 16)))
    return fail(HMOE_ERR_ALIGN, "outputs must be 16-byte aligned");
  if (hmoe_status st = check_weights(L, weights)) return st;
  hipError_t err = hmoe::launch_dequant(L, *weights, expert, tensor, out_f32, out_bf16, stream);
  if (err != hipSuccess) return hip_fail(err, "dequant launch");
  return HMOE_OK;
}

hmoe_status moe_repack(const hmoe_layer* layer, const hmoe_expert_src* experts,
                       const hmoe_weights* dst, hipStream_t stream) {
  if (hmoe_status st = check_layer(layer)) return st;
  const hmoe::Layer& L = layer->L;
  if (!experts) return fail(HMOE_ERR_INVALID_ARG, "experts is NULL");
  if (hmoe_status st = check_weights(L, dst)) return st;
  const bool nv = L.kept_format == HMOE_KEPT_NVFP4;
  struct Tensor {
    long rows;
    int K;
  };
  const Tensor ts[2] = {{2L * L.I, L.H}, {(long)L.H, L.I}};
  // validate every expert before the first copy
  for (int e = 0; e < L.E; ++e) {
    const hmoe_expert_src& s = experts[e];
    const bool nf3 = (L.nf3_mask[e >> 5] >> (e & 31)) & 1u;
    if (!s.w13_q || !s.w13_s || !s.w2_q || !s.w2_s)
      return fail(HMOE_ERR_INVALID_ARG, "expert " + std::to_string(e) + ": a code or scale pointer is NULL");
    if (nf3 && (!s.w13_hi || !s.w2_hi))
      return fail(HMOE_ERR_INVALID_ARG, "NF3 expert " + std::to_string(e) + ": a high code plane is NULL");
    if (nf3 && (!aligned(s.w13_q, 4) || !aligned(s.w13_hi, 4) || !aligned(s.w2_q, 4) ||
                !aligned(s.w2_hi, 4)))
      return fail(HMOE_ERR_ALIGN, "NF3 expert " + std::to_string(e) + ": code planes need 4-byte alignment");
    if (!nf3 && nv && (!s.w13_g || !s.w2_g))
      return fail(HMOE_ERR_INVALID_ARG, "NVFP4 expert " + std::to_string(e) + ": a per-tensor scale is NULL");
  }
  uint8_t* kq[2] = {const_cast<uint8_t*>(dst->kept_w13_q), const_cast<uint8_t*>(dst->kept_w2_q)};
  uint8_t* ks[2] = {const_cast<uint8_t*>(dst->kept_w13_s), const_cast<uint8_t*>(dst->kept_w2_s)};
  float* kg[2] = {const_cast<float*>(dst->kept_w13_g), const_cast<float*>(dst->kept_w2_g)};
  uint8_t* nq[2] = {const_cast<uint8_t*>(dst->nf3_w13_q), const_cast<uint8_t*>(dst->nf3_w2_q)};
  uint16_t* ns[2] = {const_cast<uint16_t*>(dst->nf3_w13_s), const_cast<uint16_t*>(dst->nf3_w2_s)};
  int below[2] = {0, 0};  // experts of each tier so far: the tier-local index
  hmoe::RepackBatch batch{};
  auto add = [&](const void* src, const void* hi, void* out, long n, int kind) -> hipError_t {
    batch.job[batch.njobs++] = {src, hi, out, n, kind, 0};
    if (batch.njobs < hmoe::kRepackJobs) return hipSuccess;
    hipError_t err = hmoe::launch_repack(batch, stream);
    batch.njobs = 0;
    return err;
  };
  for (int e = 0; e < L.E; ++e) {
    const hmoe_expert_src& s = experts[e];
    const int tier = ((L.nf3_mask[e >> 5] >> (e & 31)) & 1u) ? 1 : 0;
    const long loc = below[tier]++;
    const uint8_t* sq[2] = {s.w13_q, s.w2_q};
    const uint8_t* shi[2] = {s.w13_hi, s.w2_hi};
    const void* ss[2] = {s.w13_s, s.w2_s};
    const float* sg[2] = {s.w13_g, s.w2_g};
    for (int t = 0; t < 2; ++t) {
      const long rows = ts[t].rows;
      const int K = ts[t].K;
      hipError_t err = hipSuccess;
      if (tier == 0) {
        const long qb = rows * (K / 2), sb = rows * (K / (nv ? 16 : 32));
        err = add(sq[t], nullptr, kq[t] + loc * qb, qb, hmoe::kRepackCopy);
        if (err == hipSuccess) err = add(ss[t], nullptr, ks[t] + loc * sb, sb, hmoe::kRepackCopy);
        if (err == hipSuccess && nv && kg[t])
          err = add(sg[t], nullptr, kg[t] + loc, (long)sizeof(float), hmoe::kRepackCopy);
      } else {
        const long qb = rows * (3L * K / 8), sn = rows * (K / 64);
        err = add(sq[t], shi[t], nq[t] + loc * qb, rows * (K / 32), hmoe::kRepackNf3);
        if (err == hipSuccess) err = add(ss[t], nullptr, ns[t] + loc * sn, sn * 2, hmoe::kRepackCopy);
      }
      if (err != hipSuccess) return hip_fail(err, "repack");
    }
  }
  if (batch.njobs > 0) {
    hipError_t err = hmoe::launch_repack(batch, stream);
    if (err != hipSuccess) return hip_fail(err, "repack");
  }
  return HMOE_OK;
}

hmoe_status moe_quantize_mxfp4(const float* in, int32_t rows, int32_t K, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32) return fail(HMOE_ERR_INVALID_ARG, "rows >= 0 and K a positive multiple of 32");
  if (rows == 0) return HMOE_OK;
  if (!in || !codes || !scales || !aligned(in, 16) || !aligned(codes, 16))
    return fail(HMOE_ERR_ALIGN, "in, codes and scales must be non-NULL, in and codes 16-byte aligned");
  hipError_t err = hmoe::launch_mx_quant(in, false, rows, K, nullptr, codes, scales, stream);
  if (err != hipSuccess) return hip_fail(err, "quantise launch");
  return HMOE_OK;
}

const char* moe_status_string(hmoe_status s) {
  switch (s) {
    case HMOE_OK: return "HMOE_OK";
    case HMOE_ERR_INVALID_ARG: return "HMOE_ERR_INVALID_ARG";
    case HMOE_ERR_UNSUPPORTED: return "HMOE_ERR_UNSUPPORTED";
    case HMOE_ERR_ALIGN: return "HMOE_ERR_ALIGN";
    case HMOE_ERR_CAPACITY: return "HMOE_ERR_CAPACITY";
    case HMOE_ERR_SCRATCH: return "HMOE_ERR_SCRATCH";
    case HMOE_ERR_HIP: return "HMOE_ERR_HIP";
  }
  return "HMOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
