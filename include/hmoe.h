/*
 * hmoe.h - C ABI of the hybrid-precision W4A16 fused MoE layer for AMD MI355X (gfx950).
 *
 * One MoE layer whose experts each live in one of two weight tiers, chosen per
 * expert by a bit map (4 = kept tier, 3 = NF3 tail). The kept tier is NVFP4
 * (E2M1 values, an E4M3 scale per 16 along K, an fp32 per-tensor scale) or, when
 * the kept format says so, MXFP4 (E2M1 values, an E8M0 scale per 32). The NF3
 * tail stores 3-bit NormalFloat codes with an fp16 absmax scale per 64 along K.
 * Tokens are bf16, routing is softmax top-k renormalised, the experts are SwiGLU
 * MLPs, and both tiers add into one shared top-k weighted sum.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] local-inference-lab/vllm PR #92 "quant: nvfp4_nf3_hybrid", "How it works":
 *        two prepared weight objects per layer, launches sharing one route geometry
 *        and one top-k sum, the second accumulating into the first, graph-safe, an
 *        M <= 8 decode path addressed by the top-k result, layers absent from the map
 *        run uniform NVFP4, no environment variables, scratch sized from the maximum
 *        number of batched tokens.
 *   [P2] local-inference-lab/vllm PR #104, description and "Summary": bit map values
 *        4 = kept, 3 = NF3; a kept format that may switch the kept tier to MXFP4;
 *        expert weights demultiplexed into compact tier-local storage.
 *   [P3] vllm-project/vllm PR #42428 "W4A16 NVFP4 fused MoE", "What's in this PR":
 *        W4A16 keeps activations in 16 bits, with no activation scales.
 *
 * Conventions shared by every call:
 *   - Device pointers are allocated and owned by the caller; the library never
 *     allocates, frees, synchronises or reads device memory back on any call that
 *     takes a stream, so those calls can be captured into a HIP graph at fixed M.
 *   - Every call that takes a stream enqueues its kernels on that stream and returns
 *     before they run. A kernel fault surfaces at the caller's next synchronisation.
 *   - Errors are status codes; moe_last_error() gives a thread-local message for the
 *     last failing call. No C++ exception crosses this boundary.
 *   - Layout of every weight tensor: row-major [rows, K] with K (the reduction axis)
 *     contiguous. W13 has 2I rows, gate rows [0, I) then up rows [I, 2I), K = H.
 *     W2 has H rows, K = I. Tier-local arrays hold that tier's experts in ascending
 *     global id ([P2] "compact tier-local storage").
 *   - Packed bytes: FP4 codes put element 2j in the low nibble of byte j; NF3 codes
 *     are a little-endian bit stream per row with element j at bits [3j, 3j+3).
 *   - Device pointers passed to moe_route, moe_align and hybrid_moe_forward must be
 *     16-byte aligned (HMOE_ERR_ALIGN otherwise); the scratch buffer 256-byte aligned.
 */
#ifndef HMOE_H
#define HMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hmoe_status {
    HMOE_OK = 0,
    HMOE_ERR_INVALID_ARG = 1,  /* a null, negative or inconsistent argument */
    HMOE_ERR_UNSUPPORTED = 2,  /* a shape or option this build does not handle */
    HMOE_ERR_ALIGN = 3,        /* a device pointer is null or misaligned */
    HMOE_ERR_CAPACITY = 4,     /* M exceeds the layer's max_tokens */
    HMOE_ERR_SCRATCH = 5,      /* scratch buffer smaller than moe_scratch_bytes() */
    HMOE_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed */
} hmoe_status;

enum { HMOE_KEPT_NVFP4 = 0, HMOE_KEPT_MXFP4 = 1 };
/* Activations of the kept tier's matmuls: 16-bit (W4A16) or MXFP4 (W4A4). */
enum { HMOE_ACT_16BIT = 0, HMOE_ACT_MXFP4 = 1 };
/* How hybrid_moe_forward runs the decode path (M <= 8). */
enum { HMOE_DECODE_STAGED = 0, HMOE_DECODE_SINGLE_LAUNCH = 1 };
enum { HMOE_TIER_KEPT = 0, HMOE_TIER_NF3 = 1 };
enum { HMOE_TENSOR_W13 = 0, HMOE_TENSOR_W2 = 1 };
/* Stages of the forward, in launch order (see hybrid_moe_forward_stage). */
enum { HMOE_STAGE_ROUTE = 0, HMOE_STAGE_W13 = 1, HMOE_STAGE_W2 = 2, HMOE_STAGE_COMBINE = 3 };

/* Largest M served by the decode path (M <= 8, [P1] "How it works"). */
#define HMOE_DECODE_MAX_M 8

/* Layer descriptor, read once by moe_layer_create ([P2]: tier assignment comes
 * from the bit map; [P1]: scratch sizing from the maximum batched tokens).
 *   num_experts  E, 1..1024
 *   hidden       H, a multiple of 128
 *   inter        I, a multiple of 128
 *   top_k        k, 1..16 and <= E
 *   max_tokens   the largest M any call will pass; sizes the scratch buffer (>= 1)
 *   kept_format  HMOE_KEPT_NVFP4 or HMOE_KEPT_MXFP4; with a NULL bit map the layer
 *                runs uniform NVFP4 whatever this says ([P1])
 *   bit_map      host array of E bytes, each 4 (kept) or 3 (NF3); copied; NULL means
 *                every expert is in the kept tier, as NVFP4
 *   block_m      prefill rows per expert block for moe_align: 16, 32, 64 or 128; 0 lets
 *                the library pick from t = max_tokens * top_k / E: 16 below t = 4, 32
 *                below 24, else 128. The prefill GEMM runs a block whose real slots
 *                fit in 16, 32 or 64 rows as a tile of that many rows.
 *   decode_launch HMOE_DECODE_STAGED (0): the decode path as four kernels (routing, W13,
 *                W2, combine), the faster form on MI355X at every measured shape;
 *                HMOE_DECODE_SINGLE_LAUNCH (1): the whole decode forward in one
 *                persistent kernel ([P1] "How it works": the M <= 8 direct top-k path);
 *                both give the same bits.
 *   act_format   HMOE_ACT_16BIT (0): every expert W4A16 (x and h stay 16-bit, [P3]);
 *                HMOE_ACT_MXFP4 (1): the kept tier, which must be MXFP4 (a bit map and
 *                kept_format MXFP4), runs W4A4 ([P3] "What's in this PR": the W4A4
 *                backends beside the W4A16 path): x before W13 and h (in fp32) before W2
 *                are rounded to MXFP4 along K, blocks of 32, by the OCP MX v1.0
 *                conversion, on MX-scaled matrix cores; the NF3 tail stays W4A16. Every
 *                M then takes the grouped-GEMM path; decode_launch must be 0. */
typedef struct hmoe_layer_desc {
    int32_t num_experts;
    int32_t hidden;
    int32_t inter;
    int32_t top_k;
    int32_t max_tokens;
    int32_t kept_format;
    const uint8_t* bit_map;
    int32_t block_m;
    int32_t decode_launch;
    int32_t act_format;
} hmoe_layer_desc;

/* Opaque, immutable after creation: concurrent calls on different streams with
 * separate scratch buffers are safe. */
typedef struct hmoe_layer hmoe_layer;

/* Host-visible facts about a created layer. */
typedef struct hmoe_layer_info {
    int32_t num_experts, hidden, inter, top_k, max_tokens;
    int32_t kept_format;       /* effective format: NVFP4 when the bit map was NULL */
    int32_t num_kept, num_nf3; /* E4 and E3 */
    int32_t block_m;           /* effective block_m */
    int32_t max_distinct;      /* min(8 * top_k, E): decode group capacity */
    int32_t cap_kept, cap_nf3; /* align capacity per tier at max_tokens */
    int32_t fused_decode;      /* 1: hybrid_moe_forward runs M <= 8 as one launch */
    int32_t single_launch_available; /* 1: a single-launch decode exists for H and I */
    int32_t act_format;        /* HMOE_ACT_16BIT or HMOE_ACT_MXFP4 */
} hmoe_layer_info;

/* Packed weights of both tiers, in the layouts above. Device pointers, owned by the
 * caller and only read. Arrays of an empty tier may be NULL.
 *   Kept tier, NVFP4: w13_q u8 [E4, 2I, H/2], w13_s u8 [E4, 2I, H/16] (E4M3),
 *                     w13_g f32 [E4] (per-tensor multiplier); w2_q u8 [E4, H, I/2],
 *                     w2_s u8 [E4, H, I/16], w2_g f32 [E4].
 *   Kept tier, MXFP4: as NVFP4 with scales u8 [.., K/32] (E8M0); the _g arrays are
 *                     not read and may be NULL.
 *   NF3 tier:         w13_q u8 [E3, 2I, 3H/8], w13_s u16 [E3, 2I, H/64] (fp16 bits);
 *                     w2_q u8 [E3, H, 3I/8], w2_s u16 [E3, H, I/64]. */
typedef struct hmoe_weights {
    const uint8_t* kept_w13_q;
    const uint8_t* kept_w13_s;
    const float* kept_w13_g;
    const uint8_t* kept_w2_q;
    const uint8_t* kept_w2_s;
    const float* kept_w2_g;
    const uint8_t* nf3_w13_q;
    const uint16_t* nf3_w13_s;
    const uint8_t* nf3_w2_q;
    const uint16_t* nf3_w2_s;
} hmoe_weights;

/* Device pointers into a scratch buffer: the align result of one tier, valid after
 * moe_align or a prefill hybrid_moe_forward (M > 8) has run on that scratch.
 *   sorted_slots  int32 [capacity]: slots s = t * k + j of the tier's experts, grouped by
 *                 tier-local expert in ascending local id, ascending s inside an expert,
 *                 each expert's run padded to a multiple of block_m with the sentinel M*k;
 *                 only the first *num_padded entries are defined
 *   block_expert  int32 [capacity / block_m]: tier-local expert of each block of block_m
 *                 entries; only the first *num_padded / block_m entries are defined
 *   expert_off    int32 [E_tier + 1]: exclusive prefix of the padded run lengths
 *   num_padded    int32 [1] */
typedef struct hmoe_align_view {
    int32_t* sorted_slots;
    int32_t* block_expert;
    int32_t* expert_off;
    int32_t* num_padded;
    int32_t capacity;
    int32_t num_experts_tier;
} hmoe_align_view;

/* Device pointers into a scratch buffer: the decode grouping ([P1] "M <= 8 ...
 * direct-topk path"), valid after a decode hybrid_moe_forward (M <= 8).
 *   counts      int32 [2]: number of distinct touched experts, and how many of them are
 *               in the kept tier
 *   experts     int32 [max_distinct]: distinct touched global expert ids ordered by
 *               (tier, tier-local id); first counts[0] entries defined
 *   num_slots   int32 [max_distinct]: number of slots routed to each
 *   slots       int32 [max_distinct, 8]: those slots, ascending
 *   expert_tier int32 [E]: (tier << 16) | tier-local id of every expert
 *   passes      int32 [M * k, 4]: one record per slot, in slot order: (slot,
 *               (tier << 16) | tier-local id, token, expert); the staged decode GEMVs
 *               split their work over these records (written by the ROUTE stage; the
 *               other fields by the COMBINE stage, off the critical path; the single
 *               launch writes all of them from a block of its own)
 *   sync_timeouts int32 [1]: how many bounded waits of the single-launch decode gave up
 *               (cumulative over the scratch's life; 0 unless its grid could not be
 *               resident at once, e.g. beside another persistent kernel) */
typedef struct hmoe_decode_view {
    int32_t* counts;
    int32_t* experts;
    int32_t* num_slots;
    int32_t* slots;
    int32_t* expert_tier;
    int32_t* passes;
    int32_t max_distinct;
    int32_t* sync_timeouts;
} hmoe_decode_view;

/* Creates a layer from a descriptor (host only; no device call). *out receives a
 * handle owned by the library until moe_layer_destroy.
 * Errors: HMOE_ERR_INVALID_ARG (null pointers, E < 1, k < 1, k > E, max_tokens < 1,
 * a bit map value other than 3 or 4, an unknown kept format, block_m or decode_launch);
 * HMOE_ERR_UNSUPPORTED (E > 1024, k > 16, H or I not a multiple of 128, a K for
 * which no decode tiling exists, HMOE_DECODE_SINGLE_LAUNCH for an H and I it is not built
 * for (see single_launch_available), max_tokens * top_k > 2^24, max_tokens * H or the
 * prefill h rows * I reaching 2^31, or a prefill GEMM grid of 2^31 blocks or more
 * at max_tokens). */
hmoe_status moe_layer_create(const hmoe_layer_desc* desc, hmoe_layer** out);

/* Frees the handle's host memory. NULL is a no-op. */
void moe_layer_destroy(hmoe_layer* layer);

hmoe_status moe_layer_query(const hmoe_layer* layer, hmoe_layer_info* out);

/* Scratch planner ([P1] "scratch sizing from max_num_batched_tokens"): bytes of
 * device scratch that moe_align and hybrid_moe_forward need for any M <= the layer's
 * max_tokens. Pure host arithmetic. Covers: top-k ids and weights, the expert tier
 * map, the decode groups and decode intermediates (h and per-slot outputs for 8 * k
 * slots, fp32), per-tier align arrays at their capacity, and, when max_tokens > 8,
 * the prefill intermediate h [sum of capacities, I] (fp16) and the per-slot prefill
 * outputs [max_tokens * k, H] (fp32); each region is 256-byte aligned. The caller
 * allocates the buffer and passes it to every call. */
hmoe_status moe_scratch_bytes(const hmoe_layer* layer, size_t* bytes);

/* Prepares a scratch buffer for this layer's forwards: zero-fills the counters the
 * single-launch decode synchronises its workgroups with (every forward leaves them
 * zero again). A scratch buffer that was allocated zero-filled and serves only this layer
 * needs no call; one that other layers or other work also write needs a call before each
 * of this layer's M <= 8 forwards that follows such a write. Enqueued on `stream` (a fill
 * kernel, no memset, so it may be captured).
 * Errors: HMOE_ERR_INVALID_ARG, HMOE_ERR_ALIGN, HMOE_ERR_SCRATCH, HMOE_ERR_HIP. */
hmoe_status moe_scratch_init(const hmoe_layer* layer, void* scratch, size_t scratch_bytes,
                             hipStream_t stream);

/* Softmax top-k routing, renormalised. logits: fp32 [M, E] (device). For each token,
 * experts are ranked by logit, descending, ties to the lower expert id; topk_ids
 * int32 [M, k] receives them in that order and topk_w fp32 [M, k] the softmax over
 * the selected logits (= full softmax, top-k, renormalise). M = 0 is a no-op.
 * Errors: HMOE_ERR_INVALID_ARG (M < 0, E outside 1..1024, k outside 1..min(16, E));
 * HMOE_ERR_ALIGN; HMOE_ERR_HIP. */
hmoe_status moe_route(const float* logits, int32_t M, int32_t E, int32_t k,
                      int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Per-tier align for the prefill path: from topk_ids int32 [M, k] (device, values in
 * [0, E)), writes both tiers' align arrays (see hmoe_align_view) and the tier map
 * into scratch. Deterministic; the grid is sized from max_tokens, not from data.
 * Errors: HMOE_ERR_INVALID_ARG, HMOE_ERR_CAPACITY (M > max_tokens), HMOE_ERR_SCRATCH,
 * HMOE_ERR_ALIGN, HMOE_ERR_HIP. */
hmoe_status moe_align(const hmoe_layer* layer, const int32_t* topk_ids, int32_t M,
                      void* scratch, size_t scratch_bytes, hipStream_t stream);

/* Pointers to one tier's align arrays inside scratch (host arithmetic only). */
hmoe_status moe_align_view(const hmoe_layer* layer, void* scratch, int32_t tier,
                           hmoe_align_view* out);

/* Pointers to the decode grouping inside scratch (host arithmetic only). */
hmoe_status moe_decode_view(const hmoe_layer* layer, void* scratch, hmoe_decode_view* out);

/* Pointers to the top-k ids (int32 [max_tokens, k]) and weights (fp32) that
 * hybrid_moe_forward leaves in scratch (host arithmetic only). */
hmoe_status moe_topk_view(const hmoe_layer* layer, void* scratch, int32_t** topk_ids,
                          float** topk_w);

/* The layer forward ([P1] "How it works", [P2] "Summary"): y = sum over each token's
 * top-k experts of w[t, j] * SwiGLU_expert(x[t]), both tiers sharing one routing result
 * and one sum. x: bf16 bits [M, H]; router_logits: fp32 [M, E]; y: bf16 bits [M, H],
 * fully overwritten. M <= 8 takes the decode path: the four launches of
 * hybrid_moe_forward_stage, or, for a layer created with HMOE_DECODE_SINGLE_LAUNCH, one
 * launch (routing in every workgroup, W13 + SwiGLU, W2, and the weighted combine by
 * whichever workgroup finishes a 64-row output group last); both give the same bits. M > 8 takes the prefill path (route, per-tier align, grouped GEMM W13 +
 * SwiGLU, grouped GEMM W2 + weighted combine). M = 0 is a no-op returning HMOE_OK.
 * Never allocates, synchronises or reads back: capturable in a HIP graph at fixed M.
 * The single-launch decode needs its counters in the scratch at zero when it starts:
 * every forward leaves them zero, so a buffer that was zero-filled or passed through
 * moe_scratch_init once needs nothing more, as long as nothing else writes it; after the
 * buffer served another layer (whose regions differ) or any other use, call
 * moe_scratch_init again before this layer's next M <= 8 forward.
 * Errors: HMOE_ERR_INVALID_ARG (null layer/weights, M < 0, a needed weight array NULL),
 * HMOE_ERR_CAPACITY, HMOE_ERR_SCRATCH, HMOE_ERR_ALIGN, HMOE_ERR_HIP. */
hmoe_status hybrid_moe_forward(const hmoe_layer* layer, const hmoe_weights* weights,
                               const uint16_t* x, const float* router_logits, int32_t M,
                               uint16_t* y, void* scratch, size_t scratch_bytes,
                               hipStream_t stream);

/* hybrid_moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the same kernels,
 * with the scratch taken from a fixed 64 MiB array in the library's device memory, one
 * per GPU, held until the process ends (its address is looked up with
 * hipGetSymbolAddress on the first call on each device; the current device must be the
 * stream's). Allocates nothing. All calls on one GPU share that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other threads) race; serialise them.
 * The array keeps the last call's contents: before a single-launch decode forward the
 * call clears that layer's counters (a fill kernel on the stream), so layers of any
 * kind can take turns on it.
 * Arguments and results as hybrid_moe_forward.
 * Errors: HMOE_ERR_SCRATCH when moe_scratch_bytes(layer) exceeds 64 MiB (checked before
 * any device call), HMOE_ERR_HIP when the array's address cannot be obtained, and the
 * errors of hybrid_moe_forward. */
hmoe_status hybrid_moe_forward_static(const hmoe_layer* layer, const hmoe_weights* weights,
                                      const uint16_t* x, const float* router_logits, int32_t M,
                                      uint16_t* y, hipStream_t stream);

/* One stage of the forward, for profiling: with the same arguments, calling
 * HMOE_STAGE_ROUTE, _W13, _W2 and _COMBINE in that order on one stream computes what
 * hybrid_moe_forward computes, bit for bit (for M <= 8 as four launches where the forward
 * may use one). ROUTE is routing plus the per-slot pass records (M <= 8) or
 * routing, the per-tier align and the tokens' conversion to scaled fp16 (M > 8); W13 is
 * the expert up projection with the fused SwiGLU; W2 the down projection with the
 * routing weight; COMBINE the fixed-order top-k sum into y (plus, for M <= 8, the
 * decode grouping of moe_decode_view). Each stage reads what the previous stages left in scratch, so a
 * stage run out of order computes from stale scratch contents (no fault, since every
 * index it reads is bounds-checked or produced by ROUTE for this layer).
 * Errors: as hybrid_moe_forward, plus HMOE_ERR_INVALID_ARG for an unknown stage. */
hmoe_status hybrid_moe_forward_stage(const hmoe_layer* layer, const hmoe_weights* weights,
                                     const uint16_t* x, const float* router_logits, int32_t M,
                                     uint16_t* y, void* scratch, size_t scratch_bytes,
                                     int32_t stage, hipStream_t stream);

/* Test hook: dequantises one whole expert tensor (W13: [2I, H] or W2: [H, I]) of global
 * expert `expert` and writes the canonical values. It shares the format primitives of
 * the forward kernels (the hardware E2M1 and E4M3 conversions, the E8M0 scale, the NF3
 * level constants) but not their decode paths, which fold block scales into 16-bit
 * operands, scaled level tables or fp32 partials and are checked through the layer
 * output. Writes: out_f32 fp32 [rows, K] and/or out_bf16 bf16 bits
 * [rows, K] (either may be NULL). Canonical values: NVFP4 fp32(e2m1 * e4m3) * g (one
 * rounding), MXFP4 e2m1 * 2^(b - 127) (exact), NF3 level[q] * fp16 scale (one
 * rounding); the bf16 form is the fp32 value rounded to nearest even.
 * Errors: HMOE_ERR_INVALID_ARG (expert or tensor out of range, both outputs NULL, the
 * tier's arrays NULL), HMOE_ERR_HIP. */
hmoe_status moe_dequant(const hmoe_layer* layer, const hmoe_weights* weights,
                        int32_t expert, int32_t tensor, float* out_f32, uint16_t* out_bf16,
                        hipStream_t stream);

/* One expert's weight tensors as a checkpoint keeps them, addressed by global expert id
 * (device pointers, owned by the caller, only read). The layer loader of the pages
 * classifies experts by the bit map, loads each tier's tensors and repacks them into the
 * kernels' formats ([P1] review walkthrough: the hybrid quant method's weight loading;
 * [P2] "Summary": compact tier-local storage). Row layouts per expert:
 *   kept tier: w13_q u8 [2I, H/2], w13_s u8 [2I, H/16] (E4M3) or [2I, H/32] (E8M0),
 *              w13_g f32 [1] (NVFP4 only); w2_* likewise with [H, I/...];
 *   NF3 tier:  w13_q = the low code plane u8 [2I, H/4] (element j at bits 2 (j mod 4)
 *              of byte j / 4), w13_hi = the high plane u8 [2I, H/8] (element j at bit
 *              j mod 8 of byte j / 8), code = low | high << 2; w13_s u16 [2I, H/64] fp16
 *              bits; w2_* likewise with [H, I/...]. w13_g / w2_g are not read. */
typedef struct hmoe_expert_src {
    const uint8_t* w13_q;
    const uint8_t* w13_hi;
    const void* w13_s;
    const float* w13_g;
    const uint8_t* w2_q;
    const uint8_t* w2_hi;
    const void* w2_s;
    const float* w2_g;
} hmoe_expert_src;

/* Load-time demux and repack: writes every expert of `experts` (host array of E
 * entries, index = global expert id) into the tier-local arrays of `dst` (device
 * pointers in the layouts of hmoe_weights, allocated by the caller): expert e goes to
 * its tier at index = number of experts below e in the same tier; kept-tier tensors are
 * copied, NF3 code planes become the 3-bit stream of the kernels. Asynchronous on
 * `stream` (batched kernel launches, no allocation); source and destination must not
 * overlap. Errors:
 * HMOE_ERR_INVALID_ARG (null layer/experts/dst, a pointer the expert's tier needs is
 * NULL, dst arrays of a non-empty tier NULL), HMOE_ERR_HIP. */
hmoe_status moe_repack(const hmoe_layer* layer, const hmoe_expert_src* experts,
                       const hmoe_weights* dst, hipStream_t stream);

/* The W4A4 activation quantiser on its own (test hook): rows x K fp32 values (device,
 * K a multiple of 32, row-major) to MXFP4 by the OCP MX v1.0 conversion the layer uses
 * for W4A4 activations ([P3]): per 32-block the shared exponent floor(log2 amax) - 2
 * clamped to [-127, 127] (E8M0 byte 127 for an all-zero block), elements scaled by 2^-e
 * and rounded to E2M1 nearest-even, saturating at 6, zero as code 0. codes: u8 [rows,
 * K/2] (element 2j in the low nibble of byte j); scales: u8 [rows, K/32]. Pointers 16-byte
 * aligned. Errors: HMOE_ERR_INVALID_ARG (rows < 0, K not a positive multiple of 32),
 * HMOE_ERR_ALIGN, HMOE_ERR_HIP. */
hmoe_status moe_quantize_mxfp4(const float* in, int32_t rows, int32_t K, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);

/* Static string naming a status code. */
const char* moe_status_string(hmoe_status status);

/* Thread-local message describing the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HMOE_H */
