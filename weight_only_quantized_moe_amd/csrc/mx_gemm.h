// The kept tier's W4A4 grouped-GEMM tile on gfx950's MX-scaled matrix cores (MXFP4
// weights times MXFP4 activations), shared by the launches that run it. vllm-project/vllm
// PR #42428, "What's in this PR": W4A4 backends beside the W4A16 path.
#pragma once

#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMxThreads = 256;
constexpr int kMxBN = 128;   // weight rows per block tile (W13: 64 gate + the 64 matching up rows)
constexpr int kMxBK = 128;   // K per MFMA step: four 32-blocks

struct MxArgs {
  const uint8_t* wq;    // kept-tier codes [E4, rows_w, K/2]
  const uint8_t* ws;    // E8M0 scales [E4, rows_w, K/32]
  int rows_w, K;
  const uint8_t* aq;    // activation codes [arows, K/2]: W13 x per token, W2 h per align row
  const uint8_t* as;    // [arows, K/32]
  int k, nslot;
  const int32_t* slots; // kept-tier align: sorted slots, block -> expert, num_padded
  const int32_t* bexp;
  const int32_t* npad;
  int nblk;             // align blocks this launch covers
  int E4, I, H;
  float* h_out;         // W13: fp32 [cap_kept, I]
  float* o_out;         // W2: fp32 [nslot, H]
  const float* topk_w;
};

// column tiles of a kept-tier W4A4 GEMM: W13 64 h columns per tile, W2 128 outputs
inline int mx_tiles(const Layer& L, bool w13) { return w13 ? L.I / (kMxBN / 2) : L.H / kMxBN; }

// the kept-tier W4A4 GEMM arguments of one stage (HMOE_STAGE_W13 or _W2) at batch M
MxArgs mx_args(const Layer& L, const hmoe_weights& W, int M, void* scratch, int stage);

// Block: BM slot rows of one kept-tier align block x kMxBN weight rows (W13: 64 gate
// rows and the matching 64 up rows, so the block makes 64 h columns; W2: 128 output
// columns). Four waves split it 2 x 2 (1 x 4 for BM = 16); each wave keeps MT x NT
// 16x16 tiles in registers and loads, per 128-K step, one 16-byte fragment and one scale
// byte per tile row and per tile column, the next step's already in flight.
template <int BM, bool W13>
__device__ __forceinline__ void mx_gemm_tile(const MxArgs& a, int blk, int tile) {
  constexpr int WAVES_M = BM >= 32 ? 2 : 1;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int MT = BM / WAVES_M / 16;
  constexpr int NT = kMxBN / WAVES_N / 16;
  if (blk >= a.nblk || blk * BM >= a.npad[0]) return;
  const int loc = a.bexp[blk];
  if ((unsigned)loc >= (unsigned)a.E4) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int j = lane & 15, g = lane >> 4;
  const int r0 = blk * BM;
  const int n0 = tile * (W13 ? kMxBN / 2 : kMxBN);
  const int KB = a.K / 2, SB = a.K / 32;   // code and scale bytes per row

  // tile row (within the block's weight rows) of column tile nt; W13 pairs gate tile nt
  // with up tile nt + NT / 2 in the same lanes
  auto wrow = [&](int nt) {
    if constexpr (W13) {
      constexpr int HALF = NT / 2;
      const int base = wn * (kMxBN / 2 / WAVES_N);
      return nt < HALF ? n0 + base + 16 * nt : a.I + n0 + base + 16 * (nt - HALF);
    } else {
      return n0 + wn * (kMxBN / WAVES_N) + 16 * nt;
    }
  };
  const uint8_t* bq[NT];
  const uint8_t* bs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const size_t row = (size_t)loc * a.rows_w + wrow(nt) + j;
    bq[nt] = a.wq + row * KB + 16 * g;
    bs[nt] = a.ws + row * SB + g;
  }
  // activation rows: W13 the token of the slot (padding rows read row 0; a GEMM never
  // mixes rows and padding outputs are dropped), W2 the align row
  const uint8_t* aqp[MT];
  const uint8_t* asp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = (wm * MT + mt) * 16 + j;
    size_t row;
    if constexpr (W13) {
      const int slot = a.slots[r0 + m];
      row = (unsigned)slot < (unsigned)a.nslot ? (size_t)(slot / a.k) : 0;
    } else {
      row = (size_t)(r0 + m);
    }
    aqp[mt] = a.aq + row * KB + 16 * g;
    asp[mt] = a.as + row * SB + g;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Frag {
    uint4 aq[MT], bq[NT];
    uint32_t as[MT], bs[NT];
  };
  auto load = [&](int st, Frag& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.aq[mt] = *reinterpret_cast<const uint4*>(aqp[mt] + st * (kMxBK / 2));
      f.as[mt] = asp[mt][st * (kMxBK / 32)];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f.bq[nt] = *reinterpret_cast<const uint4*>(bq[nt] + st * (kMxBK / 2));
      f.bs[nt] = bs[nt][st * (kMxBK / 32)];
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const i32x8 av = {(int)f.aq[mt].x, (int)f.aq[mt].y, (int)f.aq[mt].z, (int)f.aq[mt].w, 0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const i32x8 bv = {(int)f.bq[nt].x, (int)f.bq[nt].y, (int)f.bq[nt].z, (int)f.bq[nt].w, 0, 0, 0, 0};
        // operand formats 4 = FP4 (E2M1); scales: E8M0 in byte 0 of each lane's word
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bv, acc[mt][nt], 4, 4, 0, (int)f.as[mt], 0, (int)f.bs[nt]);
      }
    }
  };
  const int steps = a.K / kMxBK;
  Frag f0, f1;
  load(0, f0);
  int st = 0;
  for (; st + 2 <= steps; st += 2) {
    load(st + 1, f1);
    mma(f0);
    if (st + 2 < steps) load(st + 2, f0);
    mma(f1);
  }
  if (st < steps) mma(f0);

  // epilogue: lane holds rows 4 g + q of each 16-row tile, column j
#pragma unroll
  for (int nt = 0; nt < (W13 ? NT / 2 : NT); ++nt) {
    const int n = wrow(nt) + j;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = (wm * MT + mt) * 16 + 4 * g + q;
        if constexpr (W13) {
          const float gate = acc[mt][nt][q], up = acc[mt][nt + NT / 2][q];
          a.h_out[(size_t)(r0 + m) * a.I + n] = silu(gate) * up;
        } else {
          const int slot = a.slots[r0 + m];
          if ((unsigned)slot < (unsigned)a.nslot)
            a.o_out[(size_t)slot * a.H + n] = acc[mt][nt][q] * a.topk_w[slot];
        }
      }
    }
  }
}

}  // namespace hmoe
