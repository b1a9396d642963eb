// The kept tier's W4A4 grouped-GEMM tile on gfx950's MX-scaled matrix cores (MXFP4
// weights times MXFP4 activations), shared by the launches that run it. vllm-project/vllm
// PR #42428, "What's in this PR": W4A4 backends beside the W4A16 path.
#pragma once

#include <type_traits>

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
  float* row_fac;       // [cap_kept]: each align row's routing weight (0 for padding),
                        // written by W13's first column tile, read by W2
};

// column tiles of a kept-tier W4A4 GEMM: W13 64 h columns per tile, W2 128 outputs
inline int mx_tiles(const Layer& L, bool w13) { return w13 ? L.I / (kMxBN / 2) : L.H / kMxBN; }

// the kept-tier W4A4 GEMM arguments of one stage (HMOE_STAGE_W13 or _W2) at batch M
MxArgs mx_args(const Layer& L, const hmoe_weights& W, int M, void* scratch, int stage);

// Block: BM slot rows of one kept-tier align block x kMxBN weight rows (W13: 64 gate
// rows and the matching 64 up rows, so the block makes 64 h columns; W2: 128 output
// columns). Four waves split it 2 x 2 (1 x 4 up to 32 rows, so that no two waves load
// the same weight fragments); each wave keeps MT x NT 16x16 tiles in registers and
// loads, per 128-K step, one 16-byte fragment per tile row and per tile column, the next
// step's already in flight, and the E8M0 bytes of its rows (see below).
template <int BM, bool W13>
__device__ __forceinline__ void mx_gemm_tile(const MxArgs& a, int blk, int tile) {
  constexpr int WAVES_M = BM >= 64 ? 2 : 1;
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
  // W2: the epilogue's rows (slot and routing weight), requested now so that their
  // latency hides under the K loop instead of adding to the tile's end (up to 64-row
  // tiles; the 128-row tile has no registers to spare and loads them at the end)
  constexpr bool PRE = !W13 && MT <= 2;
  int eslot[PRE ? MT : 1][4];
  float efac[PRE ? MT : 1][4];
  if constexpr (PRE) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = (wm * MT + mt) * 16 + 4 * g + q;
        eslot[mt][q] = a.slots[r0 + m];
        efac[mt][q] = a.row_fac[r0 + m];
      }
  }

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
  // Tiles of up to 32 rows, whose waves issue one scale load per MFMA or more, with
  // scale rows of whole, aligned 16-byte vectors (K a multiple of 512): a lane's E8M0
  // bytes of four consecutive steps (byte g of dword i is block g of step 4 q + i) come
  // in one 16-byte load per tile row and tile column, a quarter of the scale loads.
  // Every load of that loop is unconditional (steps past the last re-read the last
  // group), so the compiler's waits count exactly the loads each use needs.
  const bool vs = BM <= 32 && SB % 16 == 0 && (reinterpret_cast<uintptr_t>(a.as) % 16) == 0 &&
                  (reinterpret_cast<uintptr_t>(a.ws) % 16) == 0;
  if (BM <= 32 && vs) {
    struct Codes {
      uint4 aq[MT], bq[NT];
    };
    struct SVec {
      uint4 a[MT], b[NT];
    };
    auto load_codes = [&](int st, Codes& c) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c.aq[mt] = *reinterpret_cast<const uint4*>(aqp[mt] + st * (kMxBK / 2));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) c.bq[nt] = *reinterpret_cast<const uint4*>(bq[nt] + st * (kMxBK / 2));
    };
    // the rows' scale vectors of steps 4 q .. 4 q + 3 (asp / bs point at byte g)
    auto load_sv = [&](int q, SVec& v) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) v.a[mt] = *reinterpret_cast<const uint4*>(asp[mt] - g + 16 * q);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) v.b[nt] = *reinterpret_cast<const uint4*>(bs[nt] - g + 16 * q);
    };
    auto word = [](const uint4& v, auto I) -> uint32_t {
      if constexpr (decltype(I)::value == 0) return v.x;
      else if constexpr (decltype(I)::value == 1) return v.y;
      else if constexpr (decltype(I)::value == 2) return v.z;
      else return v.w;
    };
    auto mma_v = [&](const Codes& c, const SVec& v, auto I) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x8 av = {(int)c.aq[mt].x, (int)c.aq[mt].y, (int)c.aq[mt].z, (int)c.aq[mt].w, 0, 0, 0, 0};
        const int sa = (int)__builtin_amdgcn_ubfe(word(v.a[mt], I), 8 * g, 8);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const i32x8 bv = {(int)c.bq[nt].x, (int)c.bq[nt].y, (int)c.bq[nt].z, (int)c.bq[nt].w, 0, 0, 0, 0};
          const int sb = (int)__builtin_amdgcn_ubfe(word(v.b[nt], I), 8 * g, 8);
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt][nt], 4, 4, 0,
                                                                          sa, 0, sb);
        }
      }
    };
    const int last = steps - 1, nq = steps / 4;
    Codes c0, c1;
    SVec v0, v1;
    load_sv(0, v0);
    load_codes(0, c0);
    for (int q = 0; q < nq; ++q) {
      const int st = 4 * q;
      load_sv(min(q + 1, nq - 1), v1);
      load_codes(st + 1, c1);
      mma_v(c0, v0, std::integral_constant<int, 0>{});
      load_codes(st + 2, c0);
      mma_v(c1, v0, std::integral_constant<int, 1>{});
      load_codes(st + 3, c1);
      mma_v(c0, v0, std::integral_constant<int, 2>{});
      load_codes(min(st + 4, last), c0);
      mma_v(c1, v0, std::integral_constant<int, 3>{});
      v0 = v1;
    }
  } else {
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
  }

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
          const int slot = PRE ? eslot[PRE ? mt : 0][q] : a.slots[r0 + m];
          const float fac = PRE ? efac[PRE ? mt : 0][q] : a.row_fac[r0 + m];
          if ((unsigned)slot < (unsigned)a.nslot)
            a.o_out[(size_t)slot * a.H + n] = acc[mt][nt][q] * fac;
        }
      }
    }
  }
  // W13's first column tile: the rows' routing weights for the W2 epilogue (at the end,
  // where the two dependent loads delay only this one tile of the align block)
  if constexpr (W13) {
    if (tile == 0) {
      for (int t = threadIdx.x; t < BM; t += kMxThreads) {
        const int slot = a.slots[r0 + t];
        a.row_fac[r0 + t] = (unsigned)slot < (unsigned)a.nslot ? a.topk_w[slot] : 0.0f;
      }
    }
  }
}

}  // namespace hmoe
