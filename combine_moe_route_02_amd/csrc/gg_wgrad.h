// Shared pieces of the BF16 expert weight gradients (wgrad.hip: the split-capable lists;
// rows_wgrad.hip: the row-grouped GEMM merged with the light experts' dW2 tiles): the argument
// block, the output staging, the split threshold and the scratch layout.
#pragma once
#include "gg_engine.h"

namespace moe {
namespace gg {

struct WgradArgs {
  const uint16_t* A;      // [P, M]
  const uint16_t* B;      // [P, N]
  uint16_t* C;            // per expert [M, N]
  int64_t lda, ldb, strideC;
  int M, N;
  const int32_t* offsets; // per-chunk local offsets
  int El, n_chunks;
  int64_t P_c;
  float* part;            // partial slots (FP32 tiles), may be null when slots = 0
  int* cnt;               // per (expert, tile) arrival counters, zero between launches
  int slots;
  // a split list's next-item counter, then its exit counter (zero between launches)
  int* queue;
  // 1: only the experts whose rows exceed the split threshold Ks0 (the layer schedule computes the
  // others' tiles in the merged row-grouped launch before this one)
  int heavy_only;
};

// Waves that issue the weight gradients' operand loads: one per SIMD, right after the stage
// barrier, so that the other wave of each SIMD goes on issuing MFMAs while the loading wave waits
// to issue its loads (both operands of a weight gradient are K-slow).
constexpr int kWgradLoadWaves = kWaves / 2;
constexpr int kWgradMinSplitRows = 512;  // never split an expert's K below this many rows
constexpr int kWgradRefWorkers = 256;    // workers the split size is planned for

template <int BM, int BN>
MOE_DEV int wgrad_tiles_per_expert(const WgradArgs& a) { return ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN); }

// Split threshold before any doubling: Ks0 = max(kWgradMinSplitRows, ceil(total rows x tiles per
// expert / kWgradRefWorkers)). Experts with more rows are the "heavy" ones.
MOE_DEV long long wgrad_ks0(long long total, int T) {
  const long long k = (total * T + kWgradRefWorkers - 1) / kWgradRefWorkers;
  return k < kWgradMinSplitRows ? kWgradMinSplitRows : k;
}

// Accumulator group gq of block (tm, tn) of this lane (four consecutive columns of one row) into the
// BF16 staging tile in LDS.
template <int BM, int BN>
MOE_DEV void wgrad_stage4(char* ring, int tm, int tn, int gq, float a0, float a1, float a2, float a3, int lane,
                          int wave) {
  constexpr int WTM = BM / kWM, WTN = BN / kWN;
  const int wm = wave / kWN, wn = wave % kWN;
  const int row = wm * WTM + tm * 32 + out_row(lane);
  const int nl = wn * WTN + tn * 32 + out_col(gq, lane);
  *(uint2*)(ring + row * pitch<BN>() + 2 * nl) = pack4(a0, a1, a2, a3);
}

// Store the staged tile as BF16 rows of C[grp] (the ring holds it).
template <int BM, int BN>
MOE_DEV void wgrad_store(const WgradArgs& a, int grp, int m0, int n0, char* ring, int tid) {
  lds_barrier();
  store_staged<BM, BN, true>(ring, a.C + (int64_t)grp * a.strideC + (int64_t)m0 * a.N + n0, a.N,
                             min(BM, a.M - m0), min(BN, a.N - n0), tid);
  lds_barrier();
}

}  // namespace gg

using gg::WgradArgs;

// Weight-gradient partial slots: 256 x 256 FP32 tiles of dW1 and of dW2 after the counter area
// (launch.h: gemm_queue).
constexpr int kWgradTile = 256;
constexpr int kWgradSlots = 192;  // partial tiles per weight gradient at most
inline int64_t wgrad_slots(int64_t tiles_per_expert, int El) {
  const int64_t cap = 4 * tiles_per_expert * El;
  return cap < kWgradSlots ? cap : kWgradSlots;
}
inline int64_t wgrad_counter_bytes(int H, int I, int El) {
  return (((int64_t)El * (wgrad_tiles_1(H, I) + wgrad_tiles_2(H, I)) + kQueueBlocks * kQueueInts) * 4 + 255) / 256 * 256;
}


// dW1[e] [2I, H] = sum dgu^T xd (the longer tile list, first) and dW2[e] [H, I] = sum dyd^T h
inline void wgrad_args(const ExpertGemm& g, WgradArgs& w1, WgradArgs& w2) {
  w1 = WgradArgs{};
  w1.A = (const uint16_t*)g.dgu; w1.B = (const uint16_t*)g.xd; w1.C = (uint16_t*)g.dw1; w1.lda = 2 * g.I;
  w1.ldb = g.H; w1.strideC = (int64_t)2 * g.I * g.H; w1.M = 2 * g.I; w1.N = g.H; w1.offsets = g.offsets;
  w1.El = g.El; w1.n_chunks = g.n_chunks; w1.P_c = g.P_c;
  w2 = WgradArgs{};
  w2.A = (const uint16_t*)g.dyd; w2.B = (const uint16_t*)g.h; w2.C = (uint16_t*)g.dw2; w2.lda = g.H;
  w2.ldb = g.I; w2.strideC = (int64_t)g.H * g.I; w2.M = g.H; w2.N = g.I; w2.offsets = g.offsets;
  w2.El = g.El; w2.n_chunks = g.n_chunks; w2.P_c = g.P_c;
  if (g.wgrad_ws && g.El > 0) {
    char* ws = (char*)g.wgrad_ws;
    const int64_t t1 = wgrad_tiles_1(g.H, g.I), t2 = wgrad_tiles_2(g.H, g.I);
    const int64_t slot = (int64_t)kWgradTile * kWgradTile;  // floats
    w1.cnt = (int*)ws;
    w2.cnt = (int*)ws + g.El * t1;
    w1.queue = gemm_queue(g, kQueueWgrad1);
    w2.queue = gemm_queue(g, kQueueWgrad2);
    float* parts = (float*)(ws + wgrad_counter_bytes(g.H, g.I, g.El));
    w1.slots = (int)wgrad_slots(t1, g.El);
    w2.slots = (int)wgrad_slots(t2, g.El);
    w1.part = parts;
    w2.part = parts + w1.slots * slot;
  }
}

}  // namespace moe
