// The layer schedule's merged launch of the last chunk's gate/up dgrad with dW2 (dW2[e] = sum over
// the rows of every chunk of expert e of dyd^T h, one FP32 K loop, one BF16 conversion): the dW2
// tiles fill the dgrad's last round. It takes the experts whose rows do not exceed the weight
// gradients' split threshold Ks0 (every expert under balanced routing); the heavier ones, which
// the weight-gradient launch that follows splits along K, are left to it (wgrad.hip, heavy_only).
// A light expert's tile is the same K loop over the same rows as in wgrad.hip, so the results are
// bitwise those of the stage call.
//
// Kept in a translation unit of its own, without the split reduction: with that code in the same
// kernel or module the compiler kept fewer of the row-grouped K loop's LDS addresses in registers
// (six more address adds per stage) and the launch took 8% longer.
#include "gg_wgrad.h"

namespace moe {
namespace gg {

// Tile `tile` (expert-major) of a weight gradient over all of its expert's rows; after_k runs once
// its K loops are done (before the staging of the result).
template <int BM, int BN, class AfterK>
MOE_DEV void wgrad_tile_full(const WgradArgs& a, int grp, int t_in, char* ring, int tid, int lane, int wave,
                             AfterK&& after_k) {
  constexpr int WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  const int wm = wave / kWN, wn = wave % kWN;
  const int ntiles = (a.N + BN - 1) / BN;
  const int m0 = (t_in / ntiles) * BM, n0 = (t_in % ntiles) * BN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  for (int c = 0; c < a.n_chunks; ++c) {
    const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
    const int o0 = __builtin_amdgcn_readfirstlane(off[grp]);
    const int len = __builtin_amdgcn_readfirstlane(off[grp + 1]) - o0;
    if (len <= 0) continue;
    const int64_t row0 = (int64_t)c * a.P_c + o0;
    Loader<BM, true, kWgradLoadWaves> la;
    la.init_kslow(a.A + row0 * a.lda + m0, a.lda * 2, ((int64_t)len * a.lda - m0) * 2, wave, lane);
    Loader<BN, true, kWgradLoadWaves> lb;
    lb.init_kslow(a.B + row0 * a.ldb + n0, a.ldb * 2, ((int64_t)len * a.ldb - n0) * 2, wave, lane);
    const int nks = (len + kKRows - 1) / kKRows;
    kloop<false, true, true, BM, BN, TM, TN, TM>(la, lb, ring, nks, wm * WTM, wn * WTN, lane, acc);
  }
  after_k();
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x16_t& v = acc[tm][tn];
        wgrad_stage4<BM, BN>(ring, tm, tn, gq, v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3], lane, wave);
      }
  wgrad_store<BM, BN>(a, grp, m0, n0, ring, tid);
}

// The light experts' tiles (expert-major, ceil(items / 8) per XCD as in the unsplit weight
// gradient; the heavy experts' slots stay empty). Round robin: in the slot sequence of rows_list
// from per-XCD slot `first` on; returns the slot after the last. With a queue (a.queue) every
// workgroup takes its XCD's slots from an atomic counter (fetched after each tile's K loops: a
// returning atomic in flight would hold back the K loop's load counts), and the last workgroup to
// leave resets the counters.
template <int BM, int BN>
MOE_DEV int wgrad_list_light(const WgradArgs& a, int first, char* ring, int* q) {
  if (a.El <= 0) return first;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = wgrad_tiles_per_expert<BM, BN>(a);
  const int items = a.El * T, px = (items + 7) / 8;
  long long total = 0;
  for (int c = 0; c < a.n_chunks; ++c) total += a.offsets[(int64_t)c * (a.El + 1) + a.El];
  const long long Ks0 = wgrad_ks0(total, T);
  const int xcd = blockIdx.x % 8, wg_per_xcd = gridDim.x / 8;
  int* const queue = a.queue;
  if (queue) {
    __syncthreads();  // every thread has read *q in the list before
    if (tid == 0) *q = atomicAdd(queue + xcd, 1);
  }
  int slot = first_slot(first) - first;
  for (;;) {
    if (queue) {
      __syncthreads();
      slot = *q;
      __syncthreads();  // every thread has read it before the next write
    }
    if (slot >= px) break;
    int nxt = 0;
    auto fetch_next = [&] {
      if (queue && tid == 0) nxt = atomicAdd(queue + xcd, 1);
    };
    const int item = xcd * px + slot;
    int e = -1, ke = 0;
    if (item < items) {
      e = item / T;
      for (int c = 0; c < a.n_chunks; ++c) {
        const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
        ke += off[e + 1] - off[e];
      }
    }
    if (e >= 0 && ke <= Ks0)  // heavy experts: the weight-gradient launch that follows splits them
      wgrad_tile_full<BM, BN>(a, e, item - e * T, ring, tid, lane, wave, fetch_next);
    else
      fetch_next();
    if (queue) {
      if (tid == 0) *q = nxt;
    } else {
      slot += wg_per_xcd;
    }
  }
  if (queue) {
    if (tid == 0 && atomicAdd(queue + 8, 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int x = 0; x < 9; ++x) queue[x] = 0;
    }
    return first;
  }
  return first + px;
}

template <int BM1, int BN1, int MODE1, int BM, int BN, bool Q1>
__global__ __launch_bounds__(kThreads) void rows_wgrad_kernel(RowsArgs r, WgradArgs a) {
  __shared__ RowsShared sh;
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int f = rows_list<BM1, BN1, MODE1, false, Q1>(r, 0, sh, ring);
  wgrad_list_light<BM, BN>(a, f, ring, &sh.q);
}

template <int BM1, int BN1, int MODE1, int BM, int BN>
static hipError_t run_rows_wgrad(const char* name, const RowsArgs& r, const WgradArgs& a, hipStream_t s) {
  const size_t l1 = rows_lds_bytes<BM1, BN1, MODE1>(), l2 = wgrad_lds_bytes<BM, BN>();
  const size_t lds = l1 > l2 ? l1 : l2;
  constexpr bool kQ = (MODE1 == kDown || MODE1 == kGateUpBwd) && BN1 == 256;
  auto k = (kQ && r.Cq) ? rows_wgrad_kernel<BM1, BN1, MODE1, BM, BN, kQ>
                        : rows_wgrad_kernel<BM1, BN1, MODE1, BM, BN, false>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tw = a.El > 0 ? (int64_t)a.El * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) : 0;
  const int64_t grid = persistent_grid(rows_tiles_bound<BM1, BN1, MODE1>(r) + tw);
  if (grid <= 0) return hipSuccess;
  {
    MOE_TRACE(name, s);
    MOE_LAUNCH(k, dim3((unsigned)grid), dim3(kThreads), lds, s, r, a);
  }
  return hipGetLastError();
}

}  // namespace gg

using namespace gg;

hipError_t gg_gateup_dgrad_then_wgrad2(const ExpertGemm& g, int c, hipStream_t s) {
  WgradArgs w1, w2;
  wgrad_args(g, w1, w2);
  // both lists from work queues (a queue for the row tiles alone, with the dW2 tiles then dealt
  // round robin from slot 0, measured 151 against 132 us for round robin throughout)
  RowsArgs r = gateup_dgrad_args(g, c, 1);
  r.queue = gemm_queue(g, kQueueRows1);
  w2.queue = gemm_queue(g, kQueueRows2);
  return run_rows_wgrad<MOE_GUDGRAD, 256, 256>("gemm_gateup_dgrad+wgrad_w2", r, w2, s);
}

}  // namespace moe
