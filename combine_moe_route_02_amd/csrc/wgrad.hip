// BF16 expert weight gradients on CDNA4 matrix cores: dW1[e] = dG/dU_e^T xd_e and dW2[e] = dyd_e^T h_e
// over the rows of every chunk of expert e, one FP32 K loop per tile (or per split of it), one BF16
// conversion (the FP32-accumulate-then-convert rule that token-wise ChunkedEP, Megatron-LM PR 7342,
// "Numerical status -- unresolved", states for the router weights). Built on the grouped-GEMM
// engine of gg_engine.h; kept in a translation unit of its own so that its register-heavy split
// reduction does not change the code generated for the row-grouped kernels.
#include "gg_wgrad.h"

namespace moe {
namespace gg {

// Weight gradients: C_e[m][n] = sum over the rows of every chunk of expert e of A[row][m] B[row][n]
// (both operands K-slow), accumulated in FP32 across the chunks' segments, converted once.
//
// Balance under imbalanced routing: an expert's K (its rows over every chunk) may be many times
// another's, so a tile's K loop is split when the expert holds more rows than one worker's share of
// the whole gradient. The plan depends only on the per-expert row counts (not on the launch), so
// every launch that computes a gradient gives bitwise the same result:
//   * Ks = max(kWgradMinSplitRows, ceil(total rows x tiles per expert / kWgradRefWorkers)), doubled
//     until the split experts' partial tiles fit the partial slots;
//   * expert e runs s_e = ceil(K_e / Ks) splits per tile; with q = floor(K_e / s_e) and
//     r = K_e mod s_e, split s covers its rows [s q + min(s, r), (s + 1) q + min(s + 1, r)) of the
//     concatenated chunk segments (the first r splits take one row more);
//   * an unsplit tile converts its FP32 sum to BF16 directly; a split writes its FP32 partial
//     tile to a slot, and the last split to arrive (a per-tile counter) sums the partials in split
//     order, converts once, and resets the counter to zero (the counters must be zero when first
//     used; every launch leaves them zero).
// When some expert is split, items (expert, split, tile) are ordered by descending expert rows and
// dealt to the XCDs in contiguous ranges of equal row cost, so the tiles of one expert share an
// XCD's L2 where they can (that static dealing serves the lists without a split). Items of a split
// list differ in cost by orders of magnitude, so the workgroups take them from one queue (an atomic
// counter) as they become free: the largest first, each to the first free workgroup, so that no
// workgroup holds two of the largest items while others idle (measured: with static or per-XCD
// dealing, the XCDs holding the heaviest expert's splits ran two of them on most of their
// workgroups and finished last). Which workgroup computes an item does not change its result. The
// last workgroup to leave the list resets the counters for the next launch.
// Split plan of one weight gradient, rebuilt in LDS by every workgroup. With no split expert (the
// usual case) only K and the per-wave partials are written: item i is then tile i % T of expert
// i / T, and each XCD takes ceil(items / 8) consecutive items (whole rounds of equal-cost tiles).
struct WgradPlan {
  int K[kMaxGroups];         // rows of expert e over every chunk
  int order[kMaxGroups];     // experts by descending rows, then by index
  int ipre[kMaxGroups + 1];  // items before the o-th expert of the order
  int spre[kMaxGroups];      // first partial slot of expert e (-1: not split)
  int xfirst[9];             // first item of each XCD's range
  int wsum[kWaves], wmax[kWaves];  // per-wave partial total and maximum of K
  int red[4];                // reductions and the last-arrival flag
};

MOE_DEV int block_sum_to(int v, int* dst) {  // adds v of every thread into *dst (zeroed before)
  v = wave_sum_int(v);
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(dst, v);
  return v;
}

// Builds the plan; returns Ks (then below the largest K_e, so it fits an int), 0 when no expert
// is split (then only p.K is written), or -1 for a heavy_only list without a heavy expert (no
// items). A heavy_only list takes the experts above Ks0 only, split or not; its Ks and splits are
// those of the full list, so either computes a heavy expert's tiles bitwise alike.
template <int BM, int BN>
MOE_DEV int wgrad_plan(const WgradArgs& a, WgradPlan& p) {
  const int tid = threadIdx.x, El = a.El, T = wgrad_tiles_per_expert<BM, BN>(a);
  __syncthreads();  // a previous list of this launch may still read the LDS it shares with the plan
  int part = 0, kmax = 0;
  for (int e = tid; e < El; e += kThreads) {
    int k = 0;
    for (int c = 0; c < a.n_chunks; ++c) {
      const int32_t* off = a.offsets + (int64_t)c * (El + 1);
      k += off[e + 1] - off[e];
    }
    p.K[e] = k;
    part += k;
    kmax = max(kmax, k);
  }
  part = wave_sum_int(part);
  kmax = wave_max_int(kmax);
  if ((tid & 63) == 0) {
    p.wsum[tid >> 6] = part;
    p.wmax[tid >> 6] = kmax;
  }
  __syncthreads();
  long long total = 0;
  kmax = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    total += p.wsum[w];
    kmax = max(kmax, p.wmax[w]);
  }
  const long long Ks0 = wgrad_ks0(total, T);
  long long Ks = Ks0;
  if (kmax <= Ks0) return a.heavy_only ? -1 : 0;  // uniform: every thread read the same partials
  if (tid < 4) p.red[tid] = 0;
  __syncthreads();
  int tot = 0;
  for (;;) {  // the same bound on every thread: uniform exit
    if (tid == 0) p.red[1] = 0;
    __syncthreads();
    int need = 0;
    for (int e = tid; e < El; e += kThreads) {
      const long long sp = (p.K[e] + Ks - 1) / Ks;
      if (sp > 1) need += (int)sp * T;
    }
    block_sum_to(need, &p.red[1]);
    __syncthreads();
    tot = p.red[1];
    __syncthreads();
    if (tot <= a.slots) break;
    Ks *= 2;
  }
  if (tot == 0 && !a.heavy_only) return 0;  // the slots forced a split size above every expert's rows
  // the heaviest experts first
  for (int e = tid; e < El; e += kThreads) {
    const int ke = p.K[e];
    int r = 0;
    for (int f = 0; f < El; ++f) {
      const int kf = p.K[f];
      r += (kf > ke || (kf == ke && f < e)) ? 1 : 0;
    }
    p.order[r] = e;
  }
  __syncthreads();
  if (tid == 0) {
    int ip = 0, sp = 0;
    for (int o = 0; o < El; ++o) {
      const int e = p.order[o];
      const int se = (int)((p.K[e] + Ks - 1) / Ks);
      const int s1 = (a.heavy_only && p.K[e] <= Ks0) ? 0 : (se > 1 ? se : 1);
      p.ipre[o] = ip;
      ip += s1 * T;
      p.spre[e] = se > 1 ? sp : -1;
      sp += se > 1 ? se * T : 0;
    }
    p.ipre[El] = ip;
  }
  __syncthreads();
  // XCD x takes the items whose cost midpoint lies in [x C / 8, (x + 1) C / 8), the cost of an
  // item being the rows of its split (at least 1: an empty expert's tiles still write zeros)
  if (tid < 9) {
    long long C = 0;
    for (int o = 0; o < El; ++o) {
      const int ke = p.K[p.order[o]];
      const long long se = (a.heavy_only && ke <= Ks0) ? 0 : ke > Ks ? (ke + Ks - 1) / Ks : 1;
      long long c = se ? (ke + se - 1) / se : 1;
      if (c < 1) c = 1;
      C += se * T * c;
    }
    long long cpre = 0, n = 0;
    for (int o = 0; o < El; ++o) {
      const int ke = p.K[p.order[o]];
      const long long se = (a.heavy_only && ke <= Ks0) ? 0 : ke > Ks ? (ke + Ks - 1) / Ks : 1;
      long long c = se ? (ke + se - 1) / se : 1;
      if (c < 1) c = 1;
      const long long items = se * T;
      // item j's midpoint cpre + (j + 1/2) c lies below tid C / 8  <=>  16 c j < 2 tid C - 16 cpre - 8 c
      const long long R = 2LL * tid * C - 16 * cpre - 8 * c;
      long long cnt = R <= 0 ? 0 : (R + 16 * c - 1) / (16 * c);
      if (cnt > items) cnt = items;
      n += cnt;
      cpre += items * c;
    }
    p.xfirst[tid] = (int)n;
  }
  __syncthreads();
  return (int)Ks;
}

// One work item: tile t of expert e, split s of se, over rows [k_lo, k_hi) of the expert's chunk
// segments taken in chunk order.
template <int BM, int BN>
MOE_DEV void wgrad_item(const WgradArgs& a, WgradPlan& p, int e, int s, int se, int t, int k_lo, int k_hi,
                        char* ring, int tid, int lane, int wave) {
  constexpr int WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  const int wm = wave / kWN, wn = wave % kWN;
  const int ntiles = (a.N + BN - 1) / BN;
  const int m0 = (t / ntiles) * BM, n0 = (t % ntiles) * BN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  int cum = 0;  // rows of this expert in the chunks before c
  for (int c = 0; c < a.n_chunks; ++c) {
    const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
    const int o0 = __builtin_amdgcn_readfirstlane(off[e]);
    const int seg = __builtin_amdgcn_readfirstlane(off[e + 1]) - o0;
    const int lo = k_lo > cum ? k_lo : cum, hi = k_hi < cum + seg ? k_hi : cum + seg;
    if (hi > lo) {
      const int64_t row0 = (int64_t)c * a.P_c + o0 + (lo - cum);
      const int len = hi - lo;
      Loader<BM, true, kWgradLoadWaves> la;
      la.init_kslow(a.A + row0 * a.lda + m0, a.lda * 2, ((int64_t)len * a.lda - m0) * 2, wave, lane);
      Loader<BN, true, kWgradLoadWaves> lb;
      lb.init_kslow(a.B + row0 * a.ldb + n0, a.ldb * 2, ((int64_t)len * a.ldb - n0) * 2, wave, lane);
      const int nks = (len + kKRows - 1) / kKRows;
      kloop<false, true, true, BM, BN, TM, TN, TM>(la, lb, ring, nks, wm * WTM, wn * WTN, lane, acc);
    }
    cum += seg;
  }

  if (se <= 1) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x16_t& v = acc[tm][tn];
          wgrad_stage4<BM, BN>(ring, tm, tn, gq, v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3], lane, wave);
        }
    wgrad_store<BM, BN>(a, e, m0, n0, ring, tid);
    return;
  }
  // Split: the FP32 partial tile, each lane's 4-register groups stored contiguously per wave
  // (the last split reads back, per thread, the elements it holds itself).
  constexpr int NG = TM * TN * 4;  // 4-register groups per lane
  const int T = wgrad_tiles_per_expert<BM, BN>(a);
  const int64_t slot0 = p.spre[e] + (int64_t)t;
  auto group_ptr = [&](int sp, int g) {
    return (float4*)(a.part + (slot0 + (int64_t)sp * T) * (BM * BN)) + ((int64_t)wave * NG + g) * 64 + lane;
  };
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x16_t& v = acc[tm][tn];
        *group_ptr(s, (tm * TN + tn) * 4 + gq) = make_float4(v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]);
      }
  __threadfence();  // this thread's partial is visible device-wide before the arrival count
  __syncthreads();
  if (tid == 0) p.red[2] = (atomicAdd(a.cnt + e * T + t, 1) == se - 1) ? 1 : 0;
  __syncthreads();
  const bool last = p.red[2] != 0;
  __syncthreads();
  if (!last) return;
  __threadfence();  // the other splits' partials are visible before they are read
  // sum the partials in split order (the result does not depend on which split arrives last),
  // four values at a time, straight into the BF16 staging tile
#pragma unroll 1
  for (int g = 0; g < NG; ++g) {
    float4 v = *group_ptr(0, g);
#pragma unroll 1
    for (int sp = 1; sp < se; ++sp) {
      const float4 w = *group_ptr(sp, g);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    const int gq = g & 3, tn = (g >> 2) % TN, tm = (g >> 2) / TN;
    wgrad_stage4<BM, BN>(ring, tm, tn, gq, v.x, v.y, v.z, v.w, lane, wave);
  }
  if (tid == 0) a.cnt[e * T + t] = 0;  // ready for the next launch
  wgrad_store<BM, BN>(a, e, m0, n0, ring, tid);
}

// The items of one weight gradient (a.El = 0: none) from per-XCD slot `first` on, in the slot
// sequence of rows_list. Returns the slot after the last. Every thread of the workgroup calls it.
template <int BM, int BN>
MOE_DEV int wgrad_list(const WgradArgs& a, int first, char* ring, WgradPlan& p) {
  if (a.El <= 0) return first;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Ks = wgrad_plan<BM, BN>(a, p);
  if (Ks < 0) return first;  // the plan depends only on the offsets: the same on every workgroup
  const int T = wgrad_tiles_per_expert<BM, BN>(a);
  const int xcd = blockIdx.x % 8, wg_per_xcd = gridDim.x / 8;
  // item -> (expert, split, tile) and its rows
  auto run_item = [&](int item) {
    int e, j;
    if (Ks == 0) {
      e = item / T;
      j = item - e * T;
    } else {
      int lo = 0, hi = a.El;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.ipre[mid] <= item) lo = mid; else hi = mid;
      }
      e = p.order[lo];
      j = item - p.ipre[lo];
    }
    e = __builtin_amdgcn_readfirstlane(e);
    j = __builtin_amdgcn_readfirstlane(j);
    const int ke = __builtin_amdgcn_readfirstlane(p.K[e]);
    const int se = (Ks > 0 && ke > Ks) ? ke / Ks + (ke % Ks != 0) : 1;
    const int sp = j / T;
    // split sp of se covers rows [sp q + min(sp, r), (sp + 1) q + min(sp + 1, r)), q = ke / se,
    // r = ke mod se (the first r splits take one row more)
    const int q = ke / se, r = ke - q * se;
    const int k_lo = sp * q + min(sp, r), k_hi = k_lo + q + (sp < r ? 1 : 0);
    wgrad_item<BM, BN>(a, p, e, sp, se, j - sp * T, k_lo, k_hi, ring, tid, lane, wave);
  };
  if (Ks > 0 && a.queue) {
    const int n_items = p.xfirst[8];
    for (;;) {  // every thread sees the same index: uniform exit
      if (tid == 0) p.red[3] = atomicAdd(a.queue, 1);
      __syncthreads();
      const int item = p.red[3];
      __syncthreads();
      if (item >= n_items) break;
      run_item(item);
    }
    // this workgroup takes no more items of the list; the last one to leave resets the counters
    if (tid == 0 && atomicAdd(a.queue + 1, 1) == (int)gridDim.x - 1) {
      a.queue[0] = 0;
      a.queue[1] = 0;
    }
    return first;
  }
  int maxc, lo_item, hi_item;
  if (Ks == 0) {  // no split: expert-major tiles, ceil(items / 8) per XCD
    const int items = a.El * T;
    maxc = (items + 7) / 8;
    lo_item = min(items, xcd * maxc);
    hi_item = min(items, lo_item + maxc);
  } else {
    maxc = 0;
    for (int x = 0; x < 8; ++x) maxc = max(maxc, p.xfirst[x + 1] - p.xfirst[x]);
    lo_item = p.xfirst[xcd];
    hi_item = p.xfirst[xcd + 1];
  }
  for (int gs = first_slot(first); gs < first + maxc; gs += wg_per_xcd) {
    const int item = lo_item + (gs - first);
    if (item >= hi_item) continue;
    run_item(item);
  }
  return first + maxc;
}

// Up to two independent weight gradients in one persistent launch, so the second fills the
// first one's last round. TAG only names the launch (0: the stage call, 1: the layer's last
// weight-gradient launch), so that profiles tell the two apart.
template <int BM, int BN, int TAG>
__global__ __launch_bounds__(kThreads) void wgrad_kernel(WgradArgs a, WgradArgs b) {
  __shared__ WgradPlan plan;
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int f = wgrad_list<BM, BN>(a, 0, ring, plan);
  wgrad_list<BM, BN>(b, f, ring, plan);
}

// ---------------------------------------------------------------------------------------------
// Launchers

template <int BM, int BN, int TAG>
hipError_t run_wgrad(const char* name, const WgradArgs& a, const WgradArgs& b, hipStream_t s) {
  const size_t lds = wgrad_lds_bytes<BM, BN>();
  auto k = wgrad_kernel<BM, BN, TAG>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  auto tiles = [](const WgradArgs& w) {  // items at most: every tile once, plus the split partials
    return w.El > 0 ? (int64_t)w.El * ((w.M + BM - 1) / BM) * ((w.N + BN - 1) / BN) + w.slots : 0;
  };
  const int64_t grid = persistent_grid(tiles(a) + tiles(b));
  if (grid <= 0) return hipSuccess;
  {
    MOE_TRACE(name, s);
    MOE_LAUNCH(k, dim3((unsigned)grid), dim3(kThreads), lds, s, a, b);
  }
  return hipGetLastError();
}

}  // namespace gg

using namespace gg;

int64_t wgrad_scratch_bytes(int H, int I, int El) {
  if (El <= 0) return 0;
  const int64_t slot = (int64_t)kWgradTile * kWgradTile * 4;
  return wgrad_counter_bytes(H, I, El) +
         (wgrad_slots(wgrad_tiles_1(H, I), El) + wgrad_slots(wgrad_tiles_2(H, I), El)) * slot;
}
int64_t wgrad_counter_bytes_of(int H, int I, int El) { return El > 0 ? wgrad_counter_bytes(H, I, El) : 0; }

hipError_t gg_expert_wgrad_bf16(const void* dyd, const void* dgu, const void* xd, const void* h,
                                const int32_t* offsets, void* dw1, void* dw2, int H, int I, int El,
                                int n, int64_t P_c, void* wgrad_ws, hipStream_t s) {
  ExpertGemm g{};
  g.dyd = dyd; g.dgu = (void*)dgu; g.xd = xd; g.h = (void*)h; g.offsets = offsets; g.dw1 = dw1; g.dw2 = dw2;
  g.H = H; g.I = I; g.El = El; g.n_chunks = n; g.P_c = P_c; g.wgrad_ws = wgrad_ws;
  WgradArgs a, b;
  wgrad_args(g, a, b);
  return run_wgrad<256, 256, 0>("gemm_wgrad", a, b, s);
}

// The layer's last weight-gradient launch: the dW2 tiles of the experts above the split threshold
// (rows_wgrad.hip computed the others beside the last gate/up dgrad), then every dW1 tile. The
// heavy dW2 list (empty under balanced routing) goes first so that its large items are not left
// for the end of the launch behind dW1's small ones.
hipError_t gg_wgrad1(const ExpertGemm& g, hipStream_t s) {
  WgradArgs w1, w2;
  wgrad_args(g, w1, w2);
  w2.heavy_only = 1;
  return run_wgrad<256, 256, 1>("gemm_wgrad_w1", w2, w1, s);
}

}  // namespace moe
