// Router weight gradient on the expert GEMM engine: dW_r = dlogits^T x over a chunk's tokens, with
// the FP32 dlogits split into BF16 high and low parts (x = hi + lo + O(2^-17 x); x itself is exactly
// BF16), both K-slow like x. Each workgroup takes one output tile and one token range of the split-K
// partition, runs the weight gradients' K loop (K-slow operands through the LDS ring, transposing
// fragment reads) over the range, and writes the range's partial sum [S, E, H], which
// reduce_partials_kernel adds in range order. Above 128 experts: 128 x 256 tiles, a pass over the
// high plane and then one over the low plane into the same FP32 accumulator.
#include "gg_wgrad.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace gg {

struct RouterPlaneArgs {
  const uint16_t* hi;  // [len, ldl] BF16 high parts of the chunk's dlogits rows
  const uint16_t* lo;  // [len, ldl] low parts
  const uint16_t* x;   // [T, H]
  float* part;         // [S, E, H]
  int64_t t0, len;     // token range of the chunk
  int ks, ldl, E, H;   // tokens per split, plane pitch
};

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void router_wgrad_planes_kernel(RouterPlaneArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  constexpr int WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int mt = (a.E + BM - 1) / BM, nt = (a.H + BN - 1) / BN;
  const int tile = blockIdx.x % (mt * nt), s = blockIdx.x / (mt * nt);
  const int m0 = (tile / nt) * BM, n0 = (tile % nt) * BN;
  const int64_t r0 = a.t0 + (int64_t)s * a.ks;
  const int64_t rem = a.t0 + a.len - r0;
  const int len = (int)(rem < a.ks ? rem : a.ks);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  if (len > 0) {
    const int nks = (len + kKRows - 1) / kKRows;
    // K-rows past the range and columns past the plane's last row read zeros (descriptor extent);
    // columns m >= E of a K-row read the next K-rows' values, which reach only rows never stored
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      Loader<BM, true, kWgradLoadWaves> la;
      la.init_kslow((p ? a.lo : a.hi) + (r0 - a.t0) * a.ldl + m0, (int64_t)a.ldl * 2, ((int64_t)len * a.ldl - m0) * 2, wave,
                    lane);
      Loader<BN, true, kWgradLoadWaves> lb;
      lb.init_kslow(a.x + r0 * a.H + n0, (int64_t)a.H * 2, ((int64_t)len * a.H - n0) * 2, wave, lane);
      kloop<false, true, true, BM, BN, TM, TN, TM>(la, lb, ring, nks, wm * WTM, wn * WTN, lane, acc);
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m0 + wm * WTM + tm * 32 + out_row(lane);
    if (m >= a.E) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + tn * 32 + out_col(g, lane);
        if (n >= a.H) continue;
        const f32x16_t& v = acc[tm][tn];
        *(float4*)(a.part + ((int64_t)s * a.E + m) * a.H + n) =
            make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
  }
}

// Up to 128 experts the high and low planes sit side by side ([tokens, 256], the low part at column
// 128) and form one 256-row A operand, so a single K pass of a 256 x 256 tile covers both parts with
// a third fewer load bytes per MFMA than two passes of a 128-row tile. Tile rows 128 + e hold the
// low parts' sums: the second wave row stages them in LDS after the K loop and the first adds them
// to the high parts' sums (FP32) before the store.
template <int BN>
__global__ __launch_bounds__(kThreads) void router_wgrad_paired_kernel(RouterPlaneArgs a) {
  constexpr int BM = 256, WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  constexpr int kPitch = BN + 4;  // FP32 staging row pitch (floats)
  static_assert(WTM == 128, "wave row 0 holds the high parts, wave row 1 the low parts");
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int nt = (a.H + BN - 1) / BN;
  const int s = blockIdx.x / nt, n0 = (blockIdx.x % nt) * BN;
  const int64_t r0 = a.t0 + (int64_t)s * a.ks;
  const int64_t rem = a.t0 + a.len - r0;
  const int len = (int)(rem < a.ks ? rem : a.ks);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  if (len > 0) {
    Loader<BM, true, kWgradLoadWaves> la;
    la.init_kslow(a.hi + (r0 - a.t0) * 256, 512, (int64_t)len * 512, wave, lane);
    Loader<BN, true, kWgradLoadWaves> lb;
    lb.init_kslow(a.x + r0 * a.H + n0, (int64_t)a.H * 2, ((int64_t)len * a.H - n0) * 2, wave, lane);
    kloop<false, true, true, BM, BN, TM, TN, TM>(la, lb, ring, (len + kKRows - 1) / kKRows, wm * WTM, wn * WTN,
                                                 lane, acc);
  }
  // the ring is free (the K loop ends with a barrier after its last LDS reads)
  float* st = (float*)ring;
  if (wm == 1) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& v = acc[tm][tn];
          const int r = tm * 32 + out_row(lane), c = wn * WTN + tn * 32 + out_col(g, lane);
          *(float4*)(st + r * kPitch + c) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
        }
  }
  __syncthreads();
  if (wm == 0) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int m = tm * 32 + out_row(lane);
      if (m >= a.E) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wn * WTN + tn * 32 + out_col(g, lane), n = n0 + c;
          if (n >= a.H) continue;
          const f32x16_t& v = acc[tm][tn];
          const float4 l = *(const float4*)(st + m * kPitch + c);
          *(float4*)(a.part + ((int64_t)s * a.E + m) * a.H + n) =
              make_float4(v[4 * g] + l.x, v[4 * g + 1] + l.y, v[4 * g + 2] + l.z, v[4 * g + 3] + l.w);
        }
    }
  }
}

}  // namespace gg

hipError_t launch_router_wgrad_planes(const uint16_t* hi, const uint16_t* lo, int ldl, const void* x, float* partials,
                                      int64_t t0, int64_t len, int ks, int S, int E, int H, hipStream_t s) {
  using namespace gg;
  constexpr int BM = 128, BN = 256;
  if (len <= 0 || S <= 0) return hipSuccess;
  if (ldl % 8 || ldl < E || H % 64) return hipErrorInvalidValue;
  if (E <= 128) {
    // side by side: the low plane starts 128 columns after the high one, rows of 256
    if (ldl != 128 || lo != hi + 128) return hipErrorInvalidValue;
    const size_t ring = (size_t)kNst * (256 + BN) * kRowB, ep = (size_t)128 * (BN + 4) * sizeof(float);
    const size_t lds = ring > ep ? ring : ep;
    auto k = router_wgrad_paired_kernel<BN>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    RouterPlaneArgs a{hi, lo, (const uint16_t*)x, partials, t0, len, ks, ldl, E, H};
    {
      MOE_TRACE("gemm_router_wgrad", s);
      MOE_LAUNCH(k, dim3((unsigned)(S * ((H + BN - 1) / BN))), dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
  }
  const size_t lds = (size_t)kNst * (BM + BN) * kRowB;
  auto k = router_wgrad_planes_kernel<BM, BN>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  RouterPlaneArgs a{hi, lo, (const uint16_t*)x, partials, t0, len, ks, ldl, E, H};
  const int tiles = ((E + BM - 1) / BM) * ((H + BN - 1) / BN);
  {
    MOE_TRACE("gemm_router_wgrad", s);
    MOE_LAUNCH(k, dim3((unsigned)(S * tiles)), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
