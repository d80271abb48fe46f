// Grouped expert GEMMs on CDNA4 matrix cores: BF16 (v_mfma_f32_32x32x16_bf16) and FP8 e4m3
// (v_mfma_f32_32x32x64_f8f6f4) with FP32 accumulation, for the expert FFN forward, its input
// gradients and the expert weight gradients.
//
// The expert FFN is a grouped GEMM whose groups are the local experts' row segments in the
// expert-contiguous dispatch buffer (token-wise ChunkedEP, Megatron-LM PR 7342, "Summary": expert
// compute per token chunk). Group sizes exist only on the device (the offset table written by
// routing): every workgroup rebuilds the group -> tile prefix in LDS and walks its share of the
// tiles (persistent, at most one workgroup per CU); nothing returns to the host. Weight gradients
// iterate K over the rows of every chunk of one expert in one FP32 reduction and convert once
// (the FP32-accumulate-then-convert rule that ChunkedEP's "Numerical status -- unresolved" states
// for the router weights). One launch may carry the tile lists of two independent GEMMs (the
// layer schedule's merged launches): the second list's tiles continue the first's round robin,
// so the CUs that the first leaves idle in its last round start the second.
//
// The shared engine (operand ring, K loop, staging, tile walk) is in gg_engine.h; the BF16 weight
// gradients are in wgrad.hip.
#include "gg_engine.h"

namespace moe {
namespace gg {

template <int BM, int BN, int MODE, bool FP8, bool QOUT, bool GATHER>
__global__ __launch_bounds__(kThreads) void rows_kernel(RowsArgs a) {
  __shared__ RowsShared sh;
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  rows_list<BM, BN, MODE, FP8, QOUT, GATHER>(a, 0, sh, ring);
}

// Two independent row-grouped GEMMs in one persistent launch: the second's tiles fill the
// workgroups that the first leaves idle in its last round, and one kernel boundary goes away.
// Q1 / Q2: that list writes block-scaled FP8 rows. G1: the first list (a gate/up GEMM) reads its
// token rows through src_token.
template <int BM1, int BN1, int MODE1, int BM2, int BN2, int MODE2, bool Q1, bool Q2, bool G1 = false>
__global__ __launch_bounds__(kThreads) void rows_pair_kernel(RowsArgs a, RowsArgs b) {
  __shared__ RowsShared sh;
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int f = rows_list<BM1, BN1, MODE1, false, Q1, G1>(a, 0, sh, ring);
  rows_list<BM2, BN2, MODE2, false, Q2>(b, f, sh, ring);
}

// FP8 weight gradients. Both operands hold, per expert, the columns of its rows (every chunk's)
// quantised per column and stored transposed: A [M][Kp_e] at byte koff_e * M, B [N][Kp_e] at
// koff_e * N (expert_k; rows past K_e are zero codes), so both are K-major like the forward
// operands. C[e] = s_a[e][m] * s_b[e][n] * sum_k A[m][k] B[n][k], one FP32 K loop, one BF16 store.
struct WgradFp8Args {
  const uint8_t* A;
  const uint8_t* B;
  const float* sa;        // [El][M]
  const float* sb;        // [El][N]
  uint16_t* C;            // per expert [M, N]
  int64_t strideC;
  int M, N;
  const int32_t* offsets;
  int El, n_chunks;
};

template <int BM, int BN>
MOE_DEV void wgrad_fp8_tile(const WgradFp8Args& a, int tile, char* ring, int tid, int lane, int wave) {
  constexpr int WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  const int wm = wave / kWN, wn = wave % kWN;
  const int mtiles = (a.M + BM - 1) / BM, ntiles = (a.N + BN - 1) / BN;
  const int grp = tile / (mtiles * ntiles);
  const int t_in = tile % (mtiles * ntiles);
  const int m0 = (t_in / ntiles) * BM, n0 = (t_in % ntiles) * BN;
  int64_t koff;
  int K;
  expert_k(a.offsets, a.El, a.n_chunks, grp, koff, K);
  const int Kp = __builtin_amdgcn_readfirstlane((K + 63) & ~63);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;
  if (Kp > 0) {
    Loader<BM, false, kWaves, true> la;
    la.init_kmajor(a.A + koff * a.M + (int64_t)m0 * Kp, Kp, (int64_t)(a.M - m0) * Kp, wave, lane,
                   [](int r) { return r; });
    Loader<BN, false, kWaves, true> lb;
    lb.init_kmajor(a.B + koff * a.N + (int64_t)n0 * Kp, Kp, (int64_t)(a.N - n0) * Kp, wave, lane,
                   [](int r) { return r; });
    kloop_pairs<true, BM, BN, TM, TN, TM>(la, lb, ring, Kp / 64, wm * WTM, wn * WTN, lane, acc);
  }

  const int mrow = wm * WTM + out_row(lane);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const float sr = a.sa[(int64_t)grp * a.M + min(m0 + mrow + tm * 32, a.M - 1)];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int nl = wn * WTN + tn * 32 + out_col(gq, lane);
        const f32x16_t& v = acc[tm][tn];
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = v[4 * gq + q] * sr * a.sb[(int64_t)grp * a.N + min(n0 + nl + q, a.N - 1)];
        *(uint2*)(ring + (mrow + tm * 32) * pitch<BN>() + 2 * nl) = pack4(o[0], o[1], o[2], o[3]);
      }
  }
  lds_barrier();
  store_staged<BM, BN, true>(ring, a.C + (int64_t)grp * a.strideC + (int64_t)m0 * a.N + n0, a.N,
                             min(BM, a.M - m0), min(BN, a.N - n0), tid);
  lds_barrier();
}

template <int BM, int BN>
MOE_DEV int wgrad_fp8_list(const WgradFp8Args& a, int first, char* ring) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ta = a.El > 0 ? a.El * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) : 0;
  const int pxa = (ta + 7) / 8;
  const int xcd = blockIdx.x % 8, wg_per_xcd = gridDim.x / 8;
  for (int gs = first_slot(first); gs < first + pxa; gs += wg_per_xcd) {
    const int tile = xcd * pxa + (gs - first);
    if (tile < ta) wgrad_fp8_tile<BM, BN>(a, tile, ring, tid, lane, wave);
  }
  return first + pxa;
}

// dW1 and dW2 on FP8 in one persistent launch (dW1's longer list first).
template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void wgrad_fp8_kernel(WgradFp8Args a, WgradFp8Args b) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int f = wgrad_fp8_list<BM, BN>(a, 0, ring);
  wgrad_fp8_list<BM, BN>(b, f, ring);
}

// ---------------------------------------------------------------------------------------------
// Launchers

// Grid bound: per chunk at most floor(P_c / BM) + E_local row tiles (every expert adds at most
// one partial tile) times the column tiles; the device-side count decides the work.
// QOUT: a.Cq set (block-scaled FP8 output, plain-store modes only).
template <int BM, int BN, int MODE, bool FP8>
hipError_t run_rows(const char* name, const RowsArgs& a, hipStream_t s) {
  const size_t lds = rows_lds_bytes<BM, BN, MODE>();
  constexpr bool kQ = (MODE == kDown || MODE == kGateUpBwd) && BN == 256;
  constexpr bool kG = MODE == kGateUp && !FP8;
  auto k = (kQ && a.Cq)       ? rows_kernel<BM, BN, MODE, FP8, kQ, false>
           : (kG && a.gather) ? rows_kernel<BM, BN, MODE, FP8, false, kG>
                              : rows_kernel<BM, BN, MODE, FP8, false, false>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int outn = (MODE == kGateUp) ? BN / 2 : BN;
  const int64_t ntiles = (a.N + outn - 1) / outn;
  const int64_t mtiles = (int64_t)a.nc * (a.P_c / BM + a.El);
  const int64_t grid = persistent_grid(mtiles * ntiles);
  if (grid <= 0) return hipSuccess;
  {
    MOE_TRACE(name, s);
    MOE_LAUNCH(k, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace gg

using namespace gg;

template <int BM1, int BN1, int MODE1, int BM2, int BN2, int MODE2>
static hipError_t run_pair(const char* name, const RowsArgs& a, const RowsArgs& b, hipStream_t s) {
  const size_t l1 = rows_lds_bytes<BM1, BN1, MODE1>(), l2 = rows_lds_bytes<BM2, BN2, MODE2>();
  const size_t lds = l1 > l2 ? l1 : l2;
  // FP8 output rows: only the second list of a pair has them (the gate/up dgrad's dxd)
  constexpr bool kQ2 = (MODE2 == kDown || MODE2 == kGateUpBwd) && BN2 == 256;
  constexpr bool kG1 = MODE1 == kGateUp;
  if (a.Cq || (a.gather && !kG1) || b.gather) return hipErrorInvalidValue;
  auto k = (kQ2 && b.Cq)    ? rows_pair_kernel<BM1, BN1, MODE1, BM2, BN2, MODE2, false, kQ2>
           : (kG1 && a.gather) ? rows_pair_kernel<BM1, BN1, MODE1, BM2, BN2, MODE2, false, false, kG1>
                               : rows_pair_kernel<BM1, BN1, MODE1, BM2, BN2, MODE2, false, false>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t grid = persistent_grid(rows_tiles_bound<BM1, BN1, MODE1>(a) + rows_tiles_bound<BM2, BN2, MODE2>(b));
  if (grid <= 0) return hipSuccess;
  {
    MOE_TRACE(name, s);
    MOE_LAUNCH(k, dim3((unsigned)grid), dim3(kThreads), lds, s, a, b);
  }
  return hipGetLastError();
}

hipError_t gg_expert_fwd_bf16(const void* xd, const void* w1, const void* w2, const int32_t* offsets,
                              void* gu, void* h, void* yd, int H, int I, int El, int c0, int nc,
                              int64_t P_c, hipStream_t s) {
  ExpertGemm g{};
  g.xd = xd; g.w1 = w1; g.w2 = w2; g.offsets = offsets; g.gu = gu; g.h = h; g.yd = yd;
  g.H = H; g.I = I; g.El = El; g.P_c = P_c;
  hipError_t e = run_rows<MOE_GATEUP, false>("gemm_gateup_swiglu", gateup_args(g, c0, nc), s);
  if (e != hipSuccess) return e;
  return run_rows<MOE_DOWN, false>("gemm_down", down_args(g, c0, nc), s);
}

hipError_t gg_expert_dgrad_bf16(const void* dyd, const void* gu, const void* w1, const void* w2,
                                const int32_t* offsets, void* dgu, void* dxd, float* dxd_scales, int H, int I,
                                int El, int c0, int nc, int64_t P_c, hipStream_t s) {
  ExpertGemm g{};
  g.dyd = dyd; g.gu = (void*)gu; g.w1 = w1; g.w2 = w2; g.offsets = offsets; g.dgu = dgu; g.dxd = dxd;
  g.dxd_scales = dxd_scales;
  g.H = H; g.I = I; g.El = El; g.P_c = P_c;
  hipError_t e = run_rows<MOE_DDGRAD, false>("gemm_down_dgrad_swiglu", down_dgrad_args(g, c0, nc), s);
  if (e != hipSuccess) return e;
  return run_rows<MOE_GUDGRAD, false>("gemm_gateup_dgrad", gateup_dgrad_args(g, c0, nc), s);
}

// Launches of the layer schedule (one chunk each; the pairs take independent work of two steps).
// Their lists take tiles from the work queues in the expert-GEMM scratch: a workgroup that drew
// short tiles takes more, so a launch ends closer to its mean workgroup time. A pair runs the list
// with the longer tiles first and the shorter tiles fill the end (measured with per-tile timing:
// with round-robin slots the pairs ended 11-21 us after their mean workgroup).
static RowsArgs queued(RowsArgs a, const ExpertGemm& g, int which) {
  a.queue = gemm_queue(g, which);
  return a;
}
hipError_t gg_gateup(const ExpertGemm& g, int c, hipStream_t s) {
  return run_rows<MOE_GATEUP, false>("gemm_gateup_swiglu", queued(gateup_args(g, c, 1), g, kQueueRows1), s);
}
hipError_t gg_gateup_gather(const ExpertGemm& g, int c, const void* x, const int32_t* src_token, int64_t T,
                            hipStream_t s) {
  RowsArgs a = queued(gateup_args(g, c, 1), g, kQueueRows1);
  a.A = x;
  a.gather = src_token;
  a.gather_rows = T;
  return run_rows<MOE_GATEUP, false>("gemm_gateup_swiglu", a, s);
}
hipError_t gg_down(const ExpertGemm& g, int c, hipStream_t s) {
  return run_rows<MOE_DOWN, false>("gemm_down", queued(down_args(g, c, 1), g, kQueueRows1), s);
}
hipError_t gg_down_then_gateup(const ExpertGemm& g, int c, int c2, hipStream_t s) {
  return run_pair<MOE_GATEUP, MOE_DOWN>("gemm_down+gateup_swiglu",
                                        queued(gateup_args(g, c2, 1), g, kQueueRows1),
                                        queued(down_args(g, c, 1), g, kQueueRows2), s);
}
hipError_t gg_down_then_gateup_gather(const ExpertGemm& g, int c, int c2, const void* x, const int32_t* src_token,
                                      int64_t T, hipStream_t s) {
  RowsArgs a = queued(gateup_args(g, c2, 1), g, kQueueRows1);
  a.A = x;
  a.gather = src_token;
  a.gather_rows = T;
  return run_pair<MOE_GATEUP, MOE_DOWN>("gemm_down+gateup_swiglu", a, queued(down_args(g, c, 1), g, kQueueRows2),
                                        s);
}
hipError_t gg_down_dgrad(const ExpertGemm& g, int c, hipStream_t s) {
  return run_rows<MOE_DDGRAD, false>("gemm_down_dgrad_swiglu", queued(down_dgrad_args(g, c, 1), g, kQueueRows1), s);
}
hipError_t gg_gateup_dgrad_then_down_dgrad(const ExpertGemm& g, int c, int c2, hipStream_t s) {
  return run_pair<MOE_DDGRAD, MOE_GUDGRAD>("gemm_gateup_dgrad+down_dgrad_swiglu",
                                           queued(down_dgrad_args(g, c2, 1), g, kQueueRows1),
                                           queued(gateup_dgrad_args(g, c, 1), g, kQueueRows2), s);
}

// FP8 forward: gate/up on FP8 MFMA with s_row * s_col dequantisation and SwiGLU -> h (BF16);
// h quantised per row to e4m3 (codes stored after the BF16 values in the h buffer); down on FP8
// MFMA -> yd (BF16).
hipError_t launch_expert_fwd_fp8(const void* xd, const float* xd_scale, const void* w1,
                                 const float* w1_scale, const void* w2, const float* w2_scale,
                                 const int32_t* offsets, void* h, float* h_scale, void* yd, int H,
                                 int I, int El, int c0, int nc, int64_t P_c, int64_t P, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  uint8_t* hq = (uint8_t*)h + P * (int64_t)I * 2;  // codes after the BF16 values
  RowsArgs a{};
  a.A = xd; a.B = w1; a.C = (uint16_t*)h; a.C2 = nullptr;
  a.scale_a = xd_scale; a.scale_b = w1_scale; a.strideSB = 2 * (int64_t)I;
  a.lda = H; a.ldc = I; a.strideB = (int64_t)2 * I * H; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
  hipError_t e = run_rows<256, 256, kGateUp, true>("gemm_gateup_swiglu_fp8", a, s);
  if (e != hipSuccess) return e;
  e = launch_quantize_segments_fp8("quantize_h_fp8", h, hq, h_scale, offsets, El, c0, nc, P_c, I, s);
  if (e != hipSuccess) return e;
  RowsArgs b{};
  b.A = hq; b.B = w2; b.C = (uint16_t*)yd;
  b.scale_a = h_scale; b.scale_b = w2_scale; b.strideSB = H;
  b.lda = I; b.ldc = H; b.strideB = (int64_t)H * I; b.K = I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
  return run_rows<256, 256, kDown, true>("gemm_down_fp8", b, s);
}

// The weight gradients' FP8 operands that do not wait for the input gradients: dyd, h and xd.
hipError_t launch_wgrad_fp8_operands(const void* dyd, const void* xd, const void* h, const int32_t* offsets,
                                     void* dyd_t, float* dyd_cs, void* xd_t, float* xd_cs, void* h_t, float* h_cs,
                                     int H, int I, int El, int n, int64_t P_c, hipStream_t s) {
  hipError_t e = launch_quantize_expert_cols_fp8("quantize_dyd_cols_fp8", dyd, dyd_t, dyd_cs, offsets, El, n, P_c, H, s);
  if (e == hipSuccess) e = launch_quantize_expert_cols_fp8("quantize_h_cols_fp8", h, h_t, h_cs, offsets, El, n, P_c, I, s);
  if (e == hipSuccess) e = launch_quantize_expert_cols_fp8("quantize_xd_cols_fp8", xd, xd_t, xd_cs, offsets, El, n, P_c, H, s);
  return e;
}

// FP8 weight gradients: dyd, h, dgu and xd quantised per column over each expert's rows and stored
// transposed (expert_k layout), then dW1[e] = dgu_e^T xd_e and dW2[e] = dyd_e^T h_e on FP8 MFMA in one
// launch.
hipError_t launch_expert_wgrad_fp8(const void* dyd, const void* dgu, const void* xd, const void* h,
                                   const int32_t* offsets, void* dyd_t, float* dyd_cs, void* dgu_t,
                                   float* dgu_cs, void* xd_t, float* xd_cs, void* h_t, float* h_cs, void* dw1,
                                   void* dw2, int H, int I, int El, int n, int64_t P_c, hipStream_t s,
                                   bool quantize) {
  if (El <= 0) return hipSuccess;
  if (quantize) {
    hipError_t e = launch_wgrad_fp8_operands(dyd, xd, h, offsets, dyd_t, dyd_cs, xd_t, xd_cs, h_t, h_cs, H, I, El, n,
                                             P_c, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_quantize_expert_cols_fp8("quantize_dgu_cols_fp8", dgu, dgu_t, dgu_cs, offsets, El, n, P_c,
                                                 2 * (int64_t)I, s);
  if (e != hipSuccess) return e;
  WgradFp8Args a{}, b{};
  a.A = (const uint8_t*)dgu_t; a.B = (const uint8_t*)xd_t; a.sa = dgu_cs; a.sb = xd_cs; a.C = (uint16_t*)dw1;
  a.strideC = (int64_t)2 * I * H; a.M = 2 * I; a.N = H; a.offsets = offsets; a.El = El; a.n_chunks = n;
  b.A = (const uint8_t*)dyd_t; b.B = (const uint8_t*)h_t; b.sa = dyd_cs; b.sb = h_cs; b.C = (uint16_t*)dw2;
  b.strideC = (int64_t)H * I; b.M = H; b.N = I; b.offsets = offsets; b.El = El; b.n_chunks = n;
  const size_t lds = wgrad_lds_bytes<256, 256>();
  auto k = wgrad_fp8_kernel<256, 256>;
  e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = (int64_t)El * (((2 * I + 255) / 256) * ((H + 255) / 256) + ((H + 255) / 256) * ((I + 255) / 256));
  const int64_t grid = persistent_grid(tiles);
  if (grid <= 0) return hipSuccess;
  {
    MOE_TRACE("gemm_wgrad_fp8", s);
    MOE_LAUNCH(k, dim3((unsigned)grid), dim3(kThreads), lds, s, a, b);
  }
  return hipGetLastError();
}

// FP8 input gradients: dyd quantised per row (FP32 steps of dispatch); dh = deq(dyd) deq(W2t)^T on
// FP8 MFMA with the SwiGLU gradient in the epilogue -> dgu (BF16); dgu quantised per row; dxd =
// deq(dgu) deq(W1t)^T on FP8 MFMA -> BF16. W2t [El][I][H] and W1t [El][H][2I] hold the weights'
// columns as rows (per-column scales), so both products read K-contiguous operands, like the
// forward ones.
hipError_t launch_expert_dgrad_fp8(const void* dyd, const void* gu, const void* w1t, const float* w1t_scale,
                                   const void* w2t, const float* w2t_scale, const int32_t* offsets,
                                   void* dyd_q, float* dyd_scale, void* dgu, void* dgu_q, float* dgu_scale,
                                   void* dxd, float* dxd_scales, int H, int I, int El, int c0, int nc, int64_t P_c,
                                   hipStream_t s, bool quantize_dyd) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (quantize_dyd) {
    e = launch_quantize_segments_fp8("quantize_dyd_fp8", dyd, dyd_q, dyd_scale, offsets, El, c0, nc, P_c, H, s);
    if (e != hipSuccess) return e;
  }
  RowsArgs a{};
  a.A = dyd_q; a.B = w2t; a.C = (uint16_t*)dgu; a.aux = (const uint16_t*)gu;
  a.scale_a = dyd_scale; a.scale_b = w2t_scale; a.strideSB = I;
  a.lda = H; a.ldc = 2 * (int64_t)I; a.strideB = (int64_t)I * H; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
  e = run_rows<128, 256, kDownBwd, true>("gemm_down_dgrad_swiglu_fp8", a, s);
  if (e != hipSuccess) return e;
  e = launch_quantize_segments_fp8("quantize_dgu_fp8", dgu, dgu_q, dgu_scale, offsets, El, c0, nc, P_c, 2 * I, s);
  if (e != hipSuccess) return e;
  RowsArgs b{};
  b.A = dgu_q; b.B = w1t;
  if (dxd_scales) {  // block-scaled FP8 dxd
    b.Cq = (uint8_t*)dxd; b.Cs = dxd_scales; b.ldcs = (H + 255) / 256;
  } else {
    b.C = (uint16_t*)dxd;
  }
  b.scale_a = dgu_scale; b.scale_b = w1t_scale; b.strideSB = H;
  b.lda = 2 * (int64_t)I; b.ldc = H; b.strideB = (int64_t)H * 2 * I; b.K = 2 * I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
  return run_rows<256, 256, kDown, true>("gemm_gateup_dgrad_fp8", b, s);
}

}  // namespace moe
