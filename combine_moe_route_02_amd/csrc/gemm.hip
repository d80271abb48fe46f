// Token-wise ChunkedEP (Megatron-LM PR 7342, "Numerical status -- unresolved") accumulates the
// router weight gradient across chunks in FP32 and converts it once: each chunk's dlogits^T x is
// computed in FP32 (dlogits = hi + lo with hi, lo BF16, x exactly BF16; the engine kernel in
// router_wgrad.hip), its split-K partials are summed in a fixed order into the FP32 accumulator here,
// and the last chunk converts it once. FP32 SIMT grouped GEMMs serve FP32 payloads; the BF16/FP8
// expert GEMMs live in grouped_gemm.hip.
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace gemm {

constexpr int BK = 64;
constexpr int kMaxGroups = 1024;

// Sum S partial [M, N] FP32 blocks in order into acc (overwrite when first), then optionally
// convert acc once to the payload type.
template <typename TOUT>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part, int S,
                                                              int64_t MN, float* __restrict__ acc,
                                                              bool first, TOUT* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float s = first ? 0.f : acc[i];
  for (int p = 0; p < S; ++p) s += part[(int64_t)p * MN + i];
  acc[i] = s;
  if (out) st_elem<TOUT>(out + i, s);
}

// ---------------------------------------------------------------------------------------------
// FP32 SIMT path (FP32 payloads): same grouping, 64x64 tiles, 4x4 outputs per thread.
enum SimtMode { kGateUp = 0, kDown = 1, kDownBwd = 2, kGateUpBwd = 3 };

struct SimtRowsArgs {
  const float* A; const float* B; float* C; float* C2; const float* aux;
  int64_t lda, ldc, strideB;
  int K, N, I;
  const int32_t* offsets;
  int El, c0, nc;
  int64_t P_c;
  uint32_t zero;  // unused by the SIMT kernels (shared launcher code sets it)
  int one;
};

template <int MODE>
__global__ __launch_bounds__(256) void simt_rows_kernel(SimtRowsArgs a) {
  constexpr int TB = 64, TK = 16;
  __shared__ float sA[TK][TB + 4];
  __shared__ float sB[TK][TB + 4];
  __shared__ int s_pre[kMaxGroups + 1];
  __shared__ int64_t s_r0[kMaxGroups];
  __shared__ int s_len[kMaxGroups];
  constexpr bool kSwiGLU = (MODE == kGateUp);
  constexpr int OUTN = kSwiGLU ? TB / 2 : TB;
  const int tid = threadIdx.x;
  const int G = a.nc * a.El;
  const int ntiles = (a.N + OUTN - 1) / OUTN;
  for (int g = tid; g < G; g += 256) {
    const int c = a.c0 + g / a.El, e = g % a.El;
    const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
    const int len = off[e + 1] - off[e];
    s_r0[g] = (int64_t)c * a.P_c + off[e];
    s_len[g] = len;
    s_pre[g + 1] = ((len + TB - 1) / TB) * ntiles;
  }
  __syncthreads();
  if (tid == 0) { s_pre[0] = 0; for (int g = 0; g < G; ++g) s_pre[g + 1] += s_pre[g]; }
  __syncthreads();
  const int total = s_pre[G];
  const int tx = tid & 15, ty = tid >> 4;  // 16 x 16 threads, 4 x 4 outputs each
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = G;
    while (hi - lo > 1) { int mid = (lo + hi) >> 1; if (s_pre[mid] <= tile) lo = mid; else hi = mid; }
    const int g = lo, e = g % a.El;
    const int t_in = tile - s_pre[g];
    const int mt = t_in / ntiles, nt = t_in % ntiles;
    const int64_t r0 = s_r0[g] + (int64_t)mt * TB;
    const int mvalid = min(TB, s_len[g] - mt * TB);
    const int n0 = nt * OUTN;
    const float* Be = a.B + (int64_t)e * a.strideB;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < a.K; k0 += TK) {
      for (int i = tid; i < TK * TB; i += 256) {
        const int r = i / TK, kk = i % TK;
        sA[kk][r] = r < mvalid ? a.A[(r0 + r) * a.lda + k0 + kk] : 0.f;
        float bv = 0.f;
        if constexpr (kSwiGLU) {
          int j = n0 + (r < 32 ? r : r - 32);
          if (j < a.N) bv = Be[(int64_t)(r < 32 ? j : a.I + j) * a.K + k0 + kk];
        } else if constexpr (MODE == kDownBwd || MODE == kGateUpBwd) {
          if (n0 + r < a.N) bv = Be[(int64_t)(k0 + kk) * a.N + n0 + r];
        } else {
          if (n0 + r < a.N) bv = Be[(int64_t)(n0 + r) * a.K + k0 + kk];
        }
        sB[kk][r] = bv;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < TK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) { av[q] = sA[kk][ty * 4 + q]; bv[q] = sB[kk][tx + 16 * q]; }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(av[p], bv[q], acc[p][q]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int m = ty * 4 + p;
      if (m >= mvalid) continue;
      const int64_t row = r0 + m;
      if constexpr (kSwiGLU) {
        // columns tx + 16q: q = 0,1 gate columns j = n0 + tx + 16q; q = 2,3 the matching up
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = n0 + tx + 16 * q;
          if (j >= a.N) continue;
          const float gv = acc[p][q], uv = acc[p][q + 2];
          a.C[row * a.ldc + j] = gv * sigmoidf_(gv) * uv;
          if (a.C2) { a.C2[row * 2 * (int64_t)a.I + j] = gv; a.C2[row * 2 * (int64_t)a.I + a.I + j] = uv; }
        }
      } else if constexpr (MODE == kDownBwd) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = n0 + tx + 16 * q;
          if (j >= a.N) continue;
          const int64_t I2 = 2 * (int64_t)a.I;
          const float gv = a.aux[row * I2 + j], uv = a.aux[row * I2 + a.I + j];
          const float s = sigmoidf_(gv), dh = acc[p][q];
          a.C[row * I2 + j] = dh * uv * s * (1.f + gv * (1.f - s));
          a.C[row * I2 + a.I + j] = dh * gv * s;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + tx + 16 * q;
          if (n < a.N) a.C[row * a.ldc + n] = acc[p][q];
        }
      }
    }
  }
}

// FP32 SIMT weight gradients / router gradient partials: C[grp][m][n] = sum_rows A[row][m] B[row][n].
struct SimtKArgs {
  const float* A; const float* B; float* C;
  int64_t lda, ldb, strideC;
  int M, N;
  const int32_t* offsets;
  int El, n_chunks;
  int64_t P_c;
  int64_t k0, klen;
  int ksplit;
  bool router;
};

__global__ __launch_bounds__(256) void simt_kgroup_kernel(SimtKArgs a) {
  constexpr int TB = 64, TK = 16;
  __shared__ float sA[TK][TB + 4];
  __shared__ float sB[TK][TB + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int mtiles = (a.M + TB - 1) / TB, ntiles = (a.N + TB - 1) / TB;
  const int grp = blockIdx.x / (mtiles * ntiles);
  const int t_in = blockIdx.x % (mtiles * ntiles);
  const int m0 = (t_in / ntiles) * TB, n0 = (t_in % ntiles) * TB;
  float acc[4][4] = {};
  const int nseg = a.router ? 1 : a.n_chunks;
  for (int sgi = 0; sgi < nseg; ++sgi) {
    int64_t row0;
    int len;
    if (a.router) {
      row0 = a.k0 + (int64_t)grp * a.ksplit;
      int64_t rem = a.k0 + a.klen - row0;
      len = (int)(rem < a.ksplit ? (rem < 0 ? 0 : rem) : a.ksplit);
    } else {
      const int32_t* off = a.offsets + (int64_t)sgi * (a.El + 1);
      row0 = (int64_t)sgi * a.P_c + off[grp];
      len = off[grp + 1] - off[grp];
    }
    for (int k0 = 0; k0 < len; k0 += TK) {
      for (int i = tid; i < TK * TB; i += 256) {
        const int kk = i / TB, c = i % TB;
        const bool kok = k0 + kk < len;
        sA[kk][c] = (kok && m0 + c < a.M) ? a.A[(row0 + k0 + kk) * a.lda + m0 + c] : 0.f;
        sB[kk][c] = (kok && n0 + c < a.N) ? a.B[(row0 + k0 + kk) * a.ldb + n0 + c] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < TK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) { av[q] = sA[kk][ty * 4 + q]; bv[q] = sB[kk][tx + 16 * q]; }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(av[p], bv[q], acc[p][q]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + ty * 4 + p, n = n0 + tx + 16 * q;
      if (m < a.M && n < a.N) a.C[(int64_t)grp * a.strideC + (int64_t)m * a.N + n] = acc[p][q];
    }
}

}  // namespace gemm

// ---------------------------------------------------------------------------------------------
// Launchers
using namespace gemm;

namespace {
constexpr int kSimtGrid = 512;  // persistent grid of the FP32 SIMT kernels
}  // namespace

hipError_t launch_expert_fwd(bool bf16, const void* xd, const void* w1, const void* w2,
                             const int32_t* offsets, void* gu, void* h, void* yd, int H, int I,
                             int El, int c0, int nc, int64_t P_c, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  if (bf16) return gg_expert_fwd_bf16(xd, w1, w2, offsets, gu, h, yd, H, I, El, c0, nc, P_c, s);
  SimtRowsArgs a{};
  a.A = (const float*)xd; a.B = (const float*)w1; a.C = (float*)h; a.C2 = (float*)gu;
  a.lda = H; a.ldc = I; a.strideB = (int64_t)2 * I * H; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c; a.one = 1; a.zero = 0;
  {
    MOE_TRACE("gemm_gateup_swiglu_f32", s);
    MOE_LAUNCH(simt_rows_kernel<kGateUp>, dim3(kSimtGrid), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtRowsArgs b{};
  b.A = (const float*)h; b.B = (const float*)w2; b.C = (float*)yd;
  b.lda = I; b.ldc = H; b.strideB = (int64_t)H * I; b.K = I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c; b.one = 1; b.zero = 0;
  {
    MOE_TRACE("gemm_down_f32", s);
    MOE_LAUNCH(simt_rows_kernel<kDown>, dim3(kSimtGrid), dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

hipError_t launch_expert_dgrad(bool bf16, const void* dyd, const void* gu, const void* w1,
                               const void* w2, const int32_t* offsets, void* dgu, void* dxd, float* dxd_scales,
                               int H, int I, int El, int c0, int nc, int64_t P_c, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  if (bf16) return gg_expert_dgrad_bf16(dyd, gu, w1, w2, offsets, dgu, dxd, dxd_scales, H, I, El, c0, nc, P_c, s);
  if (dxd_scales) return hipErrorInvalidValue;  // FP8 dxd rows are a BF16-path format
  SimtRowsArgs a{};
  a.A = (const float*)dyd; a.B = (const float*)w2; a.C = (float*)dgu; a.aux = (const float*)gu;
  a.lda = H; a.ldc = 2 * I; a.strideB = (int64_t)H * I; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c; a.one = 1; a.zero = 0;
  {
    MOE_TRACE("gemm_down_dgrad_swiglu_f32", s);
    MOE_LAUNCH(simt_rows_kernel<kDownBwd>, dim3(kSimtGrid), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtRowsArgs b{};
  b.A = (const float*)dgu; b.B = (const float*)w1; b.C = (float*)dxd;
  b.lda = 2 * I; b.ldc = H; b.strideB = (int64_t)2 * I * H; b.K = 2 * I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c; b.one = 1; b.zero = 0;
  {
    MOE_TRACE("gemm_gateup_dgrad_f32", s);
    MOE_LAUNCH(simt_rows_kernel<kGateUpBwd>, dim3(kSimtGrid), dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

hipError_t launch_expert_wgrad(bool bf16, const void* dyd, const void* dgu, const void* xd,
                               const void* h, const int32_t* offsets, void* dw1, void* dw2, int H,
                               int I, int El, int n, int64_t P_c, void* wgrad_ws, hipStream_t s) {
  if (El <= 0) return hipSuccess;
  if (bf16) return gg_expert_wgrad_bf16(dyd, dgu, xd, h, offsets, dw1, dw2, H, I, El, n, P_c, wgrad_ws, s);
  SimtKArgs a{};
  a.A = (const float*)dyd; a.B = (const float*)h; a.C = (float*)dw2; a.lda = H; a.ldb = I;
  a.strideC = (int64_t)H * I; a.M = H; a.N = I; a.offsets = offsets; a.El = El; a.n_chunks = n; a.P_c = P_c;
  {
    MOE_TRACE("gemm_wgrad_down_f32", s);
    MOE_LAUNCH(simt_kgroup_kernel, dim3(El * ((H + 63) / 64) * ((I + 63) / 64)), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtKArgs b{};
  b.A = (const float*)dgu; b.B = (const float*)xd; b.C = (float*)dw1; b.lda = 2 * I; b.ldb = H;
  b.strideC = (int64_t)2 * I * H; b.M = 2 * I; b.N = H; b.offsets = offsets; b.El = El; b.n_chunks = n; b.P_c = P_c;
  {
    MOE_TRACE("gemm_wgrad_gateup_f32", s);
    MOE_LAUNCH(simt_kgroup_kernel, dim3(El * ((2 * I + 63) / 64) * ((H + 63) / 64)), dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

int router_ksplit(int64_t tokens) {
  // split the chunk's tokens so that about 256 workgroups run; multiples of the LDS stage
  int64_t per = (tokens + 15) / 16;
  per = ((per + BK - 1) / BK) * BK;
  return (int)(per < BK ? BK : per);
}

// Upper bound of the split count over every chunk length <= Tc: a split holds at least 64
// tokens and there are at most 16 splits.
int64_t router_partials_bytes(int64_t Tc, int E, int H) {
  int64_t S = (Tc + BK - 1) / BK;
  if (S > 16) S = 16;
  if (S < 1) S = 1;
  return S * (int64_t)E * H * (int64_t)sizeof(float);
}

hipError_t launch_router_wgrad(bool bf16, const float* dlogits, const uint16_t* dl_hi, const uint16_t* dl_lo,
                               int ldl, const void* x, float* partials, float* dwr_acc, bool first, void* dwr,
                               int64_t t0, int64_t t1, int E, int H, hipStream_t s) {
  const int64_t len = t1 - t0;
  const int ks = router_ksplit(len);
  int S = (int)((len + ks - 1) / ks);
  if (S < 1) S = 1;
  if (len > 0) {
    if (bf16) {
      if (!dl_hi || !dl_lo) return hipErrorInvalidValue;
      hipError_t e = launch_router_wgrad_planes(dl_hi, dl_lo, ldl, x, partials, t0, len, ks, S, E, H, s);
      if (e != hipSuccess) return e;
    } else {
      SimtKArgs a{};
      a.A = dlogits; a.B = (const float*)x; a.C = partials; a.lda = E; a.ldb = H;
      a.strideC = (int64_t)E * H; a.M = E; a.N = H; a.k0 = t0; a.klen = len; a.ksplit = ks; a.router = true;
      {
        MOE_TRACE("gemm_router_wgrad_f32", s);
        MOE_LAUNCH(simt_kgroup_kernel, dim3(S * ((E + 63) / 64) * ((H + 63) / 64)), dim3(256), 0, s, a);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    S = 0;
  }
  const int64_t MN = (int64_t)E * H;
  dim3 g((unsigned)((MN + 255) / 256));
  if (bf16)
    {
      MOE_TRACE("router_reduce", s);
      MOE_LAUNCH(reduce_partials_kernel<uint16_t>, g, dim3(256), 0, s, partials, S, MN, dwr_acc,
                         first, (uint16_t*)dwr);
    }
  else
    {
      MOE_TRACE("router_reduce", s);
      MOE_LAUNCH(reduce_partials_kernel<float>, g, dim3(256), 0, s, partials, S, MN, dwr_acc,
                         first, (float*)dwr);
    }
  return hipGetLastError();
}

}  // namespace moe
