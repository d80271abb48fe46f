// Row-copy kernels of the layer share: dispatch, combine and their transposes, plus the
// per-token part of the routing backward. All are HBM-bound, with 64-bit indexing throughout.
//
// Dispatch, combine and combine backward run one 256-thread block per token: thread i moves the
// 16-byte vectors i, i + 256, ... of the token's row (one vector per thread at H = 2048 BF16), and
// the token's slot rows and gates are broadcast from lanes 0..k-1 with v_readlane (scalar), so
// every wave issues few memory instructions and many waves keep HBM busy. Dispatch backward and
// the FP8 dispatch keep one wave per token (the FP8 quantiser needs the row's absmax in one wave).
//
// torchtitan PR 5541 ("AI-Generated Details") describes its BF16/FP8 row-copy kernels with
// multi-row tiles, tail masks and 64-bit addressing; these kernels keep those properties for the
// gather/scatter between token order and expert-contiguous order. ART PR 971 (description)
// gives combine's fresh [P, H] output cropped to the logical rows: only rows t < T are written.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {

constexpr int kTokPerBlock = 4;   // one wave per token (wave-per-token kernels)
constexpr int kBatch = 4;         // 16-byte vectors per lane kept in flight
constexpr int kBlockThreads = 256;  // block-per-token kernels

// Broadcast lane j's value to the wave (scalar register).
MOE_DEV int bcast_i(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
MOE_DEV float bcast_f(float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); }

// ---------------------------------------------------------------------------------------------
// Dispatch (F32 / BF16): scatter x[t] to xd[row_of[t][j]] for every local slot; bitwise copy. A
// token without a local expert is not read at all.
template <int K>
__global__ __launch_bounds__(kBlockThreads) void dispatch_copy_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ row_of, u32x4* __restrict__ xd,
    int64_t t0, int64_t t1, int64_t nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + blockIdx.x;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  if (__ballot(myrow >= 0) == 0) return;
  for (int64_t i = threadIdx.x; i < nvec; i += kBlockThreads) {
    const u32x4 v = x[t * nvec + i];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int32_t r = bcast_i(myrow, j);
      if (r >= 0) xd[(int64_t)r * nvec + i] = v;
    }
  }
}


// Dispatch (FP8): per token absmax over the BF16 row, codes = e4m3(x * (448/amax)),
// xd_scale[row] = amax/448 (1 for a zero row); h_scale[row] cleared. Row of <= 16 vectors/lane.
constexpr int kFp8MaxVec = 16;
__global__ __launch_bounds__(256) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ row_of, uint2* __restrict__ xd,
    float* __restrict__ xd_scale, float* __restrict__ h_scale, int64_t t0, int64_t t1, int K,
    int64_t nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  if (__ballot(myrow >= 0) == 0) return;
  const u32x4* src = x + t * nvec;
  u32x4 v[kFp8MaxVec];
  float m = 0.f;
#pragma unroll
  for (int b = 0; b < kFp8MaxVec; ++b) {
    int64_t i = b * 64 + lane;
    if (i < nvec) { v[b] = src[i]; m = fmaxf(m, absmax8(v[b])); }
  }
  const float amax = wave_max(m);
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  uint2 q[kFp8MaxVec];
#pragma unroll
  for (int b = 0; b < kFp8MaxVec; ++b) {
    int64_t i = b * 64 + lane;
    if (i < nvec) q[b] = quant8(v[b], inv);
  }
  for (int j = 0; j < K; ++j) {
    int32_t r = __shfl(myrow, j, 64);
    if (r < 0) continue;
    uint2* dst = xd + (int64_t)r * nvec;
#pragma unroll
    for (int b = 0; b < kFp8MaxVec; ++b) {
      int64_t i = b * 64 + lane;
      if (i < nvec) dst[i] = q[b];
    }
    if (lane == 0) { xd_scale[r] = scale; h_scale[r] = 0.f; }
  }
}

// Row quantisation of a [rows, cols] BF16 matrix (weights), same FP32 steps as dispatch.
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(
    const u32x4* __restrict__ src, uint2* __restrict__ codes, float* __restrict__ scale,
    int64_t rows, int64_t nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;
  const u32x4* s = src + r * nvec;
  float m = 0.f;
  for (int64_t i = lane; i < nvec; i += 64) m = fmaxf(m, absmax8(s[i]));
  const float amax = wave_max(m);
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  for (int64_t i = lane; i < nvec; i += 64) codes[r * nvec + i] = quant8(s[i], inv);
  if (lane == 0) scale[r] = amax > 0.f ? amax / 448.0f : 1.0f;
}

// Per-row quantisation of the dispatch rows [c*P_c, c*P_c + N_c) of chunk c (N_c from the offset
// table, so the row count stays on the device): one wave per row, grid-stride over the rows, the
// FP32 steps of dispatch. With kRegs (rows of at most kFp8MaxVec vectors per lane) the row stays in
// registers between the absmax and the quantisation, so it is read once.
template <bool kRegs>
__global__ __launch_bounds__(256) void quantize_segments_fp8_kernel(
    const u32x4* __restrict__ src, uint2* __restrict__ codes, float* __restrict__ scale,
    const int32_t* __restrict__ offsets, int El, int c0, int64_t P_c, int64_t nvec) {
  const int lane = threadIdx.x & 63;
  const int c = c0 + (int)blockIdx.y;
  const int64_t n = offsets[(int64_t)c * (El + 1) + El];
  for (int64_t r = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6); r < n;
       r += (int64_t)gridDim.x * kTokPerBlock) {
    const int64_t row = (int64_t)c * P_c + r;
    const u32x4* s = src + row * nvec;
    float m = 0.f;
    if constexpr (kRegs) {
      u32x4 v[kFp8MaxVec];
#pragma unroll
      for (int b = 0; b < kFp8MaxVec; ++b) {
        const int64_t i = b * 64 + lane;
        if (i < nvec) { v[b] = s[i]; m = fmaxf(m, absmax8(v[b])); }
      }
      const float amax = wave_max(m);
      const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
      for (int b = 0; b < kFp8MaxVec; ++b) {
        const int64_t i = b * 64 + lane;
        if (i < nvec) codes[row * nvec + i] = quant8(v[b], inv);
      }
      if (lane == 0) scale[row] = amax > 0.f ? amax / 448.0f : 1.0f;
    } else {
      for (int64_t i = lane; i < nvec; i += 64) m = fmaxf(m, absmax8(s[i]));
      const float amax = wave_max(m);
      const float inv = amax > 0.f ? 448.0f / amax : 0.f;
      for (int64_t i = lane; i < nvec; i += 64) codes[row * nvec + i] = quant8(s[i], inv);
      if (lane == 0) scale[row] = amax > 0.f ? amax / 448.0f : 1.0f;
    }
  }
}

// Per-column quantisation of a batch of [rows, cols] BF16 matrices stored transposed: codes
// [batch, cols, rows] (the column's values contiguous) and scale [batch, cols], each column with
// the FP32 steps of dispatch. One block per 64 columns of one matrix: the 256 threads (8 column
// vectors of 8 values x 32 row groups) first reduce the 64 column maxima through LDS, then walk
// 64-row tiles, quantise, transpose the bytes in LDS and store 16 code bytes per thread.
// rows % 16 == 0 and cols % 8 == 0 (checked on the host).
constexpr int kColTile = 64, kColPitch = kColTile + 16;
__global__ __launch_bounds__(256) void quantize_cols_fp8_kernel(
    const u32x4* __restrict__ src, uint8_t* __restrict__ codes, float* __restrict__ scale,
    int64_t rows, int64_t cols) {
  __shared__ float red[32][kColTile];
  __shared__ float s_inv[kColTile];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTile * kColPitch];
  const int t = threadIdx.x, cv = t & 7, rg = t >> 3;
  const int64_t b = blockIdx.y, c0 = (int64_t)blockIdx.x * kColTile;
  const int64_t nvec = cols / 8;
  const bool cin = c0 + cv * 8 < cols;
  const u32x4* s = src + b * rows * nvec + c0 / 8 + cv;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (cin)
    for (int64_t r = rg; r < rows; r += 32) {
      const u32x4 v = s[r * nvec];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = fmaxf(m[2 * i], fabsf(bf2f(w[i] & 0xffff)));
        m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(bf2f(w[i] >> 16)));
      }
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rg][cv * 8 + i] = m[i];
  __syncthreads();
  if (t < kColTile) {
    float amax = 0.f;
    for (int g = 0; g < 32; ++g) amax = fmaxf(amax, red[g][t]);
    s_inv[t] = amax > 0.f ? 448.0f / amax : 0.f;
    if (c0 + t < cols) scale[b * cols + c0 + t] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
  __syncthreads();
  float inv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) inv[i] = s_inv[cv * 8 + i];
  const int oc = t >> 2, orow = (t & 3) * 16;   // output: column oc, 16 rows from orow
  uint8_t* out = codes + (b * cols + c0 + oc) * rows;
  for (int64_t r0 = 0; r0 < rows; r0 += kColTile) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = rg + 32 * h;
      if (cin && r0 + rl < rows) {
        const u32x4 v = s[(r0 + rl) * nvec];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf2f(w[i] & 0xffff); f[2 * i + 1] = bf2f(w[i] >> 16); }
        const uint32_t lo = pack_fp8x4(clamp448(f[0] * inv[0]), clamp448(f[1] * inv[1]), clamp448(f[2] * inv[2]),
                                       clamp448(f[3] * inv[3]));
        const uint32_t hi = pack_fp8x4(clamp448(f[4] * inv[4]), clamp448(f[5] * inv[5]), clamp448(f[6] * inv[6]),
                                       clamp448(f[7] * inv[7]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tile[(cv * 8 + i) * kColPitch + rl] = (uint8_t)(lo >> (8 * i));
          tile[(cv * 8 + 4 + i) * kColPitch + rl] = (uint8_t)(hi >> (8 * i));
        }
      }
    }
    __syncthreads();
    if (c0 + oc < cols && r0 + orow < rows)
      *(u32x4*)(out + r0 + orow) = *(const u32x4*)(tile + oc * kColPitch + orow);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Vector helpers over a 16-byte payload vector: 4 FP32 or 8 BF16 values.
template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  MOE_DEV static void to_f(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  MOE_DEV static u32x4 from_f(const float* f) {
    return {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  MOE_DEV static void to_f(const u32x4& v, float* f) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf2f(w[i] & 0xffff); f[2 * i + 1] = bf2f(w[i] >> 16); }
  }
  MOE_DEV static u32x4 from_f(const float* f) {
    return {pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]), pack_bf2(f[6], f[7])};
  }
};

// Combine: out[t] = RNE(sum_j g_tj * yd[row_of[t][j]]), FP32 accumulation, j ascending; a token
// without a local expert gets a zero row.
template <typename T, int K>
__global__ __launch_bounds__(kBlockThreads) void combine_kernel(
    const u32x4* __restrict__ yd, const float* __restrict__ gates, const int32_t* __restrict__ row_of,
    u32x4* __restrict__ out, int64_t t0, int64_t t1, int64_t nvec) {
  using V = Vec<T>;
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + blockIdx.x;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  const float mygate = lane < K ? gates[t * K + lane] : 0.f;
  for (int64_t i = threadIdx.x; i < nvec; i += kBlockThreads) {
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int32_t r = bcast_i(myrow, j);
      if (r >= 0) v[j] = yd[(int64_t)r * nvec + i];
    }
    float acc[V::N];
#pragma unroll
    for (int q = 0; q < V::N; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (bcast_i(myrow, j) < 0) continue;
      const float g = bcast_f(mygate, j);
      float f[V::N];
      V::to_f(v[j], f);
#pragma unroll
      for (int q = 0; q < V::N; ++q) acc[q] = fmaf(g, f[q], acc[q]);
    }
    out[t * nvec + i] = V::from_f(acc);
  }
}

// Combine backward: dyd[row_of[t][j]] = g_tj * dy[t]; dgates[t][j] = <dy[t], yd[row]> (FP32): each
// thread's partial over its vectors, a wave sum, then the four waves' sums in order (no atomics).
// The slots' yd loads are issued four at a time, and the kernel is capped at 64 VGPRs (eight waves
// per SIMD) so that its waves fit beside the persistent expert GEMMs of the other stream.
template <typename T, int K>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(8))) void combine_bwd_kernel(
    const u32x4* __restrict__ dy, const u32x4* __restrict__ yd, const float* __restrict__ gates,
    const int32_t* __restrict__ row_of, u32x4* __restrict__ dyd, float* __restrict__ dgates,
    int64_t t0, int64_t t1, int64_t nvec) {
  using V = Vec<T>;
  constexpr int NW = kBlockThreads / 64;
  __shared__ float part[NW][K];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = t0 + blockIdx.x;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  const float mygate = lane < K ? gates[t * K + lane] : 0.f;
  const uint64_t local = __ballot(myrow >= 0);
  float dg[K];
#pragma unroll
  for (int j = 0; j < K; ++j) dg[j] = 0.f;
  if (local) {
    for (int64_t i = threadIdx.x; i < nvec; i += kBlockThreads) {
      float d[V::N];
      V::to_f(dy[t * nvec + i], d);
      constexpr int G = K < 4 ? K : 4;  // slots whose loads are in flight together
#pragma unroll
      for (int j0 = 0; j0 < K; j0 += G) {
        u32x4 v[G];
#pragma unroll
        for (int jj = 0; jj < G && j0 + jj < K; ++jj) {
          const int32_t r = bcast_i(myrow, j0 + jj);
          if (r >= 0) v[jj] = yd[(int64_t)r * nvec + i];
        }
#pragma unroll
        for (int jj = 0; jj < G && j0 + jj < K; ++jj) {
          const int j = j0 + jj;
          const int32_t r = bcast_i(myrow, j);
          if (r < 0) continue;
          const float g = bcast_f(mygate, j);
          float f[V::N], o[V::N];
          V::to_f(v[jj], f);
#pragma unroll
          for (int q = 0; q < V::N; ++q) { dg[j] = fmaf(d[q], f[q], dg[j]); o[q] = g * d[q]; }
          dyd[(int64_t)r * nvec + i] = V::from_f(o);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (!((local >> j) & 1)) continue;
    const float w = wave_sum(dg[j]);
    if (lane == 0) part[wave][j] = w;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int j = threadIdx.x;
    float sum = 0.f;
    if ((local >> j) & 1) {
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += part[w][j];
    }
    dgates[t * K + j] = sum;
  }
}

// Combine backward of BF16 rows that also quantises every written dyd row to e4m3 with the FP32
// steps of dispatch (the FP8 input gradients take them). The row's absmax is that of the BF16
// values RNE(g * dy), which equals RNE(|g| * max|dy|) because the FP32 product and the rounding are
// monotone, so one block reduction of max|dy[t]| gives every slot's scale, and the codes equal those
// of quantising the stored dyd rows. Each thread holds NV vectors of the token's row (H <= NV * 2048
// BF16 values): dy and the slots' yd are loaded before the one barrier, then dyd, its codes and the
// dgates partials follow from registers.
constexpr int kCombineQMaxVec = kCombineQMaxH / 8 / kBlockThreads;
template <int K, int NV>
__global__ __launch_bounds__(kBlockThreads) void combine_bwd_q_kernel(
    const u32x4* __restrict__ dy, const u32x4* __restrict__ yd, const float* __restrict__ gates,
    const int32_t* __restrict__ row_of, u32x4* __restrict__ dyd, float* __restrict__ dgates,
    uint2* __restrict__ dq, float* __restrict__ dq_scale, int64_t t0, int64_t t1, int64_t nvec) {
  using V = Vec<uint16_t>;
  constexpr int NW = kBlockThreads / 64;
  __shared__ float part[NW][K];
  __shared__ float amx[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = t0 + blockIdx.x;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  const float mygate = lane < K ? gates[t * K + lane] : 0.f;
  const uint64_t local = __ballot(myrow >= 0);   // the same in every wave of the block
  if (!local) {
    if (threadIdx.x < K) dgates[t * K + threadIdx.x] = 0.f;
    return;
  }
  u32x4 dv[NV], yv[NV][K];
  float m = 0.f;
#pragma unroll
  for (int b = 0; b < NV; ++b) {
    const int64_t i = threadIdx.x + (int64_t)b * kBlockThreads;
    if (i < nvec) {
      dv[b] = dy[t * nvec + i];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int32_t r = bcast_i(myrow, j);
        if (r >= 0) yv[b][j] = yd[(int64_t)r * nvec + i];
      }
      m = fmaxf(m, absmax8(dv[b]));
    }
  }
  m = wave_max(m);
  if (lane == 0) amx[wave] = m;
  __syncthreads();
  m = amx[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, amx[w]);
  float inv[K], dg[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    dg[j] = 0.f;
    const float a = bf2f(f2bf(fabsf(bcast_f(mygate, j)) * m));
    inv[j] = a > 0.f ? 448.0f / a : 0.f;
    const int32_t r = bcast_i(myrow, j);
    if (threadIdx.x == 0 && r >= 0) dq_scale[r] = a > 0.f ? a / 448.0f : 1.0f;
  }
#pragma unroll
  for (int b = 0; b < NV; ++b) {
    const int64_t i = threadIdx.x + (int64_t)b * kBlockThreads;
    if (i >= nvec) continue;
    float d[V::N];
    V::to_f(dv[b], d);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int32_t r = bcast_i(myrow, j);
      if (r < 0) continue;
      const float g = bcast_f(mygate, j);
      float f[V::N], o[V::N];
      V::to_f(yv[b][j], f);
#pragma unroll
      for (int q = 0; q < V::N; ++q) { dg[j] = fmaf(d[q], f[q], dg[j]); o[q] = g * d[q]; }
      const u32x4 ov = V::from_f(o);
      dyd[(int64_t)r * nvec + i] = ov;
      dq[(int64_t)r * nvec + i] = quant8(ov, inv[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (!((local >> j) & 1)) continue;
    const float w = wave_sum(dg[j]);
    if (lane == 0) part[wave][j] = w;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int j = threadIdx.x;
    float sum = 0.f;
    if ((local >> j) & 1) {
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += part[w][j];
    }
    dgates[t * K + j] = sum;
  }
}

// Route backward, per token: dlogits[t][e] = g_j (dg_j - sum_i g_i dg_i) where e = idx[t][j],
// zero for every other expert (the full row of E columns is written): the row is cleared with
// coalesced stores, then lanes 0..K-1 store their slot's value (same wave, program order).
__global__ __launch_bounds__(256) void route_bwd_dlogits_kernel(
    const float* __restrict__ dgates, const float* __restrict__ gates, const int32_t* __restrict__ idx,
    float* __restrict__ dlogits, uint16_t* __restrict__ dl_hi, uint16_t* __restrict__ dl_lo, int ldl, int64_t pitch,
    int64_t t0, int64_t t1, int K, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const float g = lane < K ? gates[t * K + lane] : 0.f;
  const float d = lane < K ? dgates[t * K + lane] : 0.f;
  const int id = lane < K ? idx[t * K + lane] : -1;
  float s = 0.f;  // sum_i g_i dg_i, slots in ascending order
  for (int j = 0; j < K; ++j)
    s = fmaf(bcast_f(g, j), bcast_f(d, j), s);
  float* row = dlogits + t * (int64_t)E;
  for (int e = lane; e < E; e += 64) row[e] = 0.f;
  const float v = g * (d - s);
  if (lane < K) row[id] = v;
  if (dl_hi) {
    // BF16 high and low parts of the row for the router weight gradient (row t - t0 of the
    // planes; zeros past E up to ldl columns)
    int ids[8];
    float vs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ids[j] = j < K ? bcast_i(id, j) : -1;
      vs[j] = j < K ? bcast_f(v, j) : 0.f;
    }
    // two columns per lane (the pitch is a multiple of 8), one 4-byte store per plane
    uint32_t* hr = (uint32_t*)(dl_hi + (t - t0) * pitch);
    uint32_t* lr = (uint32_t*)(dl_lo + (t - t0) * pitch);
    for (int e = 2 * lane; e < ldl; e += 128) {
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ids[j] == e) x0 = vs[j];
        if (ids[j] == e + 1) x1 = vs[j];
      }
      const uint16_t h0 = f2bf(x0), h1 = f2bf(x1);
      hr[e / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lr[e / 2] = (uint32_t)f2bf(x0 - bf2f(h0)) | ((uint32_t)f2bf(x1 - bf2f(h1)) << 16);
    }
  }
}

// Dispatch backward: dx[t] = RNE(sum_j local dxd[row_of[t][j]] + sum_j dlogits[t][e_j] W_r[e_j]).
// Capped at 64 VGPRs (eight waves per SIMD): it runs on the aux stream beside the persistent
// expert GEMMs, whose two waves per SIMD hold up to 448 of a SIMD's 512 VGPRs, so only a wave of at
// most 64 VGPRs can share a CU with them instead of waiting for a GEMM workgroup to exit.
template <typename T, int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void dispatch_bwd_kernel(
    const u32x4* __restrict__ dxd, const int32_t* __restrict__ row_of, const int32_t* __restrict__ idx,
    const float* __restrict__ dlogits, const u32x4* __restrict__ w_r, u32x4* __restrict__ dx,
    int64_t t0, int64_t t1, int E, int64_t nvec) {
  using V = Vec<T>;
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  const int myid = lane < K ? idx[t * K + lane] : 0;
  const float mydl = lane < K ? dlogits[t * E + myid] : 0.f;
  const uint64_t local = __ballot(myrow >= 0);
  u32x4* dst = dx + t * nvec;
  // NB vectors i0, i0 + 64, ... per lane; each slot's loads are issued together before use
  auto pass = [&](int64_t i0, auto nb) {
    constexpr int NB = decltype(nb)::value;
    float acc[NB][V::N];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < V::N; ++q) acc[b][q] = 0.f;
    // expert path: the local slots' dxd rows, j ascending
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (!((local >> j) & 1)) continue;
      const u32x4* src = dxd + (int64_t)bcast_i(myrow, j) * nvec;
      u32x4 v[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) v[b] = src[i0 + 64 * b];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float f[V::N];
        V::to_f(v[b], f);
#pragma unroll
        for (int q = 0; q < V::N; ++q) acc[b][q] += f[q];
      }
    }
    // router path: dlogits[t][e_j] * W_r[e_j] for every slot, j ascending (W_r stays in L2)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const u32x4* wr = w_r + (int64_t)bcast_i(myid, j) * nvec;
      const float dl = bcast_f(mydl, j);
      u32x4 w[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) w[b] = wr[i0 + 64 * b];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float f[V::N];
        V::to_f(w[b], f);
#pragma unroll
        for (int q = 0; q < V::N; ++q) acc[b][q] = fmaf(dl, f[q], acc[b][q]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) dst[i0 + 64 * b] = V::from_f(acc[b]);
  };
  // vectors per lane in flight: kBatch, or fewer where the 64-VGPR cap would spill at kBatch
  constexpr int NBV = (sizeof(T) == 2 && K >= 3 && K <= 5) ? 1
                    : ((sizeof(T) == 2 && K == 2) || (sizeof(T) == 4 && K == 6)) ? 2 : kBatch;
  int64_t i0 = lane;
  for (; i0 + 64 * (NBV - 1) < nvec; i0 += 64 * NBV) pass(i0, std::integral_constant<int, NBV>());
  for (; i0 < nvec; i0 += 64) pass(i0, std::integral_constant<int, 1>());
}

// Dispatch backward on block-scaled FP8 dxd rows (e4m3 codes [., H], one FP32 scale per row and
// 256-column block): dx[t] = RNE(sum_j deq(dxd[row_of[t][j]]) + sum_j dlogits[t][e_j] W_r[e_j]),
// each code dequantised as code value * its block's scale in FP32, slots in ascending order. Eight
// columns per lane and vector (8 code bytes, one BF16 vector of W_r and dx). Capped at 64 VGPRs like
// the BF16 kernel.
template <int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void dispatch_bwd_fp8_kernel(
    const uint2* __restrict__ dxq, const float* __restrict__ dxs, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ idx, const float* __restrict__ dlogits, const u32x4* __restrict__ w_r,
    u32x4* __restrict__ dx, int64_t t0, int64_t t1, int E, int64_t nvec, int nblk) {
  using V = Vec<uint16_t>;
  const int lane = threadIdx.x & 63;
  const int64_t t = t0 + (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= t1) return;
  const int32_t myrow = lane < K ? row_of[t * K + lane] : -1;
  const int myid = lane < K ? idx[t * K + lane] : 0;
  const float mydl = lane < K ? dlogits[t * E + myid] : 0.f;
  const uint64_t local = __ballot(myrow >= 0);
  u32x4* dst = dx + t * nvec;
  auto pass = [&](int64_t i0, auto nb) {
    constexpr int NB = decltype(nb)::value;
    float acc[NB][8];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[b][q] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (!((local >> j) & 1)) continue;
      const int64_t row = bcast_i(myrow, j);
      const uint2* src = dxq + row * nvec;
      const float* sc = dxs + row * nblk;
      uint2 c[NB];
      float s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        c[b] = src[i0 + 64 * b];
        s[b] = sc[(i0 + 64 * b) >> 5];  // 32 vectors of 8 columns per 256-column block
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float f[8];
        deq8(c[b], s[b], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b][q] += f[q];
      }
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const u32x4* wr = w_r + (int64_t)bcast_i(myid, j) * nvec;
      const float dl = bcast_f(mydl, j);
      u32x4 w[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) w[b] = wr[i0 + 64 * b];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float f[8];
        V::to_f(w[b], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b][q] = fmaf(dl, f[q], acc[b][q]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) dst[i0 + 64 * b] = V::from_f(acc[b]);
  };
  constexpr int NB2 = 2;  // vectors per lane in flight (the 64-VGPR cap spills at 4)
  int64_t i0 = lane;
  for (; i0 + 64 * (NB2 - 1) < nvec; i0 += 64 * NB2) pass(i0, std::integral_constant<int, NB2>());
  for (; i0 < nvec; i0 += 64) pass(i0, std::integral_constant<int, 1>());
}

// ---------------------------------------------------------------------------------------------
// Launchers. Token range [t0, t1); nvec = 16-byte vectors per row.
static inline dim3 tok_grid(int64_t ntok) { return dim3((unsigned)((ntok + kTokPerBlock - 1) / kTokPerBlock)); }

// K (top-k, 1..8) is a template parameter of the row kernels so that the slot loops unroll.
#define MOE_SWITCH_K(K, ...)                     \
  switch (K) {                                   \
    case 1: { constexpr int KK = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int KK = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int KK = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int KK = 4; __VA_ARGS__; } break; \
    case 5: { constexpr int KK = 5; __VA_ARGS__; } break; \
    case 6: { constexpr int KK = 6; __VA_ARGS__; } break; \
    case 7: { constexpr int KK = 7; __VA_ARGS__; } break; \
    case 8: { constexpr int KK = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;      \
  }

hipError_t launch_dispatch(const void* x, const int32_t* row_of, void* xd, int64_t t0, int64_t t1,
                           int K, int64_t row_bytes, hipStream_t s) {
  if (t1 <= t0) return hipSuccess;
  {
    MOE_TRACE("dispatch", s);
    MOE_SWITCH_K(K, MOE_LAUNCH(dispatch_copy_kernel<KK>, dim3((unsigned)(t1 - t0)), dim3(kBlockThreads), 0, s,
                                       (const u32x4*)x, row_of, (u32x4*)xd, t0, t1, row_bytes / 16));
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const void* x, const int32_t* row_of, void* xd, float* xd_scale,
                               float* h_scale, int64_t t0, int64_t t1, int K, int H, hipStream_t s) {
  if (t1 <= t0) return hipSuccess;
  {
    MOE_TRACE("dispatch_fp8", s);
    MOE_LAUNCH(dispatch_fp8_kernel, tok_grid(t1 - t0), dim3(256), 0, s, (const u32x4*)x,
                       row_of, (uint2*)xd, xd_scale, h_scale, t0, t1, K, (int64_t)H / 8);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows_fp8(const void* src, void* codes, float* scale, int64_t rows,
                                    int cols, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  {
    MOE_TRACE("quantize_rows_fp8", s);
    MOE_LAUNCH(quantize_rows_fp8_kernel, tok_grid(rows), dim3(256), 0, s, (const u32x4*)src,
                       (uint2*)codes, scale, rows, (int64_t)cols / 8);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_segments_fp8(const char* name, const void* src, void* codes, float* scale,
                                        const int32_t* offsets, int El, int c0, int nc, int64_t P_c,
                                        int cols, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  // enough waves for every row of a chunk up to 16K rows (the row count is on the device)
  const int64_t nvec = cols / 8;
  const unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>((P_c + kTokPerBlock - 1) / kTokPerBlock, 4096));
  {
    MOE_TRACE(name, s);
    if (nvec <= 64 * kFp8MaxVec)
      MOE_LAUNCH(quantize_segments_fp8_kernel<true>, dim3(gx, (unsigned)nc), dim3(256), 0, s,
                 (const u32x4*)src, (uint2*)codes, scale, offsets, El, c0, P_c, nvec);
    else
      MOE_LAUNCH(quantize_segments_fp8_kernel<false>, dim3(gx, (unsigned)nc), dim3(256), 0, s,
                 (const u32x4*)src, (uint2*)codes, scale, offsets, El, c0, P_c, nvec);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_cols_fp8(const void* src, void* codes_t, float* scale, int64_t batch, int64_t rows,
                                    int64_t cols, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  {
    MOE_TRACE("quantize_cols_fp8", s);
    MOE_LAUNCH(quantize_cols_fp8_kernel, dim3((unsigned)((cols + kColTile - 1) / kColTile), (unsigned)batch),
               dim3(256), 0, s, (const u32x4*)src, (uint8_t*)codes_t, scale, rows, cols);
  }
  return hipGetLastError();
}

// Per-expert, per-column quantisation of dispatch rows for the FP8 weight gradients: expert e's rows
// of every chunk (chunk order) are quantised per column (absmax over those rows, the FP32 steps of
// dispatch) and stored transposed and zero-padded: codes[koff_e * C + c * Kp_e + k] (expert_k) and
// scale[e * C + c]. One 1024-thread block per 64 columns of one expert (8 column vectors x 128 row
// groups, so that enough rows are in flight): the column maxima through LDS, then 128-row tiles
// quantised, transposed in LDS and stored 8 bytes a thread.
constexpr int kEcThreads = 1024, kEcRG = kEcThreads / 8, kEcPitch = kEcRG + 16;
__global__ __launch_bounds__(kEcThreads) void quantize_expert_cols_fp8_kernel(
    const u32x4* __restrict__ src, uint8_t* __restrict__ codes, float* __restrict__ scale,
    const int32_t* __restrict__ offsets, int El, int n_chunks, int64_t P_c, int64_t cols) {
  __shared__ float red[kEcRG][kColTile + 1];
  __shared__ float s_inv[kColTile];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTile * kEcPitch];
  const int t = threadIdx.x, cv = t & 7, rg = t >> 3;
  const int e = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * kColTile;
  const int64_t nvec = cols / 8;
  const bool cin = c0 + cv * 8 < cols;
  int64_t koff;
  int K;
  expert_k(offsets, El, n_chunks, e, koff, K);
  const int Kp = (K + 63) & ~63;
  // dispatch row of the expert's k-th row
  auto row_of_k = [&](int k) -> int64_t {
    for (int c = 0; c < n_chunks; ++c) {
      const int32_t* off = offsets + (int64_t)c * (El + 1);
      const int len = off[e + 1] - off[e];
      if (k < len) return (int64_t)c * P_c + off[e] + k;
      k -= len;
    }
    return -1;
  };
  const u32x4* s = src + c0 / 8 + cv;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (cin) {
#pragma unroll 4
    for (int k = rg; k < K; k += kEcRG) {
      const u32x4 v = s[row_of_k(k) * nvec];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = fmaxf(m[2 * i], fabsf(bf2f(w[i] & 0xffff)));
        m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(bf2f(w[i] >> 16)));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rg][cv * 8 + i] = m[i];
  __syncthreads();
  if (t < kColTile) {
    float amax = 0.f;
    for (int g = 0; g < kEcRG; ++g) amax = fmaxf(amax, red[g][t]);
    s_inv[t] = amax > 0.f ? 448.0f / amax : 0.f;
    if (c0 + t < cols) scale[(int64_t)e * cols + c0 + t] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
  __syncthreads();
  float inv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) inv[i] = s_inv[cv * 8 + i];
  const int oc = t >> 4, orow = (t & 15) * 8;   // output: column oc, 8 rows from orow
  uint8_t* out = codes + koff * cols + (c0 + oc) * Kp;
  for (int k0 = 0; k0 < Kp; k0 += kEcRG) {
    if (cin) {
      uint32_t lo = 0, hi = 0;   // rows past K_e: zero codes
      if (k0 + rg < K) {
        const u32x4 v = s[row_of_k(k0 + rg) * nvec];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf2f(w[i] & 0xffff); f[2 * i + 1] = bf2f(w[i] >> 16); }
        lo = pack_fp8x4(clamp448(f[0] * inv[0]), clamp448(f[1] * inv[1]), clamp448(f[2] * inv[2]),
                        clamp448(f[3] * inv[3]));
        hi = pack_fp8x4(clamp448(f[4] * inv[4]), clamp448(f[5] * inv[5]), clamp448(f[6] * inv[6]),
                        clamp448(f[7] * inv[7]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tile[(cv * 8 + i) * kEcPitch + rg] = (uint8_t)(lo >> (8 * i));
        tile[(cv * 8 + 4 + i) * kEcPitch + rg] = (uint8_t)(hi >> (8 * i));
      }
    }
    __syncthreads();
    if (c0 + oc < cols && k0 + orow < Kp) *(uint2*)(out + k0 + orow) = *(const uint2*)(tile + oc * kEcPitch + orow);
    __syncthreads();
  }
}

hipError_t launch_quantize_expert_cols_fp8(const char* name, const void* src, void* codes, float* scale,
                                           const int32_t* offsets, int El, int n_chunks, int64_t P_c, int64_t cols,
                                           hipStream_t s) {
  if (El <= 0 || cols <= 0) return hipSuccess;
  {
    MOE_TRACE(name, s);
    MOE_LAUNCH(quantize_expert_cols_fp8_kernel, dim3((unsigned)((cols + kColTile - 1) / kColTile), (unsigned)El),
               dim3(kEcThreads), 0, s, (const u32x4*)src, (uint8_t*)codes, scale, offsets, El, n_chunks, P_c, cols);
  }
  return hipGetLastError();
}

hipError_t launch_combine(bool bf16, const void* yd, const float* gates, const int32_t* row_of,
                          void* out, int64_t t0, int64_t t1, int K, int64_t row_bytes, hipStream_t s) {
  if (t1 <= t0) return hipSuccess;
  if (bf16)
    {
      MOE_TRACE("combine", s);
      MOE_SWITCH_K(K, MOE_LAUNCH((combine_kernel<uint16_t, KK>), dim3((unsigned)(t1 - t0)), dim3(kBlockThreads), 0, s,
                         (const u32x4*)yd, gates, row_of, (u32x4*)out, t0, t1, row_bytes / 16));
    }
  else
    {
      MOE_TRACE("combine", s);
      MOE_SWITCH_K(K, MOE_LAUNCH((combine_kernel<float, KK>), dim3((unsigned)(t1 - t0)), dim3(kBlockThreads), 0, s,
                         (const u32x4*)yd, gates, row_of, (u32x4*)out, t0, t1, row_bytes / 16));
    }
  return hipGetLastError();
}

hipError_t launch_combine_bwd(bool bf16, const void* dy, const void* yd, const float* gates,
                              const int32_t* row_of, void* dyd, float* dgates, int64_t t0,
                              int64_t t1, int K, int64_t row_bytes, hipStream_t s, void* dyd_q,
                              float* dyd_scale) {
  if (t1 <= t0) return hipSuccess;
  const int64_t nvec = row_bytes / 16;
  if (bf16 && dyd_q) {
    if (nvec > kCombineQMaxVec * kBlockThreads) return hipErrorInvalidValue;  // the host checks H first
    MOE_TRACE("combine_bwd_q", s);
#define MOE_CBQ(NV_)                                                                                            \
    MOE_SWITCH_K(K, MOE_LAUNCH((combine_bwd_q_kernel<KK, NV_>), dim3((unsigned)(t1 - t0)), dim3(kBlockThreads), 0, s, \
                               (const u32x4*)dy, (const u32x4*)yd, gates, row_of, (u32x4*)dyd, dgates,           \
                               (uint2*)dyd_q, dyd_scale, t0, t1, nvec))
    if (nvec <= kBlockThreads) {
      MOE_CBQ(1);
    } else if (nvec <= 2 * kBlockThreads) {
      MOE_CBQ(2);
    } else {
      MOE_CBQ(4);
    }
#undef MOE_CBQ
  } else if (bf16) {
    MOE_TRACE("combine_bwd", s);
    MOE_SWITCH_K(K, MOE_LAUNCH((combine_bwd_kernel<uint16_t, KK>), dim3((unsigned)(t1 - t0)), dim3(kBlockThreads),
                               0, s, (const u32x4*)dy, (const u32x4*)yd, gates, row_of, (u32x4*)dyd, dgates,
                               t0, t1, nvec));
  } else {
    MOE_TRACE("combine_bwd", s);
    MOE_SWITCH_K(K, MOE_LAUNCH((combine_bwd_kernel<float, KK>), dim3((unsigned)(t1 - t0)), dim3(kBlockThreads),
                               0, s, (const u32x4*)dy, (const u32x4*)yd, gates, row_of, (u32x4*)dyd, dgates,
                               t0, t1, nvec));
  }
  return hipGetLastError();
}

hipError_t launch_route_bwd_dlogits(const float* dgates, const float* gates, const int32_t* idx,
                                    float* dlogits, int64_t t0, int64_t t1, int K, int E,
                                    hipStream_t s, uint16_t* dl_hi, uint16_t* dl_lo, int ldl, int64_t pitch) {
  if (dl_hi && (!dl_lo || ldl < E || ldl % 8 || pitch % 2 || pitch < ldl)) return hipErrorInvalidValue;
  if (t1 <= t0) return hipSuccess;
  {
    MOE_TRACE("route_bwd_dlogits", s);
    MOE_LAUNCH(route_bwd_dlogits_kernel, tok_grid(t1 - t0), dim3(256), 0, s, dgates, gates,
                       idx, dlogits, dl_hi, dl_lo, ldl, pitch, t0, t1, K, E);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd(bool bf16, const void* dxd, const float* dxd_scales, const int32_t* row_of,
                               const int32_t* idx, const float* dlogits, const void* w_r, void* dx, int64_t t0,
                               int64_t t1, int K, int E, int H, int64_t row_bytes, hipStream_t s) {
  if (t1 <= t0) return hipSuccess;
  if (dxd_scales) {
    if (!bf16 || H % 8) return hipErrorInvalidValue;
    MOE_TRACE("dispatch_bwd_fp8", s);
    MOE_SWITCH_K(K, MOE_LAUNCH((dispatch_bwd_fp8_kernel<KK>), tok_grid(t1 - t0), dim3(256), 0, s,
                               (const uint2*)dxd, dxd_scales, row_of, idx, dlogits, (const u32x4*)w_r, (u32x4*)dx,
                               t0, t1, E, (int64_t)H / 8, (H + 255) / 256));
    return hipGetLastError();
  }
  if (bf16)
    {
      MOE_TRACE("dispatch_bwd", s);
      MOE_SWITCH_K(K, MOE_LAUNCH((dispatch_bwd_kernel<uint16_t, KK>), tok_grid(t1 - t0), dim3(256), 0, s,
                         (const u32x4*)dxd, row_of, idx, dlogits, (const u32x4*)w_r, (u32x4*)dx,
                         t0, t1, E, row_bytes / 16));
    }
  else
    {
      MOE_TRACE("dispatch_bwd", s);
      MOE_SWITCH_K(K, MOE_LAUNCH((dispatch_bwd_kernel<float, KK>), tok_grid(t1 - t0), dim3(256), 0, s,
                         (const u32x4*)dxd, row_of, idx, dlogits, (const u32x4*)w_r, (u32x4*)dx,
                         t0, t1, E, row_bytes / 16));
    }
  return hipGetLastError();
}

}  // namespace moe
