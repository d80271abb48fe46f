// Routing kernels: per-token top-k over FP32 logits with renormalised gates, per-chunk expert
// histograms, and the stable expert-contiguous permutation.
//
// Token-wise ChunkedEP (Megatron-LM PR 7342, "Summary") routes each token chunk with top-k
// (no auxiliary loss, "Tests and limitations"). The pages print no formula; the reading is:
// select the k largest logits (ties to the lower expert index, NaN lowest), gates = softmax over
// the selected logits. The permutation is the stable sort of (token, slot) pairs by expert inside
// each chunk: within an expert, rows follow ascending token index.
//
// Two launches, both deterministic:
//   route_topk   one lane per token: top-k, gates, and a per-64-token-block histogram of all
//                E experts (LDS integer adds: the sum does not depend on their order).
//   route_layout per block: prefix of the earlier blocks' histograms (exclusive scan), local
//                offsets, then each token's rank among the block's earlier tokens choosing the
//                same expert from a 64-bit ballot mask (popcount below the lane).
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {

constexpr int kRouteBlock = 64;   // tokens per block: one wave
constexpr int kLogitTile = 128;   // logits per token staged in LDS at a time

// One wave per 64 tokens. The wave stages a [64, 128] tile of logits through LDS with coalesced
// 16-byte loads (rows padded to 129 floats so that each lane reading its own row is
// conflict-free), then every lane runs an unrolled top-K insertion over its token's logits.
template <int K>
__global__ __launch_bounds__(kRouteBlock) void route_topk_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ gates,
    int32_t* __restrict__ block_hist, int64_t T, int E, int n, int chunk0, int nbpc) {
  __shared__ float tile[kRouteBlock][kLogitTile + 1];
  extern __shared__ int hist[];  // [E]
  const int lane = threadIdx.x;
  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  for (int e = lane; e < E; e += kRouteBlock) hist[e] = 0;
  const int64_t tb = cr.t0 + (int64_t)bl * kRouteBlock;
  const int ntok = (int)max((int64_t)0, min((int64_t)kRouteBlock, cr.t1 - tb));
  const int64_t t = tb + lane;
  const bool valid = lane < ntok;

  float v[K];
  int id[K];
#pragma unroll
  for (int s = 0; s < K; ++s) { v[s] = -__builtin_huge_valf(); id[s] = 0x7fffffff; }
  for (int e0 = 0; e0 < E; e0 += kLogitTile) {
    const int w = min(kLogitTile, E - e0);
    __syncthreads();
    if ((E & 3) == 0 && w == kLogitTile) {
      // full tile: 32 float4 per token row; two rows per wave instruction, all loads in flight
      constexpr int kQ = kLogitTile / 4;
#pragma unroll 8
      for (int i = lane; i < kRouteBlock * kQ; i += kRouteBlock) {
        const int r = i / kQ, q = i % kQ;
        if (r < ntok) {
          const float4 f = *(const float4*)(logits + (tb + r) * (int64_t)E + e0 + 4 * q);
          tile[r][4 * q] = f.x; tile[r][4 * q + 1] = f.y; tile[r][4 * q + 2] = f.z; tile[r][4 * q + 3] = f.w;
        }
      }
    } else if ((E & 3) == 0) {
      const int w4 = w >> 2;
      for (int i = lane; i < ntok * w4; i += kRouteBlock) {
        const int r = i / w4, q = i % w4;
        const float4 f = *(const float4*)(logits + (tb + r) * (int64_t)E + e0 + 4 * q);
        tile[r][4 * q] = f.x; tile[r][4 * q + 1] = f.y; tile[r][4 * q + 2] = f.z; tile[r][4 * q + 3] = f.w;
      }
    } else {
      for (int i = lane; i < ntok * w; i += kRouteBlock) {
        const int r = i / w, q = i % w;
        tile[r][q] = logits[(tb + r) * (int64_t)E + e0 + q];
      }
    }
    __syncthreads();
    if (valid) {
      for (int q = 0; q < w; ++q) {
        float x = tile[lane][q];
        if (x != x) x = -__builtin_huge_valf();  // NaN ranks lowest
        int xi = e0 + q;
        // candidate beats slot s if larger, or equal with a lower index (only sentinels)
        if (x > v[K - 1] || (x == v[K - 1] && xi < id[K - 1])) {
#pragma unroll
          for (int s = 0; s < K; ++s) {
            bool take = x > v[s] || (x == v[s] && xi < id[s]);
            float tv = v[s];
            int ti = id[s];
            v[s] = take ? x : v[s];
            id[s] = take ? xi : id[s];
            x = take ? tv : x;
            xi = take ? ti : xi;
          }
        }
      }
    }
  }
  if (valid) {
    float p[K];
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < K; ++s) { p[s] = expf(v[s] - v[0]); sum += p[s]; }
#pragma unroll
    for (int s = 0; s < K; ++s) {
      topk_idx[t * K + s] = id[s];
      gates[t * K + s] = p[s] / sum;
      atomicAdd(&hist[id[s]], 1);
    }
  }
  __syncthreads();
  int32_t* out = block_hist + ((int64_t)c * nbpc + bl) * E;
  for (int e = lane; e < E; e += kRouteBlock) out[e] = hist[e];
}

// One wave per 64 tokens: local offsets from the chunk's block histograms, then each token's
// rank among the block's earlier tokens choosing the same expert from a 64-bit ballot mask.
__global__ __launch_bounds__(kRouteBlock) void route_layout_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_token, int64_t T, int E, int e0, int El, int K, int n, int chunk0,
    int nbpc, int64_t P_c) {
  extern __shared__ unsigned char smem[];
  // layout: base[El] int, off[El+1] int, mask[El] u64
  int* base = (int*)smem;
  int* off = base + El;
  uint64_t* mask = (uint64_t*)(((uintptr_t)(off + El + 1) + 7) & ~(uintptr_t)7);

  const int lane = threadIdx.x;
  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  const int32_t* bh = block_hist + (int64_t)c * nbpc * E;

  // per local expert: rows owned by earlier blocks of this chunk, and the chunk total; lanes
  // stride over the blocks and a wave reduction sums them
  for (int el = 0; el < El; ++el) {
    int before = 0, total = 0;
    for (int b = lane; b < nbpc; b += kRouteBlock) {
      const int h = bh[(int64_t)b * E + e0 + el];
      before += (b < bl) ? h : 0;
      total += h;
    }
    before = wave_sum_int(before);
    total = wave_sum_int(total);
    if (lane == 0) { base[el] = before; off[el + 1] = total; }
  }
  for (int el = lane; el < El; el += kRouteBlock) mask[el] = 0;
  __syncthreads();
  if (lane == 0) {  // exclusive scan over local experts (El is small)
    int run = 0;
    for (int el = 0; el < El; ++el) { int cnt = off[el + 1]; off[el] = run; run += cnt; }
    off[El] = run;
  }
  __syncthreads();
  const int N_c = off[El];
  if (bl == 0) {
    for (int e = lane; e < E; e += kRouteBlock) {
      int total = 0;
#pragma unroll 16
      for (int b = 0; b < nbpc; ++b) total += bh[(int64_t)b * E + e];
      counts[(int64_t)c * E + e] = total;
    }
    for (int el = lane; el <= El; el += kRouteBlock) offsets[(int64_t)c * (El + 1) + el] = off[el];
  }

  const int64_t t = cr.t0 + (int64_t)bl * kRouteBlock + lane;
  const bool valid = t < cr.t1;
  if (valid) {
    for (int j = 0; j < K; ++j) {
      int el = topk_idx[t * K + j] - e0;
      if (el >= 0 && el < El) atomicOr((unsigned long long*)&mask[el], 1ull << lane);
    }
  }
  __syncthreads();
  if (valid) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j) {
      int el = topk_idx[t * K + j] - e0;
      int32_t row = -1;
      if (el >= 0 && el < El) {
        int rank = __popcll(mask[el] & below);
        int64_t r = (int64_t)c * P_c + off[el] + base[el] + rank;
        src_token[r] = (int32_t)t;
        row = (int32_t)r;
      }
      row_of[t * K + j] = row;
    }
  }
  // rows N_c..P_c-1 of this chunk's region hold no token
  for (int64_t r = N_c + (int64_t)bl * kRouteBlock + lane; r < P_c; r += (int64_t)nbpc * kRouteBlock)
    src_token[(int64_t)c * P_c + r] = -1;
}

int route_blocks_per_chunk(int64_t T, int n) {
  int64_t tc = (T + n - 1) / n;
  int64_t nb = (tc + kRouteBlock - 1) / kRouteBlock;
  return (int)(nb < 1 ? 1 : nb);
}

int64_t route_scratch_bytes(int64_t T, int n, int E) {
  return (int64_t)n * route_blocks_per_chunk(T, n) * E * (int64_t)sizeof(int32_t);
}

hipError_t launch_route(const float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* src_token, int32_t* scratch,
                        int64_t T, int E, int e0, int El, int K, int n, int chunk0, int nchunks,
                        int64_t P_c, hipStream_t s) {
  const int nbpc = route_blocks_per_chunk(T, n);
  dim3 grid(nbpc * nchunks), block(kRouteBlock);
  size_t sm1 = (size_t)E * sizeof(int);
  switch (K) {
#define MOE_ROUTE_K(KK)                                                                      \
  case KK: {                                                                                 \
    MOE_TRACE("route_topk", s);                                                              \
    hipLaunchKernelGGL(route_topk_kernel<KK>, grid, block, sm1, s, logits, topk_idx, gates, \
                       scratch, T, E, n, chunk0, nbpc);                                      \
    break;                                                                                   \
  }
    MOE_ROUTE_K(1) MOE_ROUTE_K(2) MOE_ROUTE_K(3) MOE_ROUTE_K(4)
    MOE_ROUTE_K(5) MOE_ROUTE_K(6) MOE_ROUTE_K(7) MOE_ROUTE_K(8)
#undef MOE_ROUTE_K
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  size_t sm2 = (size_t)El * 4 + (size_t)(El + 1) * 4 + 8 + (size_t)El * 8;
  {
    MOE_TRACE("route_layout", s);
    hipLaunchKernelGGL(route_layout_kernel, grid, block, sm2, s, topk_idx, scratch, counts, offsets,
                       row_of, src_token, T, E, e0, El, K, n, chunk0, nbpc, P_c);
  }
  return hipGetLastError();
}

}  // namespace moe
