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
//   route_topk   one thread per token: top-k, gates, and a per-256-token-block histogram of
//                all E experts (LDS integer adds: the sum does not depend on their order).
//   route_layout per block: prefix of the earlier blocks' histograms (exclusive scan), local
//                offsets, then each token's rank among the block's earlier tokens choosing the
//                same expert from per-wave 64-bit ballot masks (popcount below the lane).
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {

constexpr int kRouteBlock = 256;  // tokens per block (4 waves)

template <int K>
__global__ __launch_bounds__(kRouteBlock) void route_topk_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ gates,
    int32_t* __restrict__ block_hist, int64_t T, int E, int n, int chunk0, int nbpc) {
  extern __shared__ int hist[];  // [E]
  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t t = cr.t0 + (int64_t)bl * kRouteBlock + threadIdx.x;
  if (t < cr.t1) {
    float v[K];
    int id[K];
#pragma unroll
    for (int s = 0; s < K; ++s) { v[s] = -__builtin_huge_valf(); id[s] = 0x7fffffff; }
    const float* row = logits + t * (int64_t)E;
    for (int e = 0; e < E; ++e) {
      float x = row[e];
      if (x != x) x = -__builtin_huge_valf();  // NaN ranks lowest
      int xi = e;
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
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

__global__ __launch_bounds__(kRouteBlock) void route_layout_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_token, int64_t T, int E, int e0, int El, int K, int n, int chunk0,
    int nbpc, int64_t P_c) {
  extern __shared__ unsigned char smem[];
  // layout: base[El] int, off[El+1] int, mask[4][El] u64, wprefix[4][El] int
  int* base = (int*)smem;
  int* off = base + El;
  uint64_t* mask = (uint64_t*)(((uintptr_t)(off + El + 1) + 7) & ~(uintptr_t)7);
  int* wpre = (int*)(mask + 4 * El);

  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  const int32_t* bh = block_hist + (int64_t)c * nbpc * E;

  // per local expert: rows owned by earlier blocks of this chunk, and the chunk total
  for (int el = threadIdx.x; el < El; el += blockDim.x) {
    int before = 0, total = 0;
    for (int b = 0; b < nbpc; ++b) {
      int h = bh[(int64_t)b * E + e0 + el];
      before += (b < bl) ? h : 0;
      total += h;
    }
    base[el] = before;
    off[el + 1] = total;
  }
  for (int i = threadIdx.x; i < 4 * El; i += blockDim.x) mask[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive scan over local experts (El is small)
    int run = 0;
    for (int el = 0; el < El; ++el) { int cnt = off[el + 1]; off[el] = run; run += cnt; }
    off[El] = run;
  }
  __syncthreads();
  const int N_c = off[El];
  if (bl == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int total = 0;
      for (int b = 0; b < nbpc; ++b) total += bh[(int64_t)b * E + e];
      counts[(int64_t)c * E + e] = total;
    }
    for (int el = threadIdx.x; el <= El; el += blockDim.x) offsets[(int64_t)c * (El + 1) + el] = off[el];
  }

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t = cr.t0 + (int64_t)bl * kRouteBlock + threadIdx.x;
  const bool valid = t < cr.t1;
  if (valid) {
    for (int j = 0; j < K; ++j) {
      int el = topk_idx[t * K + j] - e0;
      if (el >= 0 && el < El) atomicOr((unsigned long long*)&mask[w * El + el], 1ull << lane);
    }
  }
  __syncthreads();
  for (int el = threadIdx.x; el < El; el += blockDim.x) {
    int run = 0;
    for (int ww = 0; ww < 4; ++ww) {
      wpre[ww * El + el] = run;
      run += __popcll(mask[ww * El + el]);
    }
  }
  __syncthreads();
  if (valid) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j) {
      int el = topk_idx[t * K + j] - e0;
      int32_t row = -1;
      if (el >= 0 && el < El) {
        int rank = wpre[w * El + el] + __popcll(mask[w * El + el] & below);
        int64_t r = (int64_t)c * P_c + off[el] + base[el] + rank;
        src_token[r] = (int32_t)t;
        row = (int32_t)r;
      }
      row_of[t * K + j] = row;
    }
  }
  // rows N_c..P_c-1 of this chunk's region hold no token
  for (int64_t r = N_c + (int64_t)bl * kRouteBlock + threadIdx.x; r < P_c; r += (int64_t)nbpc * kRouteBlock)
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
  size_t sm2 = (size_t)El * 4 + (size_t)(El + 1) * 4 + 8 + (size_t)4 * El * 8 + (size_t)4 * El * 4;
  {
    MOE_TRACE("route_layout", s);
    hipLaunchKernelGGL(route_layout_kernel, grid, block, sm2, s, topk_idx, scratch, counts, offsets,
                       row_of, src_token, T, E, e0, El, K, n, chunk0, nbpc, P_c);
  }
  return hipGetLastError();
}

}  // namespace moe
