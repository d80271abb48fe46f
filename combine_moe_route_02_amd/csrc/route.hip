// Routing kernels: per-token top-k over FP32 logits with renormalised gates, per-chunk expert
// histograms, and the stable expert-contiguous permutation.
//
// Token-wise ChunkedEP (Megatron-LM PR 7342, "Summary") routes each token chunk with top-k
// (no auxiliary loss, "Tests and limitations"). The pages print no formula; the reading is:
// select the k largest logits (ties to the lower expert index, NaN lowest), gates = softmax over
// the selected logits. The permutation is the stable sort of (token, slot) pairs by expert inside
// each chunk: within an expert, rows follow ascending token index.
//
// Two launches per chunk range, both deterministic:
//   route_topk   16 lanes per token (4 tokens per wave, 16 tokens per 256-thread block). Each
//                lane keeps a sorted top-K list of its share of the experts as 64-bit keys
//                (order-preserving logit bits above the complemented expert index, so ties go to
//                the lower index), then K rounds of a 16-lane max merge the lists. A histogram
//                over all E experts per 16 tokens is summed in LDS with integer atomics (the sum
//                does not depend on their order).
//   route_layout per 64-token block: rows that earlier tokens of the chunk give each local expert
//                (one wave per expert, lanes over the 16-token histograms), local offsets, then
//                each token's rank among
//                the block's earlier tokens choosing the same expert from a 64-bit ballot mask
//                (popcount below the lane); one wave per top-k slot.
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {

constexpr int kRouteBlock = 64;     // tokens per route_layout block (one ballot wave)
constexpr int kRouteThreads = 1024; // route_layout: 16 waves
constexpr int kGroup = 16;          // lanes per token in route_topk
constexpr int kTopkThreads = 256;   // route_topk block
constexpr int kHistTok = kTopkThreads / kGroup;  // tokens per histogram (16)
constexpr int kSub = kRouteBlock / kHistTok;     // histograms per route_layout block (4)

// Order-preserving map of a logit to 32 bits: larger logit -> larger key; NaN ranks as -inf and
// -0 equals +0.
MOE_DEV uint32_t logit_key(float x) {
  if (x != x) x = -__builtin_huge_valf();
  if (x == 0.f) x = 0.f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Full key: logit key above the complemented expert index, so equal logits rank the lower index
// higher. Every real key is > 0; 0 marks an empty list slot.
MOE_DEV uint64_t full_key(float x, int e) {
  return ((uint64_t)logit_key(x) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

template <int K>
MOE_DEV void insert_key(uint64_t (&l)[K], uint64_t key) {
#pragma unroll
  for (int s = 0; s < K; ++s) {
    const uint64_t cur = l[s];
    const bool take = key > cur;
    l[s] = take ? key : cur;
    key = take ? cur : key;
  }
}

MOE_DEV uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}

template <int K>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ gates,
    int32_t* __restrict__ block_hist, int64_t T, int E, int n, int chunk0, int nbpc) {
  extern __shared__ int hist[];  // [E]
  const int tid = threadIdx.x;
  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  for (int e = tid; e < E; e += kTopkThreads) hist[e] = 0;
  __syncthreads();
  const int q = tid & (kGroup - 1);                 // lane within the token's group
  const int64_t t = cr.t0 + (int64_t)bl * kHistTok + (tid / kGroup);
  const bool valid = t < cr.t1;

  uint64_t l[K];
#pragma unroll
  for (int s = 0; s < K; ++s) l[s] = 0;
  if (valid) {
    const float* row = logits + t * (int64_t)E;
    if ((E & 3) == 0) {
      // lane q reads experts [base + 4q, base + 4q + 4): 256 contiguous bytes per group
      for (int base = 0; base < E; base += 4 * kGroup) {
        const int e = base + 4 * q;
        if (e < E) {
          const float4 f = *(const float4*)(row + e);
          insert_key<K>(l, full_key(f.x, e));
          insert_key<K>(l, full_key(f.y, e + 1));
          insert_key<K>(l, full_key(f.z, e + 2));
          insert_key<K>(l, full_key(f.w, e + 3));
        }
      }
    } else {
      for (int e = q; e < E; e += kGroup) insert_key<K>(l, full_key(row[e], e));
    }
  }
  // K rounds: the group's largest head wins and its lane pops it (keys are distinct)
  uint64_t sel[K];
#pragma unroll
  for (int s = 0; s < K; ++s) {
    uint64_t m = l[0];
#pragma unroll
    for (int o = kGroup / 2; o > 0; o >>= 1) {
      const uint64_t other = shfl_xor_u64(m, o);
      m = other > m ? other : m;
    }
    sel[s] = m;
    if (l[0] == m) {
#pragma unroll
      for (int r = 0; r + 1 < K; ++r) l[r] = l[r + 1];
      l[K - 1] = 0;
    }
  }
  if (valid && q < K) {
    const float v0 = key_logit((uint32_t)(sel[0] >> 32));
    float sum = 0.f, mine = 0.f;
    int myid = 0;
#pragma unroll
    for (int s = 0; s < K; ++s) {
      const float p = expf(key_logit((uint32_t)(sel[s] >> 32)) - v0);
      sum += p;
      if (s == q) { mine = p; myid = (int)(0xffffffffu - (uint32_t)sel[s]); }
    }
    topk_idx[t * K + q] = myid;
    gates[t * K + q] = mine / sum;
    atomicAdd(&hist[myid], 1);
  }
  __syncthreads();
  // expert-major: the counts of expert e over the chunk's histograms are contiguous
  int32_t* out = block_hist + (int64_t)c * E * nbpc + bl;
  for (int e = tid; e < E; e += kTopkThreads) out[(int64_t)e * nbpc] = hist[e];
}

__global__ __launch_bounds__(kRouteThreads) void route_layout_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_token, int64_t T, int E, int e0, int El, int K, int n, int chunk0,
    int nbpc, int64_t P_c) {
  extern __shared__ unsigned char smem[];
  // layout: base[El] int, off[El+1] int, mask[El] u64
  int* base = (int*)smem;
  int* off = base + El;
  uint64_t* mask = (uint64_t*)(((uintptr_t)(off + El + 1) + 7) & ~(uintptr_t)7);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kRouteThreads / 64;
  const int c = chunk0 + blockIdx.x / nbpc;
  const int bl = blockIdx.x % nbpc;
  const ChunkRange cr = chunk_range(T, n, c);
  const int nh = nbpc * kSub;  // 16-token histograms of the chunk
  const int32_t* bh = block_hist + (int64_t)c * E * nh;  // [E][nh]

  // one wave per local expert: rows owned by earlier tokens of this chunk, and the chunk total
  for (int el = wave; el < El; el += kWaves) {
    int before = 0, total = 0;
    const int32_t* he = bh + (int64_t)(e0 + el) * nh;
    for (int b0 = 0; b0 < nh; b0 += 256) {  // four loads in flight per lane
      int h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) h[u] = (b0 + 64 * u + lane < nh) ? he[b0 + 64 * u + lane] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        before += (b0 + 64 * u + lane < bl * kSub) ? h[u] : 0;
        total += h[u];
      }
    }
    before = wave_sum_int(before);
    total = wave_sum_int(total);
    if (lane == 0) { base[el] = before; off[el + 1] = total; }
  }
  for (int el = tid; el < El; el += kRouteThreads) mask[el] = 0;
  __syncthreads();
  if (tid == 0) {  // exclusive scan over the local experts
    int run = 0;
    for (int el = 0; el < El; ++el) { int cnt = off[el + 1]; off[el] = run; run += cnt; }
    off[El] = run;
  }
  __syncthreads();
  const int N_c = off[El];
  // per-expert counts over all E experts, spread over the chunk's blocks, one wave per expert
  // (integer sums: the order does not matter)
  for (int e = bl + nbpc * wave; e < E; e += nbpc * kWaves) {
    const int32_t* he = bh + (int64_t)e * nh;
    int total = 0;
    for (int b0 = 0; b0 < nh; b0 += 256) {
      int h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) h[u] = (b0 + 64 * u + lane < nh) ? he[b0 + 64 * u + lane] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) total += h[u];
    }
    total = wave_sum_int(total);
    if (lane == 0) counts[(int64_t)c * E + e] = total;
  }
  if (bl == 0)
    for (int el = tid; el <= El; el += kRouteThreads) offsets[(int64_t)c * (El + 1) + el] = off[el];

  // wave j < K owns slot j of the block's 64 tokens (lane = token)
  const int64_t t = cr.t0 + (int64_t)bl * kRouteBlock + lane;
  const bool valid = t < cr.t1;
  const int j = wave;
  int el = -1;
  if (valid && j < K) {
    el = topk_idx[t * K + j] - e0;
    if (el >= 0 && el < El) atomicOr((unsigned long long*)&mask[el], 1ull << lane);
    else el = -1;
  }
  __syncthreads();
  if (valid && j < K) {
    int32_t row = -1;
    if (el >= 0) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int rank = __popcll(mask[el] & below);
      const int64_t r = (int64_t)c * P_c + off[el] + base[el] + rank;
      src_token[r] = (int32_t)t;
      row = (int32_t)r;
    }
    row_of[t * K + j] = row;
  }
  // rows N_c..P_c-1 of this chunk's region hold no token
  for (int64_t r = N_c + (int64_t)bl * kRouteThreads + tid; r < P_c; r += (int64_t)nbpc * kRouteThreads)
    src_token[(int64_t)c * P_c + r] = -1;
}

int route_blocks_per_chunk(int64_t T, int n) {
  int64_t tc = (T + n - 1) / n;
  int64_t nb = (tc + kRouteBlock - 1) / kRouteBlock;
  return (int)(nb < 1 ? 1 : nb);
}

int64_t route_scratch_bytes(int64_t T, int n, int E) {
  return (int64_t)n * route_blocks_per_chunk(T, n) * kSub * E * (int64_t)sizeof(int32_t);
}

hipError_t launch_route(const float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* src_token, int32_t* scratch,
                        int64_t T, int E, int e0, int El, int K, int n, int chunk0, int nchunks,
                        int64_t P_c, hipStream_t s) {
  const int nbpc = route_blocks_per_chunk(T, n);
  dim3 grid(nbpc * nchunks), block(kRouteThreads);
  dim3 grid1(nbpc * kSub * nchunks), block1(kTopkThreads);
  size_t sm1 = (size_t)E * sizeof(int);
  switch (K) {
#define MOE_ROUTE_K(KK)                                                                      \
  case KK: {                                                                                 \
    MOE_TRACE("route_topk", s);                                                              \
    hipLaunchKernelGGL(route_topk_kernel<KK>, grid1, block1, sm1, s, logits, topk_idx, gates, \
                       scratch, T, E, n, chunk0, nbpc * kSub);                               \
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
