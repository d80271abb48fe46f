// Routing kernels: per-token top-k over FP32 logits with renormalised gates, per-chunk expert
// histograms, and the stable expert-contiguous permutation.
//
// Token-wise ChunkedEP (Megatron-LM PR 7342, "Summary") routes each token chunk with top-k
// (no auxiliary loss, "Tests and limitations"). The pages print no formula; the reading is:
// select the k largest logits (ties to the lower expert index, NaN lowest), gates = softmax over
// the selected logits. The permutation is the stable sort of (token, slot) pairs by expert inside
// each chunk: within an expert, rows follow ascending token index.
//
// Two or three launches per chunk range, all deterministic (route_topk, or route_proj_topk when
// routing starts from x and the router weight):
//   route_topk   16 lanes per token (4 tokens per wave, 16 tokens per 256-thread block). Each
//                lane keeps a sorted top-K list of its share of the experts as 64-bit keys
//                (order-preserving logit bits above the complemented expert index, so ties go to
//                the lower index), then K rounds of a 16-lane max merge the lists. A histogram
//                over all E experts per 16 tokens is summed in LDS with integer atomics (the sum
//                does not depend on their order).
//   route_scan   (chunks of more than 128 64-token blocks) one wave per expert and chunk: the
//                chunk's total per expert (counts) and, per 64-token block, the rows that the
//                chunk's earlier blocks give the expert (an exclusive scan of the block sums, one
//                block per lane), so the work is linear in the chunk's tokens.
//   route_layout per 64-token block: local offsets from the counts, then each token's rank among
//                the block's earlier tokens choosing the same expert from a 64-bit ballot mask
//                (popcount below the lane) plus the rows of the earlier blocks; one wave per top-k
//                slot. For shorter chunks the block sums the earlier blocks' histograms itself
//                (one launch fewer).
#include <mutex>
#include <type_traits>

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

// Top-K of one token's logits row (nullptr: no token) for the 16-lane group of lane q: each lane
// keeps a sorted list of its share of the experts, then K rounds of a 16-lane max merge the
// lists (keys are distinct). Every lane of the group must call it (it shuffles).
template <int K>
MOE_DEV void select_topk(const float* row, int E, int q, uint64_t (&sel)[K]) {
  uint64_t l[K];
#pragma unroll
  for (int s = 0; s < K; ++s) l[s] = 0;
  if (row) {
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
}

// Lane q < K of a token's group writes slot q (descending logit): the expert, its gate
// exp(l_q - l_0) / sum_s exp(l_s - l_0) over the K selected logits, and one histogram count.
template <int K>
MOE_DEV void emit_topk(const uint64_t (&sel)[K], int q, int64_t t, int32_t* topk_idx, float* gates, int* hist) {
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
  uint64_t sel[K];
  select_topk<K>(valid ? logits + t * (int64_t)E : nullptr, E, q, sel);
  if (valid && q < K) emit_topk<K>(sel, q, t, topk_idx, gates, hist);
  __syncthreads();
  // expert-major: the counts of expert e over the chunk's histograms are contiguous
  int32_t* out = block_hist + (int64_t)c * E * nbpc + bl;
  for (int e = tid; e < E; e += kTopkThreads) out[(int64_t)e * nbpc] = hist[e];
}

// Router projection fused with the top-K: logits = x . W_r^T for 32 tokens and all E experts
// (E <= 256) on BF16 MFMA with FP32 accumulation, then the same selection as route_topk from LDS.
// The K loop streams 64-wide K stages of the 32 x rows and the E W_r rows through a 4-stage LDS
// ring with direct-to-LDS 16-byte loads: one wave instruction moves 8 whole 128-byte row
// segments, and each stage holds (32 + E) rows of 128 bytes whose 16-byte chunks are
// XOR-swizzled by (row & 7), so the 32-row fragment reads hit every bank once. Loads run three
// stages ahead with one barrier per stage, spread over all eight waves (measured faster than
// four waves issuing them). Wave w multiplies the 32-expert blocks w % 4,
// w % 4 + 4, ... over the K steps 2 (w / 4), 2 (w / 4) + 1 of each stage; the two partial tiles
// are added in LDS in a fixed order.
constexpr int kProjTok = 32;
constexpr int kRxThreads = 512;
constexpr int kRxNst = 4;        // LDS ring stages
constexpr int kRxRowB = 128;     // bytes of K per row per stage (64 BF16)

MOE_DEV int rx_off(int row, int chunk) { return row * kRxRowB + ((chunk ^ (row & 7)) << 4); }

template <int N>
MOE_DEV void rx_wait(int loads_per_stage) {  // vmcnt(2 * loads_per_stage), 1 <= loads_per_stage <= N
  if (loads_per_stage >= N) { wait_vm<2 * N>(); return; }
  if constexpr (N > 1) rx_wait<N - 1>(loads_per_stage);
}

template <int K, int NB>
__global__ __launch_bounds__(kRxThreads) void route_proj_topk_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ w_r, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ gates, int32_t* __restrict__ block_hist, int64_t T,
    int E, int H, int n, int chunk0, int nb32) {
  extern __shared__ __attribute__((aligned(1024))) char rx_smem[];
  char* smem = rx_smem;
  const int SS = (kProjTok + E) * kRxRowB;        // stage bytes
  int* hist = (int*)(smem + kRxNst * SS);          // [2][E], outside the ring
  float* lg = (float*)smem;                        // [kProjTok][E + 4] logits, on the ring after the K loop
  const int ldl = E + 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = chunk0 + blockIdx.x / nb32, bl = blockIdx.x % nb32;
  const ChunkRange cr = chunk_range(T, n, c);
  const int64_t tb = cr.t0 + (int64_t)bl * kProjTok;  // first token of the block
  const int ntok = (int)max((int64_t)0, min((int64_t)kProjTok, cr.t1 - tb));
  for (int e = tid; e < 2 * E; e += kRxThreads) hist[e] = 0;
  const int neb = E / 32, kp = wave / 4;
  const int r = lane & 31, h = lane >> 5;
  if (ntok > 0) {
    // loads: the stage's M = (32 + E) / 8 wave instructions (8 rows each) are dealt round-robin
    // to the 8 waves; rows 0..31 are x (masked past ntok), rows 32.. are W_r
    const int M = (kProjTok + E) / 8;
    const int mine = (M - wave + 7) / 8;           // this wave's instructions per stage (>= 1)
    const __amdgpu_buffer_rsrc_t rsx = make_rsrc(x + tb * (int64_t)H, (int64_t)ntok * H * 2);
    const __amdgpu_buffer_rsrc_t rsw = make_rsrc(w_r, (int64_t)E * H * 2);
    auto issue = [&](int stage) {
      char* slot = smem + (stage % kRxNst) * SS;
      for (int q = wave; q < M; q += 8) {
        const int row = 8 * q + (lane >> 3);
        const int g = (lane & 7) ^ (row & 7);                 // global chunk this lane fetches
        const bool isx = row < kProjTok;
        const int grow = isx ? row : row - kProjTok;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isx ? rsx : rsw, (lds_void_t*)(slot + q * 1024), 16,
                                                 grow * H * 2 + g * 16, stage * kRxRowB, 0, 0);
      }
    };
    f32x16_t acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    const int nks = H / 64;
    for (int s0 = 0; s0 < kRxNst - 1; ++s0) issue(s0);
    for (int st = 0; st < nks; ++st) {
      rx_wait<5>(mine);              // this wave's loads of stage st have landed (two younger in flight)
      __builtin_amdgcn_s_barrier();  // stage st is in LDS for every wave; stage st-1 is consumed
      issue(st + kRxNst - 1);        // into the slot of stage st-1 (past the end: masked or unused)
      const char* slot = smem + (st % kRxNst) * SS;
#pragma unroll
      for (int s = 2 * kp; s < 2 * kp + 2; ++s) {
        const bf16x8_t fa = *(const bf16x8_t*)(slot + rx_off(r, 2 * s + h));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int eb = wave % 4 + 4 * i;
          if (eb < neb) {
            const bf16x8_t fb = *(const bf16x8_t*)(slot + rx_off(kProjTok + 32 * eb + r, 2 * s + h));
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc[i], 0, 0, 0);
          }
        }
      }
    }
    wait_vm<0>();
    __syncthreads();  // ring free
    // acc[i][4g + q] is (token r, expert 32 eb + 8g + 4 h + q): K part 1 stores, part 0 adds
    for (int pass = 1; pass >= 0; --pass) {
      if (kp == pass) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int eb = wave % 4 + 4 * i;
          if (eb >= neb) continue;
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float* d = lg + r * ldl + eb * 32 + 8 * g + 4 * h + q;
              *d = pass ? acc[i][4 * g + q] : acc[i][4 * g + q] + *d;
            }
        }
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
  }
  // top-K: 16 lanes per token, all 32 tokens at once
  const int q = tid & (kGroup - 1);
  const int tl = tid / kGroup;
  const bool valid = tl < ntok;
  uint64_t sel[K];
  select_topk<K>(valid ? lg + tl * ldl : nullptr, E, q, sel);
  if (valid && q < K) emit_topk<K>(sel, q, tb + tl, topk_idx, gates, hist + (tl / kHistTok) * E);
  if (logits)
    for (int i = tid; i < ntok * E; i += kRxThreads)
      logits[(tb + i / E) * (int64_t)E + i % E] = lg[(i / E) * ldl + i % E];
  __syncthreads();
  // this block's two 16-token histograms, expert-major
  const int nh = 2 * nb32;
  for (int i = tid; i < 2 * E; i += kRxThreads)
    block_hist[((int64_t)c * E + i % E) * nh + 2 * bl + i / E] = hist[i];
}

// Per chunk c and expert e (one wave each): counts[c][e] = the chunk's rows of e, and
// pre[c][e][b] = rows of e in the chunk's 64-token blocks before b. Lane l of an iteration owns
// block b0 + l, whose four 16-token histograms it reads as one 16-byte load.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(const int32_t* __restrict__ block_hist,
                                                                   int32_t* __restrict__ pre,
                                                                   int32_t* __restrict__ counts, int E,
                                                                   int chunk0, int nbpc) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kScanThreads / 64) + (threadIdx.x >> 6);
  const int c = chunk0 + blockIdx.y;
  if (e >= E) return;
  const int nh = nbpc * kSub;
  const int4* he = (const int4*)(block_hist + ((int64_t)c * E + e) * nh);
  int32_t* pe = pre + ((int64_t)c * E + e) * nbpc;
  int carry = 0;
  for (int b0 = 0; b0 < nbpc; b0 += 64) {
    const int b = b0 + lane;
    int v = 0;
    if (b < nbpc) {
      const int4 h = he[b];
      v = h.x + h.y + h.z + h.w;
    }
    int incl = v;  // inclusive scan over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (b < nbpc) pe[b] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) counts[(int64_t)c * E + e] = carry;
}

// kScanned: the prefixes and counts come from route_scan (long chunks). Otherwise (chunks of at
// most kLayoutDirectBlocks blocks) each block sums the histograms before it itself, one wave per
// local expert, and the blocks share the counts of all E experts between them: quadratic in the
// chunk length but one launch fewer, which is the cheaper form for short chunks.
constexpr int kLayoutDirectBlocks = 128;
template <bool kScanned>
__global__ __launch_bounds__(kRouteThreads) void route_layout_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_hist, const int32_t* __restrict__ pre,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_token, int64_t T, int E, int e0, int El, int K, int n, int chunk0, int nbpc,
    int64_t P_c) {
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

  if constexpr (kScanned) {
    for (int el = tid; el < El; el += kRouteThreads) {
      base[el] = pre[((int64_t)c * E + e0 + el) * nbpc + bl];
      off[el + 1] = counts[(int64_t)c * E + e0 + el];
      mask[el] = 0;
    }
  } else {
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
    // per-expert counts over all E experts, spread over the chunk's blocks, one wave per expert
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
  }
  __syncthreads();
  if (tid == 0) {  // exclusive scan over the local experts
    int run = 0;
    for (int el = 0; el < El; ++el) { int cnt = off[el + 1]; off[el] = run; run += cnt; }
    off[El] = run;
  }
  __syncthreads();
  const int N_c = off[El];
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

// Routing scratch for callers that cannot allocate (moe_route_noalloc): the per-16-token expert
// histograms of one call live in this file-scope array instead of a caller workspace. Each GPU
// holds its own copy until the process ends; every call on that GPU shares it (route_topk
// overwrites every entry the layout kernel reads, so nothing needs clearing between calls).
static __device__ __align__(256) int32_t scratch[kNoAllocRouteScratchBytes / sizeof(int32_t)];

// Device address of `scratch` on the current device, looked up once per device with that device
// current (in host code the array's name is only a host-side stand-in).
hipError_t route_noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

int route_blocks_per_chunk(int64_t T, int n) {
  int64_t tc = (T + n - 1) / n;
  int64_t nb = (tc + kRouteBlock - 1) / kRouteBlock;
  return (int)(nb < 1 ? 1 : nb);
}

// Routing scratch: the 16-token histograms [n][E][nbpc * 4], then the per-64-token-block prefixes
// [n][E][nbpc].
static int64_t route_hist_ints(int64_t T, int n, int E) { return (int64_t)n * route_blocks_per_chunk(T, n) * kSub * E; }
int64_t route_scratch_bytes(int64_t T, int n, int E) {
  return (route_hist_ints(T, n, E) + (int64_t)n * route_blocks_per_chunk(T, n) * E) * (int64_t)sizeof(int32_t);
}

static hipError_t launch_layout(const int32_t* topk_idx, int32_t* scratch, int32_t* counts,
                               int32_t* offsets, int32_t* row_of, int32_t* src_token, int64_t T, int E,
                               int e0, int El, int K, int n, int chunk0, int nchunks, int64_t P_c,
                               hipStream_t s) {
  const int nbpc = route_blocks_per_chunk(T, n);
  int32_t* pre = scratch + route_hist_ints(T, n, E);
  const bool scanned = nbpc > kLayoutDirectBlocks;
  if (scanned) {
    MOE_TRACE("route_scan", s);
    MOE_LAUNCH(route_scan_kernel, dim3((unsigned)((E + kScanThreads / 64 - 1) / (kScanThreads / 64)), (unsigned)nchunks),
               dim3(kScanThreads), 0, s, scratch, pre, counts, E, chunk0, nbpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  size_t sm2 = (size_t)El * 4 + (size_t)(El + 1) * 4 + 8 + (size_t)El * 8;
  MOE_TRACE("route_layout", s);
  if (scanned)
    MOE_LAUNCH(route_layout_kernel<true>, dim3(nbpc * nchunks), dim3(kRouteThreads), sm2, s, topk_idx, scratch,
               pre, counts, offsets, row_of, src_token, T, E, e0, El, K, n, chunk0, nbpc, P_c);
  else
    MOE_LAUNCH(route_layout_kernel<false>, dim3(nbpc * nchunks), dim3(kRouteThreads), sm2, s, topk_idx, scratch,
               pre, counts, offsets, row_of, src_token, T, E, e0, El, K, n, chunk0, nbpc, P_c);
  return hipGetLastError();
}

size_t route_x_lds_bytes(int E) { return (size_t)kRxNst * (kProjTok + E) * kRxRowB + (size_t)2 * E * 4; }

hipError_t launch_route_x(const void* x, const void* w_r, float* logits, int32_t* topk_idx, float* gates,
                          int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_token,
                          int32_t* scratch, int64_t T, int E, int H, int e0, int El, int K, int n, int chunk0,
                          int nchunks, int64_t P_c, hipStream_t s) {
  const int nb32 = route_blocks_per_chunk(T, n) * (kRouteBlock / kProjTok);
  const int NB = (E + 127) / 128;  // 32-expert blocks per wave (E <= 256)
  const size_t lds = route_x_lds_bytes(E);
  dim3 grid(nb32 * nchunks);
  {
    MOE_TRACE("route_proj_topk", s);
    switch (K * 8 + NB) {
#define MOE_RX(KK, NN)                                                                                 \
  case KK * 8 + NN: {                                                                                 \
    auto k = route_proj_topk_kernel<KK, NN>;                                                          \
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                                    \
    MOE_LAUNCH(k, grid, dim3(kRxThreads), lds, s, (const __bf16*)x, (const __bf16*)w_r, logits, \
                       topk_idx, gates, scratch, T, E, H, n, chunk0, nb32);                            \
    break;                                                                                            \
  }
#define MOE_RX_K(KK) MOE_RX(KK, 1) MOE_RX(KK, 2)
      MOE_RX_K(1) MOE_RX_K(2) MOE_RX_K(3) MOE_RX_K(4) MOE_RX_K(5) MOE_RX_K(6) MOE_RX_K(7) MOE_RX_K(8)
#undef MOE_RX_K
#undef MOE_RX
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_layout(topk_idx, scratch, counts, offsets, row_of, src_token, T, E, e0, El, K, n, chunk0, nchunks,
                       P_c, s);
}

hipError_t launch_route(const float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* src_token, int32_t* scratch,
                        int64_t T, int E, int e0, int El, int K, int n, int chunk0, int nchunks,
                        int64_t P_c, hipStream_t s) {
  const int nbpc = route_blocks_per_chunk(T, n);
  dim3 grid1(nbpc * kSub * nchunks), block1(kTopkThreads);
  size_t sm1 = (size_t)E * sizeof(int);
  switch (K) {
#define MOE_ROUTE_K(KK)                                                                      \
  case KK: {                                                                                 \
    MOE_TRACE("route_topk", s);                                                              \
    MOE_LAUNCH(route_topk_kernel<KK>, grid1, block1, sm1, s, logits, topk_idx, gates, \
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
  return launch_layout(topk_idx, scratch, counts, offsets, row_of, src_token, T, E, e0, El, K, n, chunk0, nchunks,
                       P_c, s);
}

}  // namespace moe
