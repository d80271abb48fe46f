// Router weight gradient on BF16 matrix cores (FP32 dlogits split into BF16 high and low parts,
// FP32 accumulation, split-K partials reduced in order) and FP32 SIMT grouped GEMMs for FP32
// payloads; the BF16/FP8 expert GEMMs live in grouped_gemm.hip.
//
// Token-wise ChunkedEP (Megatron-LM PR 7342, "Numerical status -- unresolved") accumulates the
// router weight gradient across chunks in FP32 and converts it once: each chunk's dlogits^T x is
// computed in FP32 (dlogits = hi + lo with hi, lo BF16, x exactly BF16), its split-K partials are
// summed in a fixed order into the FP32 accumulator, and the last chunk converts it once.
//
// Router tile engine: 256 threads (4 waves, 2 x 2), LDS stages of BK = 64, double-buffered,
// K-contiguous 128-byte rows with 16-byte chunks XOR-swizzled by the row index; operands whose K
// runs along HBM rows are transposed in registers while staging (8 K-rows x V columns per
// thread).
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace gemm {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kMaxGroups = 1024;

// LDS tile address (in BF16 elements) of 16-byte chunk `chunk` of tile row `row`: rows of 128 bytes
// with the chunk XOR-swizzled by row % 8, so that 8 consecutive rows read at one chunk (MFMA
// fragments) and the 8 chunks of one row (staging writes) each cover all banks; row % 8 does
// not change between 32-row MFMA blocks, so their addresses differ by constants.
MOE_DEV int sw(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

MOE_DEV u32x4 zero4() { return {0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------------------------------------
// Operand staging (global -> registers -> LDS)

// Operands are staged with raw buffer loads: the tile's base address and its valid extent
// live in a scalar buffer descriptor (reads past num_records return zero, which masks rows
// beyond an expert's segment or a matrix edge), each lane keeps one 32-bit byte offset, and
// the per-row / per-stage offsets are wave-uniform scalar offsets.
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor word 3

MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(bytes < 0 ? 0 : (bytes > lim ? lim : bytes)),
                                           kBufferWord3);
}

// K-contiguous rows, R rows x 64 BF16 per stage; thread tid stages rows tid/8 + 32*i (i < R/32),
// 16-byte chunk tid%8 of each. SWIGLU_WTN > 0 maps tile rows to interleaved gate/up weight rows
// (per wave column block of SWIGLU_WTN rows: first half gate rows j, second half up rows I + j).
template <int R, bool MASK_K = true>
struct KSlow {
  static constexpr int V = R / 32;
  static constexpr int W = V / 2;  // dwords per loaded K-row (V BF16 values)
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;                   // (8 * kblk) K-rows + this lane's mn block, in bytes
  uint32_t ldb;                    // bytes between K-rows
  uint32_t v[8][W];
  MOE_DEV int mnblk(int tid) const { return tid >> 3; }
  MOE_DEV int kblk(int tid) const { return tid & 7; }
  // base: element (k = 0, mn = 0) of the tile; valid_k: K-rows readable (later rows load 0)
  MOE_DEV void init(const uint16_t* base, int64_t ld, int64_t valid_k, int tid) {
    ldb = (uint32_t)(ld * 2);
    rsrc = make_rsrc(base, valid_k * ld * 2);
    voff = (uint32_t)(8 * kblk(tid)) * ldb + (uint32_t)(mnblk(tid) * V * 2);
  }
  MOE_DEV void fetch(int k0, int /*tid*/) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int so = (int)((uint32_t)(k0 + i) * ldb);
      if constexpr (W == 4) {
        i32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff, so, 0);
        v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
      } else if constexpr (W == 2) {
        i32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (int)voff, so, 0);
        v[i][0] = t.x; v[i][1] = t.y;
      } else {
        v[i][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)voff, so, 0);
      }
    }
  }
  // Column pair (2p, 2p+1) comes from dword p of every loaded K-row.
  MOE_DEV void commit(uint16_t* lds, int tid) const {
    const int mb = mnblk(tid), kb = kblk(tid);
#pragma unroll
    for (int p = 0; p < V / 2; ++p) {
      uint32_t e[4], o[4];  // even column 2p and odd column 2p+1, 8 K values each
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[q] = (v[2 * q][p] & 0xffffu) | (v[2 * q + 1][p] << 16);
        o[q] = (v[2 * q][p] >> 16) | (v[2 * q + 1][p] & 0xffff0000u);
      }
      const int r0 = mb * V + 2 * p;
      *(u32x4*)(lds + sw(r0, kb)) = u32x4{e[0], e[1], e[2], e[3]};
      *(u32x4*)(lds + sw(r0 + 1, kb)) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
};

// FP32 operand with K along HBM rows, split into BF16 high and low parts (x = hi + lo + O(2^-17 x)).
template <int R>
struct KSlowSplit {
  static constexpr int V = R / 32;  // floats per K-row (V/4 16-byte loads)
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff, ldb;
  float v[8][V];
  MOE_DEV void init(const float* base, int64_t ld, int64_t valid_k, int tid) {
    ldb = (uint32_t)(ld * 4);
    rsrc = make_rsrc(base, valid_k * ld * 4);
    voff = (uint32_t)(8 * (tid & 7)) * ldb + (uint32_t)((tid >> 3) * V * 4);
  }
  MOE_DEV void fetch(int k0, int /*tid*/) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int c = 0; c < V; c += 4) {
        i32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff + 4 * c, (int)((uint32_t)(k0 + i) * ldb), 0);
        v[i][c] = __int_as_float(t.x); v[i][c + 1] = __int_as_float(t.y);
        v[i][c + 2] = __int_as_float(t.z); v[i][c + 3] = __int_as_float(t.w);
      }
  }
  MOE_DEV void commit(uint16_t* lds_hi, uint16_t* lds_lo, int tid) const {
    const int mb = tid >> 3, kb = tid & 7;
#pragma unroll
    for (int c = 0; c < V; ++c) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float a = v[2 * q][c], b = v[2 * q + 1][c];
        uint16_t ah = f2bf(a), bh = f2bf(b);
        uint16_t al = f2bf(a - bf2f(ah)), bl = f2bf(b - bf2f(bh));
        wh[q] = (uint32_t)ah | ((uint32_t)bh << 16);
        wl[q] = (uint32_t)al | ((uint32_t)bl << 16);
      }
      *(u32x4*)(lds_hi + sw(mb * V + c, kb)) = u32x4{wh[0], wh[1], wh[2], wh[3]};
      *(u32x4*)(lds_lo + sw(mb * V + c, kb)) = u32x4{wl[0], wl[1], wl[2], wl[3]};
    }
  }
};

// ---------------------------------------------------------------------------------------------
// MFMA inner product over one LDS stage: acc[tm][tn] += A[rows] * B[rows]^T over 64 K.
// The MFMA is issued with the B fragment as its first operand, so the 32x32 result block is
// transposed: lane l holds output row (l & 31) and, for accumulator element i, output column
// 8*(i/4) + 4*(l/32) + i%4 -- four consecutive columns per group of four elements, which the
// epilogues store as one 8-byte BF16 vector.
template <int TM, int TN, int TMA = TM>
MOE_DEV void mma_stage(const uint16_t* la, const uint16_t* lb, int arow0, int brow0, int lane,
                       f32x16_t (&acc)[TM][TN], int tma = TM) {
  const int r = lane & 31, hk = lane >> 5;
  bf16x8_t fa[2][TM], fb[2][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) fa[0][tm] = *(const bf16x8_t*)(la + sw(arow0 + tm * 32 + r, hk));
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) fb[0][tn] = *(const bf16x8_t*)(lb + sw(brow0 + tn * 32 + r, hk));
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int cb = kk & 1, nb = cb ^ 1;
    if (kk + 1 < BK / 16) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        fa[nb][tm] = *(const bf16x8_t*)(la + sw(arow0 + tm * 32 + r, 2 * (kk + 1) + hk));
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        fb[nb][tn] = *(const bf16x8_t*)(lb + sw(brow0 + tn * 32 + r, 2 * (kk + 1) + hk));
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      if (tm < tma)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cb][tn], fa[cb][tm], acc[tm][tn], 0, 0, 0);
  }
}

// Output coordinates inside a 32x32 block for lane `lane`: row, and first column of group g.
MOE_DEV int out_row(int lane) { return lane & 31; }
MOE_DEV int out_col(int g, int lane) { return 8 * g + 4 * (lane >> 5); }
MOE_DEV uint2 pack4(float a, float b, float c, float d) { return make_uint2(pack_bf2(a, b), pack_bf2(c, d)); }
MOE_DEV void unpack4(uint2 v, float* f) {
  f[0] = bf2f(v.x & 0xffff); f[1] = bf2f(v.x >> 16); f[2] = bf2f(v.y & 0xffff); f[3] = bf2f(v.y >> 16);
}

// ---------------------------------------------------------------------------------------------
// K-grouped GEMMs: weight gradients C_e[m][n] = sum over the rows of every chunk of expert e of
// A[row][m] * B[row][n] (both operands K along HBM rows), and the router weight gradient with
// an FP32 A operand split into BF16 high/low parts, written as split-K partial sums.
struct KGroupArgs {
  const void* A;          // [rows, M] (BF16, or FP32 for the router)
  const uint16_t* B;      // [rows, N]
  void* C;                // per-expert [M, N] (BF16), or partials [S, M, N] (FP32)
  int64_t lda, ldb, strideC;
  int M, N;
  const int32_t* offsets; // per-chunk local offsets (expert mode)
  int El, n_chunks;
  int64_t P_c;
  int64_t k0, klen;       // router mode: token range, split into S parts of ksplit rows
  int ksplit;
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void router_wgrad_kernel(KGroupArgs a) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  // stage s: A high/low planes at lds + s*2*BM*BK, B tile after both stages of A
#define LA(s) (lds + (s) * (2 * BM * BK))
#define LB(s) (lds + 4 * BM * BK + (s) * (BN * BK))

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int mtiles = (a.M + BM - 1) / BM, ntiles = (a.N + BN - 1) / BN;
  const int tile = blockIdx.x;
  const int grp = tile / (mtiles * ntiles);       // K split
  const int t_in = tile % (mtiles * ntiles);
  const int m0 = (t_in / ntiles) * BM, n0 = (t_in % ntiles) * BN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  const int64_t row0 = a.k0 + (int64_t)grp * a.ksplit;
  const int64_t rem = a.k0 + a.klen - row0;
  const int len = (int)(rem < a.ksplit ? (rem < 0 ? 0 : rem) : a.ksplit);
  if (len > 0) {
    KSlow<BN> ldB;
    ldB.init(a.B + row0 * a.ldb + n0, a.ldb, len, tid);
    KSlowSplit<BM> ldAs;
    ldAs.init((const float*)a.A + row0 * a.lda + m0, a.lda, len, tid);
    const int nks = (len + BK - 1) / BK;
    ldAs.fetch(0, tid);
    ldAs.commit(LA(0), LA(0) + BM * BK, tid);
    ldB.fetch(0, tid);
    ldB.commit(LB(0), tid);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nks) {
        ldAs.fetch((ks + 1) * BK, tid);
        ldB.fetch((ks + 1) * BK, tid);
      }
      mma_stage<TM, TN>(LA(cur), LB(cur), wm * WTM, wn * WTN, lane, acc);
      mma_stage<TM, TN>(LA(cur) + BM * BK, LB(cur), wm * WTM, wn * WTN, lane, acc);
      if (ks + 1 < nks) {
        ldAs.commit(LA(cur ^ 1), LA(cur ^ 1) + BM * BK, tid);
        ldB.commit(LB(cur ^ 1), tid);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m0 + wm * WTM + tm * 32 + out_row(lane);
    if (m >= a.M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + tn * 32 + out_col(g, lane);
        if (n >= a.N) continue;
        const f32x16_t& v = acc[tm][tn];
        const int64_t o = (int64_t)grp * a.strideC + (int64_t)m * a.N + n;
        *(float4*)((float*)a.C + o) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
  }
}

#undef LA
#undef LB

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

hipError_t launch_router_wgrad(bool bf16, const float* dlogits, const void* x, float* partials,
                               float* dwr_acc, bool first, void* dwr, int64_t t0, int64_t t1, int E,
                               int H, hipStream_t s) {
  const int64_t len = t1 - t0;
  const int ks = router_ksplit(len);
  int S = (int)((len + ks - 1) / ks);
  if (S < 1) S = 1;
  if (len > 0) {
    if (bf16) {
      constexpr int BM = 128, BN = 128;
      size_t lds = (size_t)2 * (2 * BM + BN) * BK * sizeof(uint16_t);
      auto k = router_wgrad_kernel<BM, BN, 2, 2>;
      hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      KGroupArgs a{};
      a.A = dlogits; a.B = (const uint16_t*)x; a.C = partials; a.lda = E; a.ldb = H;
      a.strideC = (int64_t)E * H; a.M = E; a.N = H; a.k0 = t0; a.klen = len; a.ksplit = ks;
      {
        MOE_TRACE("gemm_router_wgrad", s);
        MOE_LAUNCH(k, dim3(S * ((E + BM - 1) / BM) * ((H + BN - 1) / BN)), dim3(kThreads), lds, s, a);
      }
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
