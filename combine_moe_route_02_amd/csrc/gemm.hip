// Grouped expert GEMMs on CDNA4 matrix cores (BF16 MFMA 32x32x16, FP32 accumulation) and an
// FP32 SIMT variant for FP32 payloads.
//
// The expert FFN is a grouped GEMM whose groups are the local experts' row segments in the
// expert-contiguous dispatch buffer (token-wise ChunkedEP, Megatron-LM PR 7342, "Summary":
// expert compute per token chunk). Group sizes are only known on the device (the offset table
// written by routing), so the row-grouped kernels are persistent: every workgroup rebuilds the
// group -> tile prefix from the offset table and strides over the tiles; nothing returns to the
// host. Weight-gradient kernels iterate K over the rows of every chunk of one expert in one
// FP32 reduction and convert once (the FP32-accumulate-then-convert rule that ChunkedEP's
// "Numerical status -- unresolved" states for the router weights).
//
// Tile engine: workgroup of 256 threads (4 waves, wave grid WM x WN), LDS stages of BK = 64,
// double-buffered; both operands live in LDS K-contiguous with the eight 16-byte chunks of a row
// XOR-swizzled by the row index (conflict-free ds_read_b128 for the MFMA operand layout).
// Operands whose K runs along rows in HBM (NN dgrad weights, TN wgrad activations) are
// transposed in registers while staging (8 K-rows x V columns per thread).
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace gemm {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kMaxGroups = 1024;

MOE_DEV int sw(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

MOE_DEV u32x4 zero4() { return {0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------------------------------------
// Operand staging (global -> registers -> LDS)

// K-contiguous rows: tile row r at rowptr(r) + k. R rows x 64 BF16; R/32 vectors per thread.
template <int R>
struct KMajor {
  static constexpr int NV = R / 32;
  const uint16_t* p[NV];
  u32x4 v[NV];
  MOE_DEV void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = p[i] ? *(const u32x4*)(p[i] + k0) : zero4();
  }
  MOE_DEV void commit(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int id = tid + i * kThreads;
      *(u32x4*)(lds + sw(id >> 3, id & 7)) = v[i];
    }
  }
  // row r of thread's i-th vector
  MOE_DEV static int row_of(int tid, int i) { return (tid + i * kThreads) >> 3; }
  MOE_DEV static int chunk_of(int tid) { return tid & 7; }
};

// K along HBM rows: element (mn, k) at base[k * ld + mn]. One block of 8 K-rows x V columns per
// thread (V = R/32), transposed in registers into V K-contiguous 16-byte chunks.
template <int R>
struct KSlow {
  static constexpr int V = R / 32;
  static constexpr int W = V / 2;           // dwords per loaded K-row (V BF16 values)
  const uint16_t* base;                     // points at (k = 0, mn = this thread's first column)
  int64_t ld;
  int kvalid;                               // K rows valid in the current segment
  bool mnok;
  uint32_t v[8][W];
  MOE_DEV int mnblk(int tid) const { return tid & 31; }
  MOE_DEV int kblk(int tid) const { return tid >> 5; }
  MOE_DEV void fetch(int k0, int tid) {
    const int kb = k0 + 8 * kblk(tid);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bool ok = mnok && (kb + i) < kvalid;
      const uint16_t* q = base + (int64_t)(kb + i) * ld;
      if constexpr (W == 4) {
        u32x4 t = ok ? *(const u32x4*)q : zero4();
        v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
      } else if constexpr (W == 2) {
        uint2 t = ok ? *(const uint2*)q : make_uint2(0u, 0u);
        v[i][0] = t.x; v[i][1] = t.y;
      } else {
        v[i][0] = ok ? *(const uint32_t*)q : 0u;
      }
    }
  }
  MOE_DEV void commit(uint16_t* lds, int tid) const {
    const int mb = mnblk(tid), kb = kblk(tid);
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const int half = c & 1, wd = c >> 1;
      u32x4 o;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = half ? (v[2 * q][wd] >> 16) : (v[2 * q][wd] & 0xffffu);
        uint32_t hi = half ? (v[2 * q + 1][wd] & 0xffff0000u) : (v[2 * q + 1][wd] << 16);
        w[q] = lo | hi;
      }
      o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
      *(u32x4*)(lds + sw(mb * V + c, kb)) = o;
    }
  }
};

// FP32 operand with K along HBM rows, split into BF16 high and low parts (x = hi + lo + O(2^-17 x)).
template <int R>
struct KSlowSplit {
  static constexpr int V = R / 32;
  const float* base;
  int64_t ld;
  int kvalid;
  float v[8][V];
  MOE_DEV void fetch(int k0, int tid) {
    const int kb = k0 + 8 * (tid >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bool ok = (kb + i) < kvalid;
      const float* q = base + (int64_t)(kb + i) * ld;
#pragma unroll
      for (int c = 0; c < V; c += 4) {
        float4 t = ok ? *(const float4*)(q + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[i][c] = t.x; v[i][c + 1] = t.y; v[i][c + 2] = t.z; v[i][c + 3] = t.w;
      }
    }
  }
  MOE_DEV void commit(uint16_t* lds_hi, uint16_t* lds_lo, int tid) const {
    const int mb = tid & 31, kb = tid >> 5;
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
template <int TM, int TN>
MOE_DEV void mma_stage(const uint16_t* la, const uint16_t* lb, int arow0, int brow0, int lane,
                       f32x16_t (&acc)[TM][TN]) {
  const int r = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8_t a[TM], b[TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) a[tm] = *(const bf16x8_t*)(la + sw(arow0 + tm * 32 + r, 2 * kk + hk));
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) b[tn] = *(const bf16x8_t*)(lb + sw(brow0 + tn * 32 + r, 2 * kk + hk));
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
  }
}

// Output coordinates of accumulator element i of a 32x32 MFMA tile held by `lane`.
MOE_DEV int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
MOE_DEV int acc_col(int lane) { return lane & 31; }

// ---------------------------------------------------------------------------------------------
// Row-grouped GEMMs (forward and input-gradient), persistent over device-side groups.
//   C[r0 + m][n] = sum_k A[r0 + m][k] * B_e(n, k) for the rows of local expert e in a chunk.
enum RowsMode { kGateUp = 0, kDown = 1, kDownBwd = 2, kGateUpBwd = 3 };

struct RowsArgs {
  const uint16_t* A;     // [P, K] dispatch-ordered rows
  const uint16_t* B;     // expert weights, stride strideB per expert
  uint16_t* C;           // [P, ldc] output rows
  uint16_t* C2;          // second output (kGateUp: gu save, nullable)
  const uint16_t* aux;   // kDownBwd: gu [P, 2I]
  int64_t lda, ldc, strideB;
  int K;                 // reduction length
  int N;                 // output columns (kGateUp/kDownBwd: I)
  int I;
  const int32_t* offsets;
  int El, c0, nc;
  int64_t P_c;
};

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(kThreads) void rows_gemm_kernel(RowsArgs a) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static_assert(WM * WN == 4, "4 waves");
  constexpr bool kSwiGLU = (MODE == kGateUp);
  constexpr bool kBSlow = (MODE == kDownBwd || MODE == kGateUpBwd);
  // output columns per tile: the gate/up GEMM holds a gate and an up half per wave
  constexpr int OUTN = kSwiGLU ? BN / 2 : BN;
  __shared__ int s_pre[kMaxGroups + 1];
  __shared__ int64_t s_r0[kMaxGroups];
  __shared__ int s_len[kMaxGroups];
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  // stage s: A tile at lds + s*BM*BK, B tile at lds + 2*BM*BK + s*BN*BK
#define LA(s) (lds + (s) * (BM * BK))
#define LB(s) (lds + 2 * BM * BK + (s) * (BN * BK))

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int G = a.nc * a.El;
  const int ntiles = (a.N + OUTN - 1) / OUTN;
  for (int g = tid; g < G; g += kThreads) {
    const int c = a.c0 + g / a.El, e = g % a.El;
    const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
    const int len = off[e + 1] - off[e];
    s_r0[g] = (int64_t)c * a.P_c + off[e];
    s_len[g] = len;
    s_pre[g + 1] = ((len + BM - 1) / BM) * ntiles;
  }
  __syncthreads();
  if (tid == 0) {
    s_pre[0] = 0;
    for (int g = 0; g < G; ++g) s_pre[g + 1] += s_pre[g];
  }
  __syncthreads();
  const int total = s_pre[G];

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = G;  // find g with s_pre[g] <= tile < s_pre[g+1]
    while (hi - lo > 1) { int mid = (lo + hi) >> 1; if (s_pre[mid] <= tile) lo = mid; else hi = mid; }
    const int g = lo;
    const int e = g % a.El;
    const int t_in = tile - s_pre[g];
    const int mt = t_in / ntiles, nt = t_in % ntiles;
    const int64_t r0 = s_r0[g] + (int64_t)mt * BM;
    const int mvalid = min(BM, s_len[g] - mt * BM);
    const int n0 = nt * OUTN;
    const uint16_t* Be = a.B + (int64_t)e * a.strideB;

    KMajor<BM> ldA;
#pragma unroll
    for (int i = 0; i < KMajor<BM>::NV; ++i) {
      int r = KMajor<BM>::row_of(tid, i);
      ldA.p[i] = r < mvalid ? a.A + (r0 + r) * a.lda + KMajor<BM>::chunk_of(tid) * 8 : nullptr;
    }
    KMajor<BN> ldB;
    KSlow<BN> ldBs;
    if constexpr (!kBSlow) {
#pragma unroll
      for (int i = 0; i < KMajor<BN>::NV; ++i) {
        int r = KMajor<BN>::row_of(tid, i);
        int grow;
        if constexpr (kSwiGLU) {
          // tile row r -> wave column block r / WTN; first half gate rows, second half up rows
          int wb = r / WTN, q = r % WTN;
          int j = n0 + wb * (WTN / 2) + (q < WTN / 2 ? q : q - WTN / 2);
          grow = (q < WTN / 2) ? j : a.I + j;
          ldB.p[i] = j < a.N ? Be + (int64_t)grow * a.K + KMajor<BN>::chunk_of(tid) * 8 : nullptr;
        } else {
          grow = n0 + r;
          ldB.p[i] = grow < a.N ? Be + (int64_t)grow * a.K + KMajor<BN>::chunk_of(tid) * 8 : nullptr;
        }
      }
    } else {
      // B(n, k) = W_e[k * N + n]
      ldBs.ld = a.N;
      ldBs.kvalid = a.K;
      int col = n0 + ldBs.mnblk(tid) * KSlow<BN>::V;
      ldBs.mnok = col < a.N;
      ldBs.base = Be + col;
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

    const int nks = a.K / BK;
    ldA.fetch(0);
    if constexpr (kBSlow) ldBs.fetch(0, tid); else ldB.fetch(0);
    ldA.commit(LA(0), tid);
    if constexpr (kBSlow) ldBs.commit(LB(0), tid); else ldB.commit(LB(0), tid);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nks) {
        ldA.fetch((ks + 1) * BK);
        if constexpr (kBSlow) ldBs.fetch((ks + 1) * BK, tid); else ldB.fetch((ks + 1) * BK);
      }
      mma_stage<TM, TN>(LA(cur), LB(cur), wm * WTM, wn * WTN, lane, acc);
      if (ks + 1 < nks) {
        ldA.commit(LA(cur ^ 1), tid);
        if constexpr (kBSlow) ldBs.commit(LB(cur ^ 1), tid); else ldB.commit(LB(cur ^ 1), tid);
      }
      __syncthreads();
    }

    // epilogue
    if constexpr (kSwiGLU) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = wm * WTM + tm * 32 + acc_row(i, lane);
            const int j = n0 + wn * (WTN / 2) + tn * 32 + acc_col(lane);
            if (m < mvalid && j < a.N) {
              const float gv = acc[tm][tn][i], uv = acc[tm][tn + TN / 2][i];
              const float hv = gv * sigmoidf_(gv) * uv;
              const int64_t row = r0 + m;
              a.C[row * a.ldc + j] = f2bf(hv);
              if (a.C2) {
                a.C2[row * (2 * (int64_t)a.I) + j] = f2bf(gv);
                a.C2[row * (2 * (int64_t)a.I) + a.I + j] = f2bf(uv);
              }
            }
          }
    } else if constexpr (MODE == kDownBwd) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = wm * WTM + tm * 32 + acc_row(i, lane);
            const int j = n0 + wn * WTN + tn * 32 + acc_col(lane);
            if (m < mvalid && j < a.N) {
              const int64_t row = r0 + m;
              const int64_t I2 = 2 * (int64_t)a.I;
              const float gv = bf2f(a.aux[row * I2 + j]), uv = bf2f(a.aux[row * I2 + a.I + j]);
              const float dh = acc[tm][tn][i];
              const float s = sigmoidf_(gv);
              a.C[row * I2 + j] = f2bf(dh * uv * s * (1.f + gv * (1.f - s)));
              a.C[row * I2 + a.I + j] = f2bf(dh * gv * s);
            }
          }
    } else {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = wm * WTM + tm * 32 + acc_row(i, lane);
            const int n = n0 + wn * WTN + tn * 32 + acc_col(lane);
            if (m < mvalid && n < a.N) a.C[(r0 + m) * a.ldc + n] = f2bf(acc[tm][tn][i]);
          }
    }
    __syncthreads();
  }
}

#undef LA
#undef LB

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

template <int BM, int BN, int WM, int WN, bool ROUTER>
__global__ __launch_bounds__(kThreads) void kgroup_gemm_kernel(KGroupArgs a) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  constexpr int AS = ROUTER ? 2 : 1;  // A planes (hi, lo)
#define LA(s) (lds + (s) * (AS * BM * BK))
#define LB(s) (lds + 2 * AS * BM * BK + (s) * (BN * BK))

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int mtiles = (a.M + BM - 1) / BM, ntiles = (a.N + BN - 1) / BN;
  const int tile = blockIdx.x;
  const int grp = tile / (mtiles * ntiles);       // expert (or K split)
  const int t_in = tile % (mtiles * ntiles);
  const int m0 = (t_in / ntiles) * BM, n0 = (t_in % ntiles) * BN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

  const int nseg = ROUTER ? 1 : a.n_chunks;
  for (int sgi = 0; sgi < nseg; ++sgi) {
    int64_t row0;
    int len;
    if constexpr (ROUTER) {
      row0 = a.k0 + (int64_t)grp * a.ksplit;
      int64_t rem = a.k0 + a.klen - row0;
      len = (int)(rem < a.ksplit ? (rem < 0 ? 0 : rem) : a.ksplit);
    } else {
      const int32_t* off = a.offsets + (int64_t)sgi * (a.El + 1);
      row0 = (int64_t)sgi * a.P_c + off[grp];
      len = off[grp + 1] - off[grp];
    }
    if (len <= 0) continue;
    KSlow<BN> ldB;
    ldB.ld = a.ldb;
    ldB.kvalid = len;
    ldB.mnok = n0 + ldB.mnblk(tid) * KSlow<BN>::V < a.N;
    ldB.base = a.B + row0 * a.ldb + n0 + ldB.mnblk(tid) * KSlow<BN>::V;
    KSlow<BM> ldA;
    KSlowSplit<BM> ldAs;
    if constexpr (ROUTER) {
      ldAs.ld = a.lda;
      ldAs.kvalid = (m0 + (tid & 31) * KSlowSplit<BM>::V < a.M) ? len : 0;
      ldAs.base = (const float*)a.A + row0 * a.lda + m0 + (tid & 31) * KSlowSplit<BM>::V;
    } else {
      ldA.ld = a.lda;
      ldA.kvalid = len;
      ldA.mnok = m0 + ldA.mnblk(tid) * KSlow<BM>::V < a.M;
      ldA.base = (const uint16_t*)a.A + row0 * a.lda + m0 + ldA.mnblk(tid) * KSlow<BM>::V;
    }
    const int nks = (len + BK - 1) / BK;
    if constexpr (ROUTER) { ldAs.fetch(0, tid); ldAs.commit(LA(0), LA(0) + BM * BK, tid); }
    else { ldA.fetch(0, tid); ldA.commit(LA(0), tid); }
    ldB.fetch(0, tid);
    ldB.commit(LB(0), tid);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nks) {
        if constexpr (ROUTER) ldAs.fetch((ks + 1) * BK, tid); else ldA.fetch((ks + 1) * BK, tid);
        ldB.fetch((ks + 1) * BK, tid);
      }
      mma_stage<TM, TN>(LA(cur), LB(cur), wm * WTM, wn * WTN, lane, acc);
      if constexpr (ROUTER) mma_stage<TM, TN>(LA(cur) + BM * BK, LB(cur), wm * WTM, wn * WTN, lane, acc);
      if (ks + 1 < nks) {
        if constexpr (ROUTER) ldAs.commit(LA(cur ^ 1), LA(cur ^ 1) + BM * BK, tid);
        else ldA.commit(LA(cur ^ 1), tid);
        ldB.commit(LB(cur ^ 1), tid);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * WTM + tm * 32 + acc_row(i, lane);
        const int n = n0 + wn * WTN + tn * 32 + acc_col(lane);
        if (m >= a.M || n >= a.N) continue;
        if constexpr (ROUTER) {
          ((float*)a.C)[(int64_t)grp * a.strideC + (int64_t)m * a.N + n] = acc[tm][tn][i];
        } else {
          ((uint16_t*)a.C)[(int64_t)grp * a.strideC + (int64_t)m * a.N + n] = f2bf(acc[tm][tn][i]);
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
struct SimtRowsArgs {
  const float* A; const float* B; float* C; float* C2; const float* aux;
  int64_t lda, ldc, strideB;
  int K, N, I;
  const int32_t* offsets;
  int El, c0, nc;
  int64_t P_c;
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
constexpr int kPersistentGrid = 512;  // 256 CUs x 2 resident workgroups

template <int BM, int BN, int WM, int WN, int MODE>
hipError_t run_rows(const char* name, const RowsArgs& a, hipStream_t s) {
  size_t lds = (size_t)2 * (BM + BN) * BK * sizeof(uint16_t);
  auto k = rows_gemm_kernel<BM, BN, WM, WN, MODE>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  {
    MOE_TRACE(name, s);
    hipLaunchKernelGGL(k, dim3(kPersistentGrid), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_expert_fwd(bool bf16, const void* xd, const void* w1, const void* w2,
                             const int32_t* offsets, void* gu, void* h, void* yd, int H, int I,
                             int El, int c0, int nc, int64_t P_c, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  if (bf16) {
    RowsArgs a{};
    a.A = (const uint16_t*)xd; a.B = (const uint16_t*)w1; a.C = (uint16_t*)h; a.C2 = (uint16_t*)gu;
    a.lda = H; a.ldc = I; a.strideB = (int64_t)2 * I * H; a.K = H; a.N = I; a.I = I;
    a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
    hipError_t e = run_rows<128, 128, 2, 2, kGateUp>("gemm_gateup_swiglu", a, s);
    if (e != hipSuccess) return e;
    RowsArgs b{};
    b.A = (const uint16_t*)h; b.B = (const uint16_t*)w2; b.C = (uint16_t*)yd;
    b.lda = I; b.ldc = H; b.strideB = (int64_t)H * I; b.K = I; b.N = H; b.I = I;
    b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
    return run_rows<128, 128, 2, 2, kDown>("gemm_down", b, s);
  }
  SimtRowsArgs a{};
  a.A = (const float*)xd; a.B = (const float*)w1; a.C = (float*)h; a.C2 = (float*)gu;
  a.lda = H; a.ldc = I; a.strideB = (int64_t)2 * I * H; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
  {
    MOE_TRACE("gemm_gateup_swiglu_f32", s);
    hipLaunchKernelGGL(simt_rows_kernel<kGateUp>, dim3(kPersistentGrid), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtRowsArgs b{};
  b.A = (const float*)h; b.B = (const float*)w2; b.C = (float*)yd;
  b.lda = I; b.ldc = H; b.strideB = (int64_t)H * I; b.K = I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
  {
    MOE_TRACE("gemm_down_f32", s);
    hipLaunchKernelGGL(simt_rows_kernel<kDown>, dim3(kPersistentGrid), dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

hipError_t launch_expert_dgrad(bool bf16, const void* dyd, const void* gu, const void* w1,
                               const void* w2, const int32_t* offsets, void* dgu, void* dxd, int H,
                               int I, int El, int c0, int nc, int64_t P_c, hipStream_t s) {
  if (nc <= 0 || El <= 0) return hipSuccess;
  if (bf16) {
    RowsArgs a{};
    a.A = (const uint16_t*)dyd; a.B = (const uint16_t*)w2; a.C = (uint16_t*)dgu; a.aux = (const uint16_t*)gu;
    a.lda = H; a.ldc = 2 * I; a.strideB = (int64_t)H * I; a.K = H; a.N = I; a.I = I;
    a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
    hipError_t e = run_rows<128, 128, 2, 2, kDownBwd>("gemm_down_dgrad_swiglu", a, s);
    if (e != hipSuccess) return e;
    RowsArgs b{};
    b.A = (const uint16_t*)dgu; b.B = (const uint16_t*)w1; b.C = (uint16_t*)dxd;
    b.lda = 2 * I; b.ldc = H; b.strideB = (int64_t)2 * I * H; b.K = 2 * I; b.N = H; b.I = I;
    b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
    return run_rows<128, 128, 2, 2, kGateUpBwd>("gemm_gateup_dgrad", b, s);
  }
  SimtRowsArgs a{};
  a.A = (const float*)dyd; a.B = (const float*)w2; a.C = (float*)dgu; a.aux = (const float*)gu;
  a.lda = H; a.ldc = 2 * I; a.strideB = (int64_t)H * I; a.K = H; a.N = I; a.I = I;
  a.offsets = offsets; a.El = El; a.c0 = c0; a.nc = nc; a.P_c = P_c;
  {
    MOE_TRACE("gemm_down_dgrad_swiglu_f32", s);
    hipLaunchKernelGGL(simt_rows_kernel<kDownBwd>, dim3(kPersistentGrid), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtRowsArgs b{};
  b.A = (const float*)dgu; b.B = (const float*)w1; b.C = (float*)dxd;
  b.lda = 2 * I; b.ldc = H; b.strideB = (int64_t)2 * I * H; b.K = 2 * I; b.N = H; b.I = I;
  b.offsets = offsets; b.El = El; b.c0 = c0; b.nc = nc; b.P_c = P_c;
  {
    MOE_TRACE("gemm_gateup_dgrad_f32", s);
    hipLaunchKernelGGL(simt_rows_kernel<kGateUpBwd>, dim3(kPersistentGrid), dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

hipError_t launch_expert_wgrad(bool bf16, const void* dyd, const void* dgu, const void* xd,
                               const void* h, const int32_t* offsets, void* dw1, void* dw2, int H,
                               int I, int El, int n, int64_t P_c, hipStream_t s) {
  if (El <= 0) return hipSuccess;
  if (bf16) {
    constexpr int BM = 128, BN = 128;
    size_t lds = (size_t)2 * (BM + BN) * BK * sizeof(uint16_t);
    auto k = kgroup_gemm_kernel<BM, BN, 2, 2, false>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // dW2[e] [H, I] = sum dyd^T h
    KGroupArgs a{};
    a.A = dyd; a.B = (const uint16_t*)h; a.C = dw2; a.lda = H; a.ldb = I; a.strideC = (int64_t)H * I;
    a.M = H; a.N = I; a.offsets = offsets; a.El = El; a.n_chunks = n; a.P_c = P_c;
    {
      MOE_TRACE("gemm_wgrad_down", s);
      hipLaunchKernelGGL(k, dim3(El * ((H + BM - 1) / BM) * ((I + BN - 1) / BN)), dim3(kThreads), lds, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dW1[e] [2I, H] = sum dgu^T xd
    KGroupArgs b{};
    b.A = dgu; b.B = (const uint16_t*)xd; b.C = dw1; b.lda = 2 * I; b.ldb = H; b.strideC = (int64_t)2 * I * H;
    b.M = 2 * I; b.N = H; b.offsets = offsets; b.El = El; b.n_chunks = n; b.P_c = P_c;
    {
      MOE_TRACE("gemm_wgrad_gateup", s);
      hipLaunchKernelGGL(k, dim3(El * ((2 * I + BM - 1) / BM) * ((H + BN - 1) / BN)), dim3(kThreads), lds, s, b);
    }
    return hipGetLastError();
  }
  SimtKArgs a{};
  a.A = (const float*)dyd; a.B = (const float*)h; a.C = (float*)dw2; a.lda = H; a.ldb = I;
  a.strideC = (int64_t)H * I; a.M = H; a.N = I; a.offsets = offsets; a.El = El; a.n_chunks = n; a.P_c = P_c;
  {
    MOE_TRACE("gemm_wgrad_down_f32", s);
    hipLaunchKernelGGL(simt_kgroup_kernel, dim3(El * ((H + 63) / 64) * ((I + 63) / 64)), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SimtKArgs b{};
  b.A = (const float*)dgu; b.B = (const float*)xd; b.C = (float*)dw1; b.lda = 2 * I; b.ldb = H;
  b.strideC = (int64_t)2 * I * H; b.M = 2 * I; b.N = H; b.offsets = offsets; b.El = El; b.n_chunks = n; b.P_c = P_c;
  {
    MOE_TRACE("gemm_wgrad_gateup_f32", s);
    hipLaunchKernelGGL(simt_kgroup_kernel, dim3(El * ((2 * I + 63) / 64) * ((H + 63) / 64)), dim3(256), 0, s, b);
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
      auto k = kgroup_gemm_kernel<BM, BN, 2, 2, true>;
      hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      KGroupArgs a{};
      a.A = dlogits; a.B = (const uint16_t*)x; a.C = partials; a.lda = E; a.ldb = H;
      a.strideC = (int64_t)E * H; a.M = E; a.N = H; a.k0 = t0; a.klen = len; a.ksplit = ks;
      {
        MOE_TRACE("gemm_router_wgrad", s);
        hipLaunchKernelGGL(k, dim3(S * ((E + BM - 1) / BM) * ((H + BN - 1) / BN)), dim3(kThreads), lds, s, a);
      }
    } else {
      SimtKArgs a{};
      a.A = dlogits; a.B = (const float*)x; a.C = partials; a.lda = E; a.ldb = H;
      a.strideC = (int64_t)E * H; a.M = E; a.N = H; a.k0 = t0; a.klen = len; a.ksplit = ks; a.router = true;
      {
        MOE_TRACE("gemm_router_wgrad_f32", s);
        hipLaunchKernelGGL(simt_kgroup_kernel, dim3(S * ((E + 63) / 64) * ((H + 63) / 64)), dim3(256), 0, s, a);
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
      hipLaunchKernelGGL(reduce_partials_kernel<uint16_t>, g, dim3(256), 0, s, partials, S, MN, dwr_acc,
                         first, (uint16_t*)dwr);
    }
  else
    {
      MOE_TRACE("router_reduce", s);
      hipLaunchKernelGGL(reduce_partials_kernel<float>, g, dim3(256), 0, s, partials, S, MN, dwr_acc,
                         first, (float*)dwr);
    }
  return hipGetLastError();
}

}  // namespace moe
