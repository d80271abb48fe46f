// Shared engine of the grouped expert GEMMs on CDNA4 matrix cores (BF16 and FP8 e4m3 MFMA with
// FP32 accumulation): LDS operand ring, fragments, K loop, output staging, the row-grouped
// GEMM's tile walk, and the host-side launch helpers.
//
// Engine (one 512-thread workgroup = 8 waves in a 2 x 4 grid over a BM x BN output tile, two
// waves per SIMD, so the second wave on a SIMD issues MFMAs while the first waits; four waves
// with 128 x 128 wave tiles read a third fewer LDS bytes but measured slower on every GEMM here):
//   * Operands reach LDS by direct-to-LDS 16-byte buffer loads (buffer_load_dwordx4 ... lds):
//     no staging registers, no VALU on the load path. The scalar buffer descriptor's extent
//     masks rows past an expert's segment or a matrix edge (such loads return zero).
//   * A ring of kNst LDS stages, each holding 64 bytes of K per MN row (32 BF16 or 64 FP8
//     values); loads run kNst - 1 stages ahead. One s_barrier per stage, with an explicit
//     vmcnt wait that leaves the younger stages' loads in flight (a workgroup fence would drain
//     them). When both operands are K-major BF16 (gate/up and down), the same LDS holds two
//     slots of two stages each instead (128-byte rows), so that every load request covers a
//     whole 128-byte line; one barrier per pair of stages; the same for the FP8 GEMMs other
//     than the forward gate/up one, which keeps the stage ring. The BF16 input gradients keep
//     their K-slow weight operand in the stage ring and take the K-major A operand in pair slots.
//   * Operands with K contiguous in HBM ("K-major") live in LDS as 64-byte rows whose four
//     16-byte chunks are XOR-swizzled by (row >> 2) & 3: a ds_read_b128 of 16 consecutive rows
//     at one chunk touches all 64 banks once.
//   * Operands with K along HBM rows ("K-slow": the weights in the input-gradient GEMMs and
//     both operands of the weight gradients) live in LDS as K-rows of MN values with chunks
//     XOR-swizzled by 4 * (k & 3), and reach the MFMA through ds_read_b64_tr_b16, which
//     transposes 4 x 4 blocks of 16-bit values across each 16-lane group.
//   * The number of 32-row MFMA blocks a wave holds rows for is a template parameter of the K
//     loop (chosen once per tile), so the partial last tile of an expert issues no MFMA for empty
//     row blocks and the loop itself has no branches around MFMAs.
//   * MFMAs are issued with the B fragment as the first operand: lane l then holds output row
//     l & 31 and four consecutive columns per accumulator group, stored as one 8-byte BF16 write.
#pragma once
#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace gg {

constexpr int kWM = 2, kWN = 4;       // waves per workgroup along M and N
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = 64 * kWaves;
constexpr int kNst = 4;             // LDS ring stages
constexpr int kRowB = 64;           // K bytes per MN row per stage
constexpr int kKRows = 32;          // K rows per stage for 16-bit K-slow operands
constexpr int kMaxGroups = 1024;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// LDS byte offset of 16-byte chunk c of row r in a K-major stage.
MOE_DEV int km_off(int r, int c) { return r * kRowB + ((c ^ ((r >> 2) & 3)) << 4); }
// LDS byte offset of 16-byte chunk c of K-row k in a K-slow stage of R MN values (R >= 128).
template <int R>
MOE_DEV int ks_off(int k, int c) { return k * (2 * R) + ((c ^ ((k & 3) << 2)) << 4); }

// ---------------------------------------------------------------------------------------------
// Operand tile loader: R MN rows, one stage = R * 64 bytes = R / 16 wave instructions of 1 KiB,
// spread over the workgroup's waves.
template <int R, bool KSLOW, int LW = kWaves, bool PAIR = false>
struct Loader {
  static constexpr int kLW = LW;  // waves that issue the loads (the first LW of the workgroup)
  // PAIR (K-major): one load covers two stages of 8 rows, 128 bytes (a whole line) per row
  static constexpr int kRows = PAIR ? 8 : 16;  // rows per wave instruction
  static_assert(!(PAIR && KSLOW), "pairs of stages: K-major operands");
  static constexpr int NI = R / (kRows * LW);
  static_assert(LW == kWaves || LW == kWaves / 2, "all waves, or one per SIMD");
  static_assert(NI >= 1 && R % (kRows * LW) == 0, "tile rows must cover every loading wave");
  __amdgpu_buffer_rsrc_t rb;  // buffer descriptor
  i32x4_t rs;                 // the same as words, for the loads written in assembly
  uint32_t voff[NI];
  uint32_t step;  // HBM bytes between consecutive stages
  int wave;

  // K-major: tile row r starts at base + map(r) * ld_bytes; bytes: readable extent from base
  template <class Map>
  MOE_DEV void init_kmajor(const void* base, int64_t ld_bytes, int64_t bytes, int wv, int lane, Map map) {
    wave = wv;
    rb = make_rsrc(base, bytes);
    rs = rsrc_words(base, bytes);
    step = PAIR ? 2 * kRowB : kRowB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (PAIR) {
        const int r = 8 * (wave * NI + i) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        voff[i] = (uint32_t)((int64_t)map(r) * ld_bytes) + 16u * (uint32_t)c;
      } else {
        const int r = 16 * (wave * NI + i) + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        voff[i] = (uint32_t)((int64_t)map(r) * ld_bytes) + 16u * (uint32_t)c;
      }
    }
  }
  // K-slow: K-row k of the tile starts at base + k * ld_bytes; its R MN values are contiguous
  MOE_DEV void init_kslow(const void* base, int64_t ld_bytes, int64_t bytes, int wv, int lane) {
    static_assert(R >= 128, "K-slow tiles need >= 16 chunks per K-row");
    constexpr int CPR = 2 * R / 16;      // chunks per K-row
    constexpr int RPI = 1024 / (2 * R);  // K-rows per wave instruction
    wave = wv;
    rb = make_rsrc(base, bytes);
    rs = rsrc_words(base, bytes);
    step = (uint32_t)(kKRows * ld_bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = RPI * (wave * NI + i) + lane / CPR;
      const int c = (lane % CPR) ^ ((k & 3) << 2);
      voff[i] = (uint32_t)(k * ld_bytes) + 16u * (uint32_t)c;
    }
  }
  // Issue the loads of stage s into LDS at byte address `stage` (the operand's part of a ring
  // slot). ASM: the same loads written in assembly. Before every transposing LDS read
  // (ds_read_b64_tr_b16) the compiler waits for all outstanding direct-to-LDS loads issued
  // through its builtin (vmcnt(0)), which drains the ring's prefetch in every stage; GEMMs with a
  // K-slow operand therefore issue all of their loads in assembly, ordered with the reads of
  // their stage by the K loop's explicit vmcnt waits. M0 (the LDS destination) is saved and
  // restored; s_nop 4 covers a VALU write of an SGPR operand.
  template <bool ASM>
  MOE_DEV void issue(uint32_t stage, int s) const {
    static_assert(NI == 1 || NI % 2 == 0, "one load, or pairs of loads, per wave and operand stage");
    const uint32_t l0 = stage + (uint32_t)(wave * NI * 1024);
    if constexpr (!ASM) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(uintptr_t)(l0 + i * 1024), 16, (int)voff[i],
                                                 (int)((uint32_t)s * step), 0, 0);
    } else {
      const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)s * step);
      const uint32_t lf = __builtin_amdgcn_readfirstlane(l0);
      uint32_t m0s;
      if constexpr (NI == 1) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
            : "=&s"(m0s)
            : "s"(lf), "v"(voff[0]), "s"(rs), "s"(so)
            : "memory");
      } else {
#pragma unroll
        for (int i = 0; i < NI; i += 2) {
          const uint32_t la = lf + i * 1024, lb = la + 1024;
          asm volatile(
              "s_mov_b32 %0, m0\n\ts_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
              "buffer_load_dwordx4 %3, %5, %6 offen lds\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
              "buffer_load_dwordx4 %4, %5, %6 offen lds\n\ts_mov_b32 m0, %0"
              : "=&s"(m0s)
              : "s"(la), "s"(lb), "v"(voff[i]), "v"(voff[i + 1]), "s"(rs), "s"(so)
              : "memory");
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Fragments for one MFMA: rows mb + (lane & 31) of the operand.

// K-major BF16: 8 K values, k16 step kk of the stage, K half lane >> 5.
MOE_DEV bf16x8_t frag_km(const char* st, int mb, int kk, int lane) {
  return *(const bf16x8_t*)(st + km_off(mb + (lane & 31), 2 * kk + (lane >> 5)));
}

// K-major BF16 in a pair slot (two stages per 128-byte row, eight 16-byte chunks XOR-swizzled by
// (row >> 1) & 7: a ds_read_b128 of 16 consecutive rows at one chunk touches all 64 banks once):
// 8 K values, k16 step kk of stage half H.
MOE_DEV int km2_off(int r, int c) { return r * (2 * kRowB) + ((c ^ ((r >> 1) & 7)) << 4); }
template <int H>
MOE_DEV bf16x8_t frag_km2(const char* st, int mb, int kk, int lane) {
  return *(const bf16x8_t*)(st + km2_off(mb + (lane & 31), 4 * H + 2 * kk + (lane >> 5)));
}

MOE_DEV s16x4 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// K-slow BF16: the same 8 K values assembled by two transposing reads. In each 16-lane group
// lane q reads the 4 MN-consecutive values (k0 + (q >> 2), m + 4 (q & 3) .. +3); after the
// transpose lane q holds (k0 .. k0+3, m + q).
template <int R>
MOE_DEV bf16x8_t frag_ks(const char* st, int mb, int kk, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int cb = 2 * (mb + 16 * (g & 1) + 4 * (q & 3));  // byte of the first value in its K-row
  const int k0 = 16 * kk + 8 * (g >> 1) + (q >> 2);
  const s16x4 lo = ds_read_tr(st + ks_off<R>(k0, cb >> 4) + (cb & 15));
  const s16x4 hi = ds_read_tr(st + ks_off<R>(k0 + 4, cb >> 4) + (cb & 15));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// K-major FP8: 32 K values (bytes 32 * (lane >> 5) .. +32 of the stage row).
MOE_DEV i32x8_t frag_km8(const char* st, int mb, int lane) {
  const int r = mb + (lane & 31), hk = lane >> 5;
  const i32x4_t a = *(const i32x4_t*)(st + km_off(r, 2 * hk));
  const i32x4_t b = *(const i32x4_t*)(st + km_off(r, 2 * hk + 1));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// K-major FP8 in a pair slot: 32 K values (bytes 32 * (lane >> 5) .. +32 of stage half H).
template <int H>
MOE_DEV i32x8_t frag_km8_2(const char* st, int mb, int lane) {
  const int r = mb + (lane & 31), c = 4 * H + 2 * (lane >> 5);
  const i32x4_t a = *(const i32x4_t*)(st + km2_off(r, c));
  const i32x4_t b = *(const i32x4_t*)(st + km2_off(r, c + 1));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One LDS stage of MFMAs: acc[tm][tn] += A[rows of block tm] . B[rows of block tn]^T for
// tm < TMA (row blocks past the tile's valid rows are skipped at compile time). `loads` issues the
// global -> LDS loads of a later stage; the schedule spreads them and the fragment reads between
// the MFMAs (the default scheduler would recycle one fragment register per read and serialise).
template <bool FP8, bool AKS, bool BKS, int RA, int RB, int TM, int TN, int TMA, int VM, int HALF = -1,
          class Loads>
MOE_DEV void stage_mma(const char* sa, const char* sb, int arow0, int brow0, int lane,
                       f32x16_t (&acc)[TM][TN], Loads&& loads) {
  static_assert(HALF < 0 || (!AKS && !(FP8 && BKS)), "pair slots: K-major operands");
  if constexpr (TMA == 0) {
    loads();
  } else if constexpr (FP8) {
    i32x8_t fa[TMA], fb[TN];
#pragma unroll
    for (int tm = 0; tm < TMA; ++tm)
      fa[tm] = HALF < 0 ? frag_km8(sa, arow0 + 32 * tm, lane) : frag_km8_2<(HALF > 0)>(sa, arow0 + 32 * tm, lane);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      fb[tn] = HALF < 0 ? frag_km8(sb, brow0 + 32 * tn, lane) : frag_km8_2<(HALF > 0)>(sb, brow0 + 32 * tn, lane);
    loads();
#pragma unroll
    for (int tm = 0; tm < TMA; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[tn], fa[tm], acc[tm][tn], 0, 0,
                                                                       0, 0, 0, 0);
    constexpr int RD = 2 * (TMA + TN), MF = TMA * TN;
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int i = 0; i < VM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
  } else {
    // all fragments of k16 step 0; step 1's reads, then the loads, spread one per MFMA of step 0
    // onwards; then the remaining MFMAs
    bf16x8_t fa[2][TMA], fb[2][TN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if constexpr (HALF >= 0) {
        // A in a pair slot; B in a pair slot too, or K-slow in its own stage slot
#pragma unroll
        for (int tm = 0; tm < TMA; ++tm) fa[kk][tm] = frag_km2<HALF>(sa, arow0 + 32 * tm, kk, lane);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          fb[kk][tn] = BKS ? frag_ks<RB>(sb, brow0 + 32 * tn, kk, lane) : frag_km2<HALF>(sb, brow0 + 32 * tn, kk, lane);
      } else {
#pragma unroll
        for (int tm = 0; tm < TMA; ++tm)
          fa[kk][tm] = AKS ? frag_ks<RA>(sa, arow0 + 32 * tm, kk, lane) : frag_km(sa, arow0 + 32 * tm, kk, lane);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          fb[kk][tn] = BKS ? frag_ks<RB>(sb, brow0 + 32 * tn, kk, lane) : frag_km(sb, brow0 + 32 * tn, kk, lane);
      }
    }
    loads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int tm = 0; tm < TMA; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][tn], fa[kk][tm], acc[tm][tn], 0, 0, 0);
    constexpr int RD = ((AKS ? 2 : 1) * TMA + (BKS ? 2 : 1) * TN);  // LDS reads per k16 step
    constexpr int MF = TMA * TN;                                     // MFMAs per k16 step
    // With a K-slow weight operand (input gradients, weight gradients) the loads go out first,
    // right after the stage barrier (measured faster there); otherwise they follow the first
    // MFMAs.
    if constexpr (BKS && VM > 0) __builtin_amdgcn_sched_group_barrier(0x020, VM, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (!BKS) {
#pragma unroll
      for (int i = 0; i < VM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * MF, 0);
  }
}

// K loop over nks stages through the LDS ring. Every iteration issues the loads of stage
// s + kNst - 1; past the last stage they fetch masked (zero) or unused data into a ring slot that
// is never read again, so every iteration waits with the same count. On return all loads have
// completed and every wave has passed a barrier after its last LDS read, so the ring is free.
template <bool FP8, bool AKS, bool BKS, int RA, int RB, int TM, int TN, int TMA, class LA, class LB>
MOE_DEV void kloop(const LA& la, const LB& lb, char* ring, int nks, int arow0, int brow0, int lane,
                   f32x16_t (&acc)[TM][TN]) {
  constexpr int SA = RA * kRowB, SS = (RA + RB) * kRowB;
  constexpr int NL = LA::NI + LB::NI;  // load instructions per wave per stage
  constexpr bool kAsm = AKS || BKS;    // transposing reads follow: loads written in assembly
  const uint32_t rl = lds_addr(ring);
  static_assert(LA::kLW == LB::kLW, "one set of loading waves");
  constexpr bool kAll = LA::kLW == kWaves;
  const bool loader = kAll || la.wave < LA::kLW;
  if (loader) {
#pragma unroll
    for (int s = 0; s < kNst - 1; ++s) {
      la.template issue<kAsm>(rl + s * SS, s);
      lb.template issue<kAsm>(rl + s * SS + SA, s);
    }
  }
  for (int s = 0; s < nks; ++s) {
    wait_vm<(kNst - 2) * NL>();    // stage s has landed (this wave's loads)
    __builtin_amdgcn_s_barrier();  // every wave's part of stage s is in LDS; stage s-1 is consumed
    const int ld = s + kNst - 1;
    const uint32_t st = rl + (ld % kNst) * SS;
    const char* cur = ring + (s % kNst) * SS;
    if constexpr (kAll) {
      stage_mma<FP8, AKS, BKS, RA, RB, TM, TN, TMA, NL>(cur, cur + SA, arow0, brow0, lane, acc, [&] {
        la.template issue<kAsm>(st, ld);
        lb.template issue<kAsm>(st + SA, ld);
      });
    } else {
      // the loading waves issue the stage's loads first; the other wave on each SIMD goes
      // straight to its fragment reads and MFMAs
      if (loader) {
        la.template issue<kAsm>(st, ld);
        lb.template issue<kAsm>(st + SA, ld);
      }
      stage_mma<FP8, AKS, BKS, RA, RB, TM, TN, TMA, 0>(cur, cur + SA, arow0, brow0, lane, acc, [] {});
    }
  }
  wait_vm<0>();
  __syncthreads();
}

// K loop for two K-major operands (BF16 or FP8) over pair slots: the LDS ring holds two slots of
// two stages each (rows of 128 bytes), and each load brings a whole 128-byte line per row, half the
// load requests per byte of 64-byte stage rows (the loads' issue limits the 64-byte K loop when
// every CU runs one). Pair p+1's loads go out during the first half of pair p, into the other
// slot, which every wave finished reading before pair p's barrier; pair p+1 then waits for all of
// them. Past the last pair they fetch masked or unused data into the slot no one reads again.
template <bool FP8, int RA, int RB, int TM, int TN, int TMA, class LA, class LB>
MOE_DEV void kloop_pairs(const LA& la, const LB& lb, char* ring, int nks, int arow0, int brow0, int lane,
                         f32x16_t (&acc)[TM][TN]) {
  constexpr int SA = RA * 2 * kRowB, SS = (RA + RB) * 2 * kRowB;
  constexpr int NL = LA::NI + LB::NI;  // load instructions per wave per pair
  const uint32_t rl = lds_addr(ring);
  const int np = (nks + 1) / 2;
  la.template issue<false>(rl, 0);
  lb.template issue<false>(rl + SA, 0);
  for (int p = 0; p < np; ++p) {
    wait_vm<0>();                  // pair p has landed (this wave's loads)
    __builtin_amdgcn_s_barrier();  // every wave's part of pair p is in LDS; pair p-1 is consumed
    const int ld = p + 1;
    const uint32_t st = rl + (ld & 1) * SS;
    const char* cur = ring + (p & 1) * SS;
    stage_mma<FP8, false, false, RA, RB, TM, TN, TMA, NL, 0>(cur, cur + SA, arow0, brow0, lane, acc, [&] {
      la.template issue<false>(st, ld);
      lb.template issue<false>(st + SA, ld);
    });
    if (2 * p + 1 < nks) stage_mma<FP8, false, false, RA, RB, TM, TN, TMA, 0, 1>(cur, cur + SA, arow0, brow0, lane, acc, [] {});
  }
  wait_vm<0>();
  __syncthreads();
}

// K loop for a K-major BF16 A operand in pair slots (two slots of two stages, 128-byte rows) and
// a K-slow B operand in a ring of kNst stage slots (the input gradients): one barrier per stage.
// Stage 2p issues A's pair p+1 and B's stage 2p+3, stage 2p+1 issues B's stage 2p+4; each slot
// they fill was last read before that stage's barrier. Load counts complete in issue order: at an
// even stage the loads younger than its own are B's next two stages, at an odd stage also A's
// next pair, so the two stages wait with different counts.
template <int RA, int RB, int TM, int TN, int TMA, class LA, class LB>
MOE_DEV void kloop_apairs(const LA& la, const LB& lb, char* ring, int nks, int arow0, int brow0, int lane,
                          f32x16_t (&acc)[TM][TN]) {
  constexpr int SA = RA * 2 * kRowB;  // A pair slot
  constexpr int SB = RB * kRowB;      // B stage slot
  constexpr int NA = LA::NI, NB = LB::NI;
  const uint32_t rl = lds_addr(ring), rb = rl + 2 * SA;
  const char* ringb = ring + 2 * SA;
  const int np = (nks + 1) / 2;
  la.template issue<true>(rl, 0);
#pragma unroll
  for (int s = 0; s < kNst - 1; ++s) lb.template issue<true>(rb + s * SB, s);
  for (int p = 0; p < np; ++p) {
    const int s0 = 2 * p;
    const char* ca = ring + (p & 1) * SA;
    {
      wait_vm<(kNst - 2) * NB>();    // A's pair p and B's stage s0 have landed (this wave's loads)
      __builtin_amdgcn_s_barrier();  // every wave's part is in LDS; stage s0 - 1 is consumed
      const int lb0 = s0 + kNst - 1;
      stage_mma<false, false, true, RA, RB, TM, TN, TMA, NA + NB, 0>(
          ca, ringb + (s0 % kNst) * SB, arow0, brow0, lane, acc, [&] {
            la.template issue<true>(rl + ((p + 1) & 1) * SA, p + 1);
            lb.template issue<true>(rb + (lb0 % kNst) * SB, lb0);
          });
    }
    if (s0 + 1 < nks) {
      wait_vm<(kNst - 2) * NB + NA>();  // B's stage s0 + 1 has landed
      __builtin_amdgcn_s_barrier();
      const int lb1 = s0 + kNst;
      stage_mma<false, false, true, RA, RB, TM, TN, TMA, NB, 1>(
          ca, ringb + ((s0 + 1) % kNst) * SB, arow0, brow0, lane, acc, [&] {
            lb.template issue<true>(rb + (lb1 % kNst) * SB, lb1);
          });
    }
  }
  wait_vm<0>();
  __syncthreads();
}

MOE_DEV uint2 pack4(float a, float b, float c, float d) { return make_uint2(pack_bf2(a, b), pack_bf2(c, d)); }
MOE_DEV void unpack4(uint2 v, float* f) {
  f[0] = bf2f(v.x & 0xffff); f[1] = bf2f(v.x >> 16); f[2] = bf2f(v.y & 0xffff); f[3] = bf2f(v.y >> 16);
}
MOE_DEV int out_row(int lane) { return lane & 31; }
MOE_DEV int out_col(int g, int lane) { return 8 * g + 4 * (lane >> 5); }

// Workgroup barrier for the LDS staging area only: every wave's LDS accesses are complete, but its
// global stores may still be in flight (a __syncthreads fence would wait for them as well).
MOE_DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xf | (7 << 4) | (3 << 14));  // lgkmcnt(0), other counters untouched
  __builtin_amdgcn_s_barrier();
}

// Output staging: a [BM, W] BF16 tile in LDS with a row pitch of W * 2 + 16 bytes (16-byte aligned
// rows; the pad spreads the MFMA-layout writes of 32 rows over the banks).
template <int W> constexpr int pitch() { return W * 2 + 16; }
template <int BM, int W> constexpr size_t stage_bytes() { return (size_t)BM * pitch<W>(); }

// Store rows < mvalid and columns < nvalid (a multiple of 8) of a staged tile to dst (row stride
// ld elements) with 16-byte writes: each wave instruction writes whole rows. NT: non-temporal
// stores, for outputs no kernel reads soon (saved G/U, weight gradients); measured faster there,
// and slower for outputs the next kernel reads (h, yd, dG/dU, dxd), which stay normal.
template <int BM, int W, bool NT = false>
MOE_DEV void store_staged(const char* lds, uint16_t* dst, int64_t ld, int mvalid, int nvalid, int tid) {
  constexpr int CPR = W / 8, RPP = kThreads / CPR;
  const int c = tid % CPR;
#pragma unroll 4
  for (int r = tid / CPR; r < BM; r += RPP)
    if (r < mvalid && 8 * c < nvalid) {
      const i32x4_t v = *(const i32x4_t*)(lds + r * pitch<W>() + 16 * c);
      i32x4_t* p = (i32x4_t*)(dst + (int64_t)r * ld + 8 * c);
      if constexpr (NT) __builtin_nontemporal_store(v, p);
      else *p = v;
    }
}

// Load rows < mvalid, columns < nvalid of a [BM, W] BF16 tile from src into LDS staging.
template <int BM, int W>
MOE_DEV void load_staged(char* lds, const uint16_t* src, int64_t ld, int mvalid, int nvalid, int tid) {
  constexpr int CPR = W / 8, RPP = kThreads / CPR;
  const int c = tid % CPR;
#pragma unroll 4
  for (int r = tid / CPR; r < BM; r += RPP)
    if (r < mvalid && 8 * c < nvalid)
      *(uint4*)(lds + r * pitch<W>() + 16 * c) = *(const uint4*)(src + (int64_t)r * ld + 8 * c);
}

// Store rows < mvalid of a staged [BM, 256] BF16 tile as one column block of block-scaled FP8 rows:
// per row, amax over its nvalid columns, codes RNE(v * (448 / amax)) (FP32 steps, saturated), the
// scale amax / 448 (an all-zero block: codes 0, scale 1). A half-wave per row, 8 values per lane;
// every lane of a wave runs the same trip count, so the 32-lane max reduction is never divergent.
template <int BM, int W>
MOE_DEV void store_staged_q(const char* lds, uint8_t* dst, int64_t ld, float* sc, int64_t ldcs, int mvalid,
                            int nvalid, int tid) {
  static_assert(W == 256, "one 256-column block per staged tile");
  static_assert(BM % (2 * kWaves) == 0, "whole rows per half-wave");
  const int lane = tid & 63, l32 = lane & 31;
  for (int r = 2 * (tid >> 6) + (lane >> 5); r < BM; r += 2 * kWaves) {
    const bool live = r < mvalid && 8 * l32 < nvalid;
    u32x4 v{0u, 0u, 0u, 0u};
    if (live) v = *(const u32x4*)(lds + r * pitch<W>() + 16 * l32);
    float m = absmax8(v);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (live) *(uint2*)(dst + (int64_t)r * ld + 8 * l32) = m > 0.f ? quant8(v, 448.0f / m) : make_uint2(0u, 0u);
    if (l32 == 0 && r < mvalid) sc[(int64_t)r * ldcs] = m > 0.f ? m / 448.0f : 1.0f;
  }
}

// ---------------------------------------------------------------------------------------------
// Row-grouped GEMMs (forward and input gradients):
//   C[r0 + m][n] = sum_k A[r0 + m][k] * B_e(n, k) over the rows of local expert e in a chunk.
// Persistent: the grid holds at most one workgroup per CU; each loops over its XCD's tiles.
enum Mode { kGateUp = 0, kDown = 1, kDownBwd = 2, kGateUpBwd = 3 };

struct RowsArgs {
  const void* A;          // [P, K] dispatch-ordered rows (BF16, or e4m3 codes)
  const void* B;          // expert weights, strideB elements per expert
  uint16_t* C;            // [P, ldc] BF16 output rows
  uint16_t* C2;           // kGateUp: G/U save [P, 2I] (nullable)
  const uint16_t* aux;    // kDownBwd: G/U [P, 2I]
  const float* scale_a;   // FP8: per dispatch row
  const float* scale_b;   // FP8: per weight row, strideSB per expert
  int64_t lda, ldc, strideB, strideSB;
  int K, N, I;
  const int32_t* offsets;
  int El, c0, nc;
  int64_t P_c;
  // QOUT launches (block-scaled FP8 output instead of C): e4m3 codes [P, ldc] and one FP32 scale
  // per row and 256-column block, [P, ldcs]
  uint8_t* Cq;
  float* Cs;
  int64_t ldcs;
  // GATHER launches (gate/up): A holds the token rows [gather_rows, K] and dispatch row r reads
  // token row gather[r] (src_token), so the GEMM needs no dispatched copy of its operand
  const int32_t* gather;
  int64_t gather_rows;
  // per-XCD next-slot counters then the exit counter (zero between launches), or null: static
  // round-robin slots
  int* queue;
};

template <int BM, int BN, int MODE>
constexpr size_t rows_lds_bytes() {
  const size_t ring = (size_t)kNst * (BM + BN) * kRowB;
  // gate/up and down-bwd stage two [BM, W] tiles at once (G and U)
  const size_t ep = (MODE == kGateUp) ? 2 * stage_bytes<BM, BN / 2>()
                  : (MODE == kDownBwd) ? 2 * stage_bytes<BM, BN>() : stage_bytes<BM, BN>();
  return ring > ep ? ring : ep;
}

// LDS of a weight-gradient launch (BF16 or FP8): the operand ring or the BF16 output staging tile.
template <int BM, int BN>
constexpr size_t wgrad_lds_bytes() {
  const size_t ring = (size_t)kNst * (BM + BN) * kRowB, ep = stage_bytes<BM, BN>();
  return ring > ep ? ring : ep;
}

// Group -> tile prefix of one row-grouped GEMM, rebuilt in LDS by every workgroup.
struct RowsShared {
  int pre[kMaxGroups + 1];   // large tiles before group g
  int64_t r0[kMaxGroups];    // first dispatch row of group g
  int len[kMaxGroups];       // rows of group g
  int preb[kMaxGroups + 1];  // small tiles before group g
  int q;                     // the slot this workgroup takes next (queued lists)
};

// Persistent work slots. Per XCD the workgroups (block b runs on XCD b % 8; W of them per XCD)
// share one sequence of slots: slot s goes to the XCD's workgroup s % W, so that a list that
// starts at slot `first` continues the round robin where the previous list of the same launch
// ended, and a workgroup that finishes early takes the next list's tiles.
MOE_DEV int first_slot(int first) {
  const int w = gridDim.x / 8, j = blockIdx.x / 8;
  return first + ((j - first) % w + w) % w;
}

// The tiles of one row-grouped GEMM from per-XCD slot `first` on; returns the slot after its
// last. Every thread of the workgroup calls it (it contains barriers).
template <int BM, int BN, int MODE, bool FP8, bool QOUT = false, bool GATHER = false>
MOE_DEV int rows_list(const RowsArgs& a, int first, RowsShared& sh, char* ring) {
  constexpr int WTM = BM / kWM, WTN = BN / kWN, TM = WTM / 32, TN = WTN / 32;
  constexpr bool kSwiGLU = (MODE == kGateUp);
  // BF16 input gradients read W_e as stored (K-slow); FP8 ones read a transposed copy (K-major)
  constexpr bool kBKS = !FP8 && (MODE == kDownBwd || MODE == kGateUpBwd);
  constexpr int ES = FP8 ? 1 : 2;      // element bytes
  constexpr int OUTN = kSwiGLU ? BN / 2 : BN;
  static_assert(!(FP8 && MODE == kGateUpBwd), "FP8 gate/up dgrad runs as kDown on the transposed W1");
  static_assert(!QOUT || ((MODE == kDown || MODE == kGateUpBwd) && BN == 256), "FP8 output: plain 256-wide tiles");
  static_assert(!GATHER || (MODE == kGateUp && !FP8), "row gather: the BF16 gate/up GEMM");
  int* s_pre = sh.pre;
  int64_t* s_r0 = sh.r0;
  int* s_len = sh.len;
  int* s_preb = sh.preb;
  __syncthreads();  // a previous list of this launch may still read the prefix

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int G = a.nc * a.El;
  const int ntiles = (a.N + OUTN - 1) / OUTN;
  // Two tile classes, each in group order: "large" row tiles (full, or a last tile of more than
  // BM / 2 rows) and "small" last tiles (at most BM / 2 rows, cheaper: half the waves issue no
  // MFMA). Large tiles are dealt first, so the small ones fill a second round where one is needed.
  for (int g = tid; g < G; g += kThreads) {
    const int c = a.c0 + g / a.El, e = g % a.El;
    const int32_t* off = a.offsets + (int64_t)c * (a.El + 1);
    const int len = off[e + 1] - off[e];
    const int rem = len % BM;
    s_r0[g] = (int64_t)c * a.P_c + off[e];
    s_len[g] = len;
    s_pre[g + 1] = (len / BM + (rem > BM / 2 ? 1 : 0)) * ntiles;
    s_preb[g + 1] = (rem > 0 && rem <= BM / 2 ? 1 : 0) * ntiles;
  }
  __syncthreads();
  if (tid == 0) {
    s_pre[0] = 0;
    for (int g = 0; g < G; ++g) s_pre[g + 1] += s_pre[g];
  } else if (tid == 64) {
    s_preb[0] = 0;
    for (int g = 0; g < G; ++g) s_preb[g + 1] += s_preb[g];
  }
  __syncthreads();
  const int total_l = s_pre[G], total_s = s_preb[G];
  // Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8); each XCD owns a
  // contiguous range of the large tiles and one of the small tiles, so the tiles of one expert
  // share that XCD's L2. An XCD's workgroups walk its large range, then its small range.
  //
  // With a queue (a.queue) each workgroup takes its first slot round robin and every later one from
  // an atomic counter of its XCD as it becomes free, so a workgroup that drew short tiles takes
  // more. The next slot is fetched after the tile's K loop (and after the epilogue's own loads):
  // a returning atomic in flight would hold back the wave's later load counts, so fetched during
  // the K loop it would stall every stage until it returned. Which workgroup computes a tile does
  // not change its result. The last workgroup to leave the list resets the counters.
  const int pxl = (total_l + 7) / 8, pxs = (total_s + 7) / 8;
  const int xcd = blockIdx.x % 8, wg_per_xcd = gridDim.x / 8;
  int* const queue = a.queue;
  int slot = first_slot(first) - first;
  for (;;) {
    if (slot >= pxl + pxs) break;
    int nxt = 0;
    auto fetch_next = [&] {
      if (queue && tid == 0) nxt = wg_per_xcd + atomicAdd(queue + xcd, 1);
    };
    const bool large = slot < pxl;
    const int tile = large ? xcd * pxl + slot : xcd * pxs + (slot - pxl);
    if (tile < (large ? total_l : total_s)) {
      const int* pre = large ? s_pre : s_preb;
      int lo = 0, hi = G;
      while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (pre[mid] <= tile) lo = mid; else hi = mid; }
      const int g = __builtin_amdgcn_readfirstlane(lo);
      const int e = g % a.El;
      const int t_in = tile - __builtin_amdgcn_readfirstlane(pre[g]);
      const int mt = large ? t_in / ntiles : s_len[g] / BM, nt = t_in % ntiles;
      const int64_t rg = s_r0[g];
      const int64_t r0 = (((int64_t)__builtin_amdgcn_readfirstlane((int)(rg >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(rg & 0xffffffff))) + (int64_t)mt * BM;
      const int mvalid = min(BM, __builtin_amdgcn_readfirstlane(s_len[g]) - mt * BM);
      const int n0 = nt * OUTN;
      const int nvalid = min(OUTN, a.N - n0);
      const char* Be = (const char*)a.B + (int64_t)e * a.strideB * ES;

      // both operands K-major: pairs of stages, whole lines per row, except the FP8 gate/up GEMM,
      // whose short FP8 stages need the ring's three stages of loads ahead (pairs: 8% slower);
      // the BF16 input gradients take their K-major A operand in pairs as well
      constexpr bool kPair = !kBKS && !(FP8 && MODE == kGateUp);
      constexpr bool kAPair = !FP8 && kBKS;
      Loader<BM, false, kWaves, kPair || kAPair> la;
      if constexpr (GATHER) {
        // tile row r reads token row gather[r0 + r]; rows past the segment point one row past the
        // end of A, which the descriptor's extent turns into zeros
        const int32_t* gt = a.gather;
        const int64_t gr = a.gather_rows;
        la.init_kmajor((const char*)a.A, a.lda * ES, gr * a.lda * ES, wave, lane,
                       [gt, r0, mvalid, gr](int r) { return r < mvalid ? (int64_t)gt[r0 + r] : gr; });
      } else {
        la.init_kmajor((const char*)a.A + r0 * a.lda * ES, a.lda * ES, (int64_t)mvalid * a.lda * ES, wave, lane,
                       [](int r) { return r; });
      }
      Loader<BN, kBKS, kWaves, kPair> lb;
      if constexpr (kSwiGLU) {
        // tile row r -> wave column block r / WTN; its first half are gate rows j, its second half
        // the matching up rows I + j; readable rows run to the end of this expert's W1
        const int I = a.I;
        lb.init_kmajor(Be + (int64_t)n0 * a.K * ES, (int64_t)a.K * ES, (2 * (int64_t)I - n0) * a.K * ES, wave,
                       lane, [I](int r) {
                         const int q = r % WTN, hw = WTN / 2, j = (r / WTN) * hw + (q < hw ? q : q - hw);
                         return q < hw ? j : I + j;
                       });
      } else if constexpr (MODE == kDown || FP8) {
        lb.init_kmajor(Be + (int64_t)n0 * a.K * ES, (int64_t)a.K * ES, ((int64_t)a.N - n0) * a.K * ES, wave, lane,
                       [](int r) { return r; });
      } else {
        // B(n, k) = W_e[k][n]: K-rows of N values, the tile's columns start at n0
        lb.init_kslow(Be + (int64_t)n0 * 2, (int64_t)a.N * 2, ((int64_t)a.K * a.N - n0) * 2, wave, lane);
      }

      f32x16_t acc[TM][TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.f;

      const int nks = a.K / (FP8 ? 64 : 32);
      const int tma = __builtin_amdgcn_readfirstlane(max(0, min(TM, (mvalid - wm * WTM + 31) / 32)));
      const int arow0 = wm * WTM, brow0 = wn * WTN;
      static_assert(TM <= 4, "TM > 4");
      switch (tma) {
#define MOE_KL(T_)                                                                                        \
  if constexpr (kPair)                                                                                     \
    kloop_pairs<FP8, BM, BN, TM, TN, (T_ <= TM ? T_ : TM)>(la, lb, ring, nks, arow0, brow0, lane, acc);    \
  else if constexpr (kAPair)                                                                               \
    kloop_apairs<BM, BN, TM, TN, (T_ <= TM ? T_ : TM)>(la, lb, ring, nks, arow0, brow0, lane, acc);        \
  else                                                                                                     \
    kloop<FP8, false, kBKS, BM, BN, TM, TN, (T_ <= TM ? T_ : TM)>(la, lb, ring, nks, arow0, brow0, lane, acc)
        case 4: MOE_KL(4); break;
        case 3: MOE_KL(3); break;
        case 2: MOE_KL(2); break;
        case 1: MOE_KL(1); break;
        default: MOE_KL(0); break;
#undef MOE_KL
      }
      if constexpr (MODE != kDownBwd) fetch_next();

      // Epilogue through LDS staging (the ring is free): each wave writes its values in the MFMA
      // layout (row m = lane & 31 of each 32-row block, 4 consecutive columns), then the workgroup
      // stores whole rows. Rows past the expert's segment and columns past N are not stored.
      const int mrow = wm * WTM + out_row(lane);
      if constexpr (kSwiGLU) {
        constexpr int W = BN / 2;                 // h / G / U columns per tile
        char* sg = ring;                           // G, then h
        char* su = ring + stage_bytes<BM, W>();    // U
        float sr[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          sr[tm] = (FP8 && mrow + tm * 32 < mvalid) ? a.scale_a[r0 + mrow + tm * 32] : 1.f;
        const float* sb = FP8 ? a.scale_b + (int64_t)e * a.strideSB : nullptr;
        // G and U (dequantised) into the two staging tiles
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int jl = wn * (WTN / 2) + tn * 32 + out_col(gq, lane);   // column within the tile
              float gv[4], uv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                gv[q] = acc[tm][tn][4 * gq + q];
                uv[q] = acc[tm][tn + TN / 2][4 * gq + q];
                if constexpr (FP8) {
                  const int j = min(n0 + jl + q, a.N - 1);
                  gv[q] *= sr[tm] * sb[j];
                  uv[q] *= sr[tm] * sb[a.I + j];
                }
              }
              const int m = mrow + tm * 32;
              *(uint2*)(sg + m * pitch<W>() + 2 * jl) = pack4(gv[0], gv[1], gv[2], gv[3]);
              *(uint2*)(su + m * pitch<W>() + 2 * jl) = pack4(uv[0], uv[1], uv[2], uv[3]);
            }
        lds_barrier();
        if (a.C2) {
          store_staged<BM, W, true>(sg, a.C2 + r0 * 2 * (int64_t)a.I + n0, 2 * (int64_t)a.I, mvalid, nvalid, tid);
          store_staged<BM, W, true>(su, a.C2 + r0 * 2 * (int64_t)a.I + a.I + n0, 2 * (int64_t)a.I, mvalid, nvalid, tid);
        }
        lds_barrier();
        // h = silu(G) * U from the FP32 accumulators
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int jl = wn * (WTN / 2) + tn * 32 + out_col(gq, lane);
              float hv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float gv = acc[tm][tn][4 * gq + q], uv = acc[tm][tn + TN / 2][4 * gq + q];
                if constexpr (FP8) {
                  const int j = min(n0 + jl + q, a.N - 1);
                  gv *= sr[tm] * sb[j];
                  uv *= sr[tm] * sb[a.I + j];
                }
                hv[q] = gv * sigmoidf_(gv) * uv;
              }
              const int m = mrow + tm * 32;
              *(uint2*)(sg + m * pitch<W>() + 2 * jl) = pack4(hv[0], hv[1], hv[2], hv[3]);
            }
        lds_barrier();
        store_staged<BM, W>(sg, a.C + r0 * a.ldc + n0, a.ldc, mvalid, nvalid, tid);
        lds_barrier();
      } else if constexpr (MODE == kDownBwd) {
        // G and U of the tile's rows and columns, staged coalesced; dG and dU overwrite them in place
        constexpr int W = BN;
        char* sg = ring;
        char* su = ring + stage_bytes<BM, W>();
        const int64_t I2 = 2 * (int64_t)a.I;
        load_staged<BM, W>(sg, a.aux + r0 * I2 + n0, I2, mvalid, nvalid, tid);
        load_staged<BM, W>(su, a.aux + r0 * I2 + a.I + n0, I2, mvalid, nvalid, tid);
        fetch_next();
        float sr[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          sr[tm] = (FP8 && mrow + tm * 32 < mvalid) ? a.scale_a[r0 + mrow + tm * 32] : 1.f;
        lds_barrier();
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int jl = wn * WTN + tn * 32 + out_col(gq, lane);
              const int m = mrow + tm * 32;
              char* pg = sg + m * pitch<W>() + 2 * jl;
              char* pu = su + m * pitch<W>() + 2 * jl;
              float gv[4], uv[4], dg[4], du[4];
              unpack4(*(const uint2*)pg, gv);
              unpack4(*(const uint2*)pu, uv);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float dh = acc[tm][tn][4 * gq + q];
                if constexpr (FP8) dh *= sr[tm] * a.scale_b[(int64_t)e * a.strideSB + min(n0 + jl + q, a.N - 1)];
                const float sgm = sigmoidf_(gv[q]);
                dg[q] = dh * uv[q] * sgm * (1.f + gv[q] * (1.f - sgm));
                du[q] = dh * gv[q] * sgm;
              }
              *(uint2*)pg = pack4(dg[0], dg[1], dg[2], dg[3]);
              *(uint2*)pu = pack4(du[0], du[1], du[2], du[3]);
            }
        lds_barrier();
        store_staged<BM, W>(sg, a.C + r0 * I2 + n0, I2, mvalid, nvalid, tid);
        store_staged<BM, W>(su, a.C + r0 * I2 + a.I + n0, I2, mvalid, nvalid, tid);
        lds_barrier();
      } else {
        constexpr int W = BN;
        float sr[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          sr[tm] = (FP8 && mrow + tm * 32 < mvalid) ? a.scale_a[r0 + mrow + tm * 32] : 1.f;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int nl = wn * WTN + tn * 32 + out_col(gq, lane);
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = acc[tm][tn][4 * gq + q];
                if constexpr (FP8) v[q] *= sr[tm] * a.scale_b[(int64_t)e * a.strideSB + min(n0 + nl + q, a.N - 1)];
              }
              *(uint2*)(ring + (mrow + tm * 32) * pitch<W>() + 2 * nl) = pack4(v[0], v[1], v[2], v[3]);
            }
        lds_barrier();
        if constexpr (QOUT)
          store_staged_q<BM, W>(ring, a.Cq + r0 * a.ldc + n0, a.ldc, a.Cs + r0 * a.ldcs + n0 / W, a.ldcs, mvalid,
                                nvalid, tid);
        else
          store_staged<BM, W>(ring, a.C + r0 * a.ldc + n0, a.ldc, mvalid, nvalid, tid);
        lds_barrier();
      }
    } else {
      fetch_next();  // no such tile in this XCD's range
    }
    if (queue) {
      if (tid == 0) sh.q = nxt;
      __syncthreads();
      slot = sh.q;
      __syncthreads();  // every thread has read it before the next write
    } else {
      slot += wg_per_xcd;
    }
  }
  if (queue) {
    if (tid == 0 && atomicAdd(queue + 8, 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int x = 0; x < 9; ++x) queue[x] = 0;
    }
    return first;
  }
  return first + pxl + pxs;
}

// ---------------------------------------------------------------------------------------------
// Launch helpers

// Compute units of the current device (cached per device; the grids of the persistent kernels
// hold at most one workgroup per CU).
inline int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

inline int64_t persistent_grid(int64_t tiles_bound) {
  const int64_t cap = ((int64_t)cu_count() + 7) / 8 * 8;
  const int64_t g = (tiles_bound + 7) / 8 * 8;
  return g < cap ? g : cap;
}

// Argument sets of the BF16 expert GEMMs for chunks c0 .. c0 + nc - 1.
inline RowsArgs gateup_args(const ExpertGemm& g, int c0, int nc) {
  RowsArgs a{};
  a.A = g.xd; a.B = g.w1; a.C = (uint16_t*)g.h; a.C2 = (uint16_t*)g.gu;
  a.lda = g.H; a.ldc = g.I; a.strideB = (int64_t)2 * g.I * g.H; a.K = g.H; a.N = g.I; a.I = g.I;
  a.offsets = g.offsets; a.El = g.El; a.c0 = c0; a.nc = nc; a.P_c = g.P_c;
  return a;
}
inline RowsArgs down_args(const ExpertGemm& g, int c0, int nc) {
  RowsArgs b{};
  b.A = g.h; b.B = g.w2; b.C = (uint16_t*)g.yd;
  b.lda = g.I; b.ldc = g.H; b.strideB = (int64_t)g.H * g.I; b.K = g.I; b.N = g.H; b.I = g.I;
  b.offsets = g.offsets; b.El = g.El; b.c0 = c0; b.nc = nc; b.P_c = g.P_c;
  return b;
}
inline RowsArgs down_dgrad_args(const ExpertGemm& g, int c0, int nc) {
  RowsArgs a{};
  a.A = g.dyd; a.B = g.w2; a.C = (uint16_t*)g.dgu; a.aux = (const uint16_t*)g.gu;
  a.lda = g.H; a.ldc = 2 * g.I; a.strideB = (int64_t)g.H * g.I; a.K = g.H; a.N = g.I; a.I = g.I;
  a.offsets = g.offsets; a.El = g.El; a.c0 = c0; a.nc = nc; a.P_c = g.P_c;
  return a;
}
inline RowsArgs gateup_dgrad_args(const ExpertGemm& g, int c0, int nc) {
  RowsArgs b{};
  b.A = g.dgu; b.B = g.w1;
  if (g.dxd_scales) {  // block-scaled FP8 dxd
    b.Cq = (uint8_t*)g.dxd; b.Cs = g.dxd_scales; b.ldcs = (g.H + 255) / 256;
  } else {
    b.C = (uint16_t*)g.dxd;
  }
  b.lda = 2 * g.I; b.ldc = g.H; b.strideB = (int64_t)2 * g.I * g.H; b.K = 2 * g.I; b.N = g.H; b.I = g.I;
  b.offsets = g.offsets; b.El = g.El; b.c0 = c0; b.nc = nc; b.P_c = g.P_c;
  return b;
}
// Row tiles a launch of this GEMM can hold at most: per chunk floor(P_c / BM) + E_local row tiles
// (every expert adds at most one partial tile) times the column tiles; the device-side count
// decides the work.
template <int BM, int BN, int MODE>
inline int64_t rows_tiles_bound(const RowsArgs& a) {
  const int outn = (MODE == kGateUp) ? BN / 2 : BN;
  return (int64_t)a.nc * (a.P_c / BM + a.El) * ((a.N + outn - 1) / outn);
}

// Tile shapes: 256 x 256 everywhere except down dgrad (128 x 256: its N = I gives few column
// tiles, and 128-row tiles keep more CUs busy).
#define MOE_GATEUP 256, 256, kGateUp
#define MOE_DOWN 256, 256, kDown
#define MOE_DDGRAD 128, 256, kDownBwd
#define MOE_GUDGRAD 256, 256, kGateUpBwd

}  // namespace gg
}  // namespace moe
