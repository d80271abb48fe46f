// Shared device helpers for the MoE layer-share kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

struct alignas(16) u32x4 { uint32_t x, y, z, w; };

MOE_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// FP32 -> BF16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32, two values per
// instruction.
MOE_DEV uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
MOE_DEV uint16_t f2bf(float f) { return (uint16_t)(pack_bf2(f, 0.f) & 0xffffu); }

// Element load/store helpers for payload types (float or uint16_t BF16 bits).
template <typename T> MOE_DEV float ld_elem(const T* p);
template <> MOE_DEV float ld_elem<float>(const float* p) { return *p; }
template <> MOE_DEV float ld_elem<uint16_t>(const uint16_t* p) { return bf2f(*p); }
template <typename T> MOE_DEV void st_elem(T* p, float v);
template <> MOE_DEV void st_elem<float>(float* p, float v) { *p = v; }
template <> MOE_DEV void st_elem<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }

// Logistic sigmoid with the hardware exponential and reciprocal (about 1 ulp each): the SwiGLU
// epilogues evaluate it for every element of h, where an IEEE division would dominate the VALU time.
MOE_DEV float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Weight-gradient operands in expert-transposed FP8 form: expert e's rows over every chunk (chunk
// order) are its K_e rows, padded to Kp_e = K_e rounded up to 64; expert e's block starts at
// koff_e = sum of Kp over the experts before it. offsets: [n_chunks][El + 1] local offsets.
MOE_DEV void expert_k(const int32_t* offsets, int El, int n_chunks, int e, int64_t& koff, int& K) {
  koff = 0;
  K = 0;
  for (int g = 0; g <= e; ++g) {
    int kk = 0;
    for (int c = 0; c < n_chunks; ++c) kk += offsets[c * (El + 1) + g + 1] - offsets[c * (El + 1) + g];
    if (g < e) koff += (kk + 63) & ~63;
    else K = kk;
  }
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
MOE_DEV int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
MOE_DEV int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets past `bytes` return zero
// without touching memory (the extent masks rows past a segment or a matrix edge).
typedef __attribute__((address_space(3))) void lds_void_t;
MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           (int)(bytes < 0 ? 0 : (bytes > lim ? lim : bytes)),
                                           0x00020000);  // gfx9 raw buffer descriptor word 3
}

// The same descriptor as four dwords, for instructions written in assembly: base address bits
// 31:0, bits 47:32 with stride 0, num_records, word 3 (uniform values, made scalar).
MOE_DEV i32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const int64_t lim = 0x7fffffff;
  return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
                 __builtin_amdgcn_readfirstlane((int)(bytes < 0 ? 0 : (bytes > lim ? lim : bytes))), 0x00020000};
}

// LDS byte address of a pointer into LDS.
MOE_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
MOE_DEV void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Token range of chunk c (chunks of ceil(T/n) tokens, the last takes the remainder).
struct ChunkRange { int64_t t0, t1; };
MOE_DEV ChunkRange chunk_range(int64_t T, int n, int c) {
  int64_t tc = (T + n - 1) / n;
  int64_t a = c * tc, b = a + tc;
  if (a > T) a = T;
  if (b > T) b = T;
  return {a, b};
}

// FP8 conversion: OCP e4m3fn, round to nearest even; inputs are already within +-448.
MOE_DEV uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

MOE_DEV float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Quantise one 16-byte BF16 vector (8 values) with multiplier inv -> 8 e4m3 codes.
MOE_DEV uint2 quant8(const u32x4& v, float inv) {
  float f[8] = {bf2f(v.x & 0xffff), bf2f(v.x >> 16), bf2f(v.y & 0xffff), bf2f(v.y >> 16),
                bf2f(v.z & 0xffff), bf2f(v.z >> 16), bf2f(v.w & 0xffff), bf2f(v.w >> 16)};
  uint2 q;
  q.x = pack_fp8x4(clamp448(f[0] * inv), clamp448(f[1] * inv), clamp448(f[2] * inv), clamp448(f[3] * inv));
  q.y = pack_fp8x4(clamp448(f[4] * inv), clamp448(f[5] * inv), clamp448(f[6] * inv), clamp448(f[7] * inv));
  return q;
}

MOE_DEV float absmax8(const u32x4& v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf2f(w[i] & 0xffff)));
    m = fmaxf(m, fabsf(bf2f(w[i] >> 16)));
  }
  return m;
}

// Dequantise 8 e4m3 codes (OCP e4m3fn) times scale s.
MOE_DEV void deq8(uint2 q, float s, float* f) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  f[0] = a[0] * s; f[1] = a[1] * s; f[2] = b[0] * s; f[3] = b[1] * s;
  f[4] = c[0] * s; f[5] = c[1] * s; f[6] = d[0] * s; f[7] = d[1] * s;
}

}  // namespace moe
