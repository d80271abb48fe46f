// C ABI of the MoE layer share (include/moe.h): argument validation, extent bookkeeping,
// workspace sizing, the stage calls and the two-stream chunk schedule of the layer primitives.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <string>
#include <vector>

#include "launch.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY(expr)                      \
  do {                                     \
    moe_status _st = (expr);               \
    if (_st != MOE_OK) return _st;         \
  } while (0)
#define MOE_HIP(expr, what) MOE_TRY(hip_check((expr), (what)))
#define MOE_NEED(p) \
  do { if (!(p)) return fail(MOE_ERR_ARG, "%s: argument '%s' is NULL", __func__, #p); } while (0)

int64_t round4(int64_t x) { return (x + 3) / 4 * 4; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t tokens_per_chunk(const moe_desc* d) { return cdiv(d->T, d->n_chunks); }
int64_t min_pc(const moe_desc* d) {
  int64_t kk = d->k < d->E_local ? d->k : d->E_local;
  return tokens_per_chunk(d) * kk;
}
int elem_size(int dtype) { return dtype == MOE_F32 ? 4 : 2; }  // payload rows (FP8: BF16 x/yd)
constexpr int64_t kRsrcMax = 0x7fffffff;  // bytes one raw buffer descriptor addresses

moe_status validate(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_ARG, "descriptor is NULL");
  if (d->flags & ~(MOE_FLAG_FP8_DGRAD | MOE_FLAG_FP8_WGRAD | MOE_FLAG_FP8_DXD))
    return fail(MOE_ERR_ARG, "descriptor flags 0x%x hold an unknown bit", d->flags);
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16 && d->dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_ARG, "unknown dtype %d", d->dtype);
  if (d->T < 0) return fail(MOE_ERR_ARG, "T = %lld is negative", (long long)d->T);
  if (d->n_chunks < 1) return fail(MOE_ERR_ARG, "n_chunks = %d must be >= 1", d->n_chunks);
  if (d->E < 1 || d->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d outside 1..1024", d->E);
  if (d->k < 1 || d->k > d->E) return fail(MOE_ERR_ARG, "k = %d outside 1..E", d->k);
  if (d->k > 8) return fail(MOE_ERR_UNSUPPORTED, "k = %d above 8", d->k);
  if (d->e0 < 0 || d->E_local < 0 || (int64_t)d->e0 + d->E_local > d->E)
    return fail(MOE_ERR_ARG, "local experts [%d, %d) not inside [0, %d)", d->e0, d->e0 + d->E_local, d->E);
  if ((int64_t)d->n_chunks * d->E_local > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "n_chunks * E_local = %lld above 1024",
                (long long)d->n_chunks * d->E_local);
  if (d->H <= 0 || d->H % 64) return fail(MOE_ERR_UNSUPPORTED, "H = %d must be a positive multiple of 64", d->H);
  if (d->I <= 0 || d->I % 64) return fail(MOE_ERR_UNSUPPORTED, "I = %d must be a positive multiple of 64", d->I);
  if (d->dtype == MOE_BF16 && d->E % 4) return fail(MOE_ERR_UNSUPPORTED, "BF16 path needs E %% 4 == 0 (E = %d)", d->E);
  if (d->flags && d->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the FP8 backward flags need the BF16 dtype");
  if (d->dtype == MOE_FP8_E4M3 && d->H > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 dispatch keeps a row in registers: H = %d above 8192", d->H);
  if (d->P_c % 4) return fail(MOE_ERR_CAPACITY, "P_c = %lld is not a multiple of 4", (long long)d->P_c);
  if (d->P_c < min_pc(d))
    return fail(MOE_ERR_CAPACITY, "P_c = %lld below ceil(T/n)*min(k,E_local) = %lld", (long long)d->P_c,
                (long long)min_pc(d));
  if (d->P_out % 4) return fail(MOE_ERR_CAPACITY, "P_out = %lld is not a multiple of 4", (long long)d->P_out);
  if (d->P_out < d->T) return fail(MOE_ERR_CAPACITY, "P_out = %lld below T = %lld", (long long)d->P_out, (long long)d->T);
  if ((int64_t)d->n_chunks * d->P_c > INT32_MAX || d->T * d->k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "row indices exceed int32");
  // the expert GEMMs address one expert's weights through a buffer descriptor
  const int64_t wes = d->dtype == MOE_F32 ? 4 : 2;
  if (2 * (int64_t)d->I * d->H * wes > kRsrcMax)
    return fail(MOE_ERR_UNSUPPORTED, "one expert's W1 (2I x H = %lld elements) exceeds a 2 GiB buffer descriptor",
                (long long)(2 * (int64_t)d->I * d->H));
  return MOE_OK;
}

// Extents that the backward kernels address through one buffer descriptor (at most 2^31 - 1
// bytes; loads past a descriptor's extent would read zeros): a weight-gradient operand segment
// (one expert's rows of one chunk, at most P_c rows of max(H, 2I) BF16 values), the router
// weight gradient's operands of one chunk (ceil(T/n) rows of x and of FP32 dlogits) and, with
// FP8 weight gradients, one expert's transposed operand (max(H, 2I) rows of its padded rows of
// every chunk, at most n P_c + 64, FP8 codes).
moe_status bwd_extent(const moe_desc* d) {
  const int64_t es = d->dtype == MOE_F32 ? 4 : 2;
  const int64_t wide = d->H > 2 * (int64_t)d->I ? d->H : 2 * (int64_t)d->I;
  if (d->E_local > 0 && d->P_c * wide * es > kRsrcMax)
    return fail(MOE_ERR_UNSUPPORTED, "weight gradients: P_c x max(H, 2I) = %lld elements exceed a 2 GiB buffer descriptor",
                (long long)(d->P_c * wide));
  const int64_t tc = tokens_per_chunk(d);
  if (tc * d->H * es > kRsrcMax || tc * (int64_t)d->E * 4 > kRsrcMax)
    return fail(MOE_ERR_UNSUPPORTED, "router weight gradient: a chunk's %lld tokens exceed a 2 GiB buffer descriptor",
                (long long)tc);
  if ((d->flags & MOE_FLAG_FP8_WGRAD) && d->E_local > 0 && wide * ((int64_t)d->n_chunks * d->P_c + 64) > kRsrcMax)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 weight gradients: max(H, 2I) x (n_chunks P_c + 64) = %lld bytes exceed a 2 GiB buffer descriptor",
                (long long)(wide * ((int64_t)d->n_chunks * d->P_c + 64)));
  return MOE_OK;
}

moe_status check_chunk(const moe_desc* d, int chunk) {
  if (chunk < -1 || chunk >= d->n_chunks)
    return fail(MOE_ERR_ARG, "chunk = %d outside -1..%d", chunk, d->n_chunks - 1);
  return MOE_OK;
}

struct Range { int64_t t0, t1; int c0, nc; };
Range range_of(const moe_desc* d, int chunk) {
  if (chunk < 0) return {0, d->T, 0, d->n_chunks};
  int64_t tc = tokens_per_chunk(d);
  int64_t a = chunk * tc, b = a + tc;
  if (a > d->T) a = d->T;
  if (b > d->T) b = d->T;
  return {a, b, chunk, 1};
}

bool is_bf16_rows(const moe_desc* d) { return d->dtype != MOE_F32; }
// dispatch rows of the descriptor (0 when no expert is local)
int64_t rows_of(const moe_desc* d) { return d->E_local > 0 ? (int64_t)d->n_chunks * d->P_c : 0; }

// Events for the two-stream schedule, created once per host thread and device and reused (they
// live until the process ends). Per thread, so that schedules issued concurrently from several
// threads never record or wait on each other's events; within one thread the calls are issued
// one after another, and a wait always refers to the event's latest record.
struct EventPool {
  std::vector<hipEvent_t> ev;
};
thread_local std::map<int, EventPool> t_pools;

moe_status events(int count, hipEvent_t** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  EventPool& p = t_pools[dev];
  while ((int)p.ev.size() < count) {
    hipEvent_t e;
    MOE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence), "hipEventCreateWithFlags");
    p.ev.push_back(e);
  }
  *out = p.ev.data();
  return MOE_OK;
}

// Router weight-gradient scratch: the split-K partials, then (BF16 rows) the chunk's dlogits as BF16
// high and low planes [tokens per chunk, router_plane_ld(E)] at a 256-byte boundary.
int64_t router_partials_span(const moe_desc* d) {
  return (moe::router_partials_bytes(tokens_per_chunk(d), d->E, d->H) + 255) / 256 * 256;
}
int64_t router_plane_bytes(const moe_desc* d) {  // both planes
  return is_bf16_rows(d) ? 2 * tokens_per_chunk(d) * moe::router_plane_ld(d->E) * 2 : 0;
}
int64_t router_scratch(const moe_desc* d) { return router_partials_span(d) + router_plane_bytes(d); }

// Workspace layout: the routing histograms and the router weight gradient's partials share its
// start (they run in order on one stream); the expert weight gradients' scratch (BF16 path)
// follows at a 256-byte boundary, so the router and expert weight gradients may run concurrently.
int64_t wgrad_scratch(const moe_desc* d) {
  return d->dtype == MOE_BF16 ? moe::wgrad_scratch_bytes(d->H, d->I, d->E_local) : 0;
}
int64_t wgrad_offset(const moe_desc* d) {
  const int64_t a = moe::route_scratch_bytes(d->T, d->n_chunks, d->E);
  const int64_t b = d->dtype == MOE_FP8_E4M3 ? 0 : router_scratch(d);
  return ((a > b ? a : b) + 255) / 256 * 256;
}
void* wgrad_ws(const moe_desc* d, void* workspace) {
  return wgrad_scratch(d) > 0 && workspace ? (char*)workspace + wgrad_offset(d) : nullptr;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }
int32_t moe_abi_version(void) { return 4; }

moe_status moe_required_extent(int64_t T, int32_t k, int32_t E_local, int32_t n_chunks, int64_t* P_c,
                               int64_t* P_out) {
  if (!P_c || !P_out) return fail(MOE_ERR_ARG, "output pointer is NULL");
  if (T < 0 || k < 1 || E_local < 0 || n_chunks < 1) return fail(MOE_ERR_ARG, "invalid extent arguments");
  int64_t kk = k < E_local ? k : E_local;
  *P_c = round4(cdiv(T, n_chunks) * kk);
  int64_t po = round4(T * k);
  *P_out = po > round4(T) ? po : round4(T);
  return MOE_OK;
}

moe_status moe_workspace_bytes(const moe_desc* d, moe_workspace_sizes* o) {
  MOE_TRY(validate(d));
  if (!o) return fail(MOE_ERR_ARG, "output pointer is NULL");
  const int64_t T = d->T, H = d->H, I = d->I, E = d->E, El = d->E_local, K = d->k, n = d->n_chunks;
  const int64_t P = n * d->P_c;
  const int64_t es = elem_size(d->dtype);
  const bool fp8 = d->dtype == MOE_FP8_E4M3;
  *o = moe_workspace_sizes{};
  o->topk_idx = T * K * 4;
  o->gates = T * K * 4;
  o->counts = n * E * 4;
  o->offsets = n * (El + 1) * 4;
  o->row_of = T * K * 4;
  o->src_token = P * 4;
  o->xd = P * H * (fp8 ? 1 : es);
  o->xd_scale = fp8 ? P * 4 : 0;
  o->gu = fp8 ? 0 : P * 2 * I * es;
  o->h = P * I * (fp8 ? 3 : es);  // FP8: BF16 values, then e4m3 codes
  o->h_scale = fp8 ? P * 4 : 0;
  o->yd = P * H * es;
  o->out = d->P_out * H * es;
  if (!fp8) {
    o->dyd = P * H * es;
    o->dgates = T * K * 4;
    o->dlogits = T * E * 4;
    o->dwr_acc = E * H * 4;
    o->dgu = P * 2 * I * es;
    o->dxd = P * H * es;
    o->dx = T * H * es;
    o->dw1 = El * 2 * I * H * es;
    o->dw2 = El * H * I * es;
    o->dwr = E * H * es;
  }
  if (d->flags & MOE_FLAG_FP8_DGRAD) {
    o->w1t = El * H * 2 * I;
    o->w1t_scale = El * H * 4;
    o->w2t = El * I * H;
    o->w2t_scale = El * I * 4;
    o->dyd_q = P * H;
    o->dyd_scale = P * 4;
    o->dgu_q = P * 2 * I;
    o->dgu_scale = P * 4;
  }
  if (d->flags & MOE_FLAG_FP8_WGRAD) {
    const int64_t Kp = P + 64 * El;   // the padded rows of every expert together, at most
    o->dyd_t = H * Kp;
    o->dyd_cs = El * H * 4;
    o->dgu_t = 2 * I * Kp;
    o->dgu_cs = El * 2 * I * 4;
    o->xd_t = H * Kp;
    o->xd_cs = El * H * 4;
    o->h_t = I * Kp;
    o->h_cs = El * I * 4;
  }
  o->route_scratch = moe::route_scratch_bytes(T, (int)n, (int)E);
  o->route_bwd_scratch = fp8 ? 0 : router_scratch(d);
  o->wgrad_scratch = wgrad_scratch(d);
  o->wgrad_zero_bytes = d->dtype == MOE_BF16 ? moe::wgrad_counter_bytes_of(d->H, d->I, d->E_local) : 0;
  o->workspace = wgrad_offset(d) + o->wgrad_scratch;
  return MOE_OK;
}

// ----------------------------------------------------------------------------- stage calls

moe_status moe_route(const moe_desc* d, int chunk, const float* logits, int32_t* topk_idx, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_token,
                     void* workspace, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  if (d->T > 0) { MOE_NEED(logits); MOE_NEED(topk_idx); MOE_NEED(gates); MOE_NEED(row_of); }
  if ((int64_t)d->n_chunks * d->P_c > 0) MOE_NEED(src_token);  // rows past N_c are marked -1
  MOE_NEED(counts); MOE_NEED(offsets); MOE_NEED(workspace);
  Range r = range_of(d, chunk);
  MOE_HIP(moe::launch_route(logits, topk_idx, gates, counts, offsets, row_of, src_token,
                            (int32_t*)workspace, d->T, d->E, d->e0, d->E_local, d->k, d->n_chunks,
                            r.c0, r.nc, d->P_c, (hipStream_t)stream),
          "route");
  return MOE_OK;
}

moe_status moe_route_noalloc(const moe_desc* d, int chunk, const float* logits, int32_t* topk_idx, float* gates,
                             int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_token, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  if (d->T > 0) { MOE_NEED(logits); MOE_NEED(topk_idx); MOE_NEED(gates); MOE_NEED(row_of); }
  if ((int64_t)d->n_chunks * d->P_c > 0) MOE_NEED(src_token);
  MOE_NEED(counts); MOE_NEED(offsets);
  const int64_t need = moe::route_scratch_bytes(d->T, d->n_chunks, d->E);
  if (need > moe::kNoAllocRouteScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_route_noalloc: the routing histograms need %lld bytes, above its fixed %lld-byte device "
                "scratch (n_chunks * ceil(ceil(T/n_chunks)/64) * 4 * E * 4 bytes); use moe_route with a workspace",
                (long long)need, (long long)moe::kNoAllocRouteScratchBytes);
  void* ws = nullptr;
  MOE_HIP(moe::route_noalloc_scratch(&ws), "moe_route_noalloc: hipGetSymbolAddress");
  Range r = range_of(d, chunk);
  MOE_HIP(moe::launch_route(logits, topk_idx, gates, counts, offsets, row_of, src_token, (int32_t*)ws, d->T, d->E,
                            d->e0, d->E_local, d->k, d->n_chunks, r.c0, r.nc, d->P_c, (hipStream_t)stream),
          "route");
  return MOE_OK;
}

moe_status moe_route_x(const moe_desc* d, int chunk, const void* x, const void* w_r, float* logits,
                       int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                       int32_t* src_token, void* workspace, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  if (d->dtype == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "moe_route_x: x and W_r must be BF16 (dtype BF16 or FP8)");
  if (d->E % 32 || d->E > 256)
    return fail(MOE_ERR_UNSUPPORTED, "moe_route_x: E = %d must be a multiple of 32, at most 256", d->E);
  if (d->T > 0) { MOE_NEED(x); MOE_NEED(w_r); MOE_NEED(topk_idx); MOE_NEED(gates); MOE_NEED(row_of); }
  if ((int64_t)d->n_chunks * d->P_c > 0) MOE_NEED(src_token);  // rows past N_c are marked -1
  MOE_NEED(counts); MOE_NEED(offsets); MOE_NEED(workspace);
  Range r = range_of(d, chunk);
  MOE_HIP(moe::launch_route_x(x, w_r, logits, topk_idx, gates, counts, offsets, row_of, src_token,
                              (int32_t*)workspace, d->T, d->E, d->H, d->e0, d->E_local, d->k, d->n_chunks,
                              r.c0, r.nc, d->P_c, (hipStream_t)stream),
          "route_x");
  return MOE_OK;
}

moe_status moe_dispatch(const moe_desc* d, int chunk, const void* x, const int32_t* row_of, void* xd,
                        float* xd_scale, float* h_scale, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  Range r = range_of(d, chunk);
  if (r.t1 <= r.t0) return MOE_OK;
  MOE_NEED(x); MOE_NEED(row_of);
  if (rows_of(d) == 0) return MOE_OK;  // no local expert: nothing to write
  MOE_NEED(xd);
  if (d->dtype == MOE_FP8_E4M3) {
    MOE_NEED(xd_scale); MOE_NEED(h_scale);
    MOE_HIP(moe::launch_dispatch_fp8(x, row_of, xd, xd_scale, h_scale, r.t0, r.t1, d->k, d->H,
                                     (hipStream_t)stream), "dispatch_fp8");
  } else {
    MOE_HIP(moe::launch_dispatch(x, row_of, xd, r.t0, r.t1, d->k, (int64_t)d->H * elem_size(d->dtype),
                                 (hipStream_t)stream), "dispatch");
  }
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_desc* d, int chunk, const void* xd, const float* xd_scale,
                          const void* w1, const float* w1_scale, const void* w2, const float* w2_scale,
                          const int32_t* offsets, void* gu, void* h, float* h_scale, void* yd,
                          void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  Range r = range_of(d, chunk);
  if (rows_of(d) == 0) return MOE_OK;
  MOE_NEED(xd); MOE_NEED(w1); MOE_NEED(w2); MOE_NEED(offsets); MOE_NEED(h); MOE_NEED(yd);
  if (d->dtype == MOE_FP8_E4M3) {
    MOE_NEED(xd_scale); MOE_NEED(w1_scale); MOE_NEED(w2_scale); MOE_NEED(h_scale);
    MOE_HIP(moe::launch_expert_fwd_fp8(xd, xd_scale, w1, w1_scale, w2, w2_scale, offsets, h, h_scale,
                                       yd, d->H, d->I, d->E_local, r.c0, r.nc, d->P_c,
                                       rows_of(d), (hipStream_t)stream), "expert_ffn_fp8");
    return MOE_OK;
  }
  MOE_HIP(moe::launch_expert_fwd(is_bf16_rows(d), xd, w1, w2, offsets, gu, h, yd, d->H, d->I,
                                 d->E_local, r.c0, r.nc, d->P_c, (hipStream_t)stream), "expert_ffn");
  return MOE_OK;
}

moe_status moe_combine(const moe_desc* d, int chunk, const void* yd, const float* gates,
                       const int32_t* row_of, void* out, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_chunk(d, chunk));
  Range r = range_of(d, chunk);
  if (r.t1 <= r.t0) return MOE_OK;
  MOE_NEED(gates); MOE_NEED(row_of); MOE_NEED(out);
  if (rows_of(d) > 0) MOE_NEED(yd);
  MOE_HIP(moe::launch_combine(is_bf16_rows(d), yd, gates, row_of, out, r.t0, r.t1, d->k,
                              (int64_t)d->H * elem_size(d->dtype), (hipStream_t)stream), "combine");
  return MOE_OK;
}

// MOE_FLAG_FP8_DXD: the dxd buffer [n_chunks * P_c, H] (BF16-sized) holds the block-scaled e4m3
// rows: codes [n_chunks * P_c, H] from its start, then one FP32 scale per row and 256-column block.
static float* dxd_scales(const moe_desc* d, const void* dxd) {
  if (!(d->flags & MOE_FLAG_FP8_DXD) || !dxd) return nullptr;
  return (float*)((char*)dxd + (int64_t)d->n_chunks * d->P_c * d->H);
}

static moe_status no_fp8_bwd(const moe_desc* d) {
  if (d->dtype == MOE_FP8_E4M3) return fail(MOE_ERR_UNSUPPORTED, "the FP8 payload path is forward only");
  return MOE_OK;
}

// Combine backward; with dyd_q (BF16, the FP8 input-gradient layer) it also writes the e4m3 rows
// of dyd and their scales, as moe_expert_dgrad_fp8 would quantise them.
static moe_status combine_bwd_impl(const moe_desc* d, int chunk, const void* dy, const void* yd,
                                   const float* gates, const int32_t* row_of, void* dyd, float* dgates,
                                   void* dyd_q, float* dyd_scale, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(check_chunk(d, chunk));
  Range r = range_of(d, chunk);
  if (r.t1 <= r.t0) return MOE_OK;
  MOE_NEED(dy); MOE_NEED(gates); MOE_NEED(row_of); MOE_NEED(dgates);
  if (rows_of(d) > 0) { MOE_NEED(yd); MOE_NEED(dyd); }
  MOE_HIP(moe::launch_combine_bwd(is_bf16_rows(d), dy, yd, gates, row_of, dyd, dgates, r.t0, r.t1, d->k,
                                  (int64_t)d->H * elem_size(d->dtype), (hipStream_t)stream, dyd_q, dyd_scale),
          "combine_bwd");
  return MOE_OK;
}

moe_status moe_combine_bwd(const moe_desc* d, int chunk, const void* dy, const void* yd, const float* gates,
                           const int32_t* row_of, void* dyd, float* dgates, void* stream) {
  return combine_bwd_impl(d, chunk, dy, yd, gates, row_of, dyd, dgates, nullptr, nullptr, stream);
}

moe_status moe_route_bwd(const moe_desc* d, int chunk, const float* dgates, const float* gates,
                         const int32_t* topk_idx, const void* x, float* dlogits, float* dwr_acc, void* dwr,
                         void* workspace, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(bwd_extent(d));
  MOE_TRY(check_chunk(d, chunk));
  MOE_NEED(dwr_acc); MOE_NEED(workspace);
  if (d->T > 0) { MOE_NEED(dgates); MOE_NEED(gates); MOE_NEED(topk_idx); MOE_NEED(x); MOE_NEED(dlogits); }
  const int cfirst = chunk < 0 ? 0 : chunk, clast = chunk < 0 ? d->n_chunks - 1 : chunk;
  if (clast == d->n_chunks - 1) MOE_NEED(dwr);
  // BF16 rows: the dlogits planes follow the partials (each chunk's router gradient reads them
  // before the next chunk's dlogits kernel, on the same stream, rewrites them)
  uint16_t* hi = nullptr;
  uint16_t* lo = nullptr;
  const int ldl = moe::router_plane_ld(d->E);
  const int64_t pitch = moe::router_plane_pitch(d->E);
  if (router_plane_bytes(d) > 0) {
    hi = (uint16_t*)((char*)workspace + router_partials_span(d));
    lo = hi + moe::router_plane_lo_offset(d->E, tokens_per_chunk(d));
  }
  for (int c = cfirst; c <= clast; ++c) {
    Range r = range_of(d, c);
    MOE_HIP(moe::launch_route_bwd_dlogits(dgates, gates, topk_idx, dlogits, r.t0, r.t1, d->k, d->E,
                                          (hipStream_t)stream, hi, lo, ldl, pitch), "route_bwd_dlogits");
    MOE_HIP(moe::launch_router_wgrad(is_bf16_rows(d), dlogits, hi, lo, ldl, x, (float*)workspace, dwr_acc, c == 0,
                                     c == d->n_chunks - 1 ? dwr : nullptr, r.t0, r.t1, d->E, d->H,
                                     (hipStream_t)stream), "router_wgrad");
  }
  return MOE_OK;
}

moe_status moe_expert_wgrad(const moe_desc* d, const void* dyd, const void* dgu, const void* xd, const void* h,
                            const int32_t* offsets, void* dw1, void* dw2, void* workspace, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(bwd_extent(d));
  if (d->E_local == 0) return MOE_OK;
  MOE_NEED(offsets); MOE_NEED(dw1); MOE_NEED(dw2);
  if (wgrad_scratch(d) > 0) MOE_NEED(workspace);
  if (rows_of(d) > 0) { MOE_NEED(dyd); MOE_NEED(dgu); MOE_NEED(xd); MOE_NEED(h); }
  MOE_HIP(moe::launch_expert_wgrad(is_bf16_rows(d), dyd, dgu, xd, h, offsets, dw1, dw2, d->H, d->I,
                                   d->E_local, d->n_chunks, d->P_c, wgrad_ws(d, workspace), (hipStream_t)stream),
          "expert_wgrad");
  return MOE_OK;
}

moe_status moe_expert_ffn_bwd(const moe_desc* d, int chunk, const void* dyd, const void* xd, const void* gu,
                              const void* h, const void* w1, const void* w2, const int32_t* offsets,
                              void* dgu, void* dxd, void* dw1, void* dw2, void* workspace, void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(check_chunk(d, chunk));
  if (chunk < 0) MOE_TRY(bwd_extent(d));  // the weight gradients follow the input gradients
  if (d->E_local == 0) return MOE_OK;
  if (chunk < 0 && wgrad_scratch(d) > 0) MOE_NEED(workspace);
  Range r = range_of(d, chunk);
  if (rows_of(d) == 0)
    return chunk < 0 ? moe_expert_wgrad(d, dyd, dgu, xd, h, offsets, dw1, dw2, workspace, stream) : MOE_OK;
  MOE_NEED(dyd); MOE_NEED(gu); MOE_NEED(w1); MOE_NEED(w2); MOE_NEED(offsets); MOE_NEED(dgu); MOE_NEED(dxd);
  MOE_HIP(moe::launch_expert_dgrad(is_bf16_rows(d), dyd, gu, w1, w2, offsets, dgu, dxd, dxd_scales(d, dxd), d->H, d->I,
                                   d->E_local, r.c0, r.nc, d->P_c, (hipStream_t)stream), "expert_dgrad");
  if (chunk < 0) return moe_expert_wgrad(d, dyd, dgu, xd, h, offsets, dw1, dw2, workspace, stream);
  return MOE_OK;
}

static moe_status expert_dgrad_fp8_impl(const moe_desc* d, int chunk, const void* dyd, const void* gu,
                                        const void* w1t, const float* w1t_scale, const void* w2t,
                                        const float* w2t_scale, const int32_t* offsets, void* dyd_q,
                                        float* dyd_scale, void* dgu, void* dgu_q, float* dgu_scale, void* dxd,
                                        bool quantize_dyd, void* stream) {
  MOE_TRY(validate(d));
  if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "FP8 input gradients need the BF16 dtype");
  MOE_TRY(check_chunk(d, chunk));
  if (rows_of(d) == 0) return MOE_OK;
  Range r = range_of(d, chunk);
  MOE_NEED(dyd); MOE_NEED(gu); MOE_NEED(w1t); MOE_NEED(w1t_scale); MOE_NEED(w2t); MOE_NEED(w2t_scale);
  MOE_NEED(offsets); MOE_NEED(dyd_q); MOE_NEED(dyd_scale); MOE_NEED(dgu); MOE_NEED(dgu_q); MOE_NEED(dgu_scale);
  MOE_NEED(dxd);
  MOE_HIP(moe::launch_expert_dgrad_fp8(dyd, gu, w1t, w1t_scale, w2t, w2t_scale, offsets, dyd_q, dyd_scale, dgu,
                                       dgu_q, dgu_scale, dxd, dxd_scales(d, dxd), d->H, d->I, d->E_local, r.c0, r.nc, d->P_c,
                                       (hipStream_t)stream, quantize_dyd),
          "expert_dgrad_fp8");
  return MOE_OK;
}

moe_status moe_expert_dgrad_fp8(const moe_desc* d, int chunk, const void* dyd, const void* gu, const void* w1t,
                                const float* w1t_scale, const void* w2t, const float* w2t_scale,
                                const int32_t* offsets, void* dyd_q, float* dyd_scale, void* dgu, void* dgu_q,
                                float* dgu_scale, void* dxd, void* stream) {
  return expert_dgrad_fp8_impl(d, chunk, dyd, gu, w1t, w1t_scale, w2t, w2t_scale, offsets, dyd_q, dyd_scale, dgu,
                               dgu_q, dgu_scale, dxd, true, stream);
}

static moe_status expert_wgrad_fp8_impl(const moe_desc* d, const void* dyd, const void* dgu, const void* xd,
                                        const void* h, const int32_t* offsets, void* dyd_t, float* dyd_cs,
                                        void* dgu_t, float* dgu_cs, void* xd_t, float* xd_cs, void* h_t,
                                        float* h_cs, void* dw1, void* dw2, bool quantize, void* stream) {
  MOE_TRY(validate(d));
  {
    moe_desc f = *d;
    f.flags |= MOE_FLAG_FP8_WGRAD;
    MOE_TRY(bwd_extent(&f));
  }
  if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "FP8 weight gradients need the BF16 dtype");
  if (d->E_local == 0) return MOE_OK;
  MOE_NEED(offsets); MOE_NEED(dw1); MOE_NEED(dw2);
  MOE_NEED(dyd_t); MOE_NEED(dyd_cs); MOE_NEED(dgu_t); MOE_NEED(dgu_cs);
  MOE_NEED(xd_t); MOE_NEED(xd_cs); MOE_NEED(h_t); MOE_NEED(h_cs);
  if (rows_of(d) > 0) { MOE_NEED(dyd); MOE_NEED(dgu); MOE_NEED(xd); MOE_NEED(h); }
  MOE_HIP(moe::launch_expert_wgrad_fp8(dyd, dgu, xd, h, offsets, dyd_t, dyd_cs, dgu_t, dgu_cs, xd_t, xd_cs, h_t,
                                       h_cs, dw1, dw2, d->H, d->I, d->E_local, d->n_chunks, d->P_c,
                                       (hipStream_t)stream, quantize),
          "expert_wgrad_fp8");
  return MOE_OK;
}

moe_status moe_expert_wgrad_fp8(const moe_desc* d, const void* dyd, const void* dgu, const void* xd, const void* h,
                                const int32_t* offsets, void* dyd_t, float* dyd_cs, void* dgu_t, float* dgu_cs,
                                void* xd_t, float* xd_cs, void* h_t, float* h_cs, void* dw1, void* dw2,
                                void* stream) {
  return expert_wgrad_fp8_impl(d, dyd, dgu, xd, h, offsets, dyd_t, dyd_cs, dgu_t, dgu_cs, xd_t, xd_cs, h_t, h_cs,
                               dw1, dw2, true, stream);
}

moe_status moe_dispatch_bwd(const moe_desc* d, int chunk, const void* dxd, const int32_t* row_of,
                            const int32_t* topk_idx, const float* dlogits, const void* w_r, void* dx,
                            void* stream) {
  MOE_TRY(validate(d));
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(check_chunk(d, chunk));
  Range r = range_of(d, chunk);
  if (r.t1 <= r.t0) return MOE_OK;
  MOE_NEED(row_of); MOE_NEED(topk_idx); MOE_NEED(dlogits); MOE_NEED(w_r); MOE_NEED(dx);
  if (rows_of(d) > 0) MOE_NEED(dxd);
  MOE_HIP(moe::launch_dispatch_bwd(is_bf16_rows(d), dxd, dxd_scales(d, dxd), row_of, topk_idx, dlogits, w_r, dx,
                                   r.t0, r.t1, d->k, d->E, d->H, (int64_t)d->H * elem_size(d->dtype),
                                   (hipStream_t)stream),
          "dispatch_bwd");
  return MOE_OK;
}

moe_status moe_quantize_rows_fp8(int64_t rows, int32_t cols, const void* src_bf16, void* codes, float* scale,
                                 void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8) return fail(MOE_ERR_ARG, "rows/cols invalid (cols %% 8 == 0 required)");
  if (rows == 0) return MOE_OK;
  MOE_NEED(src_bf16); MOE_NEED(codes); MOE_NEED(scale);
  MOE_HIP(moe::launch_quantize_rows_fp8(src_bf16, codes, scale, rows, cols, (hipStream_t)stream),
          "quantize_rows_fp8");
  return MOE_OK;
}

moe_status moe_quantize_cols_fp8(int64_t batch, int64_t rows, int32_t cols, const void* src_bf16, void* codes_t,
                                 float* scale, void* stream) {
  if (batch < 0 || rows < 0 || rows % 16 || cols <= 0 || cols % 8)
    return fail(MOE_ERR_ARG, "batch/rows/cols invalid (rows %% 16 == 0 and cols %% 8 == 0 required)");
  if (batch > 65535) return fail(MOE_ERR_UNSUPPORTED, "batch = %lld above 65535", (long long)batch);
  if (batch == 0 || rows == 0) return MOE_OK;
  MOE_NEED(src_bf16); MOE_NEED(codes_t); MOE_NEED(scale);
  MOE_HIP(moe::launch_quantize_cols_fp8(src_bf16, codes_t, scale, batch, rows, cols, (hipStream_t)stream),
          "quantize_cols_fp8");
  return MOE_OK;
}

// ----------------------------------------------------------------------------- paged stash

static moe_status check_stash(const char* fn, const void* rows, const void* pool, const void* scale_a,
                              const void* scale_b, int64_t live_rows, int64_t row_bytes, int64_t num_pages,
                              int64_t page_rows, const int32_t* pages, int32_t max_ctas) {
  if (live_rows < 0 || num_pages < 0) return fail(MOE_ERR_ARG, "%s: negative live_rows or num_pages", fn);
  if (row_bytes <= 0 || row_bytes % 16) return fail(MOE_ERR_ARG, "%s: row_bytes = %lld is not a positive multiple of 16", fn, (long long)row_bytes);
  if (page_rows < 1) return fail(MOE_ERR_ARG, "%s: page_rows = %lld below 1", fn, (long long)page_rows);
  if (max_ctas < 0) return fail(MOE_ERR_ARG, "%s: max_ctas = %d is negative", fn, max_ctas);
  if ((scale_a == nullptr) != (scale_b == nullptr))
    return fail(MOE_ERR_ARG, "%s: the two scale pointers must both be NULL or both be set", fn);
  if (live_rows == 0) return MOE_OK;
  if (!rows || !pool || !pages) return fail(MOE_ERR_ARG, "%s: a tensor, pool or page-table pointer is NULL", fn);
  if (((uintptr_t)rows | (uintptr_t)pool) & 15) return fail(MOE_ERR_ARG, "%s: tensor and pool must be 16-byte aligned", fn);
  if (num_pages > (INT64_MAX / 2) / page_rows / row_bytes || live_rows > (INT64_MAX / 2) / row_bytes)
    return fail(MOE_ERR_ARG, "%s: pool or tensor size overflows 64-bit offsets", fn);
  if ((live_rows + page_rows - 1) / page_rows > INT32_MAX) return fail(MOE_ERR_ARG, "%s: too many pages", fn);
  return MOE_OK;
}

moe_status moe_stash_store(const void* src, const float* src_scale, int64_t live_rows, int64_t row_bytes,
                           void* pool, float* pool_scale, int64_t num_pages, int64_t page_rows,
                           const int32_t* pages, int32_t* page_meta, int32_t owner, int32_t max_ctas,
                           void* stream) {
  MOE_TRY(check_stash(__func__, src, pool, src_scale, pool_scale, live_rows, row_bytes, num_pages, page_rows,
                      pages, max_ctas));
  if (live_rows == 0) return MOE_OK;
  MOE_HIP(moe::launch_stash_copy(true, src, src_scale, pool, pool_scale, live_rows, row_bytes, num_pages,
                                 page_rows, pages, page_meta, owner, max_ctas ? max_ctas : 2048,
                                 (hipStream_t)stream),
          "stash_store");
  return MOE_OK;
}

moe_status moe_stash_load(const void* pool, const float* pool_scale, int64_t live_rows, int64_t row_bytes,
                          int64_t num_pages, int64_t page_rows, const int32_t* pages, void* dst,
                          float* dst_scale, int32_t* recycled, int32_t max_ctas, void* stream) {
  MOE_TRY(check_stash(__func__, dst, pool, pool_scale, dst_scale, live_rows, row_bytes, num_pages, page_rows,
                      pages, max_ctas));
  if (live_rows == 0) return MOE_OK;
  MOE_HIP(moe::launch_stash_copy(false, pool, pool_scale, dst, dst_scale, live_rows, row_bytes, num_pages,
                                 page_rows, pages, recycled, 0, max_ctas ? max_ctas : 2048,
                                 (hipStream_t)stream),
          "stash_load");
  return MOE_OK;
}

// ----------------------------------------------------------------------------- layer primitives

static moe_status check_fwd_tensors(const moe_desc* d, const moe_tensors* t) {
  if (!t) return fail(MOE_ERR_ARG, "tensors is NULL");
  MOE_NEED(t->counts); MOE_NEED(t->offsets); MOE_NEED(t->workspace);
  if (d->T > 0) {
    MOE_NEED(t->x); MOE_NEED(t->topk_idx); MOE_NEED(t->gates); MOE_NEED(t->row_of);
    if (!t->logits && !t->w_r)
      return fail(MOE_ERR_ARG, "layer: logits and w_r are both NULL (one of them routes the tokens)");
    MOE_NEED(t->out);
  }
  if ((int64_t)d->n_chunks * d->P_c > 0) MOE_NEED(t->src_token);  // rows past N_c are marked -1
  if (rows_of(d) > 0) {
    MOE_NEED(t->w1); MOE_NEED(t->w2); MOE_NEED(t->xd); MOE_NEED(t->h); MOE_NEED(t->yd);
    if (d->dtype == MOE_FP8_E4M3) { MOE_NEED(t->xd_scale); MOE_NEED(t->h_scale); MOE_NEED(t->w1_scale); MOE_NEED(t->w2_scale); }
  }
  return MOE_OK;
}

static moe_status check_bwd_tensors(const moe_desc* d, const moe_tensors* t) {
  MOE_TRY(no_fp8_bwd(d));
  MOE_TRY(bwd_extent(d));
  MOE_NEED(t->w_r); MOE_NEED(t->dwr_acc); MOE_NEED(t->dwr);
  if (d->T > 0) { MOE_NEED(t->dy); MOE_NEED(t->dgates); MOE_NEED(t->dlogits); MOE_NEED(t->dx); }
  if (rows_of(d) > 0) {
    MOE_NEED(t->gu); MOE_NEED(t->dyd); MOE_NEED(t->dgu); MOE_NEED(t->dxd); MOE_NEED(t->dw1); MOE_NEED(t->dw2);
    if (d->flags & MOE_FLAG_FP8_DGRAD) {
      MOE_NEED(t->w1t); MOE_NEED(t->w1t_scale); MOE_NEED(t->w2t); MOE_NEED(t->w2t_scale);
      MOE_NEED(t->dyd_q); MOE_NEED(t->dyd_scale); MOE_NEED(t->dgu_q); MOE_NEED(t->dgu_scale);
    }
    if (d->flags & MOE_FLAG_FP8_WGRAD) {
      MOE_NEED(t->dyd_t); MOE_NEED(t->dyd_cs); MOE_NEED(t->dgu_t); MOE_NEED(t->dgu_cs);
      MOE_NEED(t->xd_t); MOE_NEED(t->xd_cs); MOE_NEED(t->h_t); MOE_NEED(t->h_cs);
    }
  }
  return MOE_OK;
}

// Routing of one chunk in a layer primitive: from the given logits, or (logits NULL) from x and
// the router weight with the projection fused into the top-k.
static moe_status route_any(const moe_desc* d, int c, const moe_tensors* t, hipStream_t s) {
  if (t->logits || d->T == 0)
    return moe_route(d, c, t->logits, t->topk_idx, t->gates, t->counts, t->offsets, t->row_of, t->src_token,
                     t->workspace, s);
  return moe_route_x(d, c, t->x, t->w_r, nullptr, t->topk_idx, t->gates, t->counts, t->offsets, t->row_of,
                     t->src_token, t->workspace, s);
}

// Two-stream schedules. A wait of one stream on the other's event costs the waiting stream
// about as much as a kernel launch even when the event has already completed, so the compute
// stream waits only where it needs work of the auxiliary stream, and the work that nothing can
// overlap (the first chunk's routing and dispatch, the last chunk's combine, the first chunk's
// combine backward) runs on the compute stream itself. With one stream (cs == as) the issue order
// alone is a valid sequential order.
//
// Forward, n chunks:
//   compute: R0 D0 F0 | wait(disp1) F1 | ... | wait(disp n-1) F n-1, C n-1
//   aux:     wait(disp0) R1 D1 | wait(ffn0) C0, R2 D2 | wait(ffn1) C1, R3 D3 | ...
// Routing/dispatch of chunk c+1 overlaps the expert GEMMs of chunk c; combine c-1 overlaps F c.
// With `join` the compute stream finally waits for the auxiliary stream. Without it (the fused
// forward+backward) the last combine also runs on aux, beside the backward's first kernels.
static moe_status forward_sched(const moe_desc* d, const moe_tensors* t, hipStream_t cs, hipStream_t as,
                                bool join) {
  const int n = d->n_chunks;
  const bool two = cs != as && n > 1;
  hipEvent_t* ev = nullptr;
  MOE_TRY(events(2 * n + 1, &ev));
  hipEvent_t* disp = ev;       // n events: dispatch of chunk c done
  hipEvent_t* ffn = ev + n;    // n events: expert FFN of chunk c done
  hipEvent_t done = ev[2 * n];
  MOE_TRY(route_any(d, 0, t, cs));
  MOE_TRY(moe_dispatch(d, 0, t->x, t->row_of, t->xd, t->xd_scale, t->h_scale, cs));
  if (two) {
    MOE_HIP(hipEventRecord(disp[0], cs), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(as, disp[0], 0), "hipStreamWaitEvent");
  }
  for (int c = 0; c < n; ++c) {
    const hipStream_t side = two ? as : cs;
    if (c + 1 < n) {
      MOE_TRY(route_any(d, c + 1, t, side));
      MOE_TRY(moe_dispatch(d, c + 1, t->x, t->row_of, t->xd, t->xd_scale, t->h_scale, side));
      if (two) MOE_HIP(hipEventRecord(disp[c + 1], as), "hipEventRecord");
    }
    if (two && c >= 1) MOE_HIP(hipStreamWaitEvent(cs, disp[c], 0), "hipStreamWaitEvent");
    MOE_TRY(moe_expert_ffn(d, c, t->xd, t->xd_scale, t->w1, t->w1_scale, t->w2, t->w2_scale, t->offsets,
                           t->gu, t->h, t->h_scale, t->yd, cs));
    // combine on aux after this chunk's GEMMs; the last chunk's on compute when the forward
    // ends here (join), on aux when the backward follows (nothing there reads `out`)
    if (c + 1 < n || (two && !join)) {
      if (two) {
        MOE_HIP(hipEventRecord(ffn[c], cs), "hipEventRecord");
        MOE_HIP(hipStreamWaitEvent(as, ffn[c], 0), "hipStreamWaitEvent");
      }
      MOE_TRY(moe_combine(d, c, t->yd, t->gates, t->row_of, t->out, side));
    } else {
      MOE_TRY(moe_combine(d, c, t->yd, t->gates, t->row_of, t->out, cs));
    }
  }
  if (two && join) {
    MOE_HIP(hipEventRecord(done, as), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(cs, done, 0), "hipStreamWaitEvent");
  }
  return MOE_OK;
}

// Backward, n chunks (CB combine backward, RB route backward, DG expert dgrad, DB dispatch
// backward, W expert weight gradients):
//   compute: CB0 DG0 | wait(cb1) DG1 | ... | DG n-1, W, wait(done)
//   aux:     wait(cb0) CB1 RB0 wait(dg0) DB0 | CB2 RB1 wait(dg1) DB1 | ... | RB n-1 wait(dg n-1) DB n-1
// Route backward of chunk c runs in chunk order (the FP32 router-gradient sum is ordered), and
// every chunk's input-gradient work is issued before the weight-gradient GEMMs.
static moe_status backward_sched(const moe_desc* d, const moe_tensors* t, hipStream_t cs, hipStream_t as) {
  const int n = d->n_chunks;
  const bool two = cs != as;
  const hipStream_t side = two ? as : cs;
  hipEvent_t* ev = nullptr;
  MOE_TRY(events(4 * n + 3, &ev));
  // events [2n+1, 4n+3): distinct from the forward schedule's [0, 2n+1)
  hipEvent_t* cb = ev + 2 * n + 1;  // n events: combine backward of chunk c done
  hipEvent_t* dg = ev + 3 * n + 1;  // n events: expert dgrad of chunk c done
  hipEvent_t done = ev[4 * n + 1];
  hipEvent_t wq_done = ev[4 * n + 2];  // FP8 weight gradients: dyd, h, xd operands quantised
  // FP8 weight gradients: once every combine backward is issued, the auxiliary stream quantises
  // the operands that do not wait for the input gradients, beside the dgrad GEMMs
  const bool wq8 = (d->flags & MOE_FLAG_FP8_WGRAD) && rows_of(d) > 0;
  auto wgrad_operands = [&]() -> moe_status {
    MOE_HIP(moe::launch_wgrad_fp8_operands(t->dyd, t->xd, t->h, t->offsets, t->dyd_t, t->dyd_cs, t->xd_t, t->xd_cs,
                                           t->h_t, t->h_cs, d->H, d->I, d->E_local, d->n_chunks, d->P_c, side),
            "expert_wgrad_fp8");
    if (two) MOE_HIP(hipEventRecord(wq_done, side), "hipEventRecord");
    return MOE_OK;
  };
  // FP8 input gradients: combine backward also writes the e4m3 rows of dyd (H up to
  // kCombineQMaxH; above it the expert dgrad quantises the stored rows)
  const bool q = d->flags & MOE_FLAG_FP8_DGRAD;
  const bool qcb = q && d->H <= moe::kCombineQMaxH;
  auto combine_bwd = [&](int c, hipStream_t st) {
    return combine_bwd_impl(d, c, t->dy, t->yd, t->gates, t->row_of, t->dyd, t->dgates, qcb ? t->dyd_q : nullptr,
                            qcb ? t->dyd_scale : nullptr, st);
  };
  MOE_TRY(combine_bwd(0, cs));
  if (two) {
    MOE_HIP(hipEventRecord(cb[0], cs), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(as, cb[0], 0), "hipStreamWaitEvent");
  }
  if (wq8 && n == 1) MOE_TRY(wgrad_operands());
  for (int c = 0; c < n; ++c) {
    if (c + 1 < n) {
      MOE_TRY(combine_bwd(c + 1, side));
      if (two) MOE_HIP(hipEventRecord(cb[c + 1], as), "hipEventRecord");
      if (wq8 && c + 2 == n) MOE_TRY(wgrad_operands());
    }
    MOE_TRY(moe_route_bwd(d, c, t->dgates, t->gates, t->topk_idx, t->x, t->dlogits, t->dwr_acc, t->dwr,
                          t->workspace, side));
    if (two && c >= 1) MOE_HIP(hipStreamWaitEvent(cs, cb[c], 0), "hipStreamWaitEvent");
    if (q)
      MOE_TRY(expert_dgrad_fp8_impl(d, c, t->dyd, t->gu, t->w1t, t->w1t_scale, t->w2t, t->w2t_scale, t->offsets,
                                    t->dyd_q, t->dyd_scale, t->dgu, t->dgu_q, t->dgu_scale, t->dxd, !qcb, cs));
    else
      MOE_TRY(moe_expert_ffn_bwd(d, c, t->dyd, t->xd, t->gu, t->h, t->w1, t->w2, t->offsets, t->dgu, t->dxd,
                                 nullptr, nullptr, t->workspace, cs));
    if (two) {
      MOE_HIP(hipEventRecord(dg[c], cs), "hipEventRecord");
      MOE_HIP(hipStreamWaitEvent(as, dg[c], 0), "hipStreamWaitEvent");
    }
    MOE_TRY(moe_dispatch_bwd(d, c, t->dxd, t->row_of, t->topk_idx, t->dlogits, t->w_r, t->dx, side));
  }
  if (d->flags & MOE_FLAG_FP8_WGRAD) {
    if (wq8 && two) MOE_HIP(hipStreamWaitEvent(cs, wq_done, 0), "hipStreamWaitEvent");
    MOE_TRY(expert_wgrad_fp8_impl(d, t->dyd, t->dgu, t->xd, t->h, t->offsets, t->dyd_t, t->dyd_cs, t->dgu_t,
                                  t->dgu_cs, t->xd_t, t->xd_cs, t->h_t, t->h_cs, t->dw1, t->dw2, !wq8, cs));
  }
  else
    MOE_TRY(moe_expert_wgrad(d, t->dyd, t->dgu, t->xd, t->h, t->offsets, t->dw1, t->dw2, t->workspace, cs));
  if (two) {
    MOE_HIP(hipEventRecord(done, as), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(cs, done, 0), "hipStreamWaitEvent");
  }
  return MOE_OK;
}

// BF16 schedules with merged GEMM launches. A persistent GEMM launch leaves most CUs idle in
// its last round (the small last tiles of each expert), and every launch boundary costs a few µs;
// so the layer issues independent GEMMs of neighbouring steps as one launch: down of chunk c with
// gate/up of chunk c+1, and gate/up dgrad of chunk c with down dgrad of chunk c+1. Every tile
// computes exactly what the single launches compute, so the results are bitwise those of the
// stage calls. The weight gradients split by what they need: dW2 (dyd^T h, ready once every
// combine backward has run) shares a launch with the last chunk's gate/up dgrad, and dW1 (dgu^T
// xd) runs alone after it, beside the last chunk's dispatch backward (input gradients before the
// weight gradient that waits for them).
static moe::ExpertGemm expert_gemm(const moe_desc* d, const moe_tensors* t) {
  moe::ExpertGemm g{};
  g.xd = t->xd; g.w1 = t->w1; g.w2 = t->w2; g.gu = t->gu; g.h = t->h; g.yd = t->yd;
  g.dyd = t->dyd; g.dgu = t->dgu; g.dxd = t->dxd; g.dw1 = t->dw1; g.dw2 = t->dw2;
  g.offsets = t->offsets; g.H = d->H; g.I = d->I; g.El = d->E_local; g.n_chunks = d->n_chunks; g.P_c = d->P_c;
  g.wgrad_ws = wgrad_ws(d, t->workspace);
  g.dxd_scales = dxd_scales(d, t->dxd);
  return g;
}

static bool merged_gemms(const moe_desc* d) { return d->dtype == MOE_BF16 && d->T > 0 && rows_of(d) > 0; }
// the merged backward launches pair BF16 GEMMs; with an FP8 GEMM flag the backward runs per chunk (FP8
// dxd rows only change the gate/up dgrad's epilogue and dispatch backward, both in the merged launches)
static bool merged_bwd(const moe_desc* d) { return merged_gemms(d) && (d->flags & ~MOE_FLAG_FP8_DXD) == 0; }

//   compute: R0 D0 GU0 | wait(disp1) [DN0 GU1] | wait(disp2) [DN1 GU2] | ... | DN n-1, C n-1
//   aux:     wait(disp0) R1 D1 | R2 D2, wait(ffn0) C0 | R3 D3, wait(ffn1) C1 | ...
// and with two streams, when the token rows fit one buffer descriptor (gate/up reading x through
// src_token):
//   compute: R(all) GU0 | [DN0 GU1] | [DN1 GU2] | ... | DN n-1
//   aux:     wait(routed) D(all) | wait(ffn0) C0 | wait(ffn1) C1 | ... | wait(ffn n-1) C n-1
// defer_last (fused primitive, two streams): the aux stream waits for the last chunk's GEMMs but
// leaves that chunk's combine to the backward schedule, which issues it after the next combine
// backward (nothing in the step reads `out`).
static moe_status forward_sched_merged(const moe_desc* d, const moe_tensors* t, hipStream_t cs, hipStream_t as,
                                       bool join, bool defer_last = false) {
  const int n = d->n_chunks;
  const bool two = cs != as && n > 1;
  const hipStream_t side = two ? as : cs;
  const moe::ExpertGemm g = expert_gemm(d, t);
  hipEvent_t* ev = nullptr;
  MOE_TRY(events(2 * n + 1, &ev));
  hipEvent_t* disp = ev;
  hipEvent_t* ffn = ev + n;
  hipEvent_t done = ev[2 * n];
  auto route_dispatch = [&](int c, hipStream_t s) -> moe_status {
    MOE_TRY(route_any(d, c, t, s));
    MOE_TRY(moe_dispatch(d, c, t->x, t->row_of, t->xd, t->xd_scale, t->h_scale, s));
    return MOE_OK;
  };
  // With two streams the gate/up GEMMs read their rows straight from x through src_token: the
  // compute stream routes every chunk in one launch and then runs the expert GEMMs without waiting
  // for the auxiliary stream, which dispatches every chunk meanwhile (xd, which the backward and the
  // caller read). No forward kernel on the compute stream reads xd; the forward's final join (layer
  // forward) or the backward's first wait on the auxiliary stream (fused step; the kernels before
  // it read dyd and G/U only) orders every later reader after the dispatch.
  const bool gather = two && (int64_t)d->T * d->H * 2 <= kRsrcMax;
  if (gather) {
    MOE_TRY(route_any(d, -1, t, cs));
    MOE_HIP(hipEventRecord(disp[0], cs), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(as, disp[0], 0), "hipStreamWaitEvent");
    MOE_TRY(moe_dispatch(d, -1, t->x, t->row_of, t->xd, t->xd_scale, t->h_scale, as));
    MOE_HIP(moe::gg_gateup_gather(g, 0, t->x, t->src_token, d->T, cs), "expert_ffn");
  } else {
    MOE_TRY(route_dispatch(0, cs));
    if (two) {
      MOE_HIP(hipEventRecord(disp[0], cs), "hipEventRecord");
      MOE_HIP(hipStreamWaitEvent(as, disp[0], 0), "hipStreamWaitEvent");
    }
    if (n > 1) {
      MOE_TRY(route_dispatch(1, side));
      if (two) MOE_HIP(hipEventRecord(disp[1], as), "hipEventRecord");
    }
    MOE_HIP(moe::gg_gateup(g, 0, cs), "expert_ffn");
  }
  for (int c = 0; c < n; ++c) {
    if (c + 1 < n && gather) {
      MOE_HIP(moe::gg_down_then_gateup_gather(g, c, c + 1, t->x, t->src_token, d->T, cs), "expert_ffn");
    } else if (c + 1 < n) {
      if (two) MOE_HIP(hipStreamWaitEvent(cs, disp[c + 1], 0), "hipStreamWaitEvent");
      MOE_HIP(moe::gg_down_then_gateup(g, c, c + 1, cs), "expert_ffn");
      if (c + 2 < n) {
        MOE_TRY(route_dispatch(c + 2, side));
        if (two) MOE_HIP(hipEventRecord(disp[c + 2], as), "hipEventRecord");
      }
    } else {
      MOE_HIP(moe::gg_down(g, c, cs), "expert_ffn");
    }
    if (c + 1 < n || (two && !join)) {
      if (two) {
        MOE_HIP(hipEventRecord(ffn[c], cs), "hipEventRecord");
        MOE_HIP(hipStreamWaitEvent(as, ffn[c], 0), "hipStreamWaitEvent");
      }
      if (!(two && defer_last && c + 1 == n)) MOE_TRY(moe_combine(d, c, t->yd, t->gates, t->row_of, t->out, side));
    } else {
      MOE_TRY(moe_combine(d, c, t->yd, t->gates, t->row_of, t->out, cs));
    }
  }
  if (two && join) {
    MOE_HIP(hipEventRecord(done, as), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(cs, done, 0), "hipStreamWaitEvent");
  }
  return MOE_OK;
}

//   compute: CB0 DDG0 | wait(cb1) [DDG1 GUDG0] | ... | [GUDG n-1, dW2], dW1, wait(done)
//   aux:     CB1 (C n-1) wait(cb0) RB0 | CB2 RB1 wait(dg0) DB0 | CB3 RB2 wait(dg1) DB1 | ... | wait(dg n-1) DB n-1
// (C n-1: the fused primitive's deferred last combine of the forward)
// deferred_combine: the forward left its last chunk's combine to this schedule (fused primitive);
// it runs on aux after chunk 1's combine backward.
static moe_status backward_sched_merged(const moe_desc* d, const moe_tensors* t, hipStream_t cs, hipStream_t as,
                                        bool deferred_combine = false) {
  const int n = d->n_chunks;
  const bool two = cs != as;
  const hipStream_t side = two ? as : cs;
  const moe::ExpertGemm g = expert_gemm(d, t);
  hipEvent_t* ev = nullptr;
  MOE_TRY(events(4 * n + 2, &ev));
  hipEvent_t* cb = ev + 2 * n + 1;
  hipEvent_t* dg = ev + 3 * n + 1;
  hipEvent_t done = ev[4 * n + 1];
  auto combine_bwd = [&](int c, hipStream_t s) {
    return moe_combine_bwd(d, c, t->dy, t->yd, t->gates, t->row_of, t->dyd, t->dgates, s);
  };
  auto route_bwd = [&](int c) {
    return moe_route_bwd(d, c, t->dgates, t->gates, t->topk_idx, t->x, t->dlogits, t->dwr_acc, t->dwr,
                         t->workspace, side);
  };
  MOE_TRY(combine_bwd(0, cs));
  if (two) MOE_HIP(hipEventRecord(cb[0], cs), "hipEventRecord");
  // chunk 1's combine backward does not need chunk 0's: aux starts it at once (the compute stream
  // waits for it before the next dgrad launch), then the forward's deferred combine, then waits
  // for chunk 0's combine backward, whose dgates route backward 0 reads
  if (n > 1) {
    MOE_TRY(combine_bwd(1, side));
    if (two) MOE_HIP(hipEventRecord(cb[1], as), "hipEventRecord");
  }
  if (deferred_combine) MOE_TRY(moe_combine(d, n - 1, t->yd, t->gates, t->row_of, t->out, side));
  if (two) MOE_HIP(hipStreamWaitEvent(as, cb[0], 0), "hipStreamWaitEvent");
  MOE_TRY(route_bwd(0));
  MOE_HIP(moe::gg_down_dgrad(g, 0, cs), "expert_dgrad");
  for (int c = 0; c < n; ++c) {
    if (c + 1 < n) {
      if (two) MOE_HIP(hipStreamWaitEvent(cs, cb[c + 1], 0), "hipStreamWaitEvent");
      MOE_HIP(moe::gg_gateup_dgrad_then_down_dgrad(g, c, c + 1, cs), "expert_dgrad");
    } else {
      MOE_HIP(moe::gg_gateup_dgrad_then_wgrad2(g, c, cs), "expert_dgrad");
    }
    if (two) MOE_HIP(hipEventRecord(dg[c], cs), "hipEventRecord");
    if (c + 1 < n) {
      if (c + 2 < n) {
        MOE_TRY(combine_bwd(c + 2, side));
        if (two) MOE_HIP(hipEventRecord(cb[c + 2], as), "hipEventRecord");
      }
      MOE_TRY(route_bwd(c + 1));
    }
    if (two) MOE_HIP(hipStreamWaitEvent(as, dg[c], 0), "hipStreamWaitEvent");
    MOE_TRY(moe_dispatch_bwd(d, c, t->dxd, t->row_of, t->topk_idx, t->dlogits, t->w_r, t->dx, side));
  }
  MOE_HIP(moe::gg_wgrad1(g, cs), "expert_wgrad");
  if (two) {
    MOE_HIP(hipEventRecord(done, as), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(cs, done, 0), "hipStreamWaitEvent");
  }
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_desc* d, const moe_tensors* t, void* compute_stream, void* aux_stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_fwd_tensors(d, t));
  if (merged_gemms(d)) return forward_sched_merged(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream, true);
  return forward_sched(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream, true);
}

moe_status moe_layer_backward(const moe_desc* d, const moe_tensors* t, void* compute_stream, void* aux_stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_fwd_tensors(d, t));
  MOE_TRY(check_bwd_tensors(d, t));
  if (merged_bwd(d)) return backward_sched_merged(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream);
  return backward_sched(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream);
}

moe_status moe_layer_forward_backward(const moe_desc* d, const moe_tensors* t, void* compute_stream,
                                      void* aux_stream) {
  MOE_TRY(validate(d));
  MOE_TRY(check_fwd_tensors(d, t));
  MOE_TRY(check_bwd_tensors(d, t));
  // no join between the two: the backward's first wait of the auxiliary stream follows the
  // whole forward on the compute stream, and its final join covers the forward's aux work
  // with both schedules merged and two streams (n > 1) the forward's last combine moves behind
  // chunk 1's combine backward on aux: that combine backward gates the compute stream's next
  // dgrad launch, the combine gates nothing in the step
  const bool defer = merged_gemms(d) && merged_bwd(d) && compute_stream != aux_stream && d->n_chunks > 1;
  if (merged_gemms(d))
    MOE_TRY(forward_sched_merged(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream, false, defer));
  else
    MOE_TRY(forward_sched(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream, false));
  if (merged_bwd(d))
    return backward_sched_merged(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream, defer);
  return backward_sched(d, t, (hipStream_t)compute_stream, (hipStream_t)aux_stream);
}

// ----------------------------------------------------------------------------- extent tracker

struct moe_extent_tracker {
  std::map<int64_t, int64_t> live;  // handle -> rows
  int64_t next = 1;
};

moe_extent_tracker* moe_extent_tracker_create(void) { return new (std::nothrow) moe_extent_tracker(); }
void moe_extent_tracker_destroy(moe_extent_tracker* tr) { delete tr; }

moe_status moe_extent_acquire(moe_extent_tracker* tr, int64_t rows, int64_t* handle) {
  if (!tr || !handle) return fail(MOE_ERR_ARG, "tracker or handle pointer is NULL");
  if (rows < 0) return fail(MOE_ERR_ARG, "rows = %lld is negative", (long long)rows);
  *handle = tr->next++;
  tr->live[*handle] = rows;
  return MOE_OK;
}

moe_status moe_extent_release(moe_extent_tracker* tr, int64_t handle) {
  if (!tr) return fail(MOE_ERR_ARG, "tracker is NULL");
  auto it = tr->live.find(handle);
  if (it == tr->live.end()) return fail(MOE_ERR_ARG, "handle %lld is not live", (long long)handle);
  tr->live.erase(it);
  return MOE_OK;
}

int64_t moe_extent_current(const moe_extent_tracker* tr, int64_t required_rows) {
  int64_t m = required_rows < 0 ? 0 : required_rows;
  if (tr)
    for (const auto& kv : tr->live) m = kv.second > m ? kv.second : m;
  return round4(m);
}

}  // extern "C"
