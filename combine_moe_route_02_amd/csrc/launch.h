// Internal kernel launchers (host side). Every launcher enqueues on `s` and returns the HIP
// launch status; none allocates memory or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// routing
int route_blocks_per_chunk(int64_t T, int n);
int64_t route_scratch_bytes(int64_t T, int n, int E);
// the allocation-free routing variant's scratch: a file-scope device array of this many bytes per
// GPU; route_noalloc_scratch gives its address on the current device
constexpr int64_t kNoAllocRouteScratchBytes = 4 << 20;
hipError_t route_noalloc_scratch(void** out);
// routing from x: logits = x . W_r^T (BF16 MFMA, FP32 accumulation) fused with the top-k, then
// the layout kernel; logits may be NULL. Needs E % 32 == 0, E <= 256.
hipError_t launch_route_x(const void* x, const void* w_r, float* logits, int32_t* topk_idx, float* gates,
                          int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_token,
                          int32_t* scratch, int64_t T, int E, int H, int e0, int El, int K, int n, int chunk0,
                          int nchunks, int64_t P_c, hipStream_t s);
hipError_t launch_route(const float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* src_token, int32_t* scratch,
                        int64_t T, int E, int e0, int El, int K, int n, int chunk0, int nchunks,
                        int64_t P_c, hipStream_t s);

// row copies
hipError_t launch_dispatch(const void* x, const int32_t* row_of, void* xd, int64_t t0, int64_t t1,
                           int K, int64_t row_bytes, hipStream_t s);
hipError_t launch_dispatch_fp8(const void* x, const int32_t* row_of, void* xd, float* xd_scale,
                               float* h_scale, int64_t t0, int64_t t1, int K, int H, hipStream_t s);
hipError_t launch_quantize_rows_fp8(const void* src, void* codes, float* scale, int64_t rows,
                                    int cols, hipStream_t s);
hipError_t launch_combine(bool bf16, const void* yd, const float* gates, const int32_t* row_of,
                          void* out, int64_t t0, int64_t t1, int K, int64_t row_bytes, hipStream_t s);
constexpr int kCombineQMaxH = 8192;  // combine backward quantises dyd rows up to this H
hipError_t launch_combine_bwd(bool bf16, const void* dy, const void* yd, const float* gates,
                              const int32_t* row_of, void* dyd, float* dgates, int64_t t0,
                              int64_t t1, int K, int64_t row_bytes, hipStream_t s,
                              void* dyd_q = nullptr, float* dyd_scale = nullptr);  // BF16: also e4m3 rows
// dl_hi / dl_lo (nullable): also the rows' BF16 high and low parts, row t - t0 at t * pitch, ldl
// columns each (zeros past E)
hipError_t launch_route_bwd_dlogits(const float* dgates, const float* gates, const int32_t* idx,
                                    float* dlogits, int64_t t0, int64_t t1, int K, int E,
                                    hipStream_t s, uint16_t* dl_hi = nullptr, uint16_t* dl_lo = nullptr,
                                    int ldl = 0, int64_t pitch = 0);
// dxd_scales non-null: dxd holds block-scaled e4m3 rows (codes [., H], one FP32 scale per row
// and 256-column block, dxd_scales [., ceil(H/256)]); BF16 payloads only
hipError_t launch_dispatch_bwd(bool bf16, const void* dxd, const float* dxd_scales, const int32_t* row_of,
                               const int32_t* idx, const float* dlogits, const void* w_r, void* dx, int64_t t0,
                               int64_t t1, int K, int E, int H, int64_t row_bytes, hipStream_t s);

// grouped GEMMs
hipError_t launch_expert_fwd(bool bf16, const void* xd, const void* w1, const void* w2,
                             const int32_t* offsets, void* gu, void* h, void* yd, int H, int I,
                             int El, int c0, int nc, int64_t P_c, hipStream_t s);
// FP8: h holds [P, I] BF16 values followed by [P, I] e4m3 codes (P = n_chunks * P_c)
hipError_t launch_expert_fwd_fp8(const void* xd, const float* xd_scale, const void* w1,
                                 const float* w1_scale, const void* w2, const float* w2_scale,
                                 const int32_t* offsets, void* h, float* h_scale, void* yd, int H,
                                 int I, int El, int c0, int nc, int64_t P_c, int64_t P, hipStream_t s);
// per-row e4m3 quantisation of the BF16 rows [c*P_c, c*P_c + N_c) of chunks c0..c0+nc-1
hipError_t launch_quantize_segments_fp8(const char* name, const void* src, void* codes, float* scale,
                                        const int32_t* offsets, int El, int c0, int nc, int64_t P_c,
                                        int cols, hipStream_t s);
// per-column e4m3 quantisation of batch x [rows, cols] BF16, codes stored transposed [batch, cols, rows]
// per-expert, per-column e4m3 quantisation of dispatch rows, stored transposed and zero-padded (expert_k)
hipError_t launch_quantize_expert_cols_fp8(const char* name, const void* src, void* codes, float* scale,
                                           const int32_t* offsets, int El, int n_chunks, int64_t P_c, int64_t cols,
                                           hipStream_t s);
// the FP8 weight gradients' operands that do not depend on dgu (dyd, h, xd)
hipError_t launch_wgrad_fp8_operands(const void* dyd, const void* xd, const void* h, const int32_t* offsets,
                                     void* dyd_t, float* dyd_cs, void* xd_t, float* xd_cs, void* h_t, float* h_cs,
                                     int H, int I, int El, int n, int64_t P_c, hipStream_t s);
// FP8 expert weight gradients (dyd, h, xd quantised first unless `quantize` is false; dgu always)
hipError_t launch_expert_wgrad_fp8(const void* dyd, const void* dgu, const void* xd, const void* h,
                                   const int32_t* offsets, void* dyd_t, float* dyd_cs, void* dgu_t,
                                   float* dgu_cs, void* xd_t, float* xd_cs, void* h_t, float* h_cs, void* dw1,
                                   void* dw2, int H, int I, int El, int n, int64_t P_c, hipStream_t s,
                                   bool quantize = true);
hipError_t launch_quantize_cols_fp8(const void* src, void* codes_t, float* scale, int64_t batch, int64_t rows,
                                    int64_t cols, hipStream_t s);
// FP8 input gradients of the expert FFN for chunks c0..c0+nc-1: dyd quantised per row, dh on FP8
// MFMA against the transposed per-column-quantised W2 (w2t [El][I][H]), the SwiGLU gradient -> dgu
// (BF16), dgu quantised per row, dxd on FP8 MFMA against w1t [El][H][2I]
hipError_t launch_expert_dgrad_fp8(const void* dyd, const void* gu, const void* w1t, const float* w1t_scale,
                                   const void* w2t, const float* w2t_scale, const int32_t* offsets,
                                   void* dyd_q, float* dyd_scale, void* dgu, void* dgu_q, float* dgu_scale,
                                   void* dxd, float* dxd_scales, int H, int I, int El, int c0, int nc, int64_t P_c,
                                   hipStream_t s, bool quantize_dyd = true);  // false: dyd_q/dyd_scale written
// dxd_scales non-null (BF16 only): dxd is written as block-scaled e4m3 rows (see launch_dispatch_bwd)
hipError_t launch_expert_dgrad(bool bf16, const void* dyd, const void* gu, const void* w1,
                               const void* w2, const int32_t* offsets, void* dgu, void* dxd, float* dxd_scales,
                               int H, int I, int El, int c0, int nc, int64_t P_c, hipStream_t s);
hipError_t launch_expert_wgrad(bool bf16, const void* dyd, const void* dgu, const void* xd,
                               const void* h, const int32_t* offsets, void* dw1, void* dw2, int H,
                               int I, int El, int n, int64_t P_c, void* wgrad_ws, hipStream_t s);
// BF16 grouped GEMMs on the direct-to-LDS MFMA engine (grouped_gemm.hip)
hipError_t gg_expert_fwd_bf16(const void* xd, const void* w1, const void* w2, const int32_t* offsets,
                              void* gu, void* h, void* yd, int H, int I, int El, int c0, int nc,
                              int64_t P_c, hipStream_t s);
hipError_t gg_expert_dgrad_bf16(const void* dyd, const void* gu, const void* w1, const void* w2,
                                const int32_t* offsets, void* dgu, void* dxd, float* dxd_scales, int H, int I,
                                int El, int c0, int nc, int64_t P_c, hipStream_t s);
hipError_t gg_expert_wgrad_bf16(const void* dyd, const void* dgu, const void* xd, const void* h,
                                const int32_t* offsets, void* dw1, void* dw2, int H, int I, int El,
                                int n, int64_t P_c, void* wgrad_ws, hipStream_t s);
// Operands of the BF16 expert GEMMs as the layer schedule launches them (device pointers; the
// ones a launch does not use may be NULL).
struct ExpertGemm {
  const void* xd; const void* w1; const void* w2; void* gu; void* h; void* yd;
  const void* dyd; void* dgu; void* dxd; void* dw1; void* dw2;
  const int32_t* offsets;
  int H, I, El, n_chunks;
  int64_t P_c;
  void* wgrad_ws;  // weight-gradient scratch (counters zero between launches), wgrad_scratch_bytes
  float* dxd_scales;  // non-null: dxd holds block-scaled e4m3 codes [P, H] and these scales [P, ceil(H/256)]
};
// Expert-GEMM scratch (ExpertGemm::wgrad_ws): a zeroed counter area, then the weight gradients'
// partial tiles. The counter area holds the per-(expert, 256 x 256 tile) arrival counters of dW1
// and of dW2, then four work-queue blocks of kQueueInts counters: the split dW1 and dW2 lists,
// and the first and second row-grouped list of a layer launch. Every launch leaves them zero.
inline int64_t wgrad_tiles_1(int H, int I) { return (int64_t)((2 * I + 255) / 256) * ((H + 255) / 256); }
inline int64_t wgrad_tiles_2(int H, int I) { return (int64_t)((H + 255) / 256) * ((I + 255) / 256); }
constexpr int kQueueInts = 16;
constexpr int kQueueBlocks = 4;
enum { kQueueWgrad1 = 0, kQueueWgrad2 = 1, kQueueRows1 = 2, kQueueRows2 = 3 };
inline int* gemm_queue(const ExpertGemm& g, int which) {
  if (!g.wgrad_ws || g.El <= 0) return nullptr;
  return (int*)g.wgrad_ws + (int64_t)g.El * (wgrad_tiles_1(g.H, g.I) + wgrad_tiles_2(g.H, g.I)) + which * kQueueInts;
}
// weight-gradient scratch: its size, and the bytes of its leading counters (zero when first used)
int64_t wgrad_scratch_bytes(int H, int I, int El);
int64_t wgrad_counter_bytes_of(int H, int I, int El);
// One chunk's gate/up (+SwiGLU) or down GEMM; down of chunk c and gate/up of chunk c2 in one
// persistent launch (independent work: the second fills the first's last round).
hipError_t gg_gateup(const ExpertGemm& g, int c, hipStream_t s);
// gate/up of chunk c reading its operand rows straight from the token rows x [T, H] through
// src_token (no dispatched copy needed; T * H * 2 bytes must fit one buffer descriptor)
hipError_t gg_gateup_gather(const ExpertGemm& g, int c, const void* x, const int32_t* src_token, int64_t T,
                            hipStream_t s);
hipError_t gg_down(const ExpertGemm& g, int c, hipStream_t s);
hipError_t gg_down_then_gateup(const ExpertGemm& g, int c, int c2, hipStream_t s);
// the same, the gate/up tiles reading chunk c2's token rows from x through src_token
hipError_t gg_down_then_gateup_gather(const ExpertGemm& g, int c, int c2, const void* x, const int32_t* src_token,
                                      int64_t T, hipStream_t s);
// Input gradients: down dgrad (+SwiGLU backward) of chunk c, and gate/up dgrad of chunk c with
// down dgrad of chunk c2 in one launch.
hipError_t gg_down_dgrad(const ExpertGemm& g, int c, hipStream_t s);
hipError_t gg_gateup_dgrad_then_down_dgrad(const ExpertGemm& g, int c, int c2, hipStream_t s);
// Weight gradients split by what they need: dW2 = sum dyd^T h needs no input-gradient GEMM and
// shares a launch with the last chunk's gate/up dgrad; dW1 = sum dgu^T xd follows alone.
hipError_t gg_gateup_dgrad_then_wgrad2(const ExpertGemm& g, int c, hipStream_t s);
hipError_t gg_wgrad1(const ExpertGemm& g, hipStream_t s);
// paged activation stash (stash.hip): store = rows -> pool pages, else pool pages -> rows
hipError_t launch_stash_copy(bool store, const void* from, const float* from_scale, void* to,
                             float* to_scale, int64_t live_rows, int64_t row_bytes, int64_t num_pages,
                             int64_t page_rows, const int32_t* pages, int32_t* record, int32_t owner,
                             int32_t max_ctas, hipStream_t s);
int router_ksplit(int64_t tokens);
int64_t router_partials_bytes(int64_t Tc, int E, int H);
// BF16 rows: the BF16 high/low planes of dlogits ([tokens, ldl], from route_bwd_dlogits) feed the
// engine kernel (router_wgrad.hip); FP32 rows: the SIMT kernel reads dlogits
hipError_t launch_router_wgrad(bool bf16, const float* dlogits, const uint16_t* dl_hi, const uint16_t* dl_lo,
                               int ldl, const void* x, float* partials, float* dwr_acc, bool first, void* dwr,
                               int64_t t0, int64_t t1, int E, int H, hipStream_t s);
hipError_t launch_router_wgrad_planes(const uint16_t* hi, const uint16_t* lo, int ldl, const void* x, float* partials,
                                      int64_t t0, int64_t len, int ks, int S, int E, int H, hipStream_t s);
// The router gradient's dlogits planes: ld columns per plane (zeros past E). Up to 128 experts the
// high and low parts sit side by side in one [tokens, 256] matrix (low part at column 128), which
// one 256 x 256 GEMM tile reads whole; above 128 they are two [tokens, ld] planes.
inline int router_plane_ld(int E) { return E <= 128 ? 128 : (E + 7) / 8 * 8; }
inline int64_t router_plane_pitch(int E) { return E <= 128 ? 256 : router_plane_ld(E); }
inline int64_t router_plane_lo_offset(int E, int64_t tokens) { return E <= 128 ? 128 : tokens * router_plane_ld(E); }

}  // namespace moe
