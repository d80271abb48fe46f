/*
 * moe.h -- C ABI of one GPU's share of a Mixture-of-Experts layer on MI355X (gfx950).
 *
 * The layer share is: top-k routing over FP32 router logits, dispatch of token rows into
 * expert-contiguous rows, a grouped SwiGLU expert FFN, and combine (gate-weighted
 * gather-reduce back to token order into a fresh [P_out, H] output cropped to the logical
 * rows), forward and backward, processed in token-wise chunks.
 *
 * Sources (the pages the operation comes from; they print no formula, so each call states the
 * reading it implements):
 *   - token-wise ChunkedEP, Megatron-LM PR 7342, "Summary": three primitives (forward,
 *     backward, fused forward/backward), caller-owned output and dgrad buffers, tokens split
 *     into chunks so one chunk's dispatch overlaps another chunk's expert compute;
 *     "Numerical status -- unresolved": router weight gradients accumulate across chunks in
 *     FP32 before a single dtype conversion; "Tests and limitations": no router auxiliary loss.
 *   - "Price HybridEP recompute outputs at the live communication extent", OpenPipe/ART PR 971
 *     (description and review comments): combine writes a fresh [P, H] output at the live
 *     communication extent, rounded up to four rows, cropped to the logical rows by the caller;
 *     while an earlier larger graph is live its extent is kept as a high-water mark.
 *   - torchtitan PR 5541 (paged stash for HybridEP), "AI-Generated Details": multi-row tiles,
 *     tail masks and 64-bit addressing for BF16/FP8 row payloads.
 *   - "[graph_trainer] Overlap HybridEP and paging across combined PP graphs" (torchtitan
 *     PR 5542), "Verification": input-gradient work is issued before expert weight gradients.
 *
 * Conventions for every call below
 *   - Pointers named as device buffers are device (HBM) addresses, caller-owned; the library
 *     never allocates device memory and never synchronises the host. `stream` is a hipStream_t
 *     passed as void* (NULL = the null stream).
 *   - Host-side validation happens before any launch: on MOE_ERR_ARG, MOE_ERR_CAPACITY or
 *     MOE_ERR_UNSUPPORTED nothing was launched. MOE_ERR_HIP reports a failing HIP call; a call
 *     that issues several kernels (chunk = -1, the layer primitives) may have queued the ones
 *     before it. moe_last_error() returns a thread-local message for every non-OK status.
 *   - `chunk` selects one token chunk c in [0, n_chunks), or -1 for every chunk in order.
 *     Chunk c holds tokens [c*Tc, min(T, (c+1)*Tc)) with Tc = ceil(T / n_chunks), and owns the
 *     dispatch rows [c*P_c, (c+1)*P_c).
 *   - All arrays are row-major and dense. Element types depend on desc.dtype:
 *        tensor                         MOE_F32   MOE_BF16   MOE_FP8_E4M3 (forward only)
 *        x, dy, dx, W_r, dwr            f32       bf16       bf16 (x), -
 *        xd                             f32       bf16       e4m3 codes + xd_scale f32 [P]
 *        W1, W2                         f32       bf16       e4m3 codes + w1_scale [E_l,2I],
 *                                                            w2_scale [E_l,H] (f32)
 *        gu, h, yd, dyd, dgu, dxd       f32       bf16       h: [P,I] bf16 then [P,I] e4m3 codes
 *                                                            (3*P*I bytes), h_scale f32 [P]; yd bf16
 *        out                            f32       bf16       bf16
 *        dw1, dw2                       f32       bf16       -
 *     logits, gates, dgates, dlogits, dwr_acc are always f32; every index array is int32.
 *   - Shapes: logits [T,E]; topk_idx, gates, row_of, dgates [T,k]; counts [n,E];
 *     offsets [n,E_l+1]; src_token [P]; xd, yd, dyd, dxd [P,H]; gu, dgu [P,2I]; h [P,I];
 *     out [P_out,H]; W1, dw1 [E_l,2I,H] (rows 0..I-1 gate, I..2I-1 up); W2, dw2 [E_l,H,I];
 *     W_r, dwr, dwr_acc [E,H]; dlogits [T,E]; with P = n_chunks * P_c.
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* null pointer, bad chunk index, inconsistent shape */
  MOE_ERR_CAPACITY = -2,    /* P_c / P_out not a multiple of 4 or below the static minimum */
  MOE_ERR_UNSUPPORTED = -3, /* shape or dtype outside what the kernels handle */
  MOE_ERR_HIP = -4          /* a HIP launch/runtime error; message in moe_last_error() */
} moe_status;

/* Layer-share descriptor.
 *   T         logical tokens on this GPU (>= 0)
 *   H, I      hidden and expert intermediate size (multiples of 64)
 *   E         router width (all experts, 1..1024); e0, E_local: local experts [e0, e0+E_local)
 *   k         top-k (1..8, <= E)
 *   n_chunks  token-wise chunks (>= 1)
 *   P_c       dispatch rows per chunk region: multiple of 4, >= ceil(T/n)*min(k, E_local)
 *             (the static worst case, so no count ever returns to the host)
 *   P_out     combine output rows: multiple of 4, >= T (rows T..P_out-1 are never written)
 *   dtype     moe_dtype of the payloads (table above)
 *   flags     MOE_FLAG_* bits, 0 for the default path; an unknown bit is MOE_ERR_ARG */
typedef struct moe_desc {
  int64_t T;
  int32_t H, I, E, e0, E_local, k, n_chunks;
  int64_t P_c;
  int64_t P_out;
  int32_t dtype;
  int32_t flags;
} moe_desc;

/* Input gradients of the expert FFN on FP8 MFMA (moe_expert_dgrad_fp8) in the layer backward;
 * BF16 dtype only (MOE_ERR_UNSUPPORTED otherwise). */
#define MOE_FLAG_FP8_DGRAD 1
/* Expert weight gradients on FP8 MFMA (moe_expert_wgrad_fp8) in the layer backward; BF16 dtype
 * only. Independent of MOE_FLAG_FP8_DGRAD. */
#define MOE_FLAG_FP8_WGRAD 2
/* FP8 payload of dispatch backward (the token-row payload formats of torchtitan PR 5541,
 * "AI-Generated Details", applied to the backward's token rows); BF16 dtype only,
 * independent of the other two flags. The expert input-gradient calls (moe_expert_ffn_bwd,
 * moe_expert_dgrad_fp8 and the layer primitives) then write dxd as block-scaled e4m3 rows and
 * moe_dispatch_bwd reads them: the dxd buffer ([n_chunks * P_c, H] BF16-sized, caller-owned) holds
 * the codes [n_chunks * P_c, H] (one byte each) from its start, then one FP32 scale per row and
 * block of 256 columns ([n_chunks * P_c, ceil(H / 256)]). Each block is the BF16-rounded dxd values
 * quantised with the row quantiser's FP32 steps (amax over the block; codes RNE(v * (448 / amax))
 * saturated; scale amax / 448; an all-zero block stores codes 0 and scale 1). dx is the FP32 sum of
 * code * scale over the token's local slots plus the router term, rounded once to BF16. */
#define MOE_FLAG_FP8_DXD 4

/* ---------------------------------------------------------------------------------------
 * Stage calls
 * ------------------------------------------------------------------------------------- */

/* Routing (ChunkedEP "Summary": top-k routing per token chunk; no auxiliary loss).
 * Per token: the k largest logits (ties to the lower expert index, NaN ranks lowest), slot 0
 * the largest; gates = softmax over the k selected logits (= full softmax, top-k,
 * renormalise). counts[c][e] = slots of chunk c choosing expert e (all E experts);
 * offsets[c] = exclusive prefix sum over the local experts' counts, offsets[c][E_l] = N_c;
 * row_of[t][j] = c*P_c + offsets[c][e-e0] + (number of earlier tokens of chunk c choosing e),
 * -1 for a non-local expert; src_token[row] = the row's token, -1 for rows N_c..P_c-1.
 * workspace: device scratch of moe_workspace_bytes().route_scratch bytes (contents undefined
 * on return). Bit-exact and deterministic (no order-dependent atomics). */
moe_status moe_route(const moe_desc* d, int chunk, const float* logits, int32_t* topk_idx,
                     float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                     int32_t* src_token, void* workspace, void* stream);

/* Routing without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): moe_route with the same
 * arguments and bitwise the same outputs, but its histogram scratch is a fixed 4 MiB device array
 * inside the library (one per GPU, held until the process ends). It allocates nothing and
 * returns MOE_ERR_UNSUPPORTED when the call needs more than that scratch:
 * n_chunks * ceil(ceil(T/n_chunks)/64) * 4 * E * 4 bytes > 4 MiB (at E = 128, more than 131072
 * tokens). Every call on one GPU shares the array, so calls that overlap on one GPU (different
 * streams, or other host threads) race: order them on one stream or synchronise between them. */
moe_status moe_route_noalloc(const moe_desc* d, int chunk, const float* logits, int32_t* topk_idx,
                             float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                             int32_t* src_token, void* stream);

/* Routing from the token activations (the router projection fused into routing): logits =
 * x . W_r^T with BF16 x [T,H] and W_r [E,H], FP32 accumulation on MFMA, then the top-k of
 * moe_route on those logits, which stay in registers and LDS; `logits` (nullable, FP32 [T,E])
 * receives them. Every other argument and output is moe_route's. Needs a BF16 or FP8 descriptor
 * (x is BF16 in both) and E a multiple of 32, at most 256 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_route_x(const moe_desc* d, int chunk, const void* x, const void* w_r, float* logits,
                       int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                       int32_t* src_token, void* workspace, void* stream);

/* Dispatch (ChunkedEP "Summary": each token chunk's rows go to the experts before that chunk's
 * expert compute; torchtitan PR 5541 "AI-Generated Details": BF16/FP8 token-row payloads):
 * xd[row_of[t][j]] = x[t] for every local slot (a bitwise row copy for F32/BF16;
 * each touched token row is read once). FP8: per token amax over the BF16 row,
 * xd = e4m3(x * (448/amax)) with FP32 steps, RNE, saturating; xd_scale[row] = amax/448 (1 for
 * an all-zero row); h_scale[row] is cleared (moe_expert_ffn writes it). Rows N_c..P_c-1 are not
 * written. xd_scale/h_scale may be NULL unless dtype is FP8. */
moe_status moe_dispatch(const moe_desc* d, int chunk, const void* x, const int32_t* row_of,
                        void* xd, float* xd_scale, float* h_scale, void* stream);

/* Expert compute of a chunk (ChunkedEP "Summary": the expert FFN runs per token chunk, beside the
 * next chunk's dispatch). Grouped SwiGLU expert FFN over every local expert's rows [c*P_c + offsets[c][e],
 * c*P_c + offsets[c][e+1]): G = xd W1g^T, U = xd W1u^T (FP32 accumulation),
 * h = silu(G) * U with silu(z) = z/(1+exp(-z)), yd = h W2^T. gu (may be NULL) saves G and U
 * for the backward ([P,2I], G in columns 0..I-1). h is required ([P,I]). FP8: both GEMMs run on
 * FP8 MFMA with FP32 accumulation dequantised by s_row*s_col; h is written in BF16, then each
 * dispatch row of h is quantised to e4m3 (per-row absmax, the FP32 steps of moe_dispatch) into
 * the codes half of the h buffer with its scale in h_scale, and the down projection reads the
 * codes. gu is unused for FP8. */
moe_status moe_expert_ffn(const moe_desc* d, int chunk, const void* xd, const float* xd_scale,
                          const void* w1, const float* w1_scale, const void* w2,
                          const float* w2_scale, const int32_t* offsets, void* gu, void* h,
                          float* h_scale, void* yd, void* stream);

/* Combine (ART PR 971: fresh [P, H] output cropped to the logical rows):
 * out[t] = RNE( sum over local slots j, ascending, of gates[t][j] * yd[row_of[t][j]] ) with
 * FP32 accumulation; a token without a local expert gets a zero row. Writes rows of the chunk
 * only; rows T..P_out-1 are left untouched. */
moe_status moe_combine(const moe_desc* d, int chunk, const void* yd, const float* gates,
                       const int32_t* row_of, void* out, void* stream);

/* Combine backward (ChunkedEP "Summary": the backward primitive writes the caller's dgrad
 * buffers; ART PR 971: combine's output rows are the logical tokens, so only they carry dy):
 * dyd[row_of[t][j]] = gates[t][j] * dy[t] (rounded once to the payload type);
 * dgates[t][j] = <dy[t], yd[row_of[t][j]]> in FP32, 0 for non-local slots. */
moe_status moe_combine_bwd(const moe_desc* d, int chunk, const void* dy, const void* yd,
                           const float* gates, const int32_t* row_of, void* dyd, float* dgates,
                           void* stream);

/* Route backward (ChunkedEP "Numerical status": FP32 accumulation across chunks, then one
 * conversion). dlogits[t][idx[t][j]] = g_j * (dg_j - sum_i g_i dg_i), zero for unselected
 * experts (all E columns written for the chunk's rows). Router weight gradient of the
 * caller's projection logits = x W_r^T: the chunk's dlogits^T x is computed in FP32 (dlogits
 * split into a BF16 high and low part, x exact) and stored into dwr_acc for the first chunk,
 * added to it for later chunks; after the last chunk (or chunk = -1) dwr = dwr_acc converted
 * once (RNE) to the payload type. workspace: moe_workspace_bytes().route_bwd_scratch bytes
 * (the split-K partials and, for BF16 rows, the chunk's dlogits as BF16 high and low planes;
 * contents undefined between calls). */
moe_status moe_route_bwd(const moe_desc* d, int chunk, const float* dgates, const float* gates,
                         const int32_t* topk_idx, const void* x, float* dlogits, float* dwr_acc,
                         void* dwr, void* workspace, void* stream);

/* Expert FFN backward, input-gradient part (ChunkedEP "Summary": backward per token chunk;
 * torchtitan PR 5542 "Verification": input-gradient work is issued before the expert weight
 * gradients, which chunk = -1 runs last), per chunk: dh = dyd W2; with s = sigmoid(G):
 * dG = dh * U * s * (1 + G (1 - s)), dU = dh * silu(G) (G, U read from gu);
 * dxd = [dG dU] W1. With chunk = -1 it then runs moe_expert_wgrad over every chunk (workspace is
 * moe_expert_wgrad's; unused when chunk >= 0). */
moe_status moe_expert_ffn_bwd(const moe_desc* d, int chunk, const void* dyd, const void* xd,
                              const void* gu, const void* h, const void* w1, const void* w2,
                              const int32_t* offsets, void* dgu, void* dxd, void* dw1, void* dw2,
                              void* workspace, void* stream);

/* Expert weight gradients over the rows of every chunk in one FP32 reduction, converted once:
 * dW2[e] = sum_rows dyd^T h, dW1[e] = sum_rows dgu^T xd; an expert with no rows gets zeros
 * (ChunkedEP "Numerical status": FP32 accumulation across chunks before one conversion, read as
 * applying to every weight gradient). An expert holding many more rows than the others has its
 * row range split into parts whose FP32 partial tiles are summed in part order; the split depends
 * only on the per-expert row counts, so the result is deterministic. workspace: the
 * moe_workspace_bytes().workspace buffer (BF16 path); its first wgrad_zero_bytes bytes after the
 * wgrad offset (counters) must be zero when first used, and every call leaves them zero. */
moe_status moe_expert_wgrad(const moe_desc* d, const void* dyd, const void* dgu, const void* xd,
                            const void* h, const int32_t* offsets, void* dw1, void* dw2,
                            void* workspace, void* stream);

/* FP8 input gradients (a reading: ChunkedEP "Summary" gives FP8 for the dispatched payloads of
 * the forward only; the backward applies the same per-row quantisation to its payloads). Needs a
 * BF16 descriptor. Per chunk:
 *   dyd rows quantised per row into dyd_q [P,H] e4m3 / dyd_scale [P] (FP32 steps of moe_dispatch);
 *   dh = deq(dyd_q) deq(W2t)^T on FP8 MFMA (FP32 accumulation, s_row * s_col dequantisation);
 *   dG, dU as in moe_expert_ffn_bwd from the saved G, U (gu) -> dgu [P,2I] BF16;
 *   dgu rows quantised per row into dgu_q [P,2I] / dgu_scale [P];
 *   dxd = deq(dgu_q) deq(W1t)^T on FP8 MFMA -> BF16.
 * w2t [E_local][I][H] and w1t [E_local][H][2I] are the weights quantised per column and stored
 * transposed (moe_quantize_cols_fp8 of W2 [E_local][H][I] and W1 [E_local][2I][H]), with scales
 * w2t_scale [E_local][I] and w1t_scale [E_local][H]. dgu (BF16) is what moe_expert_wgrad then
 * reads. Rows N_c..P_c-1 of every output are not written. */
moe_status moe_expert_dgrad_fp8(const moe_desc* d, int chunk, const void* dyd, const void* gu,
                                const void* w1t, const float* w1t_scale, const void* w2t,
                                const float* w2t_scale, const int32_t* offsets, void* dyd_q,
                                float* dyd_scale, void* dgu, void* dgu_q, float* dgu_scale,
                                void* dxd, void* stream);

/* FP8 expert weight gradients (a reading: a weight gradient contracts over the expert's token rows,
 * so its operands are scaled per column over those rows). For every local expert e, its dispatch
 * rows of every chunk in chunk order are its K_e rows; dyd [P,H], h [P,I], dgu [P,2I] and xd [P,H]
 * (BF16) are each quantised per column over those rows (absmax, the FP32 steps of moe_dispatch) and
 * stored transposed, the rows contiguous and zero-padded to Kp_e = K_e rounded up to 64: with
 * koff_e the sum of Kp over the experts before e, column j of expert e starts at byte
 * koff_e * C + j * Kp_e of its *_t buffer (C its columns) and its scale is *_cs[e * C + j]. Then
 * dW2[e] = s * sum_k dyd_t h_t and dW1[e] = s * sum_k dgu_t xd_t on FP8 MFMA with FP32 accumulation,
 * dequantised by the two column scales, one BF16 store; an expert without rows gets zeros. Each
 * *_t buffer holds C * (n_chunks * P_c + 64 * E_local) bytes (moe_workspace_bytes). */
moe_status moe_expert_wgrad_fp8(const moe_desc* d, const void* dyd, const void* dgu, const void* xd,
                                const void* h, const int32_t* offsets, void* dyd_t, float* dyd_cs,
                                void* dgu_t, float* dgu_cs, void* xd_t, float* xd_cs, void* h_t,
                                float* h_cs, void* dw1, void* dw2, void* stream);

/* Dispatch backward (ChunkedEP "Summary": the backward returns each chunk's token gradients to
 * token order; the router term is the input gradient of the projection whose weight gradient
 * "Numerical status -- unresolved" accumulates): dx[t] = RNE( sum over local slots of dxd[row_of[t][j]]
 * + sum_j dlogits[t][idx[t][j]] * W_r[idx[t][j]] ) with FP32 accumulation (the second sum is
 * the router projection's input gradient; dlogits is zero off the selected experts). */
moe_status moe_dispatch_bwd(const moe_desc* d, int chunk, const void* dxd, const int32_t* row_of,
                            const int32_t* topk_idx, const float* dlogits, const void* w_r,
                            void* dx, void* stream);

/* FP8 weight quantisation (outside the timed path): per row of a [rows, cols] BF16 matrix,
 * codes = e4m3(w * (448/amax)) and scale = amax/448 with the FP32 steps of moe_dispatch. */
moe_status moe_quantize_rows_fp8(int64_t rows, int32_t cols, const void* src_bf16, void* codes,
                                 float* scale, void* stream);

/* Per-column FP8 quantisation, stored transposed (the weights of moe_expert_dgrad_fp8): for each of
 * `batch` BF16 matrices src [rows, cols] (row-major, contiguous), column j's absmax gives
 * scale[b][j] = amax/448 (1 for an all-zero column) and codes_t[b][j][i] = e4m3(src[b][i][j] *
 * (448/amax)) with the FP32 steps of moe_dispatch, so codes_t is [batch, cols, rows]. rows a
 * multiple of 16, cols a multiple of 8, batch <= 65535 (MOE_ERR_ARG / MOE_ERR_UNSUPPORTED). */
moe_status moe_quantize_cols_fp8(int64_t batch, int64_t rows, int32_t cols, const void* src_bf16,
                                 void* codes_t, float* scale, void* stream);

/* ---------------------------------------------------------------------------------------
 * Paged activation stash (torchtitan PR 5541, "AI-Generated Details": page-aligned multi-token
 * copy tiles, one page resolved per tile, the first tile of a page records or recycles it,
 * live-prefix and page-tail masks, 64-bit addressing, a bounded copy grid).
 *
 * A saved tensor is `live_rows` rows of `row_bytes` bytes (any payload: BF16, FP8 codes, FP32;
 * row_bytes a positive multiple of 16). The pool is `num_pages` pages of `page_rows` rows of
 * the same row_bytes, contiguous: page p starts at pool + p*page_rows*row_bytes. Logical page i
 * (tensor rows i*page_rows .. (i+1)*page_rows - 1) lives in physical page pages[i], for
 * i < ceil(live_rows / page_rows); the entries must be distinct. An entry outside
 * [0, num_pages) names no page: its rows are not copied (and nothing is written for it).
 * Only live rows move; rows of the last page past the live prefix keep their contents.
 * Optional FP32 per-row scales (FP8 payloads) are paged alongside: `*_scale` pointers are both
 * NULL or both set, pool scales [num_pages * page_rows].
 * The pool may be device memory or pinned host memory; src, dst and pool must be 16-byte
 * aligned. `max_ctas` caps the copy grid (0: 2048). Nothing is launched when live_rows is 0.
 * Errors: MOE_ERR_ARG for a NULL required pointer, misalignment, a negative size, row_bytes not
 * a positive multiple of 16, page_rows < 1, a scale pointer set without its pair. */

/* Store: pool rows <- tensor rows. page_meta (nullable, int32 [2 * num_pages]) receives, for every
 * logical page with a valid entry p: page_meta[2p] = owner, page_meta[2p+1] = its live rows. */
moe_status moe_stash_store(const void* src, const float* src_scale, int64_t live_rows, int64_t row_bytes,
                           void* pool, float* pool_scale, int64_t num_pages, int64_t page_rows,
                           const int32_t* pages, int32_t* page_meta, int32_t owner, int32_t max_ctas,
                           void* stream);
/* Load: tensor rows <- pool rows. recycled (nullable, int32 [ceil(live_rows / page_rows)])
 * receives the physical page of each logical page in order (-1 for an invalid entry). */
moe_status moe_stash_load(const void* pool, const float* pool_scale, int64_t live_rows, int64_t row_bytes,
                          int64_t num_pages, int64_t page_rows, const int32_t* pages, void* dst,
                          float* dst_scale, int32_t* recycled, int32_t max_ctas, void* stream);

/* ---------------------------------------------------------------------------------------
 * Layer primitives (ChunkedEP "Summary": forward, backward, fused forward/backward). They
 * own the two-stream chunk schedule: routing and dispatch of chunk c+1 on `aux` overlap the
 * expert GEMMs of chunk c on `compute`, and combine of chunk c runs on `aux` after them. The
 * first chunk's routing and dispatch, the last chunk's combine (on `aux` in the fused
 * forward+backward, where nothing after it reads `out`) and the first chunk's combine backward
 * run on `compute`, which waits on `aux` only where it consumes aux work. On return
 * all work is ordered before later work on `compute`. Both streams at the default priority;
 * with compute == aux everything runs in issue order on that one stream. With `logits` NULL the
 * forward routes from x and `w_r` (moe_route_x; BF16 or FP8 descriptor, E % 32 == 0, E <= 256).
 * The schedule's cross-stream dependencies use HIP events from a pool that the library creates
 * per host thread and device on first use and keeps until the process ends, so layer calls
 * issued from different threads never share events. Calls that share `workspace` or any saved-
 * context buffer must still be ordered by the caller.
 * With MOE_FLAG_FP8_DGRAD the backward runs moe_expert_dgrad_fp8 per chunk, and combine backward
 * also writes the e4m3 rows of dyd (H <= 8192; above that the dgrad quantises the stored rows);
 * t->w1t/w2t and their scales must hold the moe_quantize_cols_fp8 form of the current W1/W2. With
 * MOE_FLAG_FP8_WGRAD the weight gradients are moe_expert_wgrad_fp8's, whose dyd, h and xd operands
 * are quantised on `aux` once the last combine backward is issued.
 * ------------------------------------------------------------------------------------- */
typedef struct moe_tensors {
  /* inputs */
  const void* x; const float* logits; const void* w1; const float* w1_scale;
  const void* w2; const float* w2_scale; const void* w_r; const void* dy;
  /* routing state and saved context (caller-owned; kept between forward and backward) */
  int32_t* topk_idx; float* gates; int32_t* counts; int32_t* offsets; int32_t* row_of;
  int32_t* src_token; void* xd; float* xd_scale; void* gu; void* h; float* h_scale; void* yd;
  /* forward output: [P_out, H] */
  void* out;
  /* backward buffers and outputs */
  void* dyd; float* dgates; float* dlogits; float* dwr_acc; void* dgu; void* dxd;
  void* dx; void* dw1; void* dw2; void* dwr;
  /* scratch of moe_workspace_bytes().workspace bytes (its weight-gradient counters zero when first
   * used: see moe_workspace_sizes) */
  void* workspace;
  /* MOE_FLAG_FP8_DGRAD only (see moe_expert_dgrad_fp8): transposed FP8 weights and the quantised
   * backward payloads */
  const void* w1t; const float* w1t_scale; const void* w2t; const float* w2t_scale;
  void* dyd_q; float* dyd_scale; void* dgu_q; float* dgu_scale;
  /* MOE_FLAG_FP8_WGRAD only (see moe_expert_wgrad_fp8): the per-expert transposed FP8 operands */
  void* dyd_t; float* dyd_cs; void* dgu_t; float* dgu_cs; void* xd_t; float* xd_cs; void* h_t; float* h_cs;
} moe_tensors;

moe_status moe_layer_forward(const moe_desc* d, const moe_tensors* t, void* compute_stream,
                             void* aux_stream);
moe_status moe_layer_backward(const moe_desc* d, const moe_tensors* t, void* compute_stream,
                              void* aux_stream);
moe_status moe_layer_forward_backward(const moe_desc* d, const moe_tensors* t,
                                      void* compute_stream, void* aux_stream);

/* ---------------------------------------------------------------------------------------
 * Host-only helpers: they never initialise HIP.
 * ------------------------------------------------------------------------------------- */

/* Default extents: *P_c = round4(ceil(T/n) * min(k, E_local)), *P_out = round4(T * k). */
moe_status moe_required_extent(int64_t T, int32_t k, int32_t E_local, int32_t n_chunks,
                               int64_t* P_c, int64_t* P_out);

/* Bytes of every caller buffer for a descriptor (0 where the dtype does not use it). */
typedef struct moe_workspace_sizes {
  int64_t topk_idx, gates, counts, offsets, row_of, src_token;
  int64_t xd, xd_scale, gu, h, h_scale, yd, out;
  int64_t dyd, dgates, dlogits, dwr_acc, dgu, dxd, dx, dw1, dw2, dwr;
  int64_t route_scratch, route_bwd_scratch, workspace; /* workspace: see wgrad_scratch below */
  int64_t w1t, w1t_scale, w2t, w2t_scale, dyd_q, dyd_scale, dgu_q, dgu_scale; /* MOE_FLAG_FP8_DGRAD */
  int64_t dyd_t, dyd_cs, dgu_t, dgu_cs, xd_t, xd_cs, h_t, h_cs;              /* MOE_FLAG_FP8_WGRAD */
  /* the expert weight gradients' part of the workspace (BF16 path): it starts after the routing
   * and router scratch at a 256-byte boundary; its first wgrad_zero_bytes bytes are counters that
   * must be zero when the workspace is first used (every call leaves them zero) */
  int64_t wgrad_scratch, wgrad_zero_bytes;
} moe_workspace_sizes;
moe_status moe_workspace_bytes(const moe_desc* d, moe_workspace_sizes* out);

/* Live-extent tracker (ART PR 971): acquire() records a live graph's extent and returns a
 * handle; release() ends it; current(required) = round4(max(required, largest live extent)).
 * Not thread-safe per tracker. */
typedef struct moe_extent_tracker moe_extent_tracker;
moe_extent_tracker* moe_extent_tracker_create(void);
void moe_extent_tracker_destroy(moe_extent_tracker* tr);
moe_status moe_extent_acquire(moe_extent_tracker* tr, int64_t rows, int64_t* handle);
moe_status moe_extent_release(moe_extent_tracker* tr, int64_t handle);
int64_t moe_extent_current(const moe_extent_tracker* tr, int64_t required_rows);

/* Launch log and per-kernel timing (tracing; torchtitan PR 5542 "Verification" checks the issue
 * order of input-gradient work against weight-gradient GEMMs from a launch trace). After
 * moe_trace_enable(timing), every kernel the library launches from this thread is appended to
 * a thread-local log with its name and stream; with timing != 0 it is bracketed by two HIP
 * events on that stream. moe_trace_enable clears the log. moe_trace_entry returns entry i
 * (name: static string; ms: device duration, -1 without timing; waits for that entry's end
 * event). Tracing adds host work per launch; it is off by default. */
moe_status moe_trace_enable(int32_t timing);
/* As moe_trace_enable(1), but only launches whose name equals `only` (a NUL-terminated launch
 * name, copied) get timing events; the others are logged with ms = -1. Lets a caller time one
 * kernel kind with almost no instrumentation on the rest. MOE_ERR_ARG if `only` is NULL. */
moe_status moe_trace_enable_only(const char* only);
moe_status moe_trace_disable(void);
int64_t moe_trace_count(void);
moe_status moe_trace_entry(int64_t i, const char** name, void** stream, float* ms);
/* Timeline of a timed log: start and end of entry i in ms after the start of entry 0 (both
 * events are waited for). MOE_ERR_ARG for a bad index or NULL outputs, MOE_ERR_HIP without
 * timing. Entries on different streams give the overlap of their kernels. */
moe_status moe_trace_span(int64_t i, float* start_ms, float* end_ms);

/* Message for the last non-OK status on this thread ("" if none). */
const char* moe_last_error(void);
/* ABI version (incremented on any incompatible change). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
