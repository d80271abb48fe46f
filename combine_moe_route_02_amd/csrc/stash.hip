// Paged activation stash: saved rows (xd, gu, yd, ... of any payload) copied into fixed-size pages
// of a pool and back (torchtitan PR 5541, "AI-Generated Details": page-aligned multi-token tiles,
// one page resolved per tile, the first tile of a page records or recycles it, live-prefix and
// page-tail masks, 64-bit addressing, a bounded copy grid).
//
// A tile is up to kTileRows rows of one logical page, so each tile reads its page-table entry
// once (a scalar load) and all its addresses are one 64-bit base plus row/column offsets. Each
// 256-thread block walks tiles grid-stride; the grid is capped (max_ctas) so the copy can share the
// GPU with compute. Rows move as 16-byte vectors, a full tile's loads (eight rows) in flight per
// thread before their stores. The pool may be device memory or pinned host memory.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "trace.h"

namespace moe {
namespace {

constexpr int kStashThreads = 256;
constexpr int kTileRows = 8;

// Copy `rows` rows of nvec 16-byte vectors: src row i -> dst row i (row strides in vectors).
MOE_DEV void copy_rows(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int rows, int64_t nvec) {
  const int tid = threadIdx.x;
  int r = 0;
  for (; r + kTileRows <= rows; r += kTileRows) {
    for (int64_t v = tid; v < nvec; v += kStashThreads) {
      u32x4 a[kTileRows];
#pragma unroll
      for (int u = 0; u < kTileRows; ++u) a[u] = src[(int64_t)(r + u) * nvec + v];
#pragma unroll
      for (int u = 0; u < kTileRows; ++u) dst[(int64_t)(r + u) * nvec + v] = a[u];
    }
  }
  for (; r < rows; ++r)
    for (int64_t v = tid; v < nvec; v += kStashThreads) dst[(int64_t)r * nvec + v] = src[(int64_t)r * nvec + v];
}

// STORE: tensor rows -> pool pages (records written); else pool pages -> tensor rows (recycled).
template <bool STORE>
__global__ __launch_bounds__(kStashThreads) void stash_copy_kernel(
    const u32x4* __restrict__ from, const float* __restrict__ from_scale, u32x4* __restrict__ to,
    float* __restrict__ to_scale, int64_t live_rows, int64_t nvec, int64_t num_pages, int64_t page_rows,
    const int32_t* __restrict__ pages, int32_t* __restrict__ record, int32_t owner, int64_t tiles_per_page,
    int64_t ntiles) {
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t i = t / tiles_per_page, j = t % tiles_per_page;  // logical page, tile in page
    const int32_t p = pages[i];
    const bool valid = p >= 0 && p < num_pages;
    const int64_t page_live = min(page_rows, live_rows - i * page_rows);  // live rows of page i
    if (j == 0 && threadIdx.x == 0 && record) {
      if (STORE) {
        if (valid) { record[2 * (int64_t)p] = owner; record[2 * (int64_t)p + 1] = (int32_t)page_live; }
      } else {
        record[i] = valid ? p : -1;
      }
    }
    const int64_t q0 = j * kTileRows;  // first row of the tile within the page
    if (!valid || q0 >= page_live) continue;
    const int rows = (int)min((int64_t)kTileRows, page_live - q0);
    const int64_t trow = i * page_rows + q0;          // tensor row
    const int64_t prow = (int64_t)p * page_rows + q0;  // pool row
    const int64_t fr = STORE ? trow : prow, tr = STORE ? prow : trow;
    copy_rows(from + fr * nvec, to + tr * nvec, rows, nvec);
    if (from_scale && threadIdx.x < rows) to_scale[tr + threadIdx.x] = from_scale[fr + threadIdx.x];
  }
}

}  // namespace

hipError_t launch_stash_copy(bool store, const void* from, const float* from_scale, void* to,
                             float* to_scale, int64_t live_rows, int64_t row_bytes, int64_t num_pages,
                             int64_t page_rows, const int32_t* pages, int32_t* record, int32_t owner,
                             int32_t max_ctas, hipStream_t s) {
  const int64_t npages = (live_rows + page_rows - 1) / page_rows;
  const int64_t tpp = (min(page_rows, live_rows) + kTileRows - 1) / kTileRows;  // tiles per page
  const int64_t ntiles = npages * tpp;
  if (ntiles == 0) return hipSuccess;
  const int64_t grid = min(ntiles, (int64_t)max_ctas);
  const int64_t nvec = row_bytes / 16;
  if (store) {
    MOE_TRACE("stash_store", s);
    MOE_LAUNCH(stash_copy_kernel<true>, dim3((unsigned)grid), dim3(kStashThreads), 0, s,
                       (const u32x4*)from, from_scale, (u32x4*)to, to_scale, live_rows, nvec, num_pages,
                       page_rows, pages, record, owner, tpp, ntiles);
  } else {
    MOE_TRACE("stash_load", s);
    MOE_LAUNCH(stash_copy_kernel<false>, dim3((unsigned)grid), dim3(kStashThreads), 0, s,
                       (const u32x4*)from, from_scale, (u32x4*)to, to_scale, live_rows, nvec, num_pages,
                       page_rows, pages, record, owner, tpp, ntiles);
  }
  return hipGetLastError();
}

}  // namespace moe
