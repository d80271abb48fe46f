"""Paged activation stash: page-aligned stores of saved rows into a page pool and loads back.
Test infrastructure only (see the package docstring).

torchtitan PR 5541 ("AI-Generated Details") describes the copy kernel of its paged activation
stash: the copy loops work on page-aligned tiles of several tokens; each tile resolves one page;
only the first tile of a page records it (on a store) or recycles it (on a load); a live-prefix
mask and a page-tail mask keep the payload bytes exact; offsets are 64-bit; payloads are BF16 or
FP8. The plainest reading of that, written out here:

  * A tensor of rows (row_bytes bytes each, any payload) has a live prefix of `live_rows` rows.
  * Logical page i holds its rows i*page_rows .. (i+1)*page_rows - 1; it lives in physical page
    pages[i] of a pool of num_pages pages of page_rows rows.
  * store: pool row pages[r // page_rows] * page_rows + r % page_rows = src row r, for every live
    row r. Rows past the live prefix in the last page are left as they were (page-tail mask).
    With per-row FP32 scales (FP8 payloads) the scales follow the same mapping.
    Record of logical page i (when asked for): page_meta[2 p] = owner, page_meta[2 p + 1] = number
    of live rows in the page, where p = pages[i].
  * load: dst row r = the pool row above, for every live row r (rows past the prefix are left as
    they were); recycled[i] = pages[i] when asked for.
  * A page-table entry outside [0, num_pages) names no page: its rows are not copied, no record is
    written, and its recycled entry is -1.
"""
from __future__ import annotations

import numpy as np


def n_pages(live_rows: int, page_rows: int) -> int:
    """Logical pages that hold the live prefix."""
    return -(-int(live_rows) // int(page_rows))


def _valid(p: int, num_pages: int) -> bool:
    return 0 <= int(p) < int(num_pages)


def stash_store(src, live_rows, pool, page_rows, pages, num_pages, src_scale=None, pool_scale=None,
                page_meta=None, owner=0):
    """Copy the live rows of `src` ([rows, row_bytes] uint8) into `pool` ([num_pages*page_rows,
    row_bytes] uint8), in place. Returns nothing; every output array is updated in place."""
    for r in range(int(live_rows)):
        i, q = divmod(r, int(page_rows))
        p = int(pages[i])
        if not _valid(p, num_pages):
            continue
        pool[p * page_rows + q] = src[r]
        if src_scale is not None:
            pool_scale[p * page_rows + q] = src_scale[r]
    if page_meta is not None:
        for i in range(n_pages(live_rows, page_rows)):
            p = int(pages[i])
            if _valid(p, num_pages):
                page_meta[2 * p] = owner
                page_meta[2 * p + 1] = min(int(page_rows), int(live_rows) - i * int(page_rows))


def stash_load(pool, live_rows, page_rows, pages, num_pages, dst, pool_scale=None, dst_scale=None,
               recycled=None):
    """Copy the live rows back from `pool` into `dst` ([rows, row_bytes] uint8), in place."""
    for r in range(int(live_rows)):
        i, q = divmod(r, int(page_rows))
        p = int(pages[i])
        if not _valid(p, num_pages):
            continue
        dst[r] = pool[p * page_rows + q]
        if dst_scale is not None:
            dst_scale[r] = pool_scale[p * page_rows + q]
    if recycled is not None:
        for i in range(n_pages(live_rows, page_rows)):
            p = int(pages[i])
            recycled[i] = p if _valid(p, num_pages) else -1
