"""Pins for the paged-stash oracle (torchtitan PR 5541, "AI-Generated Details"): a worked
example listed by hand, the store/load round trip over random page tables, the page-tail and
live-prefix masks, page records, recycling order and invalid page-table entries."""
import numpy as np

from oracle import stash


def _rows(n, row_bytes, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(n, row_bytes), dtype=np.uint8)


def test_worked_example_listed_by_hand():
    # 5 live rows of 16 bytes, pages of 2 rows, logical pages -> physical [3, 0, 2] in a pool of 4
    src = np.arange(6 * 16, dtype=np.uint8).reshape(6, 16)
    pool = np.full((8, 16), 0xEE, dtype=np.uint8)
    meta = np.full(8, -7, dtype=np.int32)
    stash.stash_store(src, 5, pool, 2, np.array([3, 0, 2]), 4, page_meta=meta, owner=9)
    expected = np.full((8, 16), 0xEE, dtype=np.uint8)
    expected[6] = src[0]   # logical page 0 -> physical page 3, slots 0, 1
    expected[7] = src[1]
    expected[0] = src[2]   # logical page 1 -> physical page 0
    expected[1] = src[3]
    expected[4] = src[4]   # logical page 2 -> physical page 2, slot 0; slot 1 (pool row 5) untouched
    np.testing.assert_array_equal(pool, expected)
    np.testing.assert_array_equal(meta, [9, 2, -7, -7, 9, 1, 9, 2])
    dst = np.full((6, 16), 0x11, dtype=np.uint8)
    rec = np.full(3, -5, dtype=np.int32)
    stash.stash_load(pool, 5, 2, np.array([3, 0, 2]), 4, dst, recycled=rec)
    np.testing.assert_array_equal(dst[:5], src[:5])
    np.testing.assert_array_equal(dst[5], np.full(16, 0x11, dtype=np.uint8))  # past the live prefix
    np.testing.assert_array_equal(rec, [3, 0, 2])


def test_round_trip_over_random_page_tables():
    rng = np.random.default_rng(1)
    for trial in range(20):
        page_rows = int(rng.integers(1, 40))
        live = int(rng.integers(0, 300))
        npg = stash.n_pages(live, page_rows)
        num_pages = npg + int(rng.integers(0, 5))
        pages = rng.permutation(num_pages)[:npg].astype(np.int32)
        row_bytes = 16 * int(rng.integers(1, 9))
        src = _rows(live + 3, row_bytes, trial)
        scale = rng.standard_normal(live + 3).astype(np.float32)
        pool = _rows(num_pages * page_rows, row_bytes, 100 + trial)
        pool0 = pool.copy()
        pscale = np.zeros(num_pages * page_rows, dtype=np.float32)
        stash.stash_store(src, live, pool, page_rows, pages, num_pages, scale, pscale)
        # pages outside the table are untouched; inside, exactly the live slots changed
        used = np.zeros(num_pages * page_rows, dtype=bool)
        for r in range(live):
            used[pages[r // page_rows] * page_rows + r % page_rows] = True
        np.testing.assert_array_equal(pool[~used], pool0[~used])
        dst = np.zeros_like(src)
        dscale = np.zeros_like(scale)
        stash.stash_load(pool, live, page_rows, pages, num_pages, dst, pscale, dscale)
        np.testing.assert_array_equal(dst[:live], src[:live])
        np.testing.assert_array_equal(dscale[:live], scale[:live])
        assert not dst[live:].any() and not dscale[live:].any()


def test_page_counts_and_tail():
    assert stash.n_pages(0, 8) == 0 and stash.n_pages(1, 8) == 1 and stash.n_pages(8, 8) == 1
    assert stash.n_pages(9, 8) == 2
    meta = np.zeros(2 * 6, dtype=np.int32)
    src = _rows(20, 16, 3)
    pool = np.zeros((6 * 8, 16), dtype=np.uint8)
    stash.stash_store(src, 20, pool, 8, np.array([5, 1, 4]), 6, page_meta=meta, owner=-3)
    assert meta[2 * 5 + 1] == 8 and meta[2 * 1 + 1] == 8 and meta[2 * 4 + 1] == 4   # 20 = 8 + 8 + 4
    assert meta[10] == meta[2] == meta[8] == -3


def test_invalid_page_entries_are_skipped():
    src = _rows(6, 16, 4)
    pool = np.zeros((3 * 2, 16), dtype=np.uint8)
    meta = np.full(6, 7, dtype=np.int32)
    stash.stash_store(src, 6, pool, 2, np.array([2, -1, 3]), 3, page_meta=meta)
    np.testing.assert_array_equal(pool[4:6], src[0:2])
    assert not pool[:4].any()
    np.testing.assert_array_equal(meta, [7, 7, 7, 7, 0, 2])
    rec = np.zeros(3, dtype=np.int32)
    dst = np.zeros_like(src)
    stash.stash_load(pool, 6, 2, np.array([2, -1, 3]), 3, dst, recycled=rec)
    np.testing.assert_array_equal(rec, [2, -1, -1])
    np.testing.assert_array_equal(dst[0:2], src[0:2])
    assert not dst[2:].any()
