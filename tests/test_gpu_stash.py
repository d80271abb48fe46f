"""GPU parity of the paged activation stash (moe_stash_store / moe_stash_load) against the oracle,
bitwise: pool contents, page records, reloaded rows, recycled pages. Cases cover tiles that cross
no page boundary but end mid-page, pages not a multiple of the tile height, FP8-sized rows with
per-row scales, a one-block grid (grid-stride over every tile), a pinned host pool, invalid
page-table entries, an empty live prefix, and a chunk's dispatch-order rows at the bench size."""
import zlib

import numpy as np
import pytest

from oracle import stash as ostash

pytestmark = pytest.mark.gpu

CASES = [
    # name, live_rows, page_rows, row_bytes, spare pages, scales, max_ctas, host pool, bad entries
    ("bf16_rows", 1000, 64, 4096, 3, False, 0, False, 0),
    ("fp8_rows_scales", 777, 48, 7168, 2, True, 3, False, 0),
    ("tiny_one_block", 5, 2, 16, 1, True, 1, False, 0),
    ("page_not_tile_multiple", 301, 37, 1536, 0, False, 0, False, 0),
    ("host_pool", 300, 32, 512, 4, True, 0, True, 0),
    ("bad_entries", 400, 40, 256, 2, True, 0, False, 3),
    ("chunk_rows_bench_size", 8245, 256, 4096, 0, False, 2048, False, 0),
]


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()
    return torch, mh


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stash_store_load_bitwise(case):
    torch, mh = _require_gpu()
    name, live, page_rows, row_bytes, spare, scales, max_ctas, host_pool, bad = case
    print(f"[stash] {case}", flush=True)
    # a stable per-case seed (Python's str hash is salted per process)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    npg = ostash.n_pages(live, page_rows)
    num_pages = npg + spare
    pages = rng.permutation(num_pages)[:npg].astype(np.int32)
    for i in rng.choice(npg, size=min(bad, npg), replace=False):
        pages[i] = -1 if i % 2 else num_pages + int(i)
    src = rng.integers(0, 256, size=(live + 5, row_bytes), dtype=np.uint8)
    pool0 = rng.integers(0, 256, size=(num_pages * page_rows, row_bytes), dtype=np.uint8)
    sscale = rng.standard_normal(live + 5).astype(np.float32) if scales else None
    pscale0 = rng.standard_normal(num_pages * page_rows).astype(np.float32) if scales else None
    meta0 = np.full(2 * num_pages, -9, dtype=np.int32)

    # oracle
    pool_ref, pscale_ref, meta_ref = pool0.copy(), (pscale0.copy() if scales else None), meta0.copy()
    ostash.stash_store(src, live, pool_ref, page_rows, pages, num_pages, sscale, pscale_ref, meta_ref, owner=17)
    dst0 = rng.integers(0, 256, size=src.shape, dtype=np.uint8)
    dscale0 = rng.standard_normal(live + 5).astype(np.float32) if scales else None
    dst_ref, dscale_ref = dst0.copy(), (dscale0.copy() if scales else None)
    rec_ref = np.full(npg, 5, dtype=np.int32)
    ostash.stash_load(pool_ref, live, page_rows, pages, num_pages, dst_ref, pscale_ref, dscale_ref, rec_ref)

    # GPU
    dev = torch.device("cuda")
    g_src = torch.from_numpy(src).to(dev)
    if host_pool:
        g_pool = torch.from_numpy(pool0).pin_memory()
    else:
        g_pool = torch.from_numpy(pool0).to(dev)
    g_ps = torch.from_numpy(pscale0).to(dev) if scales else None
    g_ss = torch.from_numpy(sscale).to(dev) if scales else None
    g_pages = torch.from_numpy(pages).to(dev)
    g_meta = torch.from_numpy(meta0).to(dev)
    mh.moe_stash_store(g_src, g_ss, live, row_bytes, g_pool, g_ps, num_pages, page_rows, g_pages, g_meta,
                       owner=17, max_ctas=max_ctas)
    g_dst = torch.from_numpy(dst0).to(dev)
    g_ds = torch.from_numpy(dscale0).to(dev) if scales else None
    g_rec = torch.full((npg,), 5, dtype=torch.int32, device=dev)
    mh.moe_stash_load(g_pool, g_ps, live, row_bytes, num_pages, page_rows, g_pages, g_dst, g_ds, g_rec,
                      max_ctas=max_ctas)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g_pool.cpu().numpy(), pool_ref)
    np.testing.assert_array_equal(g_meta.cpu().numpy(), meta_ref)
    np.testing.assert_array_equal(g_dst.cpu().numpy(), dst_ref)
    np.testing.assert_array_equal(g_rec.cpu().numpy(), rec_ref)
    if scales:
        np.testing.assert_array_equal(g_ps.cpu().numpy().view(np.uint32), pscale_ref.view(np.uint32))
        np.testing.assert_array_equal(g_ds.cpu().numpy().view(np.uint32), dscale_ref.view(np.uint32))


def test_stash_empty_prefix_writes_nothing():
    torch, mh = _require_gpu()
    pool = torch.full((64, 32), 3, dtype=torch.uint8, device="cuda")
    dst = torch.full((8, 32), 4, dtype=torch.uint8, device="cuda")
    pages = torch.zeros(1, dtype=torch.int32, device="cuda")
    mh.moe_stash_store(dst, None, 0, 32, pool, None, 4, 16, pages)
    mh.moe_stash_load(pool, None, 0, 32, 4, 16, pages, dst)
    torch.cuda.synchronize()
    assert int((pool != 3).sum()) == 0 and int((dst != 4).sum()) == 0
