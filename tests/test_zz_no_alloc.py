"""The allocation-free routing entry point (moe_route_noalloc) against moe_route with a caller
workspace: bitwise the same outputs, on two calls in a row (the second with a smaller input that
reuses the library's fixed device scratch), over all chunks at once and chunk by chunk."""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")

KEYS = ("topk_idx", "gates", "counts", "offsets", "row_of", "src_token")


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()


def _route_both(cfg, logits, per_chunk):
    import torch
    import combine_moe_route_02_amd as mh
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0)
    lg = torch.from_numpy(logits).cuda()
    a = mh.allocate(d, backward=False, fill=-5)
    b = mh.allocate(d, backward=False, fill=-9)
    chunks = range(cfg.n_chunks) if per_chunk else [-1]
    for c in chunks:
        mh.moe_route(d, c, lg, a["topk_idx"], a["gates"], a["counts"], a["offsets"], a["row_of"], a["src_token"],
                     a["workspace"])
    for c in chunks:
        mh.moe_route_noalloc(d, c, lg, b["topk_idx"], b["gates"], b["counts"], b["offsets"], b["row_of"],
                             b["src_token"])
    torch.cuda.synchronize()
    for k in KEYS:
        np.testing.assert_array_equal(harness.bits_np(a[k]), harness.bits_np(b[k]), err_msg=k)
    return b


CASES = [
    (MoeConfig("share16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="bf16",
               seed_base=250), False),
    (MoeConfig("small_n3", T=1000, H=256, I=192, E=32, E_local=8, e0=4, k=4, n_chunks=3, dtype="bf16",
               seed_base=20), True),
]


def test_noalloc_route_matches_workspace_route_on_consecutive_calls():
    _require_gpu()
    import oracle
    for cfg, per_chunk in CASES:
        print(f"[noalloc] {cfg.name} per_chunk={per_chunk}", flush=True)
        logits = moe_inputs.make_inputs(cfg, parts=("logits",))["logits"]
        b = _route_both(cfg, logits, per_chunk)
        # and the oracle's integers
        idx, _ = oracle.route(logits, cfg.k)
        np.testing.assert_array_equal(b["topk_idx"].cpu().numpy(), idx)


def test_noalloc_route_rejects_sizes_past_its_scratch():
    _require_gpu()
    import combine_moe_route_02_amd as mh
    d = mh.make_desc(T=65536, H=128, I=64, E=1024, E_local=8, k=2, n_chunks=1, dtype="bf16")
    with pytest.raises(mh.MoeError) as ei:
        mh.moe_route_noalloc(d, -1, 1, 1, 1, 1, 1, 1, 1)
    assert ei.value.status == -3 and "scratch" in str(ei.value)
