"""GPU parity of routing where the tie and special-value rules decide the integers.

Top-k selection is on the FP32 logits: slot 0 holds the largest, equal logits go to the lower
expert index, NaN ranks as -inf and -0 equals +0 (the reading of token-wise ChunkedEP,
Megatron-LM PR 7342, "Summary", which names top-k routing and no tie rule). The inputs here are
logits rounded to multiples of 0.5, so exact ties are everywhere, including between the k-th and
(k+1)-th largest logit of most rows, with zeros of both signs, NaN entries, an all-zero row and a
row whose last selected slot falls among -inf and NaN entries. The kernel's top-k indices,
counts, offsets, row_of and src_token must equal the oracle's bit for bit and the gates must
agree within 1e-6, through the stage call and through the layer primitive, at small shapes, at
the 16K-token one-rank share, and on chunks long enough for the scanned layout (more than 128
blocks of 64 tokens)."""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()


def _tie_stats(lg, k):
    key = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    s = -np.sort(-key, axis=1)
    return {"kth_tie_rows": int(np.count_nonzero(s[:, k - 1] == s[:, k])) if lg.shape[1] > k else 0,
            "nan": int(np.count_nonzero(np.isnan(lg))),
            "neg_zero": int(np.count_nonzero((lg == 0) & np.signbit(lg))),
            "pos_zero": int(np.count_nonzero((lg == 0) & ~np.signbit(lg)))}


TIE_SMALL = [
    MoeConfig("tie_rag", T=1000, H=256, I=192, E=32, E_local=8, e0=4, k=4, n_chunks=2, dtype="bf16",
              seed_base=500, backward=True),
    MoeConfig("tie_k8_n3", T=777, H=128, I=64, E=64, E_local=16, e0=16, k=8, n_chunks=3, dtype="bf16",
              seed_base=510, backward=True),
    MoeConfig("tie_e8_k2", T=300, H=128, I=64, E=8, E_local=8, k=2, n_chunks=1, dtype="bf16", seed_base=520,
              backward=True),
    MoeConfig("tie_e1024", T=513, H=128, I=64, E=1024, E_local=64, e0=960, k=8, n_chunks=2, dtype="bf16",
              seed_base=530, backward=True),
    MoeConfig("tie_odd_e", T=400, H=128, I=64, E=30, E_local=6, e0=0, k=5, n_chunks=2, dtype="f32",
              seed_base=540, backward=True),
]


def _route_only(cfg, lg):
    """moe_route (chunk = -1) on the given logits; returns the device buffers."""
    import torch
    import combine_moe_route_02_amd as mh
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0)
    b = mh.allocate(d, backward=False, fill=-5)
    b["logits"] = torch.from_numpy(lg).cuda()
    mh.moe_route(d, -1, b["logits"], b["topk_idx"], b["gates"], b["counts"], b["offsets"], b["row_of"],
                 b["src_token"], b["workspace"])
    torch.cuda.synchronize()
    return d, b


def _check_route(cfg, d, b, lg):
    import oracle
    idx, gates = oracle.route(lg, cfg.k)
    counts, offsets, row_of, src = oracle.layout(idx, cfg.E, cfg.e0, cfg.E_local, cfg.n_chunks, int(d.P_c))
    for name, want in (("topk_idx", idx), ("counts", counts), ("offsets", offsets), ("row_of", row_of),
                       ("src_token", src)):
        got = b[name].cpu().numpy()
        assert got.shape == want.shape, name
        bad = np.count_nonzero(got != want)
        assert bad == 0, f"{cfg.name} {name}: {bad} of {got.size} entries differ"
    g = b["gates"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    err = float(np.max(np.abs(g - gates))) if g.size else 0.0
    assert err <= 1e-6, f"{cfg.name} gates: max abs {err:.3e}"
    return idx


@pytest.mark.parametrize("cfg", TIE_SMALL, ids=[c.name for c in TIE_SMALL])
def test_route_stage_ties_nan_signed_zero(cfg):
    _require_gpu()
    lg = moe_inputs.make_tie_logits(cfg)
    st = _tie_stats(lg, cfg.k)
    print(f"[ties] {cfg.name} {st}", flush=True)
    assert st["kth_tie_rows"] > cfg.T // 4 and st["nan"] > 0 and st["neg_zero"] > 0 and st["pos_zero"] > 0
    d, b = _route_only(cfg, lg)
    idx = _check_route(cfg, d, b, lg)
    # the all-zero row picks experts 0..k-1 in order; the second row ends on the lowest-index
    # -inf/NaN expert after its k - 1 finite values
    np.testing.assert_array_equal(idx[0], np.arange(cfg.k))
    fin = np.flatnonzero(np.isfinite(lg[1]))
    assert set(idx[1, :cfg.k - 1].tolist()) == set(fin.tolist())
    assert idx[1, cfg.k - 1] == np.flatnonzero(~np.isfinite(lg[1]))[0]
    assert b["gates"].cpu().numpy()[1, cfg.k - 1] == 0.0


def test_route_ties_do_not_depend_on_sign_of_zero_or_nan_payload():
    """Flipping the sign of every zero logit, or swapping NaN for -inf, changes no integer output
    (the keys treat -0 as +0 and NaN as -inf)."""
    _require_gpu()
    cfg = TIE_SMALL[1]
    lg = moe_inputs.make_tie_logits(cfg)
    _, b0 = _route_only(cfg, lg)
    lg2 = lg.copy()
    z = lg2 == 0
    lg2[z] = np.where(np.signbit(lg2[z]), np.float32(0.0), np.float32(-0.0))
    lg2[np.isnan(lg2)] = -np.inf
    _, b1 = _route_only(cfg, lg2)
    for name in ("topk_idx", "counts", "offsets", "row_of", "src_token", "gates"):
        np.testing.assert_array_equal(harness.bits_np(b0[name]), harness.bits_np(b1[name]), err_msg=name)


@pytest.mark.parametrize("cfg", TIE_SMALL[:3], ids=[c.name for c in TIE_SMALL[:3]])
def test_layer_with_tied_logits_matches_oracle(cfg):
    """The fused layer primitive on tie-heavy logits: integers bitwise, values within the BF16
    bounds, forward and backward."""
    _require_gpu()
    inp = moe_inputs.make_inputs(cfg)
    inp["logits"] = moe_inputs.make_tie_logits(cfg)
    run = harness.run_gpu(cfg, inp=inp, sentinel=-7.0)
    ref = harness.run_oracle(run)
    print("[ties layer]", cfg.name, harness.check_forward(run, ref, sentinel=-7.0),
          harness.check_backward(run, ref), flush=True)


def test_full_16k_tied_logits_routing_bitwise():
    """The 16K-token one-rank share (two chunks of 8192, 16 of 128 experts, top-8) routed on
    tie-heavy logits through the fused layer primitive: integers bitwise, forward values within
    the BF16 bounds."""
    _require_gpu()
    cfg = moe_inputs.CONFIGS["fb16k"]
    inp = moe_inputs.make_inputs(cfg, with_backward=False)
    inp["logits"] = moe_inputs.make_tie_logits(cfg)
    st = _tie_stats(inp["logits"], cfg.k)
    print(f"[ties 16k] {st}", flush=True)
    assert st["kth_tie_rows"] > cfg.T // 2
    run = harness.run_gpu(cfg, inp=inp, backward=False, sentinel=-3.0)
    ref = harness.run_oracle(run, backward=False)
    print("[ties 16k fwd]", harness.check_forward(run, ref, sentinel=-3.0), flush=True)
    # the stage call gives the same integers
    d, b = _route_only(cfg, inp["logits"])
    _check_route(cfg, d, b, inp["logits"])


LONG_CHUNKS = [
    # chunks of more than 128 64-token blocks take the scanned layout (route_scan, then the
    # layout reads each block's prefix); one just past the switch, one chunk, and a long one
    MoeConfig("long_n1_8256", T=8256, H=128, I=64, E=64, E_local=16, e0=8, k=8, n_chunks=1, dtype="bf16",
              seed_base=570),
    MoeConfig("long_n2_40000", T=40000, H=128, I=64, E=128, E_local=16, e0=112, k=8, n_chunks=2, dtype="bf16",
              seed_base=580),
    MoeConfig("long_n3_zipf", T=30001, H=128, I=64, E=32, E_local=8, e0=0, k=6, n_chunks=3, dtype="bf16",
              seed_base=590, zipf_s=1.2, n_empty=2),
]


@pytest.mark.parametrize("cfg", LONG_CHUNKS, ids=[c.name for c in LONG_CHUNKS])
def test_route_long_chunks_scanned_layout(cfg):
    """Routing of long chunks (the scanned layout) on tie-heavy and on Zipf-biased logits:
    integers bitwise against the oracle."""
    _require_gpu()
    for lg in (moe_inputs.make_tie_logits(cfg), moe_inputs.make_inputs(cfg, parts=("logits",))["logits"]):
        d, b = _route_only(cfg, lg)
        nbpc = -(-(-(-cfg.T // cfg.n_chunks)) // 64)
        assert nbpc > 128, nbpc
        print(f"[long] {cfg.name} blocks per chunk {nbpc}", flush=True)
        _check_route(cfg, d, b, lg)
