"""Determinism and stream-race checks of the two-stream layer primitives on the GPU.

* Ten repeats of the fused forward+backward on the same inputs give bitwise the same outputs and
  gradients, on balanced routing and on Zipf-biased routing whose heaviest experts take the split
  weight-gradient path (the last part of a tile to arrive sums the parts, and which part that is
  varies from run to run).
* A host-forced delay kernel (torch.cuda._sleep: a bounded spin that exits by itself) issued on
  the compute stream or on the auxiliary stream before a layer call lets the other stream run
  ahead: any cross-stream dependency without an event wait would read unfinished data. The results
  must not change, for the fused primitive, for forward then backward with the delay between
  them, with the FP8 backward flags, and with a single stream.

The overlap schedules follow token-wise ChunkedEP (Megatron-LM PR 7342, "Summary": one chunk's
dispatch overlaps another chunk's expert compute) and torchtitan PR 5542 ("Verification": input
gradients before weight gradients); the repeat count follows the "Historical single-layer OP
measurements" protocol of ChunkedEP (repeated measured runs of one layer).
"""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")

OUTPUTS = ("topk_idx", "row_of", "src_token", "out", "dgates", "dlogits", "dx", "dw1", "dw2", "dwr", "dwr_acc")

CASES = [
    MoeConfig("race_bal", T=3000, H=512, I=256, E=64, E_local=8, e0=8, k=8, n_chunks=3, dtype="bf16",
              seed_base=700, backward=True),
    MoeConfig("race_zipf", T=4096, H=512, I=256, E=32, E_local=8, e0=0, k=8, n_chunks=2, dtype="bf16",
              seed_base=710, zipf_s=1.2, n_empty=2, backward=True),
]

DELAY_CYCLES = 2_000_000


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()
    return torch, mh


def _setup(cfg, flags=0):
    torch, mh = _require_gpu()
    inp = moe_inputs.make_inputs(cfg, with_backward=True)
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0, flags=flags)
    b = mh.allocate(d, backward=True)
    for name in ("x", "logits", "w1", "w2", "w_r", "dy"):
        b[name] = harness.to_dev(inp, name, cfg.dtype)
    if flags & mh.FLAG_FP8_DGRAD:
        El, H, I = cfg.E_local, cfg.H, cfg.I
        mh.moe_quantize_cols_fp8(El, 2 * I, H, b["w1"], b["w1t"], b["w1t_scale"])
        mh.moe_quantize_cols_fp8(El, H, I, b["w2"], b["w2t"], b["w2t_scale"])
    torch.cuda.synchronize()
    return torch, mh, d, b


def _snapshot(b, cfg):
    return {k: harness.bits_np(b[k][:cfg.T] if k == "out" else b[k]).copy() for k in OUTPUTS}


def _assert_same(a, b, note):
    for k in OUTPUTS:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{k} ({note})")


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_ten_repeats_bitwise(cfg):
    torch, mh, d, b = _setup(cfg)
    cs, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    ref = None
    for r in range(10):
        mh.moe_layer_forward_backward(d, b, cs, aux)
        torch.cuda.synchronize()
        snap = _snapshot(b, cfg)
        if ref is None:
            ref = snap
            offs = b["offsets"].cpu().numpy()
            rows = offs[:, -1].sum()
            heavy = int(max(sum(int(offs[c, e + 1] - offs[c, e]) for c in range(cfg.n_chunks))
                            for e in range(cfg.E_local)))
            print(f"[repeat] {cfg.name}: {rows} local rows, heaviest expert {heavy} rows", flush=True)
        else:
            _assert_same(ref, snap, f"repeat {r}")


@pytest.mark.parametrize("delayed", ["compute", "aux"])
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_delay_on_one_stream_changes_nothing(cfg, delayed):
    torch, mh, d, b = _setup(cfg)
    cs, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    ref = _snapshot(b, cfg)
    # fused primitive, delay before the call
    with torch.cuda.stream(cs if delayed == "compute" else aux):
        torch.cuda._sleep(DELAY_CYCLES)
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    _assert_same(ref, _snapshot(b, cfg), f"fused, {delayed} delayed")
    # forward, delay, backward
    mh.moe_layer_forward(d, b, cs, aux)
    with torch.cuda.stream(cs if delayed == "compute" else aux):
        torch.cuda._sleep(DELAY_CYCLES)
    mh.moe_layer_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    _assert_same(ref, _snapshot(b, cfg), f"forward, {delayed} delayed, backward")


@pytest.mark.parametrize("delayed", ["compute", "aux"])
def test_delay_with_fp8_backward_flags(delayed):
    cfg = CASES[0]
    torch, mh, d, b = _setup(cfg, flags=1 | 2 | 4)
    cs, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    ref = _snapshot(b, cfg)
    with torch.cuda.stream(cs if delayed == "compute" else aux):
        torch.cuda._sleep(DELAY_CYCLES)
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    _assert_same(ref, _snapshot(b, cfg), f"FP8 flags, {delayed} delayed")


def test_one_stream_equals_two_streams():
    cfg = CASES[1]
    torch, mh, d, b = _setup(cfg)
    cs, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    ref = _snapshot(b, cfg)
    torch.cuda._sleep(DELAY_CYCLES)
    mh.moe_layer_forward_backward(d, b, cs, cs)
    torch.cuda.synchronize()
    _assert_same(ref, _snapshot(b, cfg), "one stream")
