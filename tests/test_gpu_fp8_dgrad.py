"""GPU parity of the FP8 input gradients (BF16 layer with MOE_FLAG_FP8_DGRAD) against the oracle.

* The transposed per-column weight quantisation: codes and scales bit for bit, on ragged shapes
  (row and column tails of the 64 x 64 transpose tiles), an all-zero column and a saturating one.
* The layer forward+backward with FP8 input gradients against the oracle's FP8-dgrad backward on
  small ragged cases (several chunks, local subsets, empty experts, partial tiles), and at the
  one-rank share (16K tokens, H 2048, 16 of 128 experts, top-8, I 768) in the layer primitive's
  two-stream configuration.
* The chunk = -1 stage calls on one stream give the layer primitive's results bit for bit, including
  the e4m3 rows of dyd, which the layer writes inside combine backward.
"""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()  # raises if the HIP library is missing: the GPU tests never fall back
    return torch, mh


@pytest.mark.parametrize("batch,rows,cols", [(3, 80, 136), (1, 16, 8), (2, 2048, 768), (4, 1536, 2048)])
def test_quantize_cols_bitwise(batch, rows, cols):
    torch, mh = _require_gpu()
    print(f"[quantize_cols] batch {batch} rows {rows} cols {cols}", flush=True)
    rng = np.random.default_rng(1000 + rows + cols)
    a = rng.standard_normal((batch, rows, cols), dtype=np.float32) * np.float32(0.02)
    a[0, :, 0] = 0.0                       # all-zero column: codes 0, scale 1
    if cols > 1:
        a[-1, rows // 2, 1] = 3.0e4        # one large value: that column's codes saturate at 448
    bits = moe_inputs.f32_to_bf16_bits(a)
    vals = moe_inputs.bf16_bits_to_f32(bits)
    src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    codes = torch.empty((batch, cols, rows), dtype=torch.uint8, device="cuda")
    scale = torch.empty((batch, cols), dtype=torch.float32, device="cuda")
    mh.moe_quantize_cols_fp8(batch, rows, cols, src, codes, scale)
    torch.cuda.synchronize()
    want_c, want_s = ofp8.quantize_cols_t(vals)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)
    np.testing.assert_array_equal(scale.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


FP8DG_SMALL = [
    MoeConfig("fp8dg_rag", T=1000, H=256, I=192, E=32, E_local=8, e0=4, k=4, n_chunks=2, dtype="bf16",
              seed_base=500, backward=True),
    MoeConfig("fp8dg_n3", T=777, H=384, I=320, E=64, E_local=16, e0=48, k=6, n_chunks=3, dtype="bf16",
              seed_base=510, backward=True),
    MoeConfig("fp8dg_n4_zipf", T=1500, H=256, I=128, E=32, E_local=8, k=8, n_chunks=4, dtype="bf16",
              seed_base=520, zipf_s=1.2, n_empty=2, backward=True),
    MoeConfig("fp8dg_n1", T=640, H=128, I=64, E=8, E_local=4, e0=2, k=2, n_chunks=1, dtype="bf16",
              seed_base=530, backward=True),
]


def _check_transposed_weights(run):
    inp = run.inp
    for w, name in (("w1", "w1t"), ("w2", "w2t")):
        want_c, want_s = ofp8.quantize_cols_t(inp[w])
        np.testing.assert_array_equal(run.bufs[name].cpu().numpy(), want_c, err_msg=name)
        np.testing.assert_array_equal(run.bufs[name + "_scale"].cpu().numpy().view(np.uint32),
                                      want_s.view(np.uint32), err_msg=name + "_scale")


@pytest.mark.parametrize("cfg", FP8DG_SMALL, ids=[c.name for c in FP8DG_SMALL])
def test_fp8_dgrad_layer_small(cfg):
    torch, mh = _require_gpu()
    print(f"[parity] {cfg} fp8 dgrad", flush=True)
    run = harness.run_gpu(cfg, sentinel=-7.0, flags=mh.FLAG_FP8_DGRAD)
    _check_transposed_weights(run)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-7.0)
    print("[fp8 dgrad]", harness.check_backward(run, ref), flush=True)


@pytest.mark.parametrize("cfg", FP8DG_SMALL[:3], ids=[c.name for c in FP8DG_SMALL[:3]])
def test_fp8_dgrad_stage_calls_match_layer(cfg):
    torch, mh = _require_gpu()
    a = harness.run_gpu(cfg, layer=True, flags=mh.FLAG_FP8_DGRAD)
    b = harness.run_gpu(cfg, layer=False, two_streams=False, flags=mh.FLAG_FP8_DGRAD)
    for name in ("dx", "dw1", "dw2", "dwr", "dlogits"):
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(b.bufs[name]), err_msg=name)
    # the layer quantises dyd inside combine backward (scale from RNE(|g| * max|dy|)), the stage
    # call quantises the stored dyd rows: codes and scales agree bit for bit on every valid row
    offsets = a.bufs["offsets"].cpu().numpy()
    for name in ("dyd_scale", "dgu_scale", "dyd_q", "dgu_q"):
        ga, gb = a.bufs[name].cpu().numpy(), b.bufs[name].cpu().numpy()
        for c in range(cfg.n_chunks):
            r0, n = c * a.desc.P_c, int(offsets[c, cfg.E_local])
            np.testing.assert_array_equal(ga[r0:r0 + n], gb[r0:r0 + n], err_msg=f"{name} chunk {c}")


@pytest.mark.timeout(300)
def test_fp8_dgrad_full_16k():
    """The one-rank share, fused forward+backward with FP8 input gradients, two chunks."""
    torch, mh = _require_gpu()
    cfg = moe_inputs.CONFIGS["fb16k"]
    print(f"[parity] {cfg} fp8 dgrad", flush=True)
    run = harness.run_gpu(cfg, flags=mh.FLAG_FP8_DGRAD)
    _check_transposed_weights(run)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref)
    print("[fb16k fp8 dgrad]", harness.check_backward(run, ref), flush=True)
