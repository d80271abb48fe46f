"""GPU parity of the FP8 backward (BF16 layer with MOE_FLAG_FP8_DGRAD and/or MOE_FLAG_FP8_WGRAD)
against the oracle.

* The transposed per-column weight quantisation: codes and scales bit for bit, on ragged shapes
  (row and column tails of the 64 x 64 transpose tiles), an all-zero column and a saturating one.
* The layer forward+backward with FP8 input gradients against the oracle's FP8-dgrad backward on
  small ragged cases (several chunks, local subsets, empty experts, partial tiles), and at the
  one-rank share (16K tokens, H 2048, 16 of 128 experts, top-8, I 768) in the layer primitive's
  two-stream configuration.
* The chunk = -1 stage calls on one stream give the layer primitive's results bit for bit, including
  the e4m3 rows of dyd, which the layer writes inside combine backward.
* FP8 weight gradients: the per-expert transposed xd operand bit for bit (codes, zero padding,
  scales), and the layer's dW1, dW2 against the oracle's FP8 weight gradients, alone and with the
  FP8 input gradients, small and at the one-rank share.
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


FP8DG_EDGE = [
    # H above the combine-backward quantiser's limit: the layer quantises the stored dyd rows, and
    # the row quantiser walks rows longer than its register tile
    MoeConfig("fp8dg_h8256", T=200, H=8256, I=64, E=8, E_local=4, e0=1, k=2, n_chunks=2, dtype="bf16",
              seed_base=540, backward=True),
    # one local expert takes every routed row of a chunk region (k = 1)
    MoeConfig("fp8dg_k1", T=333, H=192, I=128, E=4, E_local=1, e0=3, k=1, n_chunks=3, dtype="bf16",
              seed_base=550, backward=True),
    # no local expert: no dispatch row, nothing to quantise
    MoeConfig("fp8dg_none_local", T=200, H=128, I=64, E=8, E_local=0, e0=8, k=2, n_chunks=2, dtype="bf16",
              seed_base=560, backward=True),
]


@pytest.mark.parametrize("cfg", FP8DG_EDGE, ids=[c.name for c in FP8DG_EDGE])
def test_fp8_dgrad_edge_shapes(cfg):
    torch, mh = _require_gpu()
    print(f"[parity] {cfg} fp8 dgrad", flush=True)
    run = harness.run_gpu(cfg, sentinel=-3.0, flags=mh.FLAG_FP8_DGRAD)
    _check_transposed_weights(run)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-3.0)
    print("[fp8 dgrad edge]", harness.check_backward(run, ref), flush=True)


def test_fp8_dgrad_zero_tokens():
    """T = 0 with FP8 input gradients: the layer returns OK, writes no output row and gives zero
    weight gradients."""
    torch, mh = _require_gpu()
    d = mh.make_desc(T=0, H=128, I=64, E=8, E_local=4, k=2, n_chunks=2, flags=mh.FLAG_FP8_DGRAD)
    b = mh.allocate(d, backward=True, fill=7)
    for name, shape in (("x", (0, 128)), ("dy", (0, 128))):
        b[name] = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    b["logits"] = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    b["w1"] = torch.zeros((4, 128, 128), dtype=torch.bfloat16, device="cuda")
    b["w2"] = torch.zeros((4, 128, 64), dtype=torch.bfloat16, device="cuda")
    b["w_r"] = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    b["out"] = torch.full((max(4, int(d.P_out)), 128), 5.0, dtype=torch.bfloat16, device="cuda")
    mh.moe_quantize_cols_fp8(4, 128, 128, b["w1"], b["w1t"], b["w1t_scale"])
    mh.moe_quantize_cols_fp8(4, 128, 64, b["w2"], b["w2t"], b["w2t_scale"])
    mh.moe_layer_forward_backward(d, b, torch.cuda.current_stream(), torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.all(b["out"] == 5.0)
    assert torch.all(b["dw1"] == 0) and torch.all(b["dw2"] == 0) and torch.all(b["dwr"] == 0)
    # all-zero weight columns: codes 0, scale 1
    assert torch.all(b["w1t"] == 0) and torch.all(b["w1t_scale"] == 1.0)


# ----------------------------------------------------------------------------- FP8 weight gradients

def _check_xd_expert_codes(run, ref):
    """The weight gradients' transposed xd operand: per expert, every column's codes over the
    expert's rows of every chunk (then zero padding to a multiple of 64) and its scale, bit for bit."""
    cfg, d = run.cfg, run.desc
    offsets = run.bufs["offsets"].cpu().numpy()
    codes = run.bufs["xd_t"].cpu().numpy()
    scales = run.bufs["xd_cs"].cpu().numpy()
    koff = 0
    for e in range(cfg.E_local):
        rows = ofp8.expert_rows(offsets, d.P_c, e)
        K = rows.size
        Kp = (K + 63) // 64 * 64
        got = codes[koff * cfg.H: koff * cfg.H + cfg.H * Kp].reshape(cfg.H, Kp)
        want_c, want_s = ofp8.quantize_cols_t(ofp8.bf16_round(np.asarray(ref["xd"])[rows]))
        np.testing.assert_array_equal(got[:, :K], want_c, err_msg=f"expert {e}")
        assert np.all(got[:, K:] == 0), f"expert {e}: padding"
        np.testing.assert_array_equal(scales[e * cfg.H:(e + 1) * cfg.H].view(np.uint32), want_s.view(np.uint32))
        koff += Kp


@pytest.mark.parametrize("both", [False, True], ids=["wgrad", "dgrad+wgrad"])
@pytest.mark.parametrize("cfg", FP8DG_SMALL, ids=[c.name for c in FP8DG_SMALL])
def test_fp8_wgrad_layer_small(cfg, both):
    torch, mh = _require_gpu()
    flags = mh.FLAG_FP8_WGRAD | (mh.FLAG_FP8_DGRAD if both else 0)
    print(f"[parity] {cfg} flags {flags}", flush=True)
    run = harness.run_gpu(cfg, sentinel=-7.0, flags=flags)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-7.0)
    _check_xd_expert_codes(run, ref)
    print("[fp8 wgrad]", harness.check_backward(run, ref), flush=True)


@pytest.mark.parametrize("cfg", FP8DG_SMALL[:3], ids=[c.name for c in FP8DG_SMALL[:3]])
def test_fp8_wgrad_stage_calls_match_layer(cfg):
    torch, mh = _require_gpu()
    flags = mh.FLAG_FP8_WGRAD | mh.FLAG_FP8_DGRAD
    a = harness.run_gpu(cfg, layer=True, flags=flags)
    b = harness.run_gpu(cfg, layer=False, two_streams=False, flags=flags)
    for name in ("dx", "dw1", "dw2", "dwr"):
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(b.bufs[name]), err_msg=name)


@pytest.mark.timeout(300)
def test_fp8_dgrad_wgrad_full_16k():
    """The one-rank share with FP8 input and weight gradients."""
    torch, mh = _require_gpu()
    cfg = moe_inputs.CONFIGS["fb16k"]
    print(f"[parity] {cfg} fp8 dgrad + wgrad", flush=True)
    run = harness.run_gpu(cfg, flags=mh.FLAG_FP8_DGRAD | mh.FLAG_FP8_WGRAD)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref)
    print("[fb16k fp8 dgrad+wgrad]", harness.check_backward(run, ref), flush=True)


@pytest.mark.parametrize("cfg", FP8DG_SMALL[:2], ids=[c.name for c in FP8DG_SMALL[:2]])
def test_fp8_backward_launch_order_and_streams(cfg):
    """The fused primitive with FP8 input and weight gradients: per chunk, combine backward with
    the e4m3 dyd rows, the FP8 down dgrad, the dgu quantisation and the FP8 gate/up dgrad; the
    weight-gradient operands that do not wait for dgu are quantised on the auxiliary stream after
    the last combine backward; every chunk's input-gradient work is issued before the weight-
    gradient GEMM; no BF16 dgrad or wgrad launch remains."""
    torch, mh = _require_gpu()
    n = cfg.n_chunks
    mh.moe_trace_enable(False)
    try:
        harness.run_gpu(cfg, flags=mh.FLAG_FP8_DGRAD | mh.FLAG_FP8_WGRAD)
    finally:
        mh.moe_trace_disable()
    log = mh.moe_trace_entries()
    names = [nm for nm, _, _ in log]
    counts = {k: names.count(k) for k in set(names)}
    expect = {"combine_bwd_q": n, "combine_bwd": 0, "gemm_down_dgrad_swiglu_fp8": n, "quantize_dgu_fp8": n,
              "gemm_gateup_dgrad_fp8": n, "quantize_dyd_fp8": 0, "quantize_dyd_cols_fp8": 1,
              "quantize_h_cols_fp8": 1, "quantize_xd_cols_fp8": 1, "quantize_dgu_cols_fp8": 1,
              "gemm_wgrad_fp8": 1, "dispatch_bwd": n, "gemm_down_dgrad_swiglu": 0,
              "gemm_gateup_dgrad+down_dgrad_swiglu": 0, "gemm_gateup_dgrad+wgrad_w2": 0, "gemm_wgrad_w1": 0,
              "gemm_wgrad": 0}
    for k, v in expect.items():
        assert counts.get(k, 0) == v, (k, counts.get(k, 0), v)
    wg = names.index("gemm_wgrad_fp8")
    for kind in ("combine_bwd_q", "gemm_down_dgrad_swiglu_fp8", "quantize_dgu_fp8", "gemm_gateup_dgrad_fp8",
                 "dispatch_bwd", "quantize_dyd_cols_fp8", "quantize_h_cols_fp8", "quantize_xd_cols_fp8",
                 "quantize_dgu_cols_fp8"):
        assert max(i for i, nm in enumerate(names) if nm == kind) < wg, kind
    last_cb = max(i for i, nm in enumerate(names) if nm == "combine_bwd_q")
    assert names.index("quantize_dyd_cols_fp8") > last_cb

    def streams_of(kind):
        return [st for nm, st, _ in log if nm == kind]
    compute = streams_of("gemm_gateup_swiglu")[0]
    aux = streams_of("dispatch")[-1]
    assert aux != compute
    for kind in ("gemm_down_dgrad_swiglu_fp8", "quantize_dgu_fp8", "gemm_gateup_dgrad_fp8",
                 "quantize_dgu_cols_fp8", "gemm_wgrad_fp8"):
        assert set(streams_of(kind)) == {compute}, kind
    for kind in ("quantize_dyd_cols_fp8", "quantize_h_cols_fp8", "quantize_xd_cols_fp8", "dispatch_bwd"):
        assert set(streams_of(kind)) == {aux}, kind
    cbq = streams_of("combine_bwd_q")
    assert cbq[0] == compute and set(cbq[1:]) <= {aux}


def test_fp8_backward_under_hip_graph_capture():
    """The fused primitive with FP8 input and weight gradients captured into a HIP graph (both
    streams) replays to bitwise the eager results, three times, with eager work between replays."""
    torch, mh = _require_gpu()
    cfg = FP8DG_SMALL[0]
    inp = moe_inputs.make_inputs(cfg, with_backward=True)
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0, flags=mh.FLAG_FP8_DGRAD | mh.FLAG_FP8_WGRAD)
    b = mh.allocate(d, backward=True)
    for name in ("x", "w1", "w2", "w_r", "dy"):
        b[name] = torch.from_numpy(inp[name + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    b["logits"] = torch.from_numpy(inp["logits"]).cuda()
    mh.moe_quantize_cols_fp8(cfg.E_local, 2 * cfg.I, cfg.H, b["w1"], b["w1t"], b["w1t_scale"])
    mh.moe_quantize_cols_fp8(cfg.E_local, cfg.H, cfg.I, b["w2"], b["w2t"], b["w2t_scale"])
    cs, aux = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    keys = ("dx", "dw1", "dw2", "dwr", "dlogits")
    ref = {k: b[k].clone() for k in keys}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        mh.moe_layer_forward_backward(d, b, cs, aux)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in keys:
            b[k].fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(b[k], ref[k]), (rep, k)
