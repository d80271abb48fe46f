"""GPU parity of the FP8 dispatch-backward payload (MOE_FLAG_FP8_DXD: dxd written by the gate/up
dgrad epilogue as block-scaled e4m3 rows, one scale per row and 256-column block, read by dispatch
backward) against the oracle.

* The layer forward+backward with the flag alone and together with the FP8 input gradients,
  against the oracle's backward on the FP8 payload, on small ragged cases (H not a multiple of
  256, several chunks, local subsets, empty experts), edge shapes and the one-rank 16K share in the
  layer primitive's two-stream configuration (merged GEMM launches).
* Every gradient except dx is bit for bit that of the run without the flag.
* The payload itself, for every valid dispatch row: code value times its block's scale against the
  oracle's dxd (e4m3-sized rel-L2, at most one e4m3 step anywhere, most values within the pure
  quantisation bound), and every block scale within 2^-6 of the oracle block's amax / 448 (a scale
  from the wrong row or block fails by orders of magnitude). The GPU quantises its own BF16 dxd, so
  codes are compared as values, not bit for bit; dx takes the FP8 tolerance for that reason (a
  value that the BF16 path's rounding moves across an e4m3 boundary changes by a whole step).
* The chunk = -1 stage calls on one stream give the layer's dx and payload bit for bit.
"""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")

BLOCK = 256


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()  # raises if the HIP library is missing: the GPU tests never fall back
    return torch, mh


SMALL = [
    MoeConfig("dxd_rag", T=1000, H=384, I=192, E=32, E_local=8, e0=4, k=4, n_chunks=2, dtype="bf16",
              seed_base=600, backward=True),
    MoeConfig("dxd_n3", T=777, H=640, I=320, E=64, E_local=16, e0=48, k=6, n_chunks=3, dtype="bf16",
              seed_base=610, backward=True),
    MoeConfig("dxd_n4_zipf", T=1500, H=256, I=128, E=32, E_local=8, k=8, n_chunks=4, dtype="bf16",
              seed_base=620, zipf_s=1.2, n_empty=2, backward=True),
    MoeConfig("dxd_n1", T=640, H=128, I=64, E=8, E_local=4, e0=2, k=2, n_chunks=1, dtype="bf16",
              seed_base=630, backward=True),
]

EDGE = [
    # a long row: 32 full blocks and a 64-column one
    MoeConfig("dxd_h8256", T=200, H=8256, I=64, E=8, E_local=4, e0=1, k=2, n_chunks=2, dtype="bf16",
              seed_base=640, backward=True),
    # one local expert takes every routed row of a chunk region (k = 1)
    MoeConfig("dxd_k1", T=333, H=192, I=128, E=4, E_local=1, e0=3, k=1, n_chunks=3, dtype="bf16",
              seed_base=650, backward=True),
    # no local expert: no dxd row
    MoeConfig("dxd_none_local", T=200, H=128, I=64, E=8, E_local=0, e0=8, k=2, n_chunks=2, dtype="bf16",
              seed_base=660, backward=True),
]


def _payload(run):
    """(codes [P, H] uint8, scales [P, nblk] float32) read from the dxd buffer."""
    d, cfg = run.desc, run.cfg
    P, H = d.n_chunks * d.P_c, cfg.H
    nb = (H + BLOCK - 1) // BLOCK
    raw = run.bufs["dxd"].contiguous().view(-1).view(__import__("torch").uint8).cpu().numpy()
    codes = raw[:P * H].reshape(P, H)
    scales = raw[P * H:P * H + P * nb * 4].view(np.float32).reshape(P, nb)
    return codes, scales


def _check_payload(run, ref, upstream_fp8=False):
    """Each valid row's dequantised payload against the oracle's dxd (FP64), block by block.
    upstream_fp8: dxd itself comes from the FP8 input gradients, whose own code flips move it
    further from the oracle's, so only the rel-L2 and the scales are checked."""
    from oracle import fp8 as ofp8
    cfg, d = run.cfg, run.desc
    codes, scales = _payload(run)
    offsets = run.bufs["offsets"].cpu().numpy()
    want_all = np.asarray(ref["bwd"]["dxd"])
    H = cfg.H
    nb = (H + BLOCK - 1) // BLOCK
    for c in range(cfg.n_chunks):
        r0, n = c * d.P_c, int(offsets[c, cfg.E_local]) if cfg.E_local else 0
        if n == 0:
            continue
        got = ofp8.dequantize_row_blocks(codes[r0:r0 + n], scales[r0:r0 + n], BLOCK)
        want = want_all[r0:r0 + n]
        # the GPU quantises its own BF16 dxd, which differs from the oracle's by the BF16 path's
        # rounding; where that moves a value across an e4m3 rounding boundary the code differs by
        # one step, so the check is on the whole: e4m3-sized rel-L2 and a bounded share of values
        # outside the pure quantisation bound
        col_scale = np.repeat(scales[r0:r0 + n].astype(np.float64), BLOCK, axis=1)[:, :H]
        err = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert err <= 0.05, f"chunk {c}: payload rel-L2 {err:.3e}"
        if not upstream_fp8:
            bound = 2.0 ** -4 * np.abs(want) + 2.0 ** -9 * col_scale * 1.01
            out = np.count_nonzero(np.abs(got - want) > bound) / got.size
            assert out <= 0.05, f"chunk {c}: {out:.3%} of payload values outside the e4m3 bound"
            assert np.all(np.abs(got - want) <= 2.0 ** -3 * np.abs(want) + 2.0 ** -6 * col_scale * 448), \
                f"chunk {c}: a payload value is off by more than one e4m3 step"
        amax = np.stack([np.abs(want[:, b * BLOCK:(b + 1) * BLOCK]).max(1) for b in range(nb)], 1)
        live = amax > 0
        rel = np.abs(scales[r0:r0 + n][live] * 448.0 / amax[live] - 1.0)
        tol = 2.0 ** -3 if upstream_fp8 else 2.0 ** -6
        assert rel.max(initial=0.0) <= tol, f"chunk {c}: block scale off by {rel.max():.3e}"


def _same_except_dx(a, b, flags_note):
    for name in ("dgates", "dlogits", "dw1", "dw2", "dwr"):
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(b.bufs[name]),
                                      err_msg=f"{name} ({flags_note})")
    # dgu on the valid rows of every chunk region (rows past N_c are never written)
    offsets = a.bufs["offsets"].cpu().numpy()
    ga, gb = harness.bits_np(a.bufs["dgu"]), harness.bits_np(b.bufs["dgu"])
    for c in range(a.cfg.n_chunks):
        r0, n = c * a.desc.P_c, int(offsets[c, a.cfg.E_local]) if a.cfg.E_local else 0
        np.testing.assert_array_equal(ga[r0:r0 + n], gb[r0:r0 + n], err_msg=f"dgu chunk {c} ({flags_note})")


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_fp8_dxd_layer_small(cfg):
    torch, mh = _require_gpu()
    print(f"[parity] {cfg} fp8 dxd", flush=True)
    run = harness.run_gpu(cfg, sentinel=-7.0, flags=mh.FLAG_FP8_DXD)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-7.0)
    errs = harness.check_backward(run, ref)
    print("[fp8 dxd]", errs, flush=True)
    _check_payload(run, ref)
    base = harness.run_gpu(cfg, sentinel=-7.0, flags=0)
    _same_except_dx(run, base, "flag alone vs none")


@pytest.mark.parametrize("cfg", SMALL[:2], ids=[c.name for c in SMALL[:2]])
def test_fp8_dxd_with_fp8_dgrad(cfg):
    torch, mh = _require_gpu()
    flags = mh.FLAG_FP8_DXD | mh.FLAG_FP8_DGRAD
    print(f"[parity] {cfg} flags {flags}", flush=True)
    run = harness.run_gpu(cfg, sentinel=-7.0, flags=flags)
    from oracle import fp8 as ofp8
    for w, name in (("w1", "w1t"), ("w2", "w2t")):
        want_c, _ = ofp8.quantize_cols_t(run.inp[w])
        np.testing.assert_array_equal(run.bufs[name].cpu().numpy(), want_c, err_msg=name)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-7.0)
    print("[fp8 dxd + dgrad]", harness.check_backward(run, ref), flush=True)
    _check_payload(run, ref, upstream_fp8=True)
    base = harness.run_gpu(cfg, sentinel=-7.0, flags=mh.FLAG_FP8_DGRAD)
    _same_except_dx(run, base, "with FP8 dgrad")


@pytest.mark.parametrize("cfg", SMALL[:3], ids=[c.name for c in SMALL[:3]])
def test_fp8_dxd_stage_calls_match_layer(cfg):
    torch, mh = _require_gpu()
    a = harness.run_gpu(cfg, layer=True, flags=mh.FLAG_FP8_DXD)
    b = harness.run_gpu(cfg, layer=False, two_streams=False, flags=mh.FLAG_FP8_DXD)
    for name in ("dx", "dw1", "dw2", "dwr"):
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(b.bufs[name]), err_msg=name)
    ca, sa = _payload(a)
    cb, sb = _payload(b)
    offsets = a.bufs["offsets"].cpu().numpy()
    for c in range(cfg.n_chunks):
        r0, n = c * a.desc.P_c, int(offsets[c, cfg.E_local])
        np.testing.assert_array_equal(ca[r0:r0 + n], cb[r0:r0 + n], err_msg=f"codes chunk {c}")
        np.testing.assert_array_equal(sa[r0:r0 + n].view(np.uint32), sb[r0:r0 + n].view(np.uint32),
                                      err_msg=f"scales chunk {c}")


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_fp8_dxd_edge_shapes(cfg):
    torch, mh = _require_gpu()
    print(f"[parity] {cfg} fp8 dxd", flush=True)
    run = harness.run_gpu(cfg, sentinel=-3.0, flags=mh.FLAG_FP8_DXD)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref, sentinel=-3.0)
    print("[fp8 dxd edge]", harness.check_backward(run, ref), flush=True)
    if cfg.E_local:
        _check_payload(run, ref)


@pytest.mark.timeout(300)
def test_fp8_dxd_full_16k():
    """The one-rank share, fused forward+backward with the FP8 dxd payload, two chunks (merged
    launches: the payload is written by the paired gate/up dgrad epilogues)."""
    torch, mh = _require_gpu()
    cfg = moe_inputs.CONFIGS["fb16k"]
    print(f"[parity] {cfg} fp8 dxd", flush=True)
    run = harness.run_gpu(cfg, flags=mh.FLAG_FP8_DXD)
    ref = harness.run_oracle(run)
    harness.check_forward(run, ref)
    errs = harness.check_backward(run, ref)
    print("[fb16k fp8 dxd]", errs, flush=True)
    _check_payload(run, ref)
