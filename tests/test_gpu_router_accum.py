"""The router weight gradient accumulated in FP32 across token chunks, then converted once.

Token-wise ChunkedEP (Megatron-LM PR 7342, "Numerical status -- unresolved") reports that
accumulating the router weight gradient across chunks in FP32 before a single dtype conversion
brought the chunked result to within a 0.006774% relative L2 of the unchunked one, from 0.2871%
before. This test reproduces that comparison on the route backward stage call at the 32K-token
one-rank share (two chunks of 16384 tokens, 128 experts, H 2048, top-8):

  * dwr_acc (FP32) after both chunks matches the FP64 oracle dW_r = dlogits^T x within an FP32
    bound: dlogits enters the product as a BF16 high and low part, which carry it to a relative
    2^-18, and x is exactly BF16, so every product is exact to 2^-18 relative and the
    accumulation adds FP32 rounding; rel-L2 <= 1e-5;
  * the chunked BF16 dwr (FP32 across chunks, one conversion) is within rel-L2 1e-4 of the
    unchunked BF16 dwr (one chunk, one conversion): the two differ only where FP32 summation order
    moves a value across a BF16 rounding boundary;
  * per-chunk BF16 accumulation, bf16(bf16(p0) + bf16(p1)) formed on the host from the per-chunk
    FP32 partials that dwr_acc holds after each chunk's call, is more than 1e-3 away from the
    unchunked result and more than ten times further than the FP32-accumulated one.

Inputs are seeded and shared by both sides: x and the logits from the 32K-token workload, the
routing (indices, gates) from the oracle, and upstream gate gradients N(0, 1).

The same stage call at small ragged shapes covers both layouts of the split dlogits that the GPU
product reads: up to 128 experts the high and low parts side by side in one 256-column operand
(E = 32 and 128, zero columns past E), above 128 two planes with a pass over each (E = 132 and
256), with partial output tiles in both directions, one to three chunks."""
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


def _bf16(a):
    return moe_inputs.bf16_bits_to_f32(moe_inputs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


@pytest.mark.parametrize("name", ["fb32k"])
def test_router_grad_fp32_accumulation_across_chunks(name):
    _require_gpu()
    import torch
    import combine_moe_route_02_amd as mh
    import oracle
    from oracle import ffn as offn
    cfg = moe_inputs.CONFIGS[name]
    assert cfg.n_chunks == 2
    inp = moe_inputs.make_inputs(cfg, parts=("x", "logits"))
    idx, gates64 = oracle.route(inp["logits"], cfg.k)
    gates = gates64.astype(np.float32)
    dgates = moe_inputs.make_dgates(cfg)
    # oracle: FP64 VJP of the gates on the same FP32 inputs, and dW_r = dlogits^T x
    dl_ref = offn.route_bwd(dgates.astype(np.float64), gates.astype(np.float64), idx, cfg.E)
    x64 = inp["x"].astype(np.float64)
    dwr_ref = dl_ref.T @ x64

    dev = {"x": torch.from_numpy(inp["x_bits"].view(np.int16)).cuda().view(torch.bfloat16),
           "gates": torch.from_numpy(gates).cuda(), "dgates": torch.from_numpy(dgates).cuda(),
           "idx": torch.from_numpy(idx).cuda()}

    def run(n_chunks, per_chunk):
        d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=n_chunks,
                         dtype="bf16", e0=cfg.e0)
        ws = torch.empty(max(1, mh.workspace_bytes(d)["workspace"]), dtype=torch.uint8, device="cuda")
        dlogits = torch.full((cfg.T, cfg.E), 7.0, dtype=torch.float32, device="cuda")
        acc = torch.full((cfg.E, cfg.H), 7.0, dtype=torch.float32, device="cuda")
        dwr = torch.empty((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
        partial = []
        for c in (range(n_chunks) if per_chunk else [-1]):
            mh.moe_route_bwd(d, c, dev["dgates"], dev["gates"], dev["idx"], dev["x"], dlogits, acc, dwr, ws)
            torch.cuda.synchronize()
            partial.append(acc.cpu().numpy().astype(np.float64))
        return dlogits.cpu().numpy().astype(np.float64), partial, harness.to_np(dwr)

    dl2, acc2, dwr2 = run(2, per_chunk=True)
    dl1, acc1, dwr1 = run(1, per_chunk=False)

    # dlogits: FP32 arithmetic on the same FP32 inputs
    assert harness.rel_l2(dl2, dl_ref) <= 1e-6 and harness.rel_l2(dl1, dl_ref) <= 1e-6
    assert np.all(dl2[dl_ref == 0] == 0)
    # FP32 accumulator after both chunks against the FP64 product
    e_acc = harness.rel_l2(acc2[-1], dwr_ref)
    e_acc1 = harness.rel_l2(acc1[-1], dwr_ref)
    assert e_acc <= 1e-5 and e_acc1 <= 1e-5, (e_acc, e_acc1)
    # one conversion of the FP32 sum: the dwr output
    np.testing.assert_array_equal(dwr2, _bf16(acc2[-1]))
    # the chunk-0 partial is the oracle's chunk-0 product
    (s0, e0), (s1, e1) = oracle.chunk_bounds(cfg.T, 2)
    p0_ref = dl_ref[s0:e0].T @ x64[s0:e0]
    assert harness.rel_l2(acc2[0], p0_ref) <= 1e-5
    p0, p1 = acc2[0], acc2[1] - acc2[0]
    per_chunk_bf16 = _bf16(_bf16(p0) + _bf16(p1))
    chunked = harness.rel_l2(dwr2, dwr1)        # FP32 across chunks, one conversion, vs unchunked
    naive = harness.rel_l2(per_chunk_bf16, dwr1)  # per-chunk BF16 accumulation vs unchunked
    to_ref = (harness.rel_l2(dwr2, dwr_ref), harness.rel_l2(per_chunk_bf16, dwr_ref))
    print(f"[router accum] chunked vs unchunked rel-L2 {chunked:.3e} (page: 6.774e-5); per-chunk BF16 "
          f"{naive:.3e} (page, before the FP32 accumulation: 2.871e-3); FP32 acc vs FP64 {e_acc:.2e}; "
          f"BF16 results vs FP64: {to_ref[0]:.3e} / {to_ref[1]:.3e}", flush=True)
    assert chunked <= 1e-4
    assert naive >= 1e-3 and naive >= 10 * chunked
    assert to_ref[0] <= 5e-3 and to_ref[0] < to_ref[1]


ROUTER_CASES = [
    MoeConfig("rb_e32", T=1000, H=256, I=64, E=32, E_local=8, e0=4, k=4, n_chunks=2, dtype="bf16", seed_base=1210),
    MoeConfig("rb_e128_h320", T=300, H=320, I=64, E=128, E_local=16, e0=0, k=8, n_chunks=1, dtype="bf16",
              seed_base=1220),
    MoeConfig("rb_e132", T=500, H=320, I=64, E=132, E_local=12, e0=120, k=6, n_chunks=2, dtype="bf16",
              seed_base=1230),
    MoeConfig("rb_e256", T=777, H=192, I=64, E=256, E_local=16, e0=100, k=8, n_chunks=3, dtype="bf16",
              seed_base=1240),
]


@pytest.mark.parametrize("cfg", ROUTER_CASES, ids=[c.name for c in ROUTER_CASES])
def test_router_grad_small_shapes(cfg):
    """dlogits within FP32 rounding of the FP64 VJP (zero off the top-k), the FP32 accumulator over
    every chunk within rel-L2 1e-5 of dlogits^T x in FP64, and dwr its one BF16 conversion."""
    _require_gpu()
    import torch
    import combine_moe_route_02_amd as mh
    import oracle
    from oracle import ffn as offn
    inp = moe_inputs.make_inputs(cfg, parts=("x", "logits"))
    idx, gates64 = oracle.route(inp["logits"], cfg.k)
    gates = gates64.astype(np.float32)
    dgates = moe_inputs.make_dgates(cfg)
    dl_ref = offn.route_bwd(dgates.astype(np.float64), gates.astype(np.float64), idx, cfg.E)
    dwr_ref = dl_ref.T @ inp["x"].astype(np.float64)
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype="bf16", e0=cfg.e0)
    ws = torch.full((max(1, mh.workspace_bytes(d)["workspace"]),), 0xFF, dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    dlogits = torch.full((cfg.T, cfg.E), 7.0, dtype=torch.float32, device="cuda")
    acc = torch.full((cfg.E, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    dwr = torch.empty((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
    print(f"[router small] {cfg.name}: T {cfg.T} E {cfg.E} H {cfg.H} k {cfg.k} chunks {cfg.n_chunks}", flush=True)
    mh.moe_route_bwd(d, -1, torch.from_numpy(dgates).cuda(), torch.from_numpy(gates).cuda(),
                     torch.from_numpy(idx).cuda(), x, dlogits, acc, dwr, ws)
    torch.cuda.synchronize()
    dl = dlogits.cpu().numpy().astype(np.float64)
    assert harness.rel_l2(dl, dl_ref) <= 1e-6
    assert np.all(dl[dl_ref == 0] == 0)
    a64 = acc.cpu().numpy().astype(np.float64)
    err = harness.rel_l2(a64, dwr_ref)
    assert err <= 1e-5, err
    np.testing.assert_array_equal(harness.to_np(dwr), _bf16(a64))
