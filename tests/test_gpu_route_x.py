"""GPU parity of routing from x (moe_route_x: the router projection logits = x . W_r^T fused into
the top-k) against the oracle: logits within the FP32-accumulation bound of the FP64 product;
routing bit-exact when the oracle routes the GPU's own logits (the integers are decided in FP32,
by the kernel); bitwise equal to moe_route on those logits; chunk-by-chunk calls equal to one
all-chunks call. Shapes: ragged chunks, E from 32 to 256, an empty last chunk, H with a K tail
(192), k = 1, and the 16K-token one-rank share."""
import numpy as np
import pytest

import moe_inputs
import oracle
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

CASES = [
    MoeConfig("rx_rag", T=1000, H=256, I=64, E=32, E_local=8, e0=4, k=4, n_chunks=2, dtype="bf16", seed_base=700),
    MoeConfig("rx_e256", T=300, H=192, I=64, E=256, E_local=16, e0=100, k=8, n_chunks=3, dtype="bf16",
              seed_base=710),
    MoeConfig("rx_t5_n4_k1", T=5, H=128, I=64, E=64, E_local=4, k=1, n_chunks=4, dtype="bf16", seed_base=720),
    MoeConfig("rx_e96", T=777, H=384, I=64, E=96, E_local=12, e0=30, k=6, n_chunks=3, dtype="bf16", seed_base=730),
    MoeConfig("rx_16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="bf16", seed_base=250),
]


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()
    return torch, mh


def _route_bufs(torch, mh, d, cfg):
    b = mh.allocate(d, backward=False)
    keep = ("topk_idx", "gates", "counts", "offsets", "row_of", "src_token", "workspace")
    out = {k: b[k] for k in keep}
    out["logits"] = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    for k in ("topk_idx", "row_of", "src_token", "counts", "offsets"):
        out[k].fill_(-5)
    return out


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_route_from_x(cfg):
    torch, mh = _require_gpu()
    print(f"[route_x] {cfg}", flush=True)
    inp = moe_inputs.make_inputs(cfg, parts=("x", "w_r"))
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype="bf16", e0=cfg.e0)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).cuda()
    w = torch.from_numpy(inp["w_r_bits"].view(np.int16)).cuda()
    a = _route_bufs(torch, mh, d, cfg)
    mh.moe_route_x(d, -1, x, w, a["logits"], a["topk_idx"], a["gates"], a["counts"], a["offsets"], a["row_of"],
                   a["src_token"], a["workspace"])
    torch.cuda.synchronize()
    lg = a["logits"].cpu().numpy()

    # logits: FP32 accumulation of exact BF16 products, against the FP64 product
    ref = oracle.router_logits(inp["x"], inp["w_r"])
    scale = np.abs(inp["x"]).astype(np.float64) @ np.abs(inp["w_r"]).astype(np.float64).T
    err = np.abs(lg.astype(np.float64) - ref)
    assert np.all(err <= 2e-5 * scale + 1e-30), float((err / (scale + 1e-30)).max())

    # routing of the GPU's own logits: integers bit-exact, gates to FP32 rounding
    idx, gates = oracle.route(lg, cfg.k)
    counts, offsets, row_of, src_token = oracle.layout(idx, cfg.E, cfg.e0, cfg.E_local, cfg.n_chunks, d.P_c)
    np.testing.assert_array_equal(a["topk_idx"].cpu().numpy(), idx)
    np.testing.assert_array_equal(a["counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(a["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(a["row_of"].cpu().numpy(), row_of)
    np.testing.assert_array_equal(a["src_token"].cpu().numpy(), src_token)
    np.testing.assert_allclose(a["gates"].cpu().numpy(), gates, rtol=2e-6, atol=1e-7)

    # the same logits through moe_route: every output bitwise equal
    b = _route_bufs(torch, mh, d, cfg)
    mh.moe_route(d, -1, a["logits"], b["topk_idx"], b["gates"], b["counts"], b["offsets"], b["row_of"],
                 b["src_token"], b["workspace"])
    # chunk by chunk from x: equal to the all-chunks call
    c = _route_bufs(torch, mh, d, cfg)
    for ch in range(cfg.n_chunks):
        mh.moe_route_x(d, ch, x, w, c["logits"], c["topk_idx"], c["gates"], c["counts"], c["offsets"],
                       c["row_of"], c["src_token"], c["workspace"])
    torch.cuda.synchronize()
    for k in ("topk_idx", "counts", "offsets", "row_of", "src_token"):
        np.testing.assert_array_equal(b[k].cpu().numpy(), a[k].cpu().numpy(), err_msg=k)
        np.testing.assert_array_equal(c[k].cpu().numpy(), a[k].cpu().numpy(), err_msg=k)
    for k in ("gates", "logits"):
        np.testing.assert_array_equal(c[k].cpu().numpy().view(np.uint32), a[k].cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(b["gates"].cpu().numpy().view(np.uint32), a["gates"].cpu().numpy().view(np.uint32))


def test_route_x_rejects_unsupported_shapes():
    torch, mh = _require_gpu()
    d = mh.make_desc(T=64, H=128, I=64, E=48, E_local=4, k=2, n_chunks=1, dtype="bf16")
    with pytest.raises(mh.MoeError):
        mh.moe_route_x(d, -1, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)


def test_layer_routes_from_x_when_logits_are_null():
    """The fused layer primitive with logits NULL (routing from x and W_r) gives bitwise the
    results of the same primitive fed the logits that moe_route_x returns."""
    torch, mh = _require_gpu()
    cfg = MoeConfig("rx_layer", T=2048, H=512, I=256, E=64, E_local=8, e0=8, k=4, n_chunks=2, dtype="bf16",
                    seed_base=740, backward=True)
    inp = moe_inputs.make_inputs(cfg, with_backward=True)
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype="bf16", e0=cfg.e0)
    dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
           for n in ("x", "w1", "w2", "w_r", "dy")}
    r = _route_bufs(torch, mh, d, cfg)
    mh.moe_route_x(d, -1, dev["x"], dev["w_r"], r["logits"], r["topk_idx"], r["gates"], r["counts"], r["offsets"],
                   r["row_of"], r["src_token"], r["workspace"])

    def run(logits):
        b = mh.allocate(d, backward=True)
        b.update(dev)
        b["logits"] = logits
        cs, aux = torch.cuda.Stream(), torch.cuda.Stream()
        mh.moe_layer_forward_backward(d, b, cs, aux)
        torch.cuda.synchronize()
        res = {k: b[k].cpu() for k in ("topk_idx", "gates", "row_of", "dx", "dw1", "dw2", "dwr", "dlogits")}
        res["out"] = b["out"][:cfg.T].cpu()
        return res

    a, c = run(r["logits"]), run(None)
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           c[k].view(torch.int16) if c[k].dtype == torch.bfloat16 else c[k]), k
