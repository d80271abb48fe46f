"""Pins for the forward/backward oracle: per-token brute force, the dense SwiGLU special case
(torch CPU), the identity-expert combine, finite differences and autograd (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute, ffn


def _problem(T=40, H=12, I=10, E=8, El=8, e0=0, k=2, seed=0, n=1, router_consistent=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)) * 0.5
    w1 = rng.standard_normal((El, 2 * I, H)) * 0.3
    w2 = rng.standard_normal((El, H, I)) * 0.3
    w_r = rng.standard_normal((E, H)) * 0.5
    if router_consistent:
        logits = x @ w_r.T
    else:
        logits = rng.standard_normal((T, E))
    dy = rng.standard_normal((T, H))
    return dict(x=x, w1=w1, w2=w2, w_r=w_r, logits=logits.astype(np.float32) if not router_consistent else logits,
                dy=dy, k=k, e0=e0, El=El, n=n)


def _fwd(p, logits=None, x=None, w1=None, w2=None):
    return oracle.forward(p["x"] if x is None else x, p["logits"] if logits is None else logits,
                          p["w1"] if w1 is None else w1, p["w2"] if w2 is None else w2,
                          k=p["k"], e0=p["e0"], E_local=p["El"], n_chunks=p["n"])


@pytest.mark.parametrize("kw", [dict(), dict(E=8, El=4, e0=2, k=3, n=2), dict(E=6, El=6, k=6, n=3),
                                dict(E=16, El=5, e0=11, k=4, n=4, T=33)])
def test_forward_matches_brute_force(kw):
    p = _problem(**kw)
    f = _fwd(p)
    y = brute.forward(p["x"], p["logits"], p["w1"], p["w2"], p["k"], p["e0"], p["El"])
    np.testing.assert_allclose(f["out"], y, rtol=1e-12, atol=1e-13)


def test_dense_swiglu_special_case_torch():
    # E = 1, k = 1: every token goes to the single expert with gate 1 -> a dense SwiGLU MLP
    p = _problem(T=30, H=16, I=20, E=1, El=1, k=1)
    f = _fwd(p)
    x = torch.tensor(p["x"])
    w1 = torch.tensor(p["w1"][0])
    w2 = torch.tensor(p["w2"][0])
    gate, up = (x @ w1.T).chunk(2, dim=-1)
    y = (torch.nn.functional.silu(gate) * up) @ w2.T
    np.testing.assert_allclose(f["out"], y.numpy(), rtol=1e-12, atol=1e-14)


def test_identity_expert_combine_returns_input():
    # with every expert local and yd = xd, combine(dispatch(x)) = sum_j g_j x = x
    T, H, E, k = 64, 16, 8, 3
    rng = np.random.default_rng(2)
    x = rng.standard_normal((T, H))
    idx, g = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    P_c, _ = oracle.required_extent(T, k, E, 2)
    _, _, row_of, src = oracle.layout(idx, E, 0, E, 2, P_c)
    out = oracle.combine(oracle.dispatch(x, src), g, row_of)
    np.testing.assert_allclose(out, x, rtol=1e-13, atol=1e-14)


def test_tokens_without_local_expert_get_zero_rows():
    p = _problem(T=60, E=8, El=2, e0=6, k=2)
    f = _fwd(p)
    untouched = np.all(f["row_of"] < 0, axis=1)
    assert untouched.any()
    assert np.all(f["out"][untouched] == 0)


def _bwd(p, f):
    return oracle.backward(f, p["x"], p["dy"], p["w1"], p["w2"], p["w_r"])


@pytest.mark.parametrize("kw", [dict(), dict(E=8, El=4, e0=2, k=3, n=2), dict(E=5, El=3, e0=0, k=5, n=3)])
def test_backward_matches_brute_force(kw):
    p = _problem(**kw)
    f = _fwd(p)
    b = _bwd(p, f)
    bb = brute.backward(p["x"], p["logits"], p["w1"], p["w2"], p["w_r"], p["dy"], p["k"], p["e0"], p["El"])
    for name in ("dx", "dw1", "dw2", "dwr", "dlogits"):
        np.testing.assert_allclose(b[name], bb[name], rtol=1e-11, atol=1e-12, err_msg=name)


def _selection_gap_ok(logits, k, margin):
    s = -np.sort(-logits, axis=1)
    if k == logits.shape[1]:
        return True
    return np.min(s[:, k - 1] - s[:, k]) > margin


@pytest.mark.parametrize("kw", [dict(E=8, El=8, k=2, seed=1), dict(E=8, El=4, e0=0, k=2, seed=3, n=2)])
def test_backward_finite_differences(kw):
    """FP64 central differences of L = <dy, out> with the consistent router logits = x W_r^T."""
    p = _problem(T=24, H=10, I=8, router_consistent=True, **kw)
    eps = 1e-6
    assert _selection_gap_ok(p["logits"], p["k"], 1e-4)
    base_idx = oracle.route(p["logits"], p["k"])[0]

    def loss(x, w1, w2, w_r):
        f = oracle.forward(x, x @ w_r.T, w1, w2, k=p["k"], e0=p["e0"], E_local=p["El"], n_chunks=p["n"])
        np.testing.assert_array_equal(f["idx"], base_idx)     # no selection flip inside the stencil
        return float(np.sum(p["dy"] * f["out"]))

    f = oracle.forward(p["x"], p["logits"], p["w1"], p["w2"], k=p["k"], e0=p["e0"], E_local=p["El"],
                       n_chunks=p["n"])
    g = _bwd(p, f)
    rng = np.random.default_rng(77)
    args = dict(x=p["x"], w1=p["w1"], w2=p["w2"], w_r=p["w_r"])
    grads = dict(x=g["dx"], w1=g["dw1"], w2=g["dw2"], w_r=g["dwr"])
    for name in args:
        for _ in range(3):
            v = rng.standard_normal(args[name].shape)
            plus = dict(args); plus[name] = args[name] + eps * v
            minus = dict(args); minus[name] = args[name] - eps * v
            fd = (loss(**plus) - loss(**minus)) / (2 * eps)
            an = float(np.sum(grads[name] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_matches_torch_autograd():
    """The hand-written VJP against torch autograd of a plain torch forward (CPU, FP64)."""
    p = _problem(T=32, H=12, I=9, E=8, El=5, e0=1, k=3, seed=5, n=2)
    f = _fwd(p)
    b = _bwd(p, f)
    x = torch.tensor(p["x"], requires_grad=True)
    lg = torch.tensor(p["logits"].astype(np.float64), requires_grad=True)
    w1 = torch.tensor(p["w1"], requires_grad=True)
    w2 = torch.tensor(p["w2"], requires_grad=True)
    idx = torch.tensor(f["idx"].astype(np.int64))
    probs = torch.softmax(lg, dim=-1)
    sel = torch.gather(probs, 1, idx)
    gates = sel / sel.sum(-1, keepdim=True)
    I = p["w1"].shape[1] // 2
    out = torch.zeros_like(x)
    for j in range(p["k"]):
        for el in range(p["El"]):
            m = idx[:, j] == p["e0"] + el
            if m.any():
                gate, up = (x[m] @ w1[el].T).split(I, dim=-1)
                out = out.index_add(0, m.nonzero()[:, 0],
                                    gates[m, j, None] * ((torch.nn.functional.silu(gate) * up) @ w2[el].T))
    (out * torch.tensor(p["dy"])).sum().backward()
    np.testing.assert_allclose(f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dlogits"], lg.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(b["dw1"], w1.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(b["dw2"], w2.grad.numpy(), rtol=1e-10, atol=1e-13)
    dx_expert = b["dx"] - b["dlogits"] @ p["w_r"]
    np.testing.assert_allclose(dx_expert, x.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_dlogits_invariants():
    p = _problem(T=80, E=8, El=3, e0=2, k=4, seed=8, n=2)
    f = _fwd(p)
    b = _bwd(p, f)
    np.testing.assert_allclose(b["dlogits"].sum(1), 0.0, atol=1e-13)          # softmax VJP sums to 0
    mask = np.ones_like(b["dlogits"], dtype=bool)
    np.put_along_axis(mask, f["idx"].astype(np.int64), False, 1)
    assert np.all(b["dlogits"][mask] == 0)                                      # zero off the top-k set
    assert np.all(b["dgates"][f["row_of"] < 0] == 0)                            # non-local slots


def test_chunking_does_not_change_the_function():
    p = _problem(T=50, E=8, El=6, e0=1, k=3, seed=12)
    outs = []
    for n in (1, 2, 3, 4):
        q = dict(p); q["n"] = n
        f = _fwd(q)
        outs.append((f["out"], _bwd(q, f)))
    for o, b in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], rtol=1e-13, atol=1e-15)
        for name in ("dx", "dw1", "dw2", "dwr"):
            np.testing.assert_allclose(b[name], outs[0][1][name], rtol=1e-12, atol=1e-14)
