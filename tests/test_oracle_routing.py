"""Pins for the routing/layout oracle: brute force, closed forms, library special cases and
invariants (no GPU)."""
import numpy as np
import pytest
import scipy.special

import oracle
from oracle import brute, routing


def _logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E), dtype=np.float32)
    if ties:
        lg = np.round(lg * 2).astype(np.float32) / 2   # many exact ties
    return lg


@pytest.mark.parametrize("T,E,k,ties", [(37, 8, 2, False), (64, 8, 3, True), (19, 16, 8, True),
                                        (5, 4, 4, False), (23, 6, 1, True)])
def test_route_matches_brute_force(T, E, k, ties):
    lg = _logits(T, E, 11 + T, ties)
    idx, gates = oracle.route(lg, k)
    for t in range(T):
        chosen, g = brute.route_token(lg[t], k)
        assert list(idx[t]) == chosen
        np.testing.assert_allclose(gates[t], g, rtol=1e-13, atol=1e-15)


def test_route_closed_forms():
    # ties go to the lower expert index; slot 0 is the largest logit
    lg = np.array([[1.0, 1.0, 0.0, 0.0], [0.0, 2.0, 2.0, 1.0], [-1.0, -2.0, -3.0, -1.0]], np.float32)
    idx, g = oracle.route(lg, 2)
    assert idx.tolist() == [[0, 1], [1, 2], [0, 3]]
    np.testing.assert_allclose(g, 0.5, rtol=0, atol=1e-15)
    # two distinct logits a > b: gates are the logistic of the gap
    lg = np.array([[0.0, 3.0, 1.0, -5.0]], np.float32)
    idx, g = oracle.route(lg, 2)
    assert idx.tolist() == [[1, 2]]
    np.testing.assert_allclose(g[0], [1 / (1 + np.exp(-2.0)), 1 / (1 + np.exp(2.0))], rtol=1e-14)
    # NaN ranks lowest
    lg = np.array([[np.nan, 0.5, -0.5]], np.float32)
    idx, g = oracle.route(lg, 2)
    assert idx.tolist() == [[1, 2]]


def test_route_k_equals_E_is_textbook_softmax():
    lg = _logits(50, 8, 3)
    idx, g = oracle.route(lg, 8)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(ref, idx.astype(np.int64), 1), rtol=1e-13)
    np.testing.assert_array_equal(idx, np.argsort(-lg, axis=1, kind="stable"))


def test_route_k1_gate_is_one_and_argmax():
    lg = _logits(100, 16, 4)
    idx, g = oracle.route(lg, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(lg, axis=1))
    np.testing.assert_array_equal(g, 1.0)


def test_route_invariants():
    lg = _logits(300, 32, 5)
    idx, g = oracle.route(lg, 6)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 0)          # gates descending with the logits
    sel = np.take_along_axis(lg, idx.astype(np.int64), 1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    # every unselected logit is <= the smallest selected one
    mask = np.ones_like(lg, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, 1)
    assert np.all(np.where(mask, lg, -np.inf).max(1) <= sel[:, -1])
    # selection on probabilities equals selection on logits
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_array_equal(np.argsort(-p, axis=1, kind="stable")[:, :6], idx)


@pytest.mark.parametrize("T,E,e0,El,k,n", [(37, 8, 0, 8, 2, 1), (64, 8, 0, 4, 3, 2), (50, 16, 4, 6, 4, 3),
                                           (13, 8, 2, 3, 2, 4), (9, 4, 0, 4, 4, 4)])
def test_layout_matches_brute_force(T, E, e0, El, k, n):
    lg = _logits(T, E, 100 + T)
    idx, _ = oracle.route(lg, k)
    P_c, _ = oracle.required_extent(T, k, El, n)
    got = oracle.layout(idx, E, e0, El, n, P_c)
    want = brute.layout(idx.tolist(), T, E, e0, El, n, P_c)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(np.asarray(a), np.asarray(b))


@pytest.mark.parametrize("T,E,e0,El,k,n", [(257, 16, 0, 16, 4, 2), (333, 32, 8, 8, 8, 3), (128, 8, 0, 1, 2, 1)])
def test_layout_invariants(T, E, e0, El, k, n):
    lg = _logits(T, E, 7 * T)
    idx, _ = oracle.route(lg, k)
    P_c, _ = oracle.required_extent(T, k, El, n)
    counts, offsets, row_of, src = oracle.layout(idx, E, e0, El, n, P_c)
    assert counts.sum() == T * k
    bounds = oracle.chunk_bounds(T, n)
    for c, (s, e) in enumerate(bounds):
        assert counts[c].sum() == (e - s) * k
        assert offsets[c, 0] == 0
        np.testing.assert_array_equal(np.diff(offsets[c]), counts[c, e0:e0 + El])
        N_c = offsets[c, El]
        assert N_c <= P_c and P_c % 4 == 0
        region = src[c * P_c:(c + 1) * P_c]
        assert np.all(region[N_c:] == -1) and np.all(region[:N_c] >= s) and np.all(region[:N_c] < e)
        for el in range(El):
            seg = region[offsets[c, el]:offsets[c, el + 1]]
            assert np.all(np.diff(seg) > 0)                      # stable: ascending tokens
            assert np.all(np.any(idx[seg] == e0 + el, axis=1))   # each row's token chose it
    local = (idx >= e0) & (idx < e0 + El)
    assert np.all((row_of >= 0) == local)
    rows = row_of[local]
    assert np.unique(rows).size == rows.size                    # injective
    tok = np.nonzero(local)[0]
    np.testing.assert_array_equal(src[rows], tok)                # row_of and src_token inverse
    assert (src >= 0).sum() == rows.size                         # bijection onto used rows


def test_dispatch_then_unpermute_is_identity():
    T, E, H, k = 90, 8, 24, 3
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx, _ = oracle.route(_logits(T, E, 9), k)
    P_c, _ = oracle.required_extent(T, k, 5, 2)
    _, _, row_of, src = oracle.layout(idx, E, 1, 5, 2, P_c)
    xd = oracle.dispatch(x, src)
    back = oracle.unpermute(xd, row_of)
    local = row_of >= 0
    for j in range(k):
        np.testing.assert_array_equal(back[local[:, j], j], x[local[:, j]])


def test_extent_rules():
    assert [oracle.round4(v) for v in (0, 1, 4, 5, 7168, 7169)] == [0, 4, 4, 8, 7168, 7172]
    assert oracle.required_extent(256, 2, 8, 1) == (512, 512)          # tiny case: ceil(T*k/4)*4
    assert oracle.required_extent(16384, 8, 16, 2) == (65536, 131072)
    assert oracle.required_extent(32768, 8, 16, 2) == (131072, 262144)
    assert oracle.required_extent(10, 3, 2, 3) == (8, 32)              # min(k, E_local) per token
    assert oracle.chunk_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.chunk_bounds(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]


def test_router_logits_brute_force_and_one_hot_rows():
    """logits = x . W_r^T: per-element loops on a tiny case; one-hot router rows pick columns."""
    from oracle import routing
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    got = routing.router_logits(x, w)
    for t in range(5):
        for e in range(3):
            acc = 0.0
            for h in range(7):
                acc += x[t, h] * w[e, h]
            assert abs(got[t, e] - acc) <= 1e-12 * (1 + abs(acc))
    onehot = np.zeros((4, 7))
    cols = [6, 0, 3, 3]
    for e, c in enumerate(cols):
        onehot[e, c] = 1.0
    np.testing.assert_array_equal(routing.router_logits(x, onehot), x[:, cols])
    # a transposed operand would fail this shape check (T, E) = (5, 3)
    assert got.shape == (5, 3)
