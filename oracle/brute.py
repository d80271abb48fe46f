"""Per-token brute-force forms of the routing, layout, forward and backward. Pure-Python loops
(with vector dot products inside one token), for tiny inputs only. They follow the same readings
as ``routing`` and ``ffn`` but are written independently of them, token by token, so that the
vectorised oracle can be checked against them. Test infrastructure only.
"""
from __future__ import annotations

import math

import numpy as np


def route_token(logit_row, k):
    """Experts sorted by (logit descending, index ascending), NaN as -inf; gates from the full
    softmax restricted to the k chosen experts and renormalised."""
    vals = [(-math.inf if math.isnan(float(v)) else float(v)) for v in logit_row]
    order = sorted(range(len(vals)), key=lambda e: (-vals[e], e))
    chosen = order[:k]
    m = max(vals)
    p = [math.exp(v - m) for v in vals]
    z = sum(p)
    sel = [p[e] / z for e in chosen]
    s = sum(sel)
    return chosen, [q / s for q in sel]


def layout(idx, T, E, e0, E_local, n, P_c):
    tc = -(-T // n)
    k = len(idx[0]) if T else 0
    counts = [[0] * E for _ in range(n)]
    offsets = [[0] * (E_local + 1) for _ in range(n)]
    row_of = [[-1] * k for _ in range(T)]
    src = [-1] * (n * P_c)
    for c in range(n):
        s, e = min(T, c * tc), min(T, (c + 1) * tc)
        for t in range(s, e):
            for j in range(k):
                counts[c][int(idx[t][j])] += 1
        r = 0
        for el in range(E_local):
            offsets[c][el] = r
            for t in range(s, e):
                for j in range(k):
                    if int(idx[t][j]) == e0 + el:
                        row_of[t][j] = c * P_c + r
                        src[c * P_c + r] = t
                        r += 1
        offsets[c][E_local] = r
    return counts, offsets, row_of, src


def _expert(x_t, w1e, w2e):
    I = w1e.shape[0] // 2
    g = w1e[:I] @ x_t
    u = w1e[I:] @ x_t
    sg = 1.0 / (1.0 + np.exp(-g))
    h = g * sg * u
    return g, u, sg, h, w2e @ h


def forward(x, logits, w1, w2, k, e0, E_local):
    """y[t] = sum over chosen local experts of gate * W2 (silu(W1g x) * (W1u x))."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        chosen, g = route_token(logits[t], k)
        for j, e in enumerate(chosen):
            if e0 <= e < e0 + E_local:
                y[t] += g[j] * _expert(x[t], w1[e - e0], w2[e - e0])[4]
    return y


def backward(x, logits, w1, w2, w_r, dy, k, e0, E_local):
    """Token-by-token VJP of ``forward`` for L = <dy, y>, with logits = x W_r^T as the router's
    caller-side projection (router term in dx and dW_r)."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, H = x.shape
    E = w_r.shape[0]
    I = w1.shape[1] // 2
    dx = np.zeros((T, H))
    dw1 = np.zeros(w1.shape)
    dw2 = np.zeros(w2.shape)
    dwr = np.zeros((E, H))
    dlogits = np.zeros((T, E))
    for t in range(T):
        chosen, g = route_token(logits[t], k)
        dg = [0.0] * k
        for j, e in enumerate(chosen):
            if not (e0 <= e < e0 + E_local):
                continue
            el = e - e0
            gg, u, sg, h, f = _expert(x[t], w1[el], w2[el])
            dg[j] = float(dy[t] @ f)
            dyd = g[j] * dy[t]
            dh = w2[el].T @ dyd
            dgate = dh * u * sg * (1.0 + gg * (1.0 - sg))
            dup = dh * gg * sg
            dx[t] += w1[el, :I].T @ dgate + w1[el, I:].T @ dup
            dw2[el] += np.outer(dyd, h)
            dw1[el, :I] += np.outer(dgate, x[t])
            dw1[el, I:] += np.outer(dup, x[t])
        s = sum(g[j] * dg[j] for j in range(k))
        for j, e in enumerate(chosen):
            dl = g[j] * (dg[j] - s)
            dlogits[t, e] = dl
            dx[t] += dl * w_r[e]
            dwr[e] += dl * x[t]
    return dict(dx=dx, dw1=dw1, dw2=dw2, dwr=dwr, dlogits=dlogits)
