"""Vectorised FP64 forward and backward of the MoE layer share (per-expert matmuls).
Test infrastructure only (see the package header).

Readings (the pages name the operations, not their formulas):
  * Expert FFN is SwiGLU without biases: W1[e] is [2I, H] with rows 0..I-1 the gate projection
    and rows I..2I-1 the up projection, W2[e] is [H, I];
    G = xd W1g^T, U = xd W1u^T, h = silu(G) * U with silu(z) = z / (1 + exp(-z)), yd = h W2^T.
  * Combine (ART PR 971, "fresh [P, H] output ... cropped to the logical result"):
    out[t] = sum over slots j whose expert is local of gate[t, j] * yd[row_of[t, j]]; a token
    with no local expert gets a zero row.
  * Backward is the vector-Jacobian product of the forward for L = <dy, out>, with the router
    projection logits = x W_r^T being the caller's: the router term adds dlogits W_r to dx and
    dlogits^T x to dW_r. Router weight gradients are summed over all chunks before any rounding
    (token-wise ChunkedEP, "Numerical status -- unresolved": FP32 accumulation across chunks
    before a single dtype conversion; FP64 here).
"""
from __future__ import annotations

import numpy as np

from .routing import chunk_bounds, dispatch, layout, route


def silu(z):
    return z / (1.0 + np.exp(-z))


def _segments(offsets: np.ndarray, P_c: int):
    n, El1 = offsets.shape
    for c in range(n):
        for e in range(El1 - 1):
            r0 = c * P_c + int(offsets[c, e])
            r1 = c * P_c + int(offsets[c, e + 1])
            yield e, r0, r1


def expert_ffn(xd: np.ndarray, offsets: np.ndarray, P_c: int, w1: np.ndarray, w2: np.ndarray):
    """Grouped SwiGLU over every expert segment. Returns gu [P, 2I], h [P, I], yd [P, H] (FP64;
    rows outside every segment are zero)."""
    I = w1.shape[1] // 2
    P, H = xd.shape
    gu = np.zeros((P, 2 * I))
    h = np.zeros((P, I))
    yd = np.zeros((P, H))
    for e, r0, r1 in _segments(offsets, P_c):
        if r1 == r0:
            continue
        a = xd[r0:r1].astype(np.float64)
        w = w1[e].astype(np.float64)
        g = a @ w[:I].T
        u = a @ w[I:].T
        gu[r0:r1, :I] = g
        gu[r0:r1, I:] = u
        h[r0:r1] = silu(g) * u
        yd[r0:r1] = h[r0:r1] @ w2[e].astype(np.float64).T
    return gu, h, yd


def combine(yd: np.ndarray, gates: np.ndarray, row_of: np.ndarray) -> np.ndarray:
    """out [T, H] = sum_j (j ascending, local slots only) gates[t, j] * yd[row_of[t, j]]."""
    T, k = row_of.shape
    out = np.zeros((T, yd.shape[1]))
    for j in range(k):
        m = row_of[:, j] >= 0
        out[m] += gates[m, j, None] * yd[row_of[m, j]]
    return out


def forward(x, logits, w1, w2, *, k, e0, E_local, n_chunks, P_c=None):
    """Route -> layout -> dispatch -> expert FFN -> combine. Returns a dict of every intermediate."""
    T, H = x.shape
    E = logits.shape[1]
    if P_c is None:
        tc = -(-T // n_chunks)
        P_c = ((tc * min(k, E_local) + 3) // 4) * 4
    idx, gates = route(logits, k)
    counts, offsets, row_of, src_token = layout(idx, E, e0, E_local, n_chunks, P_c)
    xd = dispatch(np.asarray(x, dtype=np.float64), src_token)
    gu, h, yd = expert_ffn(xd, offsets, P_c, w1, w2)
    out = combine(yd, gates, row_of)
    return dict(idx=idx, gates=gates, counts=counts, offsets=offsets, row_of=row_of,
                src_token=src_token, xd=xd, gu=gu, h=h, yd=yd, out=out, P_c=P_c,
                k=k, e0=e0, E_local=E_local, n_chunks=n_chunks)


def combine_bwd(dy, yd, gates, row_of, P):
    """dyd[row_of[t, j]] = gates[t, j] * dy[t]; dgates[t, j] = <dy[t], yd[row_of[t, j]]> for
    local slots, 0 for the others (their expert output is not part of this share)."""
    T, k = row_of.shape
    dy = np.asarray(dy, dtype=np.float64)
    dyd = np.zeros((P, dy.shape[1]))
    dgates = np.zeros((T, k))
    for j in range(k):
        m = row_of[:, j] >= 0
        r = row_of[m, j]
        dyd[r] = gates[m, j, None] * dy[m]
        dgates[m, j] = np.einsum("th,th->t", dy[m], yd[r])
    return dyd, dgates


def route_bwd(dgates, gates, idx, E):
    """Softmax-over-selected VJP: dlogits[t, idx[t, j]] = g_j (dg_j - sum_i g_i dg_i); zero for
    unselected experts."""
    T, k = idx.shape
    s = np.sum(gates * dgates, axis=1, keepdims=True)
    dsel = gates * (dgates - s)
    dlogits = np.zeros((T, E))
    np.put_along_axis(dlogits, idx.astype(np.int64), dsel, axis=1)
    return dlogits


def ffn_bwd(dyd, xd, gu, h, offsets, P_c, w1, w2):
    """Per expert: dh = dyd W2; dG = dh * U * s * (1 + G (1 - s)) with s = sigmoid(G);
    dU = dh * silu(G); dxd = [dG dU] W1; dW2 = dyd^T h; dW1 = [dG dU]^T xd (summed over every
    chunk's rows of that expert; an expert with no row gets zero gradients)."""
    I = w1.shape[1] // 2
    P, H = xd.shape
    dgu = np.zeros((P, 2 * I))
    dxd = np.zeros((P, H))
    dw1 = np.zeros(w1.shape)
    dw2 = np.zeros(w2.shape)
    for e, r0, r1 in _segments(offsets, P_c):
        if r1 == r0:
            continue
        g = gu[r0:r1, :I]
        u = gu[r0:r1, I:]
        sg = 1.0 / (1.0 + np.exp(-g))
        dh = dyd[r0:r1] @ w2[e].astype(np.float64)
        dgu[r0:r1, :I] = dh * u * sg * (1.0 + g * (1.0 - sg))
        dgu[r0:r1, I:] = dh * g * sg
        dxd[r0:r1] = dgu[r0:r1] @ w1[e].astype(np.float64)
        dw2[e] += dyd[r0:r1].T @ h[r0:r1]
        dw1[e] += dgu[r0:r1].T @ xd[r0:r1]
    return dgu, dxd, dw1, dw2


def dispatch_bwd(dxd, row_of, dlogits, w_r):
    """dx[t] = sum over local slots of dxd[row_of[t, j]] + dlogits[t] W_r (router term)."""
    T, k = row_of.shape
    dx = np.asarray(dlogits, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64)
    for j in range(k):
        m = row_of[:, j] >= 0
        dx[m] += dxd[row_of[m, j]]
    return dx


def backward(fwd: dict, x, dy, w1, w2, w_r):
    """Full backward of :func:`forward` for L = <dy, out>."""
    T, H = np.asarray(x).shape
    P = fwd["src_token"].size
    E = np.asarray(w_r).shape[0]
    dyd, dgates = combine_bwd(dy, fwd["yd"], fwd["gates"], fwd["row_of"], P)
    dlogits = route_bwd(dgates, fwd["gates"], fwd["idx"], E)
    dgu, dxd, dw1, dw2 = ffn_bwd(dyd, fwd["xd"], fwd["gu"], fwd["h"], fwd["offsets"], fwd["P_c"], w1, w2)
    dx = dispatch_bwd(dxd, fwd["row_of"], dlogits, w_r)
    x64 = np.asarray(x, dtype=np.float64)
    dwr = np.zeros((E, H))
    for s, e in chunk_bounds(T, fwd["n_chunks"]):     # FP64 running sum over chunks
        dwr += dlogits[s:e].T @ x64[s:e]
    return dict(dyd=dyd, dgates=dgates, dlogits=dlogits, dgu=dgu, dxd=dxd, dx=dx, dw1=dw1,
                dw2=dw2, dwr=dwr)
