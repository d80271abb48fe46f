"""Routing and layout oracle: top-k selection, renormalised gates, counts, offsets and the stable
permutation into expert-contiguous rows. Test infrastructure only (see the package header).

Readings (the pages print no routing formula; token-wise ChunkedEP, Megatron-LM PR 7342,
"Summary", names top-k routing with token-wise chunks; OpenPipe/ART PR 971 names the
expert-contiguous dispatch extent rounded up to four rows):
  * selection is on the FP32 logits: slot 0 holds the largest logit, ties go to the lower expert
    index, NaN ranks as -inf;
  * gates: softmax over all E experts, keep the k selected probabilities, renormalise them to
    sum 1 (which equals a softmax over the k selected logits);
  * chunks are contiguous token ranges of ceil(T/n) tokens, the last takes the remainder;
  * local experts are the contiguous range [e0, e0 + E_local); each chunk c owns a row region
    starting at c * P_c; inside it, rows are grouped by local expert in ascending expert order
    and, within an expert, by ascending token index (a token picks an expert at most once).
"""
from __future__ import annotations

import numpy as np


def round4(x: int) -> int:
    """Round a row count up to a multiple of four (ART PR 971, extent rounded up to four rows)."""
    return ((int(x) + 3) // 4) * 4


def chunk_bounds(T: int, n: int):
    """Token ranges [start, end) of the n token-wise chunks (ChunkedEP, "Summary")."""
    if n <= 0:
        raise ValueError("n_chunks must be positive")
    tc = -(-T // n)
    return [(min(T, c * tc), min(T, (c + 1) * tc)) for c in range(n)]


def required_extent(T: int, k: int, E_local: int, n: int):
    """Default extents: P_c = round4(ceil(T/n) * min(k, E_local)) rows per chunk region and
    P_out = round4(T * k) rows of combine output (tiny-case rule P = ceil(T*k/4)*4)."""
    tc = -(-T // n)
    return round4(tc * min(k, E_local)), max(round4(T * k), round4(T))


def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """Router projection before the top-k: logits[t, e] = sum_h x[t, h] * W_r[e, h] (FP64).

    The pages give the router weight only through its gradient (ChunkedEP "Numerical status --
    unresolved": FP32 accumulation of the router-weight gradient across chunks); the projection is
    its plain forward counterpart, the linear map whose weight-gradient is dlogits^T x.
    """
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T


def route(logits: np.ndarray, k: int):
    """Top-k selection and renormalised softmax gates for every token.

    Returns idx [T, k] int32 (descending logit, ties to the lower index) and gates [T, k]
    float64 computed as: p = softmax over all E; g_j = p[idx_j] / sum_i p[idx_i].
    """
    lg = np.asarray(logits)
    if lg.dtype not in (np.float32, np.float64):
        lg = lg.astype(np.float64)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("k out of range")
    key = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    # stable argsort of the negated key: equal logits keep ascending expert order
    idx = np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)
    z = key - key.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    gates = sel / sel.sum(axis=1, keepdims=True)
    return idx, gates


def layout(idx: np.ndarray, E: int, e0: int, E_local: int, n: int, P_c: int):
    """Per-chunk expert histogram, local offsets and the stable permutation.

    counts [n, E]       number of (t, j) slots of chunk c that chose expert e (all experts)
    offsets [n, E_l+1]  exclusive prefix sum of counts[c, e0:e0+E_l]; offsets[c, E_l] = N_c
    row_of [T, k]       c*P_c + offsets[c, e-e0] + #{t' < t in chunk c choosing e}; -1 if e is
                        not local
    src_token [n*P_c]   token of each row; -1 for rows N_c..P_c-1 of every region
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros((n, E), dtype=np.int32)
    offsets = np.zeros((n, E_local + 1), dtype=np.int32)
    row_of = np.full((T, k), -1, dtype=np.int32)
    src_token = np.full(n * P_c, -1, dtype=np.int32)
    for c, (s, e) in enumerate(chunk_bounds(T, n)):
        sub = idx[s:e].reshape(-1).astype(np.int64)
        counts[c] = np.bincount(sub, minlength=E)[:E]
        loc = counts[c, e0:e0 + E_local]
        offsets[c, 1:] = np.cumsum(loc)
        N_c = int(offsets[c, E_local])
        if N_c > P_c:
            raise ValueError("P_c below the number of local assignments")
        slots = np.arange(sub.size, dtype=np.int64)            # t_local * k + j
        is_local = (sub >= e0) & (sub < e0 + E_local)
        chosen = slots[is_local]
        order = np.argsort(sub[is_local], kind="stable")        # by expert, then by slot
        rows = c * P_c + np.arange(N_c, dtype=np.int64)
        flat = row_of[s:e].reshape(-1)
        flat[chosen[order]] = rows
        row_of[s:e] = flat.reshape(e - s, k)
        src_token[rows] = s + chosen[order] // k
    return counts, offsets, row_of, src_token


def dispatch(x: np.ndarray, src_token: np.ndarray) -> np.ndarray:
    """Expert-contiguous rows: xd[row] = x[src_token[row]]; unused rows are zero here (the
    kernel leaves them unwritten and they are never compared)."""
    xd = np.zeros((src_token.size, x.shape[1]), dtype=x.dtype)
    v = src_token >= 0
    xd[v] = x[src_token[v]]
    return xd


def unpermute(xd: np.ndarray, row_of: np.ndarray) -> np.ndarray:
    """Inverse of dispatch for each local slot: returns [T, k, H] with xd[row_of[t, j]] (zero for
    non-local slots). Dispatch followed by this is the identity on every local slot."""
    T, k = row_of.shape
    out = np.zeros((T, k, xd.shape[1]), dtype=xd.dtype)
    m = row_of >= 0
    out[m] = xd[row_of[m]]
    return out
