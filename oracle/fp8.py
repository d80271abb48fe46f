"""FP8 (OCP e4m3fn) payload oracle. Test infrastructure only.

The pages name BF16/FP8 payloads for the token copy kernels (torchtitan PR 5541, "AI-Generated
Details" and "Verification") and say nothing more. Readings:
  * encoding: OCP e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinity,
    0x7F/0xFF NaN, largest finite 448, subnormals m * 2^-9), round to nearest even, saturating
    at +-448;
  * per-row absmax scaling: amax = max |a| over the row; the quantiser multiplies by the FP32
    value 448 / amax (FP32 division), rounds the FP32 product to e4m3, and stores the FP32
    dequantisation scale amax / 448; an all-zero row stores code 0 and scale 1. Both sides take
    these FP32 steps, so the codes are compared bit for bit;
  * activations are scaled per token (row of x), weights per output channel (row of W1[e] over
    H, row of W2[e] over I), h per dispatched row (over I) before the down projection;
  * products accumulate in FP32 (exactly, here in FP64) and are dequantised by s_row * s_col;
  * the dispatch-backward payload dxd (FP8 payloads extended to dispatch backward; the pages give
    the FP8 payload only as a copy-kernel format) is the BF16 dxd row
    quantised per block of 256 consecutive columns, each block taking the row quantiser's FP32
    steps on its own values (a block-scaled row: H / 256 scales per row). The block is the column
    tile of the GEMM that produces dxd, so the producer can quantise what it stores without a
    second pass over the row.
"""
from __future__ import annotations

import numpy as np

from .ffn import _segments as ffn_segments
from .ffn import combine, silu
from .routing import dispatch, layout, route

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.zeros(256)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        ex = (code >> 3) & 0xF
        m = code & 0x7
        if ex == 0xF and m == 0x7:
            vals[code] = np.nan
        elif ex == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return vals


_TABLE = e4m3_decode_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round FP32 values to e4m3fn codes: nearest, ties to even mantissa, saturating at 448.
    Elementwise; large arrays go through in blocks of 2^20 values (same result, less memory)."""
    v = np.asarray(v, dtype=np.float32)
    if v.size > 1 << 20:
        flat = np.ascontiguousarray(v).reshape(-1)
        out = np.empty(flat.size, dtype=np.uint8)
        for i in range(0, flat.size, 1 << 20):
            out[i:i + (1 << 20)] = _e4m3_encode_block(flat[i:i + (1 << 20)])
        return out.reshape(v.shape)
    return _e4m3_encode_block(v)


def _e4m3_encode_block(v: np.ndarray) -> np.ndarray:
    a = np.abs(v).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # binade of a: a = f * 2^ex with f in [0.5, 1), so floor(log2 a) = ex - 1; subnormals share
    # the 2^-6 binade's quantum 2^-9
    ex = np.frexp(a)[1].astype(np.int64) - 1
    ex = np.maximum(ex, -6)
    quantum = np.ldexp(1.0, ex - 3)
    mag = np.round(a / quantum) * quantum                 # numpy rounds half to even
    mag = np.minimum(mag, E4M3_MAX)
    # encode the rounded magnitude
    ex2 = np.frexp(np.where(mag > 0, mag, 1.0))[1].astype(np.int64) - 1
    normal = mag >= 2.0 ** -6
    efield = np.where(normal, ex2 + 7, 0)
    mfield = np.where(normal, np.round(mag / np.ldexp(1.0, ex2) * 8.0) - 8.0,
                      np.round(mag / 2.0 ** -9)).astype(np.int64)
    code = (efield << 3) | mfield
    code = np.where(np.signbit(v), code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows(a: np.ndarray):
    """Per-row absmax quantisation (FP32 steps as stated in the module header).
    Returns (codes uint8 [R, K], scale float32 [R])."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    amax = np.max(np.abs(a), axis=-1) if a.shape[-1] else np.zeros(a.shape[:-1], np.float32)
    amax = amax.astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    v = (a * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(v)
    codes[zero] = 0
    scale = np.where(zero, np.float32(1.0), (safe / np.float32(E4M3_MAX)).astype(np.float32))
    return codes, scale.astype(np.float32)


def dequantize_rows(codes, scale):
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


DXD_BLOCK = 256


def quantize_row_blocks(a: np.ndarray, block: int = DXD_BLOCK):
    """Block-scaled rows: every run of `block` consecutive columns of a row (the last run may be
    shorter) is quantised as one row by :func:`quantize_rows`. Returns codes uint8 [R, C] and
    scale float32 [R, ceil(C / block)]."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    R, C = a.shape
    nb = -(-C // block) if C else 0
    codes = np.zeros((R, C), dtype=np.uint8)
    scale = np.ones((R, nb), dtype=np.float32)
    for b in range(nb):
        c0, c1 = b * block, min(C, (b + 1) * block)
        codes[:, c0:c1], scale[:, b] = quantize_rows(a[:, c0:c1])
    return codes, scale


def dequantize_row_blocks(codes, scale, block: int = DXD_BLOCK):
    """Values of block-scaled rows: code value times its block's scale (FP64)."""
    v = e4m3_decode(codes)
    C = v.shape[-1]
    col_scale = np.repeat(np.asarray(scale, dtype=np.float64), block, axis=-1)[..., :C]
    return v * col_scale


def quantize_cols_t(a: np.ndarray):
    """Per-column absmax quantisation stored transposed: a [..., R, C] -> codes [..., C, R] and
    scale [..., C], column j taking the role of a row in :func:`quantize_rows` (same FP32 steps).
    Reading for the FP8 input gradients: they contract a weight matrix over its rows, so the
    weight's scale must sit on its columns, and the transposed store makes the contracted
    dimension contiguous."""
    return quantize_rows(np.swapaxes(np.asarray(a, dtype=np.float32), -1, -2))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round FP32 values to the nearest BF16 value, ties to even (finite inputs); FP32 out."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def ffn_bwd_fp8_dgrad(dyd, xd, gu, h, offsets, P_c, w1, w2):
    """Expert FFN backward with FP8 input gradients (the pages fix FP8 only
    for payloads, so these are readings):
      * dyd, the combine-backward payload, is stored in BF16 and quantised per row;
      * W2[e] and W1[e] are quantised per column and transposed (:func:`quantize_cols_t`);
      * dh = deq(dyd) deq(W2t[e])^T, then dG, dU as in ffn.ffn_bwd from the saved G, U;
      * dgu = [dG dU] is stored in BF16 and quantised per row; dxd = deq(dgu) deq(W1t[e])^T;
      * products accumulate exactly (FP64 here) and dequantise by s_row * s_col;
      * the weight gradients here are the BF16 ones, dW2 = dyd^T h and dW1 = dgu^T xd from the
        unquantised values (per-row payload scales sit on the dimension they contract over; the
        FP8 form with per-column scales is :func:`ffn_wgrad_fp8`).
    Returns dgu, dxd, dw1, dw2 (FP64)."""
    I = w1.shape[1] // 2
    P, H = xd.shape
    dyd = np.asarray(dyd, dtype=np.float64)
    dgu = np.zeros((P, 2 * I))
    dxd = np.zeros((P, H))
    dw1 = np.zeros(w1.shape)
    dw2 = np.zeros(w2.shape)
    wq = {}   # per expert: the dequantised transposed weights

    def wt(e):
        if e not in wq:
            wq[e] = (dequantize_rows(*quantize_cols_t(w2[e])),    # W2t [I, H]
                     dequantize_rows(*quantize_cols_t(w1[e])))    # W1t [H, 2I]
        return wq[e]

    # rows are quantised independently, so only the segments' rows are quantised
    for e, r0, r1 in ffn_segments(offsets, P_c):
        if r1 == r0:
            continue
        dyd_q = dequantize_rows(*quantize_rows(bf16_round(dyd[r0:r1])))
        w2t, w1t = wt(e)
        g = gu[r0:r1, :I]
        u = gu[r0:r1, I:]
        sg = 1.0 / (1.0 + np.exp(-g))
        dh = dyd_q @ w2t.T
        dgu[r0:r1, :I] = dh * u * sg * (1.0 + g * (1.0 - sg))
        dgu[r0:r1, I:] = dh * g * sg
        dw2[e] += dyd[r0:r1].T @ h[r0:r1]
        dw1[e] += dgu[r0:r1].T @ xd[r0:r1]
        dgu_q = dequantize_rows(*quantize_rows(bf16_round(dgu[r0:r1])))
        dxd[r0:r1] = dgu_q @ w1t.T
    return dgu, dxd, dw1, dw2


def expert_rows(offsets, P_c, e):
    """Dispatch rows of local expert e over every chunk, in chunk order."""
    offsets = np.asarray(offsets)
    return np.concatenate([np.arange(c * P_c + offsets[c, e], c * P_c + offsets[c, e + 1])
                           for c in range(offsets.shape[0])]).astype(np.int64)


def ffn_wgrad_fp8(dyd, dgu, xd, h, offsets, P_c, El):
    """Expert weight gradients on FP8 (a reading: the pages give FP8 only for
    forward payloads). A weight gradient contracts over the expert's token rows, so its operands are
    scaled per column over those rows (every chunk's rows of the expert together): for each
    operand, the BF16-rounded rows of expert e are quantised per column (:func:`quantize_cols_t`,
    the FP32 steps of the row quantiser) and
      dW2[e] = deq(dyd_e)^T deq(h_e),   dW1[e] = deq(dgu_e)^T deq(xd_e),
    accumulated exactly (FP64) and dequantised by s_col(A) * s_col(B). An expert without rows
    gets zeros. Returns dw1 [El, 2I, H], dw2 [El, H, I] (FP64)."""
    H = np.asarray(xd).shape[1]
    I = np.asarray(h).shape[1]
    dw1 = np.zeros((El, 2 * I, H))
    dw2 = np.zeros((El, H, I))

    def tq(a, rows):   # transposed, per-column dequantised operand [C, R]
        return dequantize_rows(*quantize_cols_t(bf16_round(np.asarray(a, dtype=np.float64)[rows])))

    for e in range(El):
        rows = expert_rows(offsets, P_c, e)
        if rows.size == 0:
            continue
        dw2[e] = tq(dyd, rows) @ tq(h, rows).T
        dw1[e] = tq(dgu, rows) @ tq(xd, rows).T
    return dw1, dw2


def dispatch_bwd_fp8(dxd, row_of, dlogits, w_r, block: int = DXD_BLOCK):
    """Dispatch backward on the FP8 payload: dxd (exact values) is rounded to BF16, quantised per
    row and column block (:func:`quantize_row_blocks`), and the dequantised rows replace dxd in
    oracle.ffn.dispatch_bwd (router term unchanged)."""
    from . import ffn
    pay = dequantize_row_blocks(*quantize_row_blocks(bf16_round(np.asarray(dxd, dtype=np.float64)), block),
                                block)
    return ffn.dispatch_bwd(pay, row_of, dlogits, w_r)


def backward_fp8_dgrad(fwd: dict, x, dy, w1, w2, w_r, fp8_dgrad=True, fp8_wgrad=False, fp8_dxd=False):
    """The layer backward (oracle.ffn.backward) with the expert FFN's input gradients and dW1 from
    :func:`ffn_bwd_fp8_dgrad` (fp8_dgrad) and/or the expert weight gradients from
    :func:`ffn_wgrad_fp8` (fp8_wgrad) and/or dx from the FP8 dispatch-backward payload
    (:func:`dispatch_bwd_fp8`, fp8_dxd); combine, routing and the router weight gradient are those
    of the BF16 backward, which does not depend on them."""
    from . import ffn
    base = ffn.backward(fwd, x, dy, w1, w2, w_r)
    out = dict(base)
    if fp8_dgrad:
        dgu, dxd, dw1, dw2 = ffn_bwd_fp8_dgrad(base["dyd"], fwd["xd"], fwd["gu"], fwd["h"], fwd["offsets"],
                                              fwd["P_c"], w1, w2)
        dx = ffn.dispatch_bwd(dxd, fwd["row_of"], base["dlogits"], w_r)
        out.update(dgu=dgu, dxd=dxd, dx=dx, dw1=dw1, dw2=dw2)
    if fp8_dxd:
        out["dx"] = dispatch_bwd_fp8(out["dxd"], fwd["row_of"], base["dlogits"], w_r)
    if fp8_wgrad:
        out["dw1"], out["dw2"] = ffn_wgrad_fp8(out["dyd"], out["dgu"], fwd["xd"], fwd["h"], fwd["offsets"],
                                               fwd["P_c"], np.asarray(w1).shape[0])
    return out


def forward(x, logits, w1, w2, *, k, e0, E_local, n_chunks, P_c=None, wq=None):
    """FP8 forward: quantise x per token and weights per output channel, grouped GEMMs with
    FP64 accumulation and s_row * s_col dequantisation, h quantised per row before the down
    projection; yd and combine unrounded (FP64).

    wq: optional precomputed (w1_codes, w1_scale, w2_codes, w2_scale)."""
    T, H = x.shape
    E = logits.shape[1]
    if P_c is None:
        tc = -(-T // n_chunks)
        P_c = ((tc * min(k, E_local) + 3) // 4) * 4
    idx, gates = route(logits, k)
    counts, offsets, row_of, src_token = layout(idx, E, e0, E_local, n_chunks, P_c)
    xq, xs = quantize_rows(x)                   # per token
    if wq is None:
        w1q, w1s = quantize_rows(w1)            # [E_l, 2I, H] codes, [E_l, 2I] scales
        w2q, w2s = quantize_rows(w2)            # [E_l, H, I] codes, [E_l, H] scales
    else:
        w1q, w1s, w2q, w2s = wq
    xdq = dispatch(xq.astype(np.int64), src_token).astype(np.uint8)
    xds = np.ones(src_token.size, dtype=np.float32)
    v = src_token >= 0
    xds[v] = xs[src_token[v]]
    I = w1.shape[1] // 2
    P = src_token.size
    h = np.zeros((P, I))
    yd = np.zeros((P, H))
    hq_all = np.zeros((P, I), dtype=np.uint8)
    hs_all = np.ones(P, dtype=np.float32)
    for c in range(n_chunks):
        for e in range(E_local):
            r0 = c * P_c + int(offsets[c, e])
            r1 = c * P_c + int(offsets[c, e + 1])
            if r1 == r0:
                continue
            a = e4m3_decode(xdq[r0:r1])
            acc = a @ e4m3_decode(w1q[e]).T
            gu = acc * xds[r0:r1, None].astype(np.float64) * w1s[e][None, :].astype(np.float64)
            hh = silu(gu[:, :I]) * gu[:, I:]
            h[r0:r1] = hh
            hq, hs = quantize_rows(hh.astype(np.float32))
            hq_all[r0:r1] = hq
            hs_all[r0:r1] = hs
            acc2 = e4m3_decode(hq) @ e4m3_decode(w2q[e]).T
            yd[r0:r1] = acc2 * hs[:, None].astype(np.float64) * w2s[e][None, :].astype(np.float64)
    out = combine(yd, gates, row_of)
    return dict(idx=idx, gates=gates, counts=counts, offsets=offsets, row_of=row_of,
                src_token=src_token, xq=xq, xs=xs, xdq=xdq, xds=xds, w1q=w1q, w1s=w1s,
                w2q=w2q, w2s=w2s, h=h, hq=hq_all, hs=hs_all, yd=yd, out=out, P_c=P_c)
