"""Pins for the FP8 encoder (torch's float8_e4m3fn, the OCP table, error bounds) and for the
extent bookkeeping (the numbers printed in ART PR 971's native validation)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import extent, fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_closed_forms():
    t = fp8.e4m3_decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    finite = t[np.isfinite(t)]
    assert finite.size == 254


def test_e4m3_encode_round_trips_every_code():
    t = fp8.e4m3_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    back = fp8.e4m3_encode(t[codes].astype(np.float32))
    # +0 and -0 keep their sign bit; every other code maps to itself
    np.testing.assert_array_equal(back, codes)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 50,
        (rng.uniform(-1, 1, 50000) * 2.0 ** -6).astype(np.float32),            # subnormal range
        (rng.uniform(-448, 448, 50000)).astype(np.float32),
    ])
    t = fp8.e4m3_decode_table()
    mids = [(t[c] + t[c + 1]) / 2 for c in range(0, 0x7E)]                       # exact ties
    v = np.concatenate([v, np.array(mids, np.float32), -np.array(mids, np.float32)])
    v = v[np.abs(v) <= 448]
    ours = fp8.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates():
    v = np.array([449.0, 464.0, 1e6, -500.0, 480.0], np.float32)
    np.testing.assert_array_equal(fp8.e4m3_encode(v), [0x7E, 0x7E, 0x7E, 0xFE, 0x7E])


def test_quantize_rows_error_bound_and_zero_row():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((64, 300)).astype(np.float32) * rng.uniform(0.01, 10, (64, 1)).astype(np.float32)
    a[5] = 0
    codes, scale = fp8.quantize_rows(a)
    assert np.all(codes[5] == 0) and scale[5] == 1.0
    deq = fp8.dequantize_rows(codes, scale)
    bound = 2.0 ** -4 * np.abs(a) + 2.0 ** -9 * scale[:, None] * (1 + 1e-6)
    assert np.all(np.abs(deq - a) <= bound)
    # the row maximum maps onto +-448 (up to one FP32 rounding of amax * (448 / amax))
    top = np.abs(fp8.e4m3_decode(codes)).max(1)
    assert np.all(top[np.arange(64) != 5] == 448.0)


def test_extent_tracker_reproduces_art971_fixture():
    g = json.load(open(os.path.join(GOLDEN, "extent_art971.json")))
    tr = extent.ExtentTracker()
    H, es, rows = g["H"], g["elem_size_bf16"], g["logical_rows"]
    floor0 = g["workspace_floor_sequence"][0]
    assert extent.workspace_floor(floor0, tr.current(rows), H, es) == g["workspace_floor_sequence"][0]
    hnd = tr.acquire(g["live_extent_rows"])
    P = tr.current(rows)
    assert P == g["live_extent_rows"]
    assert extent.output_bytes(P, H, es) == g["bytes_with_live_extent"]
    assert extent.workspace_floor(floor0, P, H, es) == g["workspace_floor_sequence"][1]
    tr.release(hnd)
    P = tr.current(rows)
    assert extent.output_bytes(P, H, es) == g["bytes_after_release"] == g["retained_bytes"]
    assert extent.workspace_floor(floor0, P, H, es) == g["workspace_floor_sequence"][2]
    # the live extent needs zero growth of the native buffer, yet the output is a fresh allocation
    assert g["live_extent_rows"] <= g["native_buffer_rows"]
    assert g["output_floor_bytes_review"] == 2 ** 19 * 1709


def test_extent_tracker_semantics():
    tr = extent.ExtentTracker()
    assert tr.current(0) == 0 and tr.current(5) == 8
    a = tr.acquire(101)
    b = tr.acquire(37)
    assert tr.current(10) == 104          # max with the live high-water, rounded up to 4
    assert tr.current(200) == 200         # a larger own extent wins (maximum, not sum)
    tr.release(a)
    assert tr.current(10) == 40
    tr.release(b)
    assert tr.current(10) == 12
    with pytest.raises(KeyError):
        tr.release(b)


def test_router_accum_fp32_across_chunks_reproduces_the_pages_direction():
    """Token-wise ChunkedEP (Megatron-LM PR 7342, "Numerical status -- unresolved"): the router
    weight gradient accumulated across chunks in FP32 and converted once lands within 6.774e-5
    relative L2 of the unchunked result, where per-chunk BF16 accumulation had been 2.871e-3 away
    (numbers in the golden file). On the oracle's own dlogits and x (FP64), with the two-chunk
    split of its chunk_bounds: emulating FP32 accumulation of the chunk partials, then one BF16
    conversion, stays within 1e-4 of the one-chunk BF16 result; per-chunk BF16 accumulation is
    more than 1e-3 away, within a factor of ten of the page's figure, and more than ten times
    further than the FP32 path. The oracle's backward sums dW_r over the chunks: its result does
    not depend on the chunk count."""
    import moe_inputs
    import oracle
    from oracle import ffn as offn
    g = json.load(open(os.path.join(GOLDEN, "router_fp32_accum_megatron7342.json")))
    cfg = moe_inputs.MoeConfig("racc", T=4096, H=256, I=64, E=32, E_local=8, k=4, n_chunks=2, dtype="bf16",
                               seed_base=600, backward=True)
    inp = moe_inputs.make_inputs(cfg, parts=("x", "logits"))
    idx, gates = oracle.route(inp["logits"], cfg.k)
    dg = moe_inputs.make_dgates(cfg).astype(np.float64)
    dl = offn.route_bwd(dg, gates, idx, cfg.E)
    x = inp["x"].astype(np.float64)

    def bf16(a):
        return moe_inputs.bf16_bits_to_f32(moe_inputs.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))
    (s0, e0), (s1, e1) = oracle.chunk_bounds(cfg.T, 2)
    p0, p1 = dl[s0:e0].T @ x[s0:e0], dl[s1:e1].T @ x[s1:e1]
    native = bf16(dl.T @ x)
    fp32_acc = bf16(np.float32(p0.astype(np.float32) + p1.astype(np.float32)))
    per_chunk_bf16 = bf16(bf16(p0) + bf16(p1))
    chunked, naive = rel(fp32_acc, native), rel(per_chunk_bf16, native)
    assert chunked <= 1e-4
    assert naive >= 1e-3 and naive >= 10 * chunked
    assert g["router_rel_l2_before_fix"] / 10 <= naive <= 10 * g["router_rel_l2_before_fix"]
    assert chunked <= 10 * g["router_rel_l2_fp32_accum"]
    assert abs(g["max_abs_error"] - 2.0 ** -23) < 1e-11   # the printed max error is one FP32 ulp at 1
    # the oracle's dW_r: a sum over chunks that does not depend on the chunk split
    full = moe_inputs.make_inputs(cfg, parts=("x", "logits", "w1", "w2", "w_r", "dy"))
    res = []
    for n in (1, 2, 3):
        f = oracle.forward(full["x"], full["logits"], full["w1"], full["w2"], k=cfg.k, e0=0, E_local=cfg.E_local,
                           n_chunks=n)
        res.append(oracle.backward(f, full["x"], full["dy"], full["w1"], full["w2"], full["w_r"])["dwr"])
    for r in res[1:]:
        np.testing.assert_allclose(r, res[0], rtol=1e-10, atol=1e-12)
    assert np.linalg.norm(res[0]) > 0
    np.testing.assert_allclose(p0 + p1, dl.T @ x, rtol=1e-12, atol=1e-12)


def _exact_e4m3_rows(rng, shape):
    """Random e4m3-representable values whose every row has absmax exactly 448 (scale 1)."""
    t = fp8.e4m3_decode_table()
    finite = t[np.isfinite(t)]
    a = rng.choice(finite, size=shape).astype(np.float32)
    a[..., 0] = 448.0
    return a


def test_fp8_forward_exact_when_quantisation_is_identity():
    import oracle
    rng = np.random.default_rng(21)
    T, H, I, E, k = 40, 32, 16, 4, 2
    x = _exact_e4m3_rows(rng, (T, H)) * np.float32(2.0 ** -6)        # per-row scale 2^-6 exactly
    w1 = _exact_e4m3_rows(rng, (E, 2 * I, H)) * np.float32(2.0 ** -12)
    w2 = _exact_e4m3_rows(rng, (E, H, I)) * np.float32(2.0 ** -12)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    f8 = fp8.forward(x, logits, w1, w2, k=k, e0=0, E_local=E, n_chunks=2)
    f64 = oracle.forward(x, logits, w1, w2, k=k, e0=0, E_local=E, n_chunks=2)
    np.testing.assert_array_equal(f8["xs"], np.float32(2.0 ** -6))
    np.testing.assert_array_equal(fp8.dequantize_rows(f8["xq"], f8["xs"]), x)
    used = f64["src_token"] >= 0
    np.testing.assert_allclose(f8["h"][used], f64["h"][used], rtol=1e-12, atol=1e-30)
    # the down projection sees h through one per-row quantisation: bounded relative error
    err = np.linalg.norm(f8["out"] - f64["out"]) / np.linalg.norm(f64["out"])
    assert err < 2.0 ** -4


def test_fp8_forward_close_to_exact_forward():
    import oracle
    rng = np.random.default_rng(22)
    T, H, I, E, El, k = 96, 64, 48, 8, 4, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    w1 = (rng.standard_normal((El, 2 * I, H)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((El, H, I)) * 0.05).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    f8 = fp8.forward(x, logits, w1, w2, k=k, e0=2, E_local=El, n_chunks=2)
    f64 = oracle.forward(x, logits, w1, w2, k=k, e0=2, E_local=El, n_chunks=2)
    for key in ("idx", "counts", "offsets", "row_of", "src_token"):
        np.testing.assert_array_equal(f8[key], f64[key])
    err = np.linalg.norm(f8["out"] - f64["out"]) / np.linalg.norm(f64["out"])
    # four independent e4m3 roundings (x, W1, h, W2), each about 3.6% RMS relative (3 mantissa
    # bits): sqrt(4) * 3.6% = 7.2% expected; a misplaced scale is off by orders of magnitude
    assert 1e-3 < err < 0.1
    # codes of dispatched rows are the token's codes
    v = f8["src_token"] >= 0
    np.testing.assert_array_equal(f8["xdq"][v], f8["xq"][f8["src_token"][v]])


# ----------------------------------------------------------------------------- FP8 input gradients

def test_bf16_round_ties_to_even():
    from oracle.fp8 import bf16_round
    one = 1.0
    vals = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -20,
                     -(one + 2.0 ** -8), 3.0], dtype=np.float32)
    want = np.array([one, one, one + 2.0 ** -6, one + 2.0 ** -7, -one, 3.0], dtype=np.float32)
    np.testing.assert_array_equal(bf16_round(vals), want)


def test_quantize_cols_transposed_worked_example():
    """Column j is quantised as a row would be and stored as row j of the transposed codes:
    column 0 (absmax 448, inverse 1): 448 -> 0x7E, -224 -> 0xF6; column 1 (absmax 1, inverse 448):
    1 -> 448 -> 0x7E, 0.5 -> 224 -> 0x76, scale 1/448; column 2 (all zero): codes 0, scale 1."""
    from oracle.fp8 import quantize_cols_t
    a = np.array([[448.0, 1.0, 0.0], [-224.0, 0.5, 0.0]], dtype=np.float32)
    codes, scale = quantize_cols_t(a)
    np.testing.assert_array_equal(codes, np.array([[0x7E, 0xF6], [0x7E, 0x76], [0, 0]], dtype=np.uint8))
    np.testing.assert_array_equal(scale, np.array([1.0, np.float32(1.0) / np.float32(448.0), 1.0], dtype=np.float32))


def _fp8_exact_case(seed=3):
    """Two experts whose dyd rows hold values in {0, +-1/2, +-1} and a 3.5 (scale 3.5/448 = 2^-7)
    and whose weight columns hold values in {0, +-1/4, +-1/2} and a +-1.75 (scale 2^-8): every
    scale is a power of two and every scaled value an e4m3 value, so per-row and per-column
    quantisation of these is lossless."""
    rng = np.random.default_rng(seed)
    H, I, El = 64, 32, 2
    rows = [5, 7]
    P_c = 16
    offsets = np.array([[0, rows[0], rows[0] + rows[1]]])
    dyd = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(P_c, H))
    dyd[:, 0] = 3.5
    w1 = rng.choice([0.0, 0.25, -0.25, 0.5, -0.5], size=(El, 2 * I, H))
    w1[:, 0, :] = 1.75
    w2 = rng.choice([0.0, 0.25, -0.25, 0.5, -0.5], size=(El, H, I))
    w2[:, 0, :] = -1.75
    xd = rng.normal(size=(P_c, H))
    gu = rng.normal(size=(P_c, 2 * I))
    h = rng.normal(size=(P_c, I))
    return dyd, xd, gu, h, offsets, P_c, w1, w2


def test_fp8_dgrad_oracle_is_exact_on_e4m3_exact_inputs():
    """With e4m3-exact dyd and W2, the FP8 dh (hence dgu and both weight gradients) equals the
    exact backward's: a transposed or mis-scaled W2 path fails this."""
    from oracle import ffn
    from oracle.fp8 import ffn_bwd_fp8_dgrad
    dyd, xd, gu, h, offsets, P_c, w1, w2 = _fp8_exact_case()
    dgu8, dxd8, dw18, dw28 = ffn_bwd_fp8_dgrad(dyd, xd, gu, h, offsets, P_c, w1, w2)
    dgu, dxd, dw1, dw2 = ffn.ffn_bwd(dyd, xd, gu, h, offsets, P_c, w1, w2)
    np.testing.assert_allclose(dgu8, dgu, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw18, dw1, rtol=0, atol=1e-9)
    np.testing.assert_allclose(dw28, dw2, rtol=0, atol=1e-9)


def test_fp8_dgrad_oracle_dxd_within_e4m3_bound():
    """dgu is not e4m3-exact, so dxd carries its quantisation error: each dequantised value is
    within 2^-4 relative (plus 2^-9 of the row scale) of the BF16-rounded dgu, which bounds the
    relative L2 error of dxd by about 2^-4 times the condition of the product; W1 is e4m3-exact,
    so a wrong transpose or a dropped scale (errors of order 1) fails."""
    from oracle import ffn
    from oracle.fp8 import ffn_bwd_fp8_dgrad
    dyd, xd, gu, h, offsets, P_c, w1, w2 = _fp8_exact_case()
    _, dxd8, _, _ = ffn_bwd_fp8_dgrad(dyd, xd, gu, h, offsets, P_c, w1, w2)
    _, dxd, _, _ = ffn.ffn_bwd(dyd, xd, gu, h, offsets, P_c, w1, w2)
    rows = slice(0, int(offsets[0, -1]))
    err = np.linalg.norm(dxd8[rows] - dxd[rows]) / np.linalg.norm(dxd[rows])
    assert 0 < err < 2.0 ** -4, err


def test_fp8_dgrad_layer_backward_changes_only_the_expert_input_gradients():
    """Gradients that do not pass through dgu (dgates, dlogits, dW2, the router gradient) equal
    the BF16 backward's exactly; dx and dW1 move by an e4m3-sized relative error, not more."""
    import oracle
    from oracle.fp8 import backward_fp8_dgrad
    from moe_inputs import MoeConfig, make_inputs
    cfg = MoeConfig("fp8dg", T=96, H=64, I=64, E=8, E_local=4, e0=2, k=2, n_chunks=2, dtype="bf16",
                    seed_base=70, backward=True)
    inp = make_inputs(cfg)
    f = oracle.forward(inp["x"], inp["logits"], inp["w1"], inp["w2"], k=cfg.k, e0=cfg.e0,
                       E_local=cfg.E_local, n_chunks=cfg.n_chunks)
    exact = oracle.backward(f, inp["x"], inp["dy"], inp["w1"], inp["w2"], inp["w_r"])
    q = backward_fp8_dgrad(f, inp["x"], inp["dy"], inp["w1"], inp["w2"], inp["w_r"])
    for name in ("dyd", "dgates", "dlogits", "dw2", "dwr"):
        np.testing.assert_array_equal(q[name], exact[name], err_msg=name)
    for name in ("dx", "dw1"):
        err = np.linalg.norm(q[name] - exact[name]) / np.linalg.norm(exact[name])
        assert 1e-4 < err < 2.0 ** -4, (name, err)


def _wgrad_case(exact, seed=5):
    """Two chunks of 16 rows, two local experts (rows 0-4 and 5-8 of chunk 0, 0-2 and 3-9 of
    chunk 1). exact: every column of every operand holds values in {0, +-1/2, +-1} over an expert's
    rows plus a 3.5 in the expert's first row (scale 2^-7), so per-column quantisation is lossless."""
    rng = np.random.default_rng(seed)
    P_c, H, I = 16, 32, 16
    offsets = np.array([[0, 5, 9], [0, 3, 10]])
    def draw(cols):
        if not exact:
            return rng.normal(size=(2 * P_c, cols))
        a = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(2 * P_c, cols))
        a[[0, 5]] = 3.5     # the first row of each expert (chunk 0)
        return a
    return dict(dyd=draw(H), dgu=draw(2 * I), xd=draw(H), h=draw(I), offsets=offsets, P_c=P_c, El=2)


def test_fp8_wgrad_oracle_is_exact_on_e4m3_exact_columns():
    """Against a brute-force sum of outer products over the expert's rows of both chunks."""
    from oracle.fp8 import ffn_wgrad_fp8
    c = _wgrad_case(exact=True)
    dw1, dw2 = ffn_wgrad_fp8(c["dyd"], c["dgu"], c["xd"], c["h"], c["offsets"], c["P_c"], c["El"])
    for e in range(c["El"]):
        w1 = np.zeros(dw1[e].shape)
        w2 = np.zeros(dw2[e].shape)
        for ch in range(2):
            for r in range(ch * c["P_c"] + c["offsets"][ch, e], ch * c["P_c"] + c["offsets"][ch, e + 1]):
                w2 += np.outer(c["dyd"][r], c["h"][r])
                w1 += np.outer(c["dgu"][r], c["xd"][r])
        np.testing.assert_allclose(dw2[e], w2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dw1[e], w1, rtol=0, atol=1e-12)


def test_fp8_wgrad_oracle_within_e4m3_bound():
    from oracle.fp8 import ffn_wgrad_fp8
    c = _wgrad_case(exact=False)
    dw1, dw2 = ffn_wgrad_fp8(c["dyd"], c["dgu"], c["xd"], c["h"], c["offsets"], c["P_c"], c["El"])
    for e in range(c["El"]):
        rows = np.concatenate([np.arange(ch * 16 + c["offsets"][ch, e], ch * 16 + c["offsets"][ch, e + 1])
                               for ch in range(2)])
        w2 = c["dyd"][rows].T @ c["h"][rows]
        w1 = c["dgu"][rows].T @ c["xd"][rows]
        for got, want in ((dw2[e], w2), (dw1[e], w1)):
            err = np.linalg.norm(got - want) / np.linalg.norm(want)
            assert 1e-4 < err < 2.0 ** -4, err


def test_quantize_row_blocks_one_block_is_the_row_quantiser():
    rng = np.random.default_rng(11)
    a = rng.standard_normal((40, 200)).astype(np.float32) * 3
    for block in (200, 256, 1024):
        c1, s1 = fp8.quantize_row_blocks(a, block)
        c0, s0 = fp8.quantize_rows(a)
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(s1[:, 0], s0)
        assert s1.shape == (40, 1)


def test_quantize_row_blocks_independent_bounded_ragged():
    """600 columns = blocks of 256, 256 and a ragged 88; magnitudes differ by block, one block of
    one row is all zero. Each block's maximum maps onto +-448, the error stays within the e4m3
    bound of its own block scale, and changing one block leaves the others' codes and scales."""
    rng = np.random.default_rng(12)
    R, C, B = 24, 600, 256
    mag = np.array([1e-3, 10.0, 0.5], np.float32)
    a = rng.standard_normal((R, C)).astype(np.float32)
    for b in range(3):
        a[:, b * B:(b + 1) * B] *= mag[b]
    a[7, B:2 * B] = 0
    codes, scale = fp8.quantize_row_blocks(a)
    assert codes.shape == (R, C) and scale.shape == (R, 3)
    assert np.all(codes[7, B:2 * B] == 0) and scale[7, 1] == 1.0
    deq = fp8.dequantize_row_blocks(codes, scale)
    col_scale = np.repeat(scale.astype(np.float64), B, axis=1)[:, :C]
    bound = 2.0 ** -4 * np.abs(a) + 2.0 ** -9 * col_scale * (1 + 1e-6)
    assert np.all(np.abs(deq - a) <= bound)
    for b in range(3):
        top = np.abs(fp8.e4m3_decode(codes[:, b * B:(b + 1) * B])).max(1)
        live = np.ones(R, bool)
        if b == 1:
            live[7] = False
        assert np.all(top[live] == 448.0), b
    # scales follow each block's own magnitude
    assert np.all(scale[:, 0] < scale[np.arange(R) != 7, 1].min())
    a2 = a.copy()
    a2[:, B:2 * B] *= 3.0
    c2, s2 = fp8.quantize_row_blocks(a2)
    np.testing.assert_array_equal(c2[:, :B], codes[:, :B])
    np.testing.assert_array_equal(c2[:, 2 * B:], codes[:, 2 * B:])
    np.testing.assert_array_equal(s2[:, [0, 2]], scale[:, [0, 2]])


def test_fp8_dxd_dispatch_bwd_exact_on_block_exact_rows():
    """Rows whose every 256-column block holds values in {0, +-1/2, +-1} * 2^m plus one 3.5 * 2^m,
    with m drawn per (row, block): the block scale is 2^m / 128 and every value is an e4m3 code
    times it, so the FP8 payload is lossless and dispatch backward on it equals the BF16 one
    exactly; a scale taken from the wrong block or row would break the equality."""
    from oracle import ffn
    rng = np.random.default_rng(13)
    P, H, T, k, E = 40, 768, 12, 3, 8
    m = rng.integers(-6, 4, size=(P, H // 256))
    dxd = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(P, H))
    dxd[:, ::256] = 3.5
    dxd *= np.repeat(2.0 ** m, 256, axis=1)
    row_of = rng.permutation(P)[:T * k].reshape(T, k).astype(np.int32)
    row_of[rng.random((T, k)) < 0.2] = -1
    dlogits = rng.standard_normal((T, E))
    w_r = rng.standard_normal((E, H))
    np.testing.assert_array_equal(fp8.dispatch_bwd_fp8(dxd, row_of, dlogits, w_r),
                                  ffn.dispatch_bwd(dxd, row_of, dlogits, w_r))
    # and not when one block's scale is taken from its neighbour
    codes, scale = fp8.quantize_row_blocks(dxd.astype(np.float32))
    wrong = fp8.dequantize_row_blocks(codes, np.roll(scale, 1, axis=1))
    assert not np.array_equal(wrong, dxd)


def test_fp8_dxd_layer_backward_changes_only_dx():
    """With the FP8 dispatch-backward payload every gradient but dx equals the BF16 backward's
    exactly; dx moves by an e4m3-sized relative error."""
    import oracle
    from oracle.fp8 import backward_fp8_dgrad
    from moe_inputs import MoeConfig, make_inputs
    cfg = MoeConfig("fp8dxd", T=96, H=512, I=64, E=8, E_local=4, e0=2, k=2, n_chunks=2, dtype="bf16",
                    seed_base=71, backward=True)
    inp = make_inputs(cfg)
    f = oracle.forward(inp["x"], inp["logits"], inp["w1"], inp["w2"], k=cfg.k, e0=cfg.e0,
                       E_local=cfg.E_local, n_chunks=cfg.n_chunks)
    exact = oracle.backward(f, inp["x"], inp["dy"], inp["w1"], inp["w2"], inp["w_r"])
    q = backward_fp8_dgrad(f, inp["x"], inp["dy"], inp["w1"], inp["w2"], inp["w_r"], fp8_dgrad=False,
                           fp8_dxd=True)
    for name in ("dyd", "dgates", "dlogits", "dgu", "dxd", "dw1", "dw2", "dwr"):
        np.testing.assert_array_equal(q[name], exact[name], err_msg=name)
    err = np.linalg.norm(q["dx"] - exact["dx"]) / np.linalg.norm(exact["dx"])
    assert 1e-4 < err < 2.0 ** -4, err
