"""Python binding of libmoe.so: one GPU's share of a MoE layer (route, dispatch, expert SwiGLU
FFN, combine, their backward, and the chunked layer primitives) on MI355X.

Argument marshalling only: every function here forwards to the C ABI of ``include/moe.h`` with the
same name. Tensors may be passed as torch tensors (their ``data_ptr()`` is used), raw integer
device addresses, or None (NULL). ``stream`` defaults to torch's current stream. PyTorch is used
for device memory and streams only (see :func:`allocate`); all computation runs in the HIP
library, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int, c_int32, c_int64, c_void_p
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
STATUS = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_CAPACITY", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: {STATUS.get(status, status)}: {message}")
        self.status = status


class MoeDesc(Structure):
    _fields_ = [("T", c_int64), ("H", c_int32), ("I", c_int32), ("E", c_int32), ("e0", c_int32),
                ("E_local", c_int32), ("k", c_int32), ("n_chunks", c_int32), ("P_c", c_int64),
                ("P_out", c_int64), ("dtype", c_int32), ("flags", c_int32)]


FLAG_FP8_DGRAD = 1
FLAG_FP8_WGRAD = 2
FLAG_FP8_DXD = 4  # dxd as block-scaled e4m3 rows (codes, then per-256-column scales) in the dxd buffer


TENSOR_FIELDS = ["x", "logits", "w1", "w1_scale", "w2", "w2_scale", "w_r", "dy",
                 "topk_idx", "gates", "counts", "offsets", "row_of", "src_token", "xd", "xd_scale",
                 "gu", "h", "h_scale", "yd", "out",
                 "dyd", "dgates", "dlogits", "dwr_acc", "dgu", "dxd", "dx", "dw1", "dw2", "dwr",
                 "workspace",
                 "w1t", "w1t_scale", "w2t", "w2t_scale", "dyd_q", "dyd_scale", "dgu_q", "dgu_scale",
                 "dyd_t", "dyd_cs", "dgu_t", "dgu_cs", "xd_t", "xd_cs", "h_t", "h_cs"]


class MoeTensors(Structure):
    _fields_ = [(f, c_void_p) for f in TENSOR_FIELDS]


SIZE_FIELDS = ["topk_idx", "gates", "counts", "offsets", "row_of", "src_token", "xd", "xd_scale", "gu",
               "h", "h_scale", "yd", "out", "dyd", "dgates", "dlogits", "dwr_acc", "dgu", "dxd", "dx",
               "dw1", "dw2", "dwr", "route_scratch", "route_bwd_scratch", "workspace",
               "w1t", "w1t_scale", "w2t", "w2t_scale", "dyd_q", "dyd_scale", "dgu_q", "dgu_scale",
               "dyd_t", "dyd_cs", "dgu_t", "dgu_cs", "xd_t", "xd_cs", "h_t", "h_cs",
               "wgrad_scratch", "wgrad_zero_bytes"]


class MoeWorkspaceSizes(Structure):
    _fields_ = [(f, c_int64) for f in SIZE_FIELDS]


_LIB = None

_SIGS = {
    "moe_route": [POINTER(MoeDesc), c_int] + [c_void_p] * 9,
    "moe_route_x": [POINTER(MoeDesc), c_int] + [c_void_p] * 11,
    "moe_route_noalloc": [POINTER(MoeDesc), c_int] + [c_void_p] * 8,
    "moe_dispatch": [POINTER(MoeDesc), c_int] + [c_void_p] * 6,
    "moe_expert_ffn": [POINTER(MoeDesc), c_int] + [c_void_p] * 12,
    "moe_combine": [POINTER(MoeDesc), c_int] + [c_void_p] * 5,
    "moe_combine_bwd": [POINTER(MoeDesc), c_int] + [c_void_p] * 7,
    "moe_route_bwd": [POINTER(MoeDesc), c_int] + [c_void_p] * 9,
    "moe_expert_ffn_bwd": [POINTER(MoeDesc), c_int] + [c_void_p] * 13,
    "moe_expert_wgrad": [POINTER(MoeDesc)] + [c_void_p] * 9,
    "moe_dispatch_bwd": [POINTER(MoeDesc), c_int] + [c_void_p] * 7,
    "moe_quantize_rows_fp8": [c_int64, c_int32] + [c_void_p] * 4,
    "moe_quantize_cols_fp8": [c_int64, c_int64, c_int32] + [c_void_p] * 4,
    "moe_expert_dgrad_fp8": [POINTER(MoeDesc), c_int] + [c_void_p] * 14,
    "moe_expert_wgrad_fp8": [POINTER(MoeDesc)] + [c_void_p] * 16,
    "moe_stash_store": [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                        c_void_p, c_int32, c_int32, c_void_p],
    "moe_stash_load": [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                       c_void_p, c_int32, c_void_p],
    "moe_layer_forward": [POINTER(MoeDesc), POINTER(MoeTensors), c_void_p, c_void_p],
    "moe_layer_backward": [POINTER(MoeDesc), POINTER(MoeTensors), c_void_p, c_void_p],
    "moe_layer_forward_backward": [POINTER(MoeDesc), POINTER(MoeTensors), c_void_p, c_void_p],
    "moe_required_extent": [c_int64, c_int32, c_int32, c_int32, POINTER(c_int64), POINTER(c_int64)],
    "moe_workspace_bytes": [POINTER(MoeDesc), POINTER(MoeWorkspaceSizes)],
    "moe_extent_tracker_create": [],
    "moe_extent_tracker_destroy": [c_void_p],
    "moe_extent_acquire": [c_void_p, c_int64, POINTER(c_int64)],
    "moe_extent_release": [c_void_p, c_int64],
    "moe_extent_current": [c_void_p, c_int64],
    "moe_trace_enable": [c_int32],
    "moe_trace_enable_only": [c_char_p],
    "moe_trace_disable": [],
    "moe_trace_count": [],
    "moe_trace_entry": [c_int64, POINTER(c_char_p), POINTER(c_void_p), POINTER(ctypes.c_float)],
    "moe_trace_span": [c_int64, POINTER(ctypes.c_float), POINTER(ctypes.c_float)],
    "moe_last_error": [],
    "moe_abi_version": [],
}
_RESTYPE = {"moe_extent_tracker_create": c_void_p, "moe_extent_tracker_destroy": None, "moe_trace_count": c_int64,
            "moe_extent_current": c_int64, "moe_last_error": c_char_p, "moe_abi_version": c_int32}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m combine_moe_route_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _RESTYPE.get(name, c_int)
        _LIB = L
    return _LIB


def exported_symbols():
    return list(_SIGS)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, name: str) -> None:
    if status != 0:
        raise MoeError(status, name, lib().moe_last_error().decode())


def last_error() -> str:
    return lib().moe_last_error().decode()


def make_desc(T, H, I, E, E_local, k, n_chunks, dtype="bf16", e0=0, P_c=None, P_out=None, flags=0) -> MoeDesc:
    pc, po = required_extent(T, k, E_local, n_chunks)
    return MoeDesc(T=T, H=H, I=I, E=E, e0=e0, E_local=E_local, k=k, n_chunks=n_chunks,
                   P_c=pc if P_c is None else P_c, P_out=po if P_out is None else P_out,
                   dtype=DTYPES[dtype] if isinstance(dtype, str) else dtype, flags=flags)


# ------------------------------------------------------------------ stage calls (same names)

def moe_route(d, chunk, logits, topk_idx, gates, counts, offsets, row_of, src_token, workspace, stream=None):
    _check(lib().moe_route(ctypes.byref(d), chunk, _ptr(logits), _ptr(topk_idx), _ptr(gates), _ptr(counts),
                           _ptr(offsets), _ptr(row_of), _ptr(src_token), _ptr(workspace), _stream(stream)),
           "moe_route")


def moe_route_noalloc(d, chunk, logits, topk_idx, gates, counts, offsets, row_of, src_token, stream=None):
    _check(lib().moe_route_noalloc(ctypes.byref(d), chunk, _ptr(logits), _ptr(topk_idx), _ptr(gates), _ptr(counts),
                                   _ptr(offsets), _ptr(row_of), _ptr(src_token), _stream(stream)),
           "moe_route_noalloc")


def moe_route_x(d, chunk, x, w_r, logits, topk_idx, gates, counts, offsets, row_of, src_token, workspace,
                stream=None):
    _check(lib().moe_route_x(ctypes.byref(d), chunk, _ptr(x), _ptr(w_r), _ptr(logits), _ptr(topk_idx), _ptr(gates),
                             _ptr(counts), _ptr(offsets), _ptr(row_of), _ptr(src_token), _ptr(workspace),
                             _stream(stream)), "moe_route_x")


def moe_dispatch(d, chunk, x, row_of, xd, xd_scale=None, h_scale=None, stream=None):
    _check(lib().moe_dispatch(ctypes.byref(d), chunk, _ptr(x), _ptr(row_of), _ptr(xd), _ptr(xd_scale),
                              _ptr(h_scale), _stream(stream)), "moe_dispatch")


def moe_expert_ffn(d, chunk, xd, xd_scale, w1, w1_scale, w2, w2_scale, offsets, gu, h, h_scale, yd, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(d), chunk, _ptr(xd), _ptr(xd_scale), _ptr(w1), _ptr(w1_scale),
                                _ptr(w2), _ptr(w2_scale), _ptr(offsets), _ptr(gu), _ptr(h), _ptr(h_scale),
                                _ptr(yd), _stream(stream)), "moe_expert_ffn")


def moe_combine(d, chunk, yd, gates, row_of, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(d), chunk, _ptr(yd), _ptr(gates), _ptr(row_of), _ptr(out),
                             _stream(stream)), "moe_combine")


def moe_combine_bwd(d, chunk, dy, yd, gates, row_of, dyd, dgates, stream=None):
    _check(lib().moe_combine_bwd(ctypes.byref(d), chunk, _ptr(dy), _ptr(yd), _ptr(gates), _ptr(row_of),
                                 _ptr(dyd), _ptr(dgates), _stream(stream)), "moe_combine_bwd")


def moe_route_bwd(d, chunk, dgates, gates, topk_idx, x, dlogits, dwr_acc, dwr, workspace, stream=None):
    _check(lib().moe_route_bwd(ctypes.byref(d), chunk, _ptr(dgates), _ptr(gates), _ptr(topk_idx), _ptr(x),
                               _ptr(dlogits), _ptr(dwr_acc), _ptr(dwr), _ptr(workspace), _stream(stream)),
           "moe_route_bwd")


def moe_expert_ffn_bwd(d, chunk, dyd, xd, gu, h, w1, w2, offsets, dgu, dxd, dw1=None, dw2=None, workspace=None,
                       stream=None):
    _check(lib().moe_expert_ffn_bwd(ctypes.byref(d), chunk, _ptr(dyd), _ptr(xd), _ptr(gu), _ptr(h), _ptr(w1),
                                    _ptr(w2), _ptr(offsets), _ptr(dgu), _ptr(dxd), _ptr(dw1), _ptr(dw2),
                                    _ptr(workspace), _stream(stream)), "moe_expert_ffn_bwd")


def moe_expert_wgrad(d, dyd, dgu, xd, h, offsets, dw1, dw2, workspace, stream=None):
    _check(lib().moe_expert_wgrad(ctypes.byref(d), _ptr(dyd), _ptr(dgu), _ptr(xd), _ptr(h), _ptr(offsets),
                                  _ptr(dw1), _ptr(dw2), _ptr(workspace), _stream(stream)), "moe_expert_wgrad")


def moe_dispatch_bwd(d, chunk, dxd, row_of, topk_idx, dlogits, w_r, dx, stream=None):
    _check(lib().moe_dispatch_bwd(ctypes.byref(d), chunk, _ptr(dxd), _ptr(row_of), _ptr(topk_idx),
                                  _ptr(dlogits), _ptr(w_r), _ptr(dx), _stream(stream)), "moe_dispatch_bwd")


def moe_quantize_cols_fp8(batch, rows, cols, src_bf16, codes_t, scale, stream=None):
    _check(lib().moe_quantize_cols_fp8(batch, rows, cols, _ptr(src_bf16), _ptr(codes_t), _ptr(scale),
                                       _stream(stream)), "moe_quantize_cols_fp8")


def moe_expert_dgrad_fp8(d, chunk, dyd, gu, w1t, w1t_scale, w2t, w2t_scale, offsets, dyd_q, dyd_scale, dgu,
                         dgu_q, dgu_scale, dxd, stream=None):
    _check(lib().moe_expert_dgrad_fp8(ctypes.byref(d), chunk, _ptr(dyd), _ptr(gu), _ptr(w1t), _ptr(w1t_scale),
                                      _ptr(w2t), _ptr(w2t_scale), _ptr(offsets), _ptr(dyd_q), _ptr(dyd_scale),
                                      _ptr(dgu), _ptr(dgu_q), _ptr(dgu_scale), _ptr(dxd), _stream(stream)),
           "moe_expert_dgrad_fp8")


def moe_expert_wgrad_fp8(d, dyd, dgu, xd, h, offsets, dyd_t, dyd_cs, dgu_t, dgu_cs, xd_t, xd_cs, h_t, h_cs, dw1,
                         dw2, stream=None):
    _check(lib().moe_expert_wgrad_fp8(ctypes.byref(d), _ptr(dyd), _ptr(dgu), _ptr(xd), _ptr(h), _ptr(offsets),
                                      _ptr(dyd_t), _ptr(dyd_cs), _ptr(dgu_t), _ptr(dgu_cs), _ptr(xd_t),
                                      _ptr(xd_cs), _ptr(h_t), _ptr(h_cs), _ptr(dw1), _ptr(dw2), _stream(stream)),
           "moe_expert_wgrad_fp8")


def moe_quantize_rows_fp8(rows, cols, src_bf16, codes, scale, stream=None):
    _check(lib().moe_quantize_rows_fp8(rows, cols, _ptr(src_bf16), _ptr(codes), _ptr(scale), _stream(stream)),
           "moe_quantize_rows_fp8")


def moe_stash_store(src, src_scale, live_rows, row_bytes, pool, pool_scale, num_pages, page_rows, pages,
                    page_meta=None, owner=0, max_ctas=0, stream=None):
    _check(lib().moe_stash_store(_ptr(src), _ptr(src_scale), live_rows, row_bytes, _ptr(pool), _ptr(pool_scale),
                                 num_pages, page_rows, _ptr(pages), _ptr(page_meta), owner, max_ctas,
                                 _stream(stream)), "moe_stash_store")


def moe_stash_load(pool, pool_scale, live_rows, row_bytes, num_pages, page_rows, pages, dst, dst_scale=None,
                   recycled=None, max_ctas=0, stream=None):
    _check(lib().moe_stash_load(_ptr(pool), _ptr(pool_scale), live_rows, row_bytes, num_pages, page_rows,
                                _ptr(pages), _ptr(dst), _ptr(dst_scale), _ptr(recycled), max_ctas,
                                _stream(stream)), "moe_stash_load")


def _tensors(bufs: Dict[str, object]) -> MoeTensors:
    t = MoeTensors()
    for f in TENSOR_FIELDS:
        setattr(t, f, _ptr(bufs.get(f)))
    return t


def moe_layer_forward(d, bufs, compute_stream=None, aux_stream=None):
    t = _tensors(bufs)
    _check(lib().moe_layer_forward(ctypes.byref(d), ctypes.byref(t), _stream(compute_stream),
                                   _stream(aux_stream)), "moe_layer_forward")


def moe_layer_backward(d, bufs, compute_stream=None, aux_stream=None):
    t = _tensors(bufs)
    _check(lib().moe_layer_backward(ctypes.byref(d), ctypes.byref(t), _stream(compute_stream),
                                    _stream(aux_stream)), "moe_layer_backward")


def moe_layer_forward_backward(d, bufs, compute_stream=None, aux_stream=None):
    t = _tensors(bufs)
    _check(lib().moe_layer_forward_backward(ctypes.byref(d), ctypes.byref(t), _stream(compute_stream),
                                            _stream(aux_stream)), "moe_layer_forward_backward")


# ------------------------------------------------------------------ host-only helpers

def required_extent(T, k, E_local, n_chunks):
    pc, po = c_int64(), c_int64()
    _check(lib().moe_required_extent(T, k, E_local, n_chunks, ctypes.byref(pc), ctypes.byref(po)),
           "moe_required_extent")
    return pc.value, po.value


def workspace_bytes(d) -> Dict[str, int]:
    s = MoeWorkspaceSizes()
    _check(lib().moe_workspace_bytes(ctypes.byref(d), ctypes.byref(s)), "moe_workspace_bytes")
    return {f: getattr(s, f) for f in SIZE_FIELDS}


class ExtentTracker:
    """Live-extent high-water tracker of the C ABI (one owner thread)."""

    def __init__(self):
        self._h = lib().moe_extent_tracker_create()
        if not self._h:
            raise MemoryError("moe_extent_tracker_create failed")

    def acquire(self, rows: int) -> int:
        h = c_int64()
        _check(lib().moe_extent_acquire(self._h, rows, ctypes.byref(h)), "moe_extent_acquire")
        return h.value

    def release(self, handle: int) -> None:
        _check(lib().moe_extent_release(self._h, handle), "moe_extent_release")

    def current(self, required_rows: int) -> int:
        return lib().moe_extent_current(self._h, required_rows)

    def __del__(self):
        if getattr(self, "_h", None) and _LIB is not None:
            _LIB.moe_extent_tracker_destroy(self._h)
            self._h = None


def moe_trace_enable(timing: bool = False) -> None:
    _check(lib().moe_trace_enable(1 if timing else 0), "moe_trace_enable")


def moe_trace_enable_only(name: str) -> None:
    """Log every launch, with timing events on the launches called `name` only."""
    _check(lib().moe_trace_enable_only(name.encode()), "moe_trace_enable_only")


def moe_trace_disable() -> None:
    _check(lib().moe_trace_disable(), "moe_trace_disable")


def moe_trace_entries():
    """The launch log of this thread: list of (kernel name, stream handle, device ms or -1)."""
    L = lib()
    out = []
    for i in range(L.moe_trace_count()):
        name, stream, ms = c_char_p(), c_void_p(), ctypes.c_float()
        _check(L.moe_trace_entry(i, ctypes.byref(name), ctypes.byref(stream), ctypes.byref(ms)),
               "moe_trace_entry")
        out.append((name.value.decode(), stream.value or 0, ms.value))
    return out


def moe_trace_timeline():
    """Timed launch log as (kernel name, stream handle, start ms, end ms), times after entry 0."""
    L = lib()
    out = []
    for i, (name, stream, _ms) in enumerate(moe_trace_entries()):
        t0, t1 = ctypes.c_float(), ctypes.c_float()
        _check(L.moe_trace_span(i, ctypes.byref(t0), ctypes.byref(t1)), "moe_trace_span")
        out.append((name, stream, t0.value, t1.value))
    return out


# ------------------------------------------------------------------ device buffers (torch plumbing)

def allocate(d: MoeDesc, device="cuda", backward: bool = True, fill=None):
    """Allocate every caller buffer of a descriptor with torch (fresh ``torch.empty``).

    Returns a dict name -> tensor. Payload tensors use torch.float32 / torch.bfloat16 / torch.uint8
    (FP8 codes) as the descriptor's dtype says; index arrays are int32; scales, gates and
    accumulators float32. ``out`` is a fresh [P_out, H] tensor; use ``out[:T]`` for the logical rows.
    """
    import torch
    T, H, I, E, El, k, n = d.T, d.H, d.I, d.E, d.E_local, d.k, d.n_chunks
    P = n * d.P_c
    fp8 = d.dtype == MOE_FP8_E4M3
    pay = torch.float32 if d.dtype == MOE_F32 else torch.bfloat16
    ws = workspace_bytes(d)
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    spec = {
        "topk_idx": ((T, k), i32), "gates": ((T, k), f32), "counts": ((n, E), i32),
        "offsets": ((n, El + 1), i32), "row_of": ((T, k), i32), "src_token": ((P,), i32),
        "xd": ((P, H), u8 if fp8 else pay), "h": ((P, I), pay), "yd": ((P, H), pay),
        "out": ((d.P_out, H), pay), "workspace": ((max(1, ws["workspace"]),), u8),
    }
    if fp8:
        # h: [P, I] BF16 values followed by their [P, I] e4m3 codes
        spec.update({"xd_scale": ((P,), f32), "h_scale": ((P,), f32), "h": ((3 * P * I,), u8)})
    else:
        spec["gu"] = ((P, 2 * I), pay)
    if backward and not fp8:
        spec.update({"dyd": ((P, H), pay), "dgates": ((T, k), f32), "dlogits": ((T, E), f32),
                     "dwr_acc": ((E, H), f32), "dgu": ((P, 2 * I), pay), "dxd": ((P, H), pay),
                     "dx": ((T, H), pay), "dw1": ((El, 2 * I, H), pay), "dw2": ((El, H, I), pay),
                     "dwr": ((E, H), pay)})
    if backward and (d.flags & FLAG_FP8_DGRAD):
        # transposed per-column FP8 weights (moe_quantize_cols_fp8) and the quantised payloads
        spec.update({"w1t": ((El, H, 2 * I), u8), "w1t_scale": ((El, H), f32), "w2t": ((El, I, H), u8),
                     "w2t_scale": ((El, I), f32), "dyd_q": ((P, H), u8), "dyd_scale": ((P,), f32),
                     "dgu_q": ((P, 2 * I), u8), "dgu_scale": ((P,), f32)})
    if backward and (d.flags & FLAG_FP8_WGRAD):
        # per-expert transposed FP8 operands of the weight gradients (sizes from the library)
        for name in ("dyd_t", "dgu_t", "xd_t", "h_t"):
            spec[name] = ((max(1, ws[name]),), u8)
        for name in ("dyd_cs", "dgu_cs", "xd_cs", "h_cs"):
            spec[name] = ((max(1, ws[name] // 4),), f32)
    out = {}
    for name, (shape, dt) in spec.items():
        if name == "workspace":
            # zeroed: the weight-gradient counters inside it must be zero when first used
            out[name] = torch.zeros(shape, dtype=dt, device=device)
            continue
        out[name] = torch.empty(shape, dtype=dt, device=device)
        if fill is not None:
            out[name].fill_(fill)
    return out
