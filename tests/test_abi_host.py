"""Host-only checks of the C ABI (no GPU): the library loads, exports every function declared in
include/moe.h, validates descriptors before any launch, and its host helpers (extents, workspace
sizes, live-extent tracker) agree with the oracle and with ART PR 971's printed byte counts."""
import json
import os
import re

import pytest

import oracle
from oracle import extent as oextent

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

mh = pytest.importorskip("combine_moe_route_02_amd")


def _lib_or_skip():
    if not os.path.exists(mh.LIB_PATH):
        pytest.skip("libmoe.so not built (run __graft_entry__.build())")
    return mh.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = _lib_or_skip()
    names = _declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mh.exported_symbols())
    assert L.moe_abi_version() == 4


@pytest.mark.parametrize("T,k,El,n", [(256, 2, 8, 1), (16384, 8, 16, 2), (32768, 8, 16, 2), (10, 3, 2, 3),
                                      (0, 2, 4, 2), (7, 8, 3, 4)])
def test_required_extent_matches_oracle(T, k, El, n):
    _lib_or_skip()
    assert mh.required_extent(T, k, El, n) == oracle.required_extent(T, k, El, n)


def _desc(**kw):
    base = dict(T=1000, H=256, I=192, E=32, e0=0, E_local=8, k=4, n_chunks=2, dtype="bf16")
    base.update(kw)
    if "P_c" not in base or "P_out" not in base:
        pc, po = oracle.required_extent(base["T"], max(1, base["k"]), base["E_local"], max(1, base["n_chunks"]))
        base.setdefault("P_c", pc)
        base.setdefault("P_out", po)
    dt = base.pop("dtype")
    return mh.MoeDesc(dtype=mh.DTYPES.get(dt, dt) if isinstance(dt, str) else dt, flags=0, **base)


def _status_of(fn, *a):
    try:
        fn(*a)
    except mh.MoeError as e:
        return e.status, str(e)
    return 0, ""


@pytest.mark.parametrize("kw,status", [
    (dict(k=9, E=32), -3), (dict(k=0), -1), (dict(E_local=40), -1), (dict(H=100), -3), (dict(I=32), -3),
    (dict(n_chunks=0, P_c=4, P_out=1000), -1), (dict(P_c=2002), -2), (dict(P_c=1996), -2), (dict(P_out=998), -2),
    (dict(P_out=1002), -2), (dict(dtype=7), -1), (dict(E=30, E_local=8), -3), (dict(E=2000, E_local=8), -3),
])
def test_descriptor_validation(kw, status):
    _lib_or_skip()
    d = _desc(**kw)
    st, msg = _status_of(mh.moe_route, d, 0, None, None, None, None, None, None, None, None, 0)
    assert st == status, msg
    assert mh.last_error()


def test_null_pointers_and_bad_chunk_are_rejected_before_launch():
    _lib_or_skip()
    d = _desc()
    assert _status_of(mh.moe_route, d, 0, None, None, None, None, None, None, None, None, 0)[0] == -1
    assert _status_of(mh.moe_route, d, 2, 1, 1, 1, 1, 1, 1, 1, 1, 0)[0] == -1      # chunk out of range
    assert _status_of(mh.moe_dispatch, d, -2, 1, 1, 1, None, None, 0)[0] == -1
    assert _status_of(mh.moe_combine, d, 0, None, 1, 1, 1, 0)[0] == -1
    assert _status_of(mh.moe_expert_ffn, d, 0, 1, None, 1, None, None, None, 1, None, 1, None, 1, 0)[0] == -1
    fp8 = _desc(dtype="fp8")
    assert _status_of(mh.moe_combine_bwd, fp8, 0, 1, 1, 1, 1, 1, 1, 0)[0] == -3    # FP8 is forward only
    assert _status_of(mh.moe_quantize_rows_fp8, 4, 12, 1, 1, 1, 0)[0] == -1


def test_workspace_bytes():
    _lib_or_skip()
    d = mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="bf16")
    ws = mh.workspace_bytes(d)
    P = 2 * 65536
    assert ws["xd"] == P * 2048 * 2 and ws["yd"] == P * 2048 * 2 and ws["gu"] == P * 1536 * 2
    assert ws["out"] == 131072 * 2048 * 2                     # fresh [P_out, H] BF16 output
    assert ws["dw1"] == 16 * 1536 * 2048 * 2 and ws["dwr_acc"] == 128 * 2048 * 4
    # routing / router scratch first, then the expert weight gradients' scratch at a 256-byte boundary:
    # per-(expert, tile) counters of dW1 (6 x 8 tiles) and dW2 (8 x 3 tiles), four work-queue
    # counter blocks (16 ints each: the split dW1 and dW2 lists, two row-grouped lists), then the
    # partial slots
    base = (max(ws["route_scratch"], ws["route_bwd_scratch"]) + 255) // 256 * 256
    assert ws["wgrad_zero_bytes"] == ((16 * (48 + 24) + 4 * 16) * 4 + 255) // 256 * 256
    assert ws["wgrad_scratch"] == ws["wgrad_zero_bytes"] + 2 * 192 * 256 * 256 * 4
    assert ws["workspace"] == base + ws["wgrad_scratch"] > 0
    f8 = mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="fp8")
    ws8 = mh.workspace_bytes(f8)
    assert ws8["xd"] == P * 2048 and ws8["xd_scale"] == P * 4 and ws8["dw1"] == 0
    assert ws8["wgrad_scratch"] == ws8["wgrad_zero_bytes"] == 0


def test_fp8_dgrad_flag_validation_and_sizes():
    _lib_or_skip()
    d = mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="bf16",
                     flags=mh.FLAG_FP8_DGRAD)
    ws = mh.workspace_bytes(d)
    P = 2 * 65536
    assert ws["w1t"] == 16 * 2048 * 1536 and ws["w1t_scale"] == 16 * 2048 * 4
    assert ws["w2t"] == 16 * 768 * 2048 and ws["w2t_scale"] == 16 * 768 * 4
    assert ws["dyd_q"] == P * 2048 and ws["dgu_q"] == P * 1536 and ws["dyd_scale"] == ws["dgu_scale"] == P * 4
    assert mh.workspace_bytes(mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2))["w1t"] == 0
    bad = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, flags=8)
    assert _status_of(mh.workspace_bytes, bad)[0] == -1
    f8 = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, dtype="fp8", flags=mh.FLAG_FP8_DGRAD)
    assert _status_of(mh.workspace_bytes, f8)[0] == -3
    # the stage call rejects a non-BF16 descriptor before touching any pointer
    f32 = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, dtype="f32")
    assert _status_of(mh.moe_expert_dgrad_fp8, f32, 0, *([1] * 13), 0)[0] == -3


def test_fp8_wgrad_sizes():
    _lib_or_skip()
    d = mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2, dtype="bf16",
                     flags=mh.FLAG_FP8_WGRAD | mh.FLAG_FP8_DGRAD)
    ws = mh.workspace_bytes(d)
    Kp = 2 * 65536 + 64 * 16
    assert ws["dyd_t"] == ws["xd_t"] == 2048 * Kp and ws["h_t"] == 768 * Kp and ws["dgu_t"] == 1536 * Kp
    assert ws["dyd_cs"] == ws["xd_cs"] == 16 * 2048 * 4 and ws["h_cs"] == 16 * 768 * 4 and ws["dgu_cs"] == 16 * 1536 * 4
    assert ws["w1t"] > 0   # both flags at once
    bad = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, flags=8)
    assert _status_of(mh.workspace_bytes, bad)[0] == -1
    # the FP8 dxd payload flag: accepted with the BF16 dtype, with or without the others, and the
    # sizes do not change (the payload fits the BF16 dxd buffer)
    for fl in (mh.FLAG_FP8_DXD, mh.FLAG_FP8_DXD | mh.FLAG_FP8_DGRAD | mh.FLAG_FP8_WGRAD):
        q = mh.make_desc(T=64, H=320, I=64, E=8, E_local=4, k=2, n_chunks=2, flags=fl)
        plain = mh.make_desc(T=64, H=320, I=64, E=8, E_local=4, k=2, n_chunks=2, flags=fl & ~mh.FLAG_FP8_DXD)
        assert mh.workspace_bytes(q) == mh.workspace_bytes(plain)
    assert 4 * ((320 + 255) // 256) <= 2 * 320 - 320  # scales fit after the codes in a BF16 row
    f32dxd = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, dtype="f32", flags=mh.FLAG_FP8_DXD)
    assert _status_of(mh.workspace_bytes, f32dxd)[0] == -3
    f32 = mh.make_desc(T=64, H=128, I=64, E=8, E_local=4, k=2, n_chunks=1, dtype="f32")
    assert _status_of(mh.moe_expert_wgrad_fp8, f32, *([1] * 15), 0)[0] == -3


def test_quantize_cols_argument_errors():
    _lib_or_skip()
    assert _status_of(mh.moe_quantize_cols_fp8, 1, 24, 16, 1, 1, 1, 0)[0] == -1   # rows % 16
    assert _status_of(mh.moe_quantize_cols_fp8, 1, 32, 12, 1, 1, 1, 0)[0] == -1   # cols % 8
    assert _status_of(mh.moe_quantize_cols_fp8, 1, 32, 16, None, 1, 1, 0)[0] == -1
    assert _status_of(mh.moe_quantize_cols_fp8, 0, 32, 16, None, None, None, 0)[0] == 0  # nothing to do


def test_extent_tracker_matches_art971_fixture_and_oracle():
    _lib_or_skip()
    g = json.load(open(os.path.join(GOLDEN, "extent_art971.json")))
    tr = mh.ExtentTracker()
    ot = oextent.ExtentTracker()
    H, es, rows = g["H"], g["elem_size_bf16"], g["logical_rows"]
    h = tr.acquire(g["live_extent_rows"])
    oh = ot.acquire(g["live_extent_rows"])
    assert tr.current(rows) == ot.current(rows) == g["live_extent_rows"]
    assert tr.current(rows) * H * es == g["bytes_with_live_extent"]
    tr.release(h)
    ot.release(oh)
    assert tr.current(rows) * H * es == g["bytes_after_release"]
    with pytest.raises(mh.MoeError):
        tr.release(h)
    for req, live in [(0, []), (5, []), (10, [101, 37]), (200, [101]), (3, [7, 9, 13])]:
        a, b = mh.ExtentTracker(), oextent.ExtentTracker()
        for r in live:
            a.acquire(r)
            b.acquire(r)
        assert a.current(req) == b.current(req)


def test_stash_argument_errors_before_any_launch():
    L = _lib_or_skip()
    import ctypes
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.addressof(buf)
    a16 = (a + 15) // 16 * 16
    pg = (ctypes.c_int32 * 4)()
    pa = ctypes.addressof(pg)
    # row_bytes not a multiple of 16, page_rows < 1, a scale pointer without its pair, a negative
    # size, a NULL tensor, a misaligned tensor: MOE_ERR_ARG (-1), nothing launched
    for args in [(a16, None, 4, 24, a16, None, 2, 2, pa, None, 0, 0, None),
                 (a16, None, 4, 16, a16, None, 2, 0, pa, None, 0, 0, None),
                 (a16, a16, 4, 16, a16, None, 2, 2, pa, None, 0, 0, None),
                 (a16, None, -1, 16, a16, None, 2, 2, pa, None, 0, 0, None),
                 (None, None, 4, 16, a16, None, 2, 2, pa, None, 0, 0, None),
                 (a16 + 4, None, 4, 16, a16, None, 2, 2, pa, None, 0, 0, None)]:
        assert L.moe_stash_store(*args) == -1, args
    for args in [(a16, None, 4, 16, 2, 2, pa, None, None, None, -1, None),
                 (a16, None, 4, 16, 2, 2, None, a16, None, None, 0, None)]:
        assert L.moe_stash_load(*args) == -1, args
    # an empty live prefix is valid and launches nothing (no GPU needed)
    assert L.moe_stash_store(None, None, 0, 16, None, None, 0, 1, None, None, 0, 0, None) == 0
    assert L.moe_stash_load(None, None, 0, 16, 0, 1, None, None, None, None, 0, None) == 0


def test_trace_enable_only_host_side():
    """The name-filtered launch log needs a name; enabling and disabling it touches no GPU."""
    import combine_moe_route_02_amd as mh
    L = mh.lib()
    assert L.moe_trace_enable_only(None) == -1
    mh.moe_trace_enable_only("gemm_wgrad_w1")
    assert L.moe_trace_count() == 0
    mh.moe_trace_disable()


def test_src_token_required_without_local_experts():
    """With no local expert but a non-empty dispatch region (P_c > 0), routing still marks every
    row of the region with -1, so a NULL src_token is rejected before any launch."""
    _lib_or_skip()
    d = _desc(E_local=0, e0=8, P_c=8, P_out=1000)
    st, msg = _status_of(mh.moe_route, d, 0, 1, 1, 1, 1, 1, 1, None, 1, 0)
    assert st == -1 and "src_token" in msg, msg
    st, msg = _status_of(mh.moe_route_x, _desc(E=32, E_local=0, e0=8, P_c=8, P_out=1000), 0, *([1] * 8), None, 1, 0)
    assert st == -1 and "src_token" in msg, msg
    bufs = {f: 1 for f in mh.TENSOR_FIELDS}
    bufs["src_token"] = None
    st, msg = _status_of(mh.moe_layer_forward, d, bufs, 0, 0)
    assert st == -1 and "src_token" in msg, msg


def test_extents_past_a_buffer_descriptor_are_rejected():
    """A kernel operand addressed through one buffer descriptor holds at most 2^31 - 1 bytes: the
    backward calls reject shapes whose static worst case exceeds it (MOE_ERR_UNSUPPORTED) before
    any launch, instead of reading zeros past the descriptor's extent."""
    _lib_or_skip()
    # weight-gradient segment: P_c x H x 2 = 262144 x 7168 x 2 bytes
    big = mh.make_desc(T=65536, H=7168, I=768, E=128, E_local=16, k=8, n_chunks=2)
    assert big.P_c * 7168 * 2 > 2**31 - 1
    mh.workspace_bytes(big)                       # the descriptor itself is valid
    st, msg = _status_of(mh.moe_expert_wgrad, big, *([1] * 8), 0)
    assert st == -3 and "buffer descriptor" in msg, msg
    st, _ = _status_of(mh.moe_route_bwd, big, -1, *([1] * 8), 0)
    assert st == -3
    st, _ = _status_of(mh.moe_expert_ffn_bwd, big, -1, *([1] * 12), 0)
    assert st == -3
    bufs = {f: 1 for f in mh.TENSOR_FIELDS}
    assert _status_of(mh.moe_layer_forward_backward, big, bufs, 0, 0)[0] == -3
    assert _status_of(mh.moe_layer_backward, big, bufs, 0, 0)[0] == -3
    # FP8 weight-gradient operand: max(H, 2I) x (n P_c + 64) codes, with the BF16 segment in range
    f8 = mh.make_desc(T=200000, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=4,
                      flags=mh.FLAG_FP8_WGRAD | mh.FLAG_FP8_DGRAD)
    assert f8.P_c * 2048 * 2 <= 2**31 - 1 < 2048 * (4 * f8.P_c + 64)
    assert _status_of(mh.moe_layer_backward, f8, bufs, 0, 0)[0] == -3
    plain = mh.make_desc(T=200000, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=4)
    assert _status_of(mh.moe_expert_wgrad_fp8, plain, *([1] * 15), 0)[0] == -3
    # an expert's W1 past one descriptor
    assert _status_of(mh.workspace_bytes, mh.make_desc(T=64, H=65536, I=16384, E=8, E_local=4, k=2,
                                                       n_chunks=1))[0] == -3


def test_host_helpers_do_not_initialise_hip():
    """The host-only helpers (extents, workspace sizes, the live-extent tracker, argument
    validation) never initialise the HIP runtime: a fresh process that calls them opens no GPU
    device file (/dev/kfd, /dev/dri/*) and the runtime reports no initialisation."""
    import subprocess
    import sys
    _lib_or_skip()
    code = r'''
import os, sys
sys.path.insert(0, sys.argv[1])
import combine_moe_route_02_amd as mh
d = mh.make_desc(T=16384, H=2048, I=768, E=128, E_local=16, k=8, n_chunks=2)
mh.workspace_bytes(d)
mh.required_extent(16384, 8, 16, 2)
tr = mh.ExtentTracker(); h = tr.acquire(262144); tr.current(131072); tr.release(h)
try:
    mh.moe_route(mh.make_desc(T=10, H=100, I=64, E=8, E_local=4, k=2, n_chunks=1), 0, *([None] * 8), 0)
except mh.MoeError:
    pass
mh.moe_trace_enable_only("x"); mh.moe_trace_disable()
fds = []
for f in os.listdir("/proc/self/fd"):
    try:
        fds.append(os.readlink("/proc/self/fd/" + f))
    except OSError:
        pass
bad = [p for p in fds if p.startswith("/dev/kfd") or p.startswith("/dev/dri")]
maps = open("/proc/self/maps").read()
print("OPEN_GPU_FILES", bad, "KFD_MAPPED", "/dev/kfd" in maps)
'''
    r = subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True, timeout=120,
                       env={k: v for k, v in os.environ.items() if k != "HIP_VISIBLE_DEVICES"})
    assert r.returncode == 0, r.stderr
    assert "OPEN_GPU_FILES [] KFD_MAPPED False" in r.stdout, r.stdout


def test_noalloc_route_size_limit_is_checked_on_the_host():
    """moe_route_noalloc rejects a call whose histograms exceed its fixed 4 MiB device scratch
    before touching the GPU (T = 65536, E = 1024, one chunk: 1024 blocks x 4 x 1024 x 4 = 16 MiB)."""
    _lib_or_skip()
    d = mh.make_desc(T=65536, H=128, I=64, E=1024, E_local=8, k=2, n_chunks=1, dtype="bf16")
    st, msg = _status_of(mh.moe_route_noalloc, d, -1, 1, 1, 1, 1, 1, 1, 1, 0)
    assert st == -3 and "scratch" in msg, msg
    assert _status_of(mh.moe_route_noalloc, _desc(), 0, None, None, None, None, None, None, None, 0)[0] == -1
