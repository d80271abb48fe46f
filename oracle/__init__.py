"""CPU oracle for one GPU's share of a MoE layer: route, dispatch, expert SwiGLU FFN, combine,
and their backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library (``combine_moe_route_02_amd``) and imports nothing from it.

What it computes, and where it comes from:
  * The pages (token-wise ChunkedEP, Megatron-LM PR 7342, "Summary"; HybridEP PRs in torchtitan
    and OpenPipe/ART) name the operations (top-k routing, token-wise chunks, dispatch into
    expert-contiguous buffers, expert FFN, combine into a fresh [P, H] output cropped to the
    logical rows, router-gradient accumulation in FP32 across chunks) but print no formula.
    The plain definitions written here are the readings listed in each function's docstring.
  * Floating point is FP64 throughout (the method's BF16/FP32 rounding is not modelled), except
    where an integer is decided by floating point (FP8 codes): there the FP32 steps are followed
    exactly, as the kernel takes them.

Modules:
  routing   top-k selection, renormalised gates, per-chunk counts/offsets, stable permutation,
            extent rules (rows rounded up to 4).
  ffn       vectorised forward and backward (per-expert matmuls).
  brute     per-token loops for tiny inputs (pins the vectorised forms).
  fp8       OCP e4m3fn encode/decode, per-row and per-row-block absmax quantisation; FP8 forward,
            FP8 input and weight gradients, the FP8 dispatch-backward payload.
  extent    live-extent tracker and combine-output workspace floor.
  stash     paged activation stash: page-aligned store/load of saved rows with live-prefix and
            page-tail masks.

Every function here is pinned by a ``-m "not gpu"`` test (brute force, closed forms, library
special cases, finite differences, autograd, printed numbers); none is "parity unpinned".
"""
from . import routing, ffn, brute, fp8, extent, stash  # noqa: F401
from .routing import (round4, chunk_bounds, required_extent, route, layout,  # noqa: F401
                      dispatch, unpermute, router_logits)
from .ffn import expert_ffn, combine, forward, backward  # noqa: F401
