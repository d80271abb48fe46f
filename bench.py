#!/usr/bin/env python3
"""Benchmark of one GPU's share of the MoE layer: fused forward+backward tokens/s at 16K tokens.

Workload: one EP8 rank's share, BF16, T=16384 tokens in two token-wise chunks of 8192, H=2048,
16 local of 128 experts, top-8, SwiGLU I=768, forward and backward (route, dispatch, grouped expert
GEMMs, combine, and their backward with grouped wgrad and the FP32-accumulated router gradient).
Inputs are seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line. `value` is fused forward+backward tokens/s; the forward-only rate, every
kernel's measured duration and algorithmic throughput, the dominant kernel's roofline, and the CPU
oracle's rate on a bounded token sample ride along.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (fwd, fwd+bwd) @16K tok top-k8; %HBM BW, %MFMA peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s

# launch-log name -> (source files under the package's csrc/ that its code comes from, substring of
# the kernel symbol that rocprofv3 reports for it)
KERNEL_SYMBOLS = {
    "route_topk": (("route.hip",), "route_topk_kernel"),
    "route_layout": (("route.hip",), "route_layout_kernel"),
    "dispatch": (("rows.hip",), "dispatch_copy_kernel"),
    "combine": (("rows.hip",), "combine_kernel"),
    "combine_bwd": (("rows.hip",), "combine_bwd_kernel"),
    "route_bwd_dlogits": (("rows.hip",), "route_bwd_dlogits_kernel"),
    "dispatch_bwd": (("rows.hip",), "dispatch_bwd_kernel<"),
    "gemm_gateup_swiglu": (("grouped_gemm.hip", "gg_engine.h"), "rows_kernel<256, 256, 0, false, false, false>"),
    # the same launch name in the fused step, whose chunk-0 gate/up reads token rows through src_token
    "gemm_gateup_swiglu_gather": (("grouped_gemm.hip", "gg_engine.h"), "rows_kernel<256, 256, 0, false, false, true>"),
    "gemm_down": (("grouped_gemm.hip", "gg_engine.h"), "rows_kernel<256, 256, 1, false, false, false>"),
    "gemm_down_dgrad_swiglu": (("grouped_gemm.hip", "gg_engine.h"), "rows_kernel<128, 256, 2, false, false, false>"),
    "gemm_gateup_dgrad": (("grouped_gemm.hip", "gg_engine.h"), "rows_kernel<256, 256, 3, false, false, false>"),
    # the fused step's pairs: down of chunk c with gate/up of chunk c+1 (reading token rows through
    # src_token), and down dgrad of chunk c+1 with gate/up dgrad of chunk c
    "gemm_down+gateup_swiglu": (("grouped_gemm.hip", "gg_engine.h"),
                                "rows_pair_kernel<256, 256, 0, 256, 256, 1, false, false, true>"),
    "gemm_gateup_dgrad+down_dgrad_swiglu": (("grouped_gemm.hip", "gg_engine.h"),
                                            "rows_pair_kernel<128, 256, 2, 256, 256, 3, false, false, false>"),
    "gemm_gateup_dgrad+wgrad_w2": (("rows_wgrad.hip", "gg_engine.h", "gg_wgrad.h"),
                                   "rows_wgrad_kernel<256, 256, 3, 256, 256, false>"),
    "gemm_wgrad_w1": (("wgrad.hip", "gg_engine.h", "gg_wgrad.h"), "wgrad_kernel<256, 256, 1>"),
    "gemm_wgrad": (("wgrad.hip", "gg_engine.h", "gg_wgrad.h"), "wgrad_kernel<256, 256, 0>"),
    "gemm_router_wgrad": (("router_wgrad.hip", "gg_engine.h", "gg_wgrad.h"), "router_wgrad_planes_kernel"),
    "router_reduce": (("gemm.hip",), "reduce_partials_kernel"),
}
CALIBRATION_BYTES = 64 << 20   # a plain elementwise copy of this many bytes (read and written once,
CALIBRATION_SYMBOL = "MulFunctor"  # one dispatch: y = 2 * x in FP32) runs before the timed region


def _code_only(text: str) -> str:
    """Source text without comments and whitespace (string literals in these files hold no
    comment markers), so that an edit to comments alone keeps a kernel's counters valid."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


def source_sha(name: str) -> str:
    """Short hash of a kernel's source code (and the shared header), comments and whitespace
    removed: counters taken on other code are not reported for the current code."""
    import hashlib
    csrc = os.path.join(ROOT, "combine_moe_route_02_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SYMBOLS[name][0] + ("common.h",):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def pmc_summary(fetch_dir: str, write_dir: str, cmd: str) -> str:
    """Markdown summary of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch):
    per kernel the median per dispatch, each scaled by what the counter reads for the calibration
    copy of known size, plus one machine-readable `traffic:` line per kernel for the roofline."""
    import statistics
    med = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for r in _counter_rows(d):
            if r["Counter_Name"] != tag:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        med[tag] = {k: statistics.median(v) for k, v in per.items()}

    def find(tag, sym):
        hits = [v for k, v in med[tag].items() if sym in k]
        return hits[0] if hits else None
    cal_f = find("FETCH_SIZE", CALIBRATION_SYMBOL)
    cal_w = find("WRITE_SIZE", CALIBRATION_SYMBOL)
    if not cal_f or not cal_w:
        raise SystemExit("calibration copy kernel not found in the counter runs")
    f_fetch, f_write = CALIBRATION_BYTES / cal_f, CALIBRATION_BYTES / cal_w
    out = ["# HBM traffic per launch from rocprofv3 counters", "",
           "Commands (from the repository root, MI355X):", "", "```", cmd, "```", "",
           f"Calibration: a {CALIBRATION_BYTES >> 20} MiB elementwise copy (`y = 2x`, kernel `{CALIBRATION_SYMBOL}`) reads "
           f"FETCH_SIZE {cal_f / 1024:.0f} KiB and WRITE_SIZE {cal_w / 1024:.0f} KiB, so FETCH_SIZE is scaled by "
           f"{f_fetch:.3f} and WRITE_SIZE by {f_write:.3f}.", "",
           "| kernel | fetch MB/launch (scaled) | write MB/launch (scaled) |", "|---|---:|---:|"]
    lines = []
    for name, (src, sym) in KERNEL_SYMBOLS.items():
        fv, wv = find("FETCH_SIZE", sym), find("WRITE_SIZE", sym)
        if fv is None or wv is None:
            continue
        fb, wb = fv * f_fetch, wv * f_write
        out.append(f"| `{name}` | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
        lines.append(f"traffic: kernel={name} source_sha={source_sha(name)} fetch_bytes={fb:.0f} write_bytes={wb:.0f}")
    out += ["", "Machine-readable lines (bench.py reads them when the source hash matches):", "", "```"] + lines + ["```", ""]
    return "\n".join(out)


# Counter passes for the GEMM engine: each pass stays within one rocprofv3 run's hardware limits
# (at most 8 SQ, 4 TCC, 4 TCP, 2 TA and 2 GRBM counters).
COUNTER_PASSES = {
    "mfma": "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
            "SQ_INSTS_MFMA SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY",
    "lds": "GRBM_GUI_ACTIVE SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT "
           "SQ_WAIT_INST_LDS SQ_LDS_DATA_FIFO_FULL SQ_ACTIVE_INST_LDS",
    "l2": "GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_REQ_sum TCP_TCC_READ_REQ_sum "
          "TCP_PENDING_STALL_CYCLES_sum TA_TA_BUSY_sum TA_DATA_STALLED_BY_TC_CYCLES_sum SQ_INSTS_VMEM_RD "
          "SQ_ACTIVE_INST_VMEM",
}
SIMDS, CUS = 1024, 256          # MI355X: 256 compute units of 4 SIMDs


def counter_summary(dirs, cmd: str) -> str:
    """Markdown summary of rocprofv3 --pmc runs (the COUNTER_PASSES): per kernel symbol the median
    per dispatch of every counter, and the derived MFMA, wave-state, LDS and L2 figures.
    GRBM_GUI_ACTIVE arrives summed over the 8 XCDs, so one XCD's active clocks are a eighth of it."""
    import statistics
    per, dur = {}, {}
    for d in dirs:
        for r in _counter_rows(d):
            k = r["Kernel_Name"]
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    names = {sym: n for n, (_src, sym) in KERNEL_SYMBOLS.items()}
    out = ["# Engine counters per kernel (rocprofv3 --pmc, medians per dispatch)", "",
           "Commands (from the repository root, MI355X):", "", "```", cmd, "```", "",
           "Counter runs serialise the dispatches, so every kernel here ran alone on the GPU. "
           "`clk` = GRBM_GUI_ACTIVE / 8 XCDs / duration. `mfma busy` = SQ_VALU_MFMA_BUSY_CYCLES / "
           "(clk cycles x 1024 SIMDs); `bf16 pk` = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flop / duration / 2.5 "
           "PFLOP/s (F8 MOPS against 5.0 PFLOP/s for FP8 kernels); `wait` = SQ_WAIT_ANY / SQ_WAVE_CYCLES "
           "(share of wave time stalled in s_waitcnt); `issue` = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waiting "
           "for an instruction to issue); `lds issue` = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; `lds act` = "
           "SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs) (indexed LDS traffic only: direct-to-LDS loads are not "
           "counted); `bank` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; `L2 hit` = TCC_HIT / TCC_REQ-side "
           "(HIT + MISS); `EA rd MB` = TCC_EA0_RDREQ_sum x 128 B; `TA busy` = TA_TA_BUSY_sum / (cycles x "
           "256).", "",
           "| kernel | n | us | clk GHz | mfma busy % | bf16 pk % | wait % | issue % | lds issue % | lds act % | "
           "bank % | L2 hit % | EA rd MB | TA busy % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    raw = ["", "Raw medians per dispatch:", ""]

    def med(c, key):
        v = c.get(key)
        return statistics.median(v) if v else None

    def pct(a, b):
        return f"{100.0 * a / b:.1f}" if a is not None and b else "—"
    rows = []
    for k, c in per.items():
        if not any(s in k for s in ("gg::", "gemm::", "dispatch_bwd", "combine", "route")):
            continue
        us = statistics.median(dur[k]) if k in dur else None
        gui = med(c, "GRBM_GUI_ACTIVE")
        cyc = gui / 8.0 if gui else None
        rows.append((k, us, cyc, c))
    rows.sort(key=lambda r: -(r[1] or 0))
    for (k, us, cyc, c) in rows:
        label = next((n for sym, n in names.items() if sym in k), None)
        name = f"`{label}`" if label else f"`{k.split('(')[0][:70]}`"
        n = max(len(v) for v in c.values())
        bf, f8 = med(c, "SQ_INSTS_VALU_MFMA_MOPS_BF16") or 0.0, med(c, "SQ_INSTS_VALU_MFMA_MOPS_F8") or 0.0
        rate = (bf * 512 / 2.5e15 + f8 * 512 / 5.0e15) / (us * 1e-6) if us else None
        wc = med(c, "SQ_WAVE_CYCLES")
        la = med(c, "SQ_LDS_IDX_ACTIVE")
        hit, miss = med(c, "TCC_HIT_sum"), med(c, "TCC_MISS_sum")
        ea = med(c, "TCC_EA0_RDREQ_sum")
        out.append(
            f"| {name} | {n} | {us:.1f} | {cyc / us / 1e3:.2f} | "
            f"{pct(med(c, 'SQ_VALU_MFMA_BUSY_CYCLES'), cyc * SIMDS if cyc else None)} | "
            f"{(100 * rate if rate is not None else float('nan')):.1f} | "
            f"{pct(med(c, 'SQ_WAIT_ANY'), wc)} | {pct(med(c, 'SQ_WAIT_INST_ANY'), wc)} | "
            f"{pct(med(c, 'SQ_WAIT_INST_LDS'), wc)} | {pct(la, cyc * CUS if cyc else None)} | "
            f"{pct(med(c, 'SQ_LDS_BANK_CONFLICT'), la)} | {pct(hit, (hit or 0) + (miss or 0))} | "
            f"{(ea * 128 / 1e6) if ea is not None else float('nan'):.1f} | "
            f"{pct(med(c, 'TA_TA_BUSY_sum'), cyc * CUS if cyc else None)} |")
        if "gg::" in k or "gemm::" in k:
            raw.append(f"- `{k.split('(')[0][:110]}` ({us:.1f} us): " +
                       ", ".join(f"{ck}={statistics.median(v):.4g}" for ck, v in sorted(c.items())))
    src = [f"Source hashes (code without comments): grouped_gemm.hip + gg_engine.h "
           f"{source_sha('gemm_gateup_swiglu')}, wgrad.hip + gg_engine.h + gg_wgrad.h {source_sha('gemm_wgrad')}, "
           f"rows_wgrad.hip + gg_engine.h + gg_wgrad.h {source_sha('gemm_gateup_dgrad+wgrad_w2')}, "
           f"router_wgrad.hip + gg_engine.h + gg_wgrad.h {source_sha('gemm_router_wgrad')}, "
           f"gemm.hip {source_sha('router_reduce')}, rows.hip {source_sha('dispatch')}.", ""]
    return "\n".join(out[:7] + src + out[7:] + raw) + "\n"


def committed_traffic(name: str):
    """Calibrated HBM bytes per launch for a kernel from profiles/*traffic*.md, or None when no
    summary was taken on this kernel's current source."""
    import glob
    want = source_sha(name) if name in KERNEL_SYMBOLS else None
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("traffic:"):
                    continue
                kv = dict(x.split("=", 1) for x in line.split()[1:])
                if kv.get("kernel") == name and kv.get("source_sha") == want:
                    return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    return None


GEMM_KERNELS = {"gemm_gateup_swiglu", "gemm_down", "gemm_down_dgrad_swiglu", "gemm_gateup_dgrad",
                "gemm_wgrad", "gemm_router_wgrad", "gemm_down+gateup_swiglu",
                "gemm_gateup_dgrad+down_dgrad_swiglu", "gemm_gateup_dgrad+wgrad_w2", "gemm_wgrad_w1"}


def algorithmic_work(cfg, counts, offsets, k_sel_local_tokens):
    """Per fused step: name -> (work, unit). FLOPs for GEMMs (useful multiply-adds x 2), bytes that
    the step must move for the row kernels (each tensor element read or written once)."""
    T, H, I, E, k, El = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.E_local
    N = int(offsets[:, El].sum())              # local rows over all chunks
    Tt = int(k_sel_local_tokens)               # tokens with at least one local expert
    s = 2                                      # BF16 payload bytes
    S = min(16, max(1, math.ceil(math.ceil(T / cfg.n_chunks) / 64)))
    w = {
        "gemm_gateup_swiglu": (2.0 * N * H * 2 * I, "flop"),
        "gemm_down": (2.0 * N * I * H, "flop"),
        "gemm_down_dgrad_swiglu": (2.0 * N * H * I, "flop"),
        "gemm_gateup_dgrad": (2.0 * N * 2 * I * H, "flop"),
        "gemm_wgrad": (2.0 * N * H * I + 2.0 * N * 2 * I * H, "flop"),  # dW2 and dW1, one launch
        "gemm_router_wgrad": (2.0 * T * E * H, "flop"),
        "route_topk": (T * E * 4 + T * k * 8, "byte"),
        "route_layout": (T * k * 8 + cfg.n_chunks * 0 + N * 4, "byte"),
        "dispatch": (Tt * H * s + N * H * s + T * k * 4, "byte"),
        "combine": (N * H * s + T * H * s + T * k * 8, "byte"),
        "combine_bwd": (Tt * H * s + 2 * N * H * s + T * k * 12, "byte"),
        "route_bwd_dlogits": (T * k * 12 + T * E * 4, "byte"),
        "dispatch_bwd": (N * H * s + T * H * s + T * k * 12 + E * H * s, "byte"),
        "router_reduce": (cfg.n_chunks * (S * E * H * 4 + 2 * E * H * 4) + E * H * s, "byte"),
    }
    return w, N, Tt


def fused_gemm_work(cfg, Nc):
    """The fused step's BF16 GEMM launches (the layer primitive merges independent GEMMs of
    neighbouring chunks): name -> ((flops, unit), HBM bytes) per step, from the local rows per chunk
    Nc. Gate/up and down dgrad run alone for chunk 0 and down alone for the last chunk; each pair
    launch does down (gate/up dgrad) of chunk c with gate/up (down dgrad) of c+1; the last chunk's
    gate/up dgrad runs with dW2 over all rows, then dW1 alone."""
    H, I, El, s, n = cfg.H, cfg.I, cfg.E_local, 2, len(Nc)
    w1, w2 = El * 2 * I * H * s, El * H * I * s
    gu_f = lambda m: 2.0 * m * H * 2 * I
    dn_f = lambda m: 2.0 * m * I * H
    gu_b = lambda m: m * H * s + w1 + m * I * s + m * 2 * I * s
    dn_b = lambda m: m * I * s + w2 + m * H * s
    ddg_b = lambda m: m * H * s + w2 + 2 * m * 2 * I * s
    gudg_b = lambda m: m * 2 * I * s + w1 + m * H * s
    pairs = range(n - 1)
    N = sum(Nc)
    dw2_f, dw2_b = 2.0 * N * H * I, N * H * s + N * I * s + w2
    dw1_f, dw1_b = 2.0 * N * 2 * I * H, N * 2 * I * s + N * H * s + w1
    return {
        "gemm_gateup_swiglu": ((gu_f(Nc[0]), "flop"), gu_b(Nc[0])),
        "gemm_down+gateup_swiglu": ((sum(dn_f(Nc[c]) + gu_f(Nc[c + 1]) for c in pairs), "flop"),
                                    sum(dn_b(Nc[c]) + gu_b(Nc[c + 1]) for c in pairs)),
        "gemm_down": ((dn_f(Nc[-1]), "flop"), dn_b(Nc[-1])),
        "gemm_down_dgrad_swiglu": ((dn_f(Nc[0]), "flop"), ddg_b(Nc[0])),
        "gemm_gateup_dgrad+down_dgrad_swiglu": ((sum(gu_f(Nc[c]) + dn_f(Nc[c + 1]) for c in pairs), "flop"),
                                                sum(gudg_b(Nc[c]) + ddg_b(Nc[c + 1]) for c in pairs)),
        "gemm_gateup_dgrad+wgrad_w2": ((gu_f(Nc[-1]) + dw2_f, "flop"), gudg_b(Nc[-1]) + dw2_b),
        "gemm_wgrad_w1": ((dw1_f, "flop"), dw1_b),
    }


def gemm_bytes(cfg, N):
    """HBM bytes each grouped GEMM must move per fused step, every tensor read or written once: the
    row operands, the weights once per launch (per chunk for the row-grouped GEMMs), the outputs.
    With the flops this gives the GEMM's arithmetic intensity and its attainable rate
    min(MFMA peak, intensity x HBM peak)."""
    H, I, El, n, s = cfg.H, cfg.I, cfg.E_local, cfg.n_chunks, 2
    w1, w2 = El * 2 * I * H * s, El * H * I * s
    return {
        "gemm_gateup_swiglu": N * H * s + n * w1 + N * I * s + N * 2 * I * s,
        "gemm_down": N * I * s + n * w2 + N * H * s,
        "gemm_down_dgrad_swiglu": N * H * s + n * w2 + 2 * N * 2 * I * s,
        "gemm_gateup_dgrad": N * 2 * I * s + n * w1 + N * H * s,
        "gemm_wgrad": (N * H * s + N * I * s + w2) + (N * 2 * I * s + N * H * s + w1),
    }


def cpu_baseline(cfg, inp, budget_s: float):
    """Time the CPU oracle (as it stands) on the workload: the forward and the fused forward +
    backward, one warmup and three measured runs each, median (and min) scaled to tokens/s. When
    one fused run would exceed a third of the budget, a prefix of the tokens (same shapes
    otherwise) is timed instead and scaled."""
    import numpy as np
    import oracle
    blas = {}
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = {"vendor": info[0].get("internal_api"), "version": info[0].get("version"),
                    "threads": info[0].get("num_threads")}
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def run(Ts, backward):
        x, lg = inp["x"][:Ts], inp["logits"][:Ts]
        t0 = time.perf_counter()
        f = oracle.forward(x, lg, inp["w1"], inp["w2"], k=cfg.k, e0=cfg.e0, E_local=cfg.E_local,
                           n_chunks=cfg.n_chunks)
        if backward:
            oracle.backward(f, x, inp["dy"][:Ts], inp["w1"], inp["w2"], inp["w_r"])
        return time.perf_counter() - t0
    Ts = cfg.T
    first = run(Ts, True)                     # also the warmup of the fused runs
    while first > budget_s / 4 and Ts > 1024:
        Ts //= 2
        first = run(Ts, True)
    fb = [run(Ts, True) for _ in range(3)]
    run(Ts, False)
    fw = [run(Ts, False) for _ in range(3)]
    med_fb, med_fw = statistics.median(fb), statistics.median(fw)
    sample = "all" if Ts == cfg.T else f"the first {Ts} of"
    return {"value": round(Ts / med_fb, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"FP64 NumPy oracle on {sample} {cfg.T} tokens (same H/I/E/k/chunks): fused forward+backward "
                      f"median of 3 runs after a warmup, {med_fb:.2f} s (min {min(fb):.2f} s); forward median "
                      f"{med_fw:.2f} s",
            "fwd_tokens_per_s": round(Ts / med_fw, 1), "fwd_bwd_s": [round(v, 3) for v in fb],
            "fwd_s": [round(v, 3) for v in fw], "blas": blas,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def step_stats(fn, stream, steps, torch):
    """Per-step durations (ms) of `steps` calls: HIP events recorded on the compute stream between
    the calls (each call ends with the auxiliary stream joined into it)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def imbalanced_leg(args, mh, torch, np):
    """The imbalanced-routing workload (Zipf(1.2) expert popularity, empty local experts) at the same
    shapes, fused forward+backward, with the combine output at the extent a live 32K-token graph
    holds (262144 rows): untraced step time, per-step median, per-kernel in-step durations, the
    local rows, and the time per local row against the balanced step's."""
    import moe_inputs
    cfg = moe_inputs.CONFIGS["zipf16k"]
    big = moe_inputs.CONFIGS["fb32k"]
    tr = mh.ExtentTracker()
    own = mh.required_extent(cfg.T, cfg.k, cfg.E_local, cfg.n_chunks)[1]
    live = tr.acquire(mh.required_extent(big.T, big.k, big.E_local, big.n_chunks)[1])
    P_out = tr.current(own)
    inp = moe_inputs.make_inputs(cfg, with_backward=True)
    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0, P_out=P_out)
    b = mh.allocate(d, backward=True)
    for name in ("x", "w1", "w2", "w_r", "dy"):
        b[name] = torch.from_numpy(inp[name + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    b["logits"] = torch.from_numpy(inp["logits"]).cuda()
    cs, aux = torch.cuda.Stream(), torch.cuda.Stream()

    def fb():
        mh.moe_layer_forward_backward(d, b, cs, aux)
    for _ in range(args.warmup):
        fb()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fb()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    for _ in range(args.warmup):
        fb()
    per_step = step_stats(fb, cs, args.steps, torch)
    mh.moe_trace_enable(True)
    for _ in range(args.steps):
        fb()
    torch.cuda.synchronize()
    mh.moe_trace_disable()
    per = {}
    for name, _s, t in mh.moe_trace_entries():
        p = per.setdefault(name, [0, 0.0])
        p[0] += 1
        p[1] += t
    offsets = b["offsets"].cpu().numpy()
    counts = [int(v) for v in (offsets[:, 1:] - offsets[:, :-1]).sum(axis=0)]
    N = int(offsets[:, cfg.E_local].sum())
    tr.release(live)
    out = {"workload": "Zipf(1.2)-biased routing, 3 empty local experts, same shapes as the main line",
           "P_out": int(P_out), "ms_per_step_untraced": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "step_ms_median": round(statistics.median(per_step), 4), "local_rows": N,
           "local_rows_per_expert": counts,
           "kernels_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()}}
    del b
    torch.cuda.empty_cache()
    return out


def fp8_forward(args, cfg, inp, mh, torch, np):
    """Forward-only FP8 rate at the same shapes: tokens/s and the FP8 GEMMs' TFLOP/s."""
    d8 = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                      dtype="fp8", e0=cfg.e0)
    b8 = mh.allocate(d8, backward=False)
    b8["x"] = torch.from_numpy(inp["x_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    b8["logits"] = torch.from_numpy(inp["logits"]).cuda()
    w1 = torch.from_numpy(inp["w1_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    w2 = torch.from_numpy(inp["w2_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    b8["w1"] = torch.empty(w1.shape, dtype=torch.uint8, device="cuda")
    b8["w2"] = torch.empty(w2.shape, dtype=torch.uint8, device="cuda")
    b8["w1_scale"] = torch.empty(w1.shape[:-1], dtype=torch.float32, device="cuda")
    b8["w2_scale"] = torch.empty(w2.shape[:-1], dtype=torch.float32, device="cuda")
    mh.moe_quantize_rows_fp8(cfg.E_local * 2 * cfg.I, cfg.H, w1, b8["w1"], b8["w1_scale"])
    mh.moe_quantize_rows_fp8(cfg.E_local * cfg.H, cfg.I, w2, b8["w2"], b8["w2_scale"])
    del w1, w2
    cs, aux = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(args.warmup):
        mh.moe_layer_forward(d8, b8, cs, aux)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mh.moe_layer_forward(d8, b8, cs, aux)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    mh.moe_trace_enable(True)
    for _ in range(args.steps):
        mh.moe_layer_forward(d8, b8, cs, aux)
    torch.cuda.synchronize()
    mh.moe_trace_disable()
    per = {}
    for name, _s, t in mh.moe_trace_entries():
        p = per.setdefault(name, [0, 0.0])
        p[0] += 1
        p[1] += t
    N = int(b8["offsets"].cpu().numpy()[:, cfg.E_local].sum())
    flops = {"gemm_gateup_swiglu_fp8": 2.0 * N * cfg.H * 2 * cfg.I, "gemm_down_fp8": 2.0 * N * cfg.I * cfg.H}
    out = {"tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "ms": round(ms, 4), "peak_fp8_tflops": PEAK_FP8_TFLOPS,
           "kernels": {}}
    for name, (cnt, tot) in per.items():
        e = {"avg_us": round(tot / cnt * 1e3, 3), "ms_per_step": round(tot / args.steps, 4)}
        if name in flops:
            r = flops[name] / (tot / args.steps * 1e-3) / 1e12
            e.update(achieved_tflops=round(r, 2), frac_mfma=round(r / PEAK_FP8_TFLOPS, 4))
        out["kernels"][name] = e
    del b8
    torch.cuda.empty_cache()
    return out


def fp8_dgrad(args, cfg, bufs, mh, torch, np):
    """The fused forward+backward with FP8 input gradients (MOE_FLAG_FP8_DGRAD; weights quantised
    per column, transposed, outside the timed region): tokens/s and the FP8 dgrad GEMMs' TFLOP/s."""
    dq = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                      dtype="bf16", e0=cfg.e0, flags=mh.FLAG_FP8_DGRAD)
    bq = mh.allocate(dq, backward=True)
    for name in ("x", "logits", "w1", "w2", "w_r", "dy"):
        bq[name] = bufs[name]
    mh.moe_quantize_cols_fp8(cfg.E_local, 2 * cfg.I, cfg.H, bq["w1"], bq["w1t"], bq["w1t_scale"])
    mh.moe_quantize_cols_fp8(cfg.E_local, cfg.H, cfg.I, bq["w2"], bq["w2t"], bq["w2t_scale"])
    cs, aux = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(args.warmup):
        mh.moe_layer_forward_backward(dq, bq, cs, aux)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mh.moe_layer_forward_backward(dq, bq, cs, aux)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    mh.moe_trace_enable(True)
    for _ in range(args.steps):
        mh.moe_layer_forward_backward(dq, bq, cs, aux)
    torch.cuda.synchronize()
    mh.moe_trace_disable()
    per = {}
    for name, _s, t in mh.moe_trace_entries():
        p = per.setdefault(name, [0, 0.0])
        p[0] += 1
        p[1] += t
    N = int(bq["offsets"].cpu().numpy()[:, cfg.E_local].sum())
    flops = {"gemm_down_dgrad_swiglu_fp8": 2.0 * N * cfg.H * cfg.I, "gemm_gateup_dgrad_fp8": 2.0 * N * 2 * cfg.I * cfg.H}
    out = {"tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "ms_per_step_untraced": round(ms, 4),
           "peak_fp8_tflops": PEAK_FP8_TFLOPS, "kernels": {}}
    for name, (cnt, tot) in per.items():
        e = {"avg_us": round(tot / cnt * 1e3, 3), "ms_per_step": round(tot / args.steps, 4)}
        if name in flops:
            r = flops[name] / (tot / args.steps * 1e-3) / 1e12
            e.update(achieved_tflops=round(r, 2), frac_mfma=round(r / PEAK_FP8_TFLOPS, 4))
        out["kernels"][name] = e
    # FP8 input and weight gradients together (untraced)
    dw = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                      dtype="bf16", e0=cfg.e0, flags=mh.FLAG_FP8_DGRAD | mh.FLAG_FP8_WGRAD)
    bw = mh.allocate(dw, backward=True)
    for name in ("x", "logits", "w1", "w2", "w_r", "dy", "w1t", "w1t_scale", "w2t", "w2t_scale"):
        bw[name] = bq[name]
    for _ in range(args.warmup):
        mh.moe_layer_forward_backward(dw, bw, cs, aux)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mh.moe_layer_forward_backward(dw, bw, cs, aux)
    torch.cuda.synchronize()
    ms_w = (time.perf_counter() - t0) * 1e3 / args.steps
    out["with_fp8_wgrad"] = {"tokens_per_s": round(cfg.T / (ms_w * 1e-3), 1), "ms_per_step_untraced": round(ms_w, 4)}
    # the BF16 step with the FP8 dispatch-backward payload alone (untraced)
    dx8 = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                       dtype="bf16", e0=cfg.e0, flags=mh.FLAG_FP8_DXD)
    bx = mh.allocate(dx8, backward=True)
    for name in ("x", "logits", "w1", "w2", "w_r", "dy"):
        bx[name] = bufs[name]
    for _ in range(args.warmup):
        mh.moe_layer_forward_backward(dx8, bx, cs, aux)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mh.moe_layer_forward_backward(dx8, bx, cs, aux)
    torch.cuda.synchronize()
    ms_x = (time.perf_counter() - t0) * 1e3 / args.steps
    out["bf16_with_fp8_dxd"] = {"tokens_per_s": round(cfg.T / (ms_x * 1e-3), 1), "ms_per_step_untraced": round(ms_x, 4)}
    del bq, bw, bx
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30)  # the clocks take some tens of ms of load to settle
    ap.add_argument("--workload", default="fb16k")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-imbalanced", action="store_true", help="skip the imbalanced-routing leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COMMANDS"),
                    help="write the markdown traffic summary of two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR_OR_COMMANDS",
                    help="counter directories of the COUNTER_PASSES runs, then the commands text: write the "
                         "markdown engine-counter summary and exit (no GPU)")
    ap.add_argument("--counter-pass", choices=sorted(COUNTER_PASSES),
                    help="print the counters of one COUNTER_PASSES entry (for rocprofv3 --pmc) and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary[:-1], args.counter_summary[-1]))
        return
    if args.counter_pass:
        print(COUNTER_PASSES[args.counter_pass])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              f"(the library runs on one GPU: run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import moe_inputs
    import combine_moe_route_02_amd as mh

    mh.lib()  # the HIP library must be present: there is no other path
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = moe_inputs.CONFIGS[args.workload]
    inp = moe_inputs.make_inputs(cfg, with_backward=True)

    d = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=cfg.n_chunks,
                     dtype=cfg.dtype, e0=cfg.e0)
    bufs = mh.allocate(d, backward=True)

    def dev(name):
        if name == "logits":
            return torch.from_numpy(inp["logits"]).cuda()
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)

    for name in ("x", "logits", "w1", "w2", "w_r", "dy"):
        bufs[name] = dev(name)
    cs = torch.cuda.Stream()
    aux = torch.cuda.Stream()
    torch.cuda.synchronize()

    # calibration for the HBM byte counters: one elementwise kernel that reads and writes a known
    # number of bytes once
    cal_src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    for _ in range(2):
        torch.mul(cal_src, 2.0, out=cal_dst)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    def fb():
        mh.moe_layer_forward_backward(d, bufs, cs, aux)

    def fwd():
        mh.moe_layer_forward(d, bufs, cs, aux)

    for _ in range(args.warmup):
        fb()
    torch.cuda.synchronize()

    # per-kernel pass (before the timed region): `steps` fused steps with every kernel launch
    # bracketed by HIP events on the stream it runs on; it gives each kernel's in-step duration
    # and picks the dominant kernel, the largest share of the compute stream, whose work sets the
    # step time (aux-stream kernels run beside a GEMM, so their in-step durations mostly measure
    # how much that GEMM slowed them)
    mh.moe_trace_enable(True)
    torch.cuda.synchronize()
    p0 = time.perf_counter()
    for _ in range(args.steps):
        fb()
    torch.cuda.synchronize()
    ms_traced = (time.perf_counter() - p0) * 1e3 / args.steps
    mh.moe_trace_disable()
    entries = mh.moe_trace_entries()
    comp = int(cs.cuda_stream)
    on_compute = {n for n, st, _ in entries if int(st or 0) == comp}
    on_compute -= {n for n, st, _ in entries if int(st or 0) != comp}
    step_ms = {}
    for n, _st, ms in entries:
        step_ms[n] = step_ms.get(n, 0.0) + ms
    dom = max((n for n in step_ms if n in on_compute), key=lambda n: step_ms[n])

    # timed region: exactly `steps` fused steps; HIP events bracket the dominant kernel's launches
    # only, so the rest of the step runs without instrumentation. Reading the log above left the
    # GPU idle for some ms, so it is warmed up again first (the clocks drop when it idles).
    for _ in range(args.warmup):
        fb()
    mh.moe_trace_enable_only(dom)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fb()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mh.moe_trace_disable()
    dom_ms = [ms for n, _st, ms in mh.moe_trace_entries() if n == dom]
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # the same loop without any launch log (warmed up again after reading the log)
    for _ in range(args.warmup):
        fb()
    torch.cuda.synchronize()
    u0 = time.perf_counter()
    for _ in range(args.steps):
        fb()
    torch.cuda.synchronize()
    ms_untraced = (time.perf_counter() - u0) * 1e3 / args.steps

    # per-step durations: HIP events on the compute stream between steps (after each step's join)
    for _ in range(args.warmup):
        fb()
    per_step = step_stats(fb, cs, args.steps, torch)

    # forward only
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    ms_fwd = (time.perf_counter() - f0) * 1e3 / args.steps

    # isolated: the same stage calls chunk by chunk on one stream (no two-stream overlap), for
    # each kernel's own cost
    def stages():
        b = bufs
        for c in range(cfg.n_chunks):
            mh.moe_route(d, c, b["logits"], b["topk_idx"], b["gates"], b["counts"], b["offsets"], b["row_of"],
                         b["src_token"], b["workspace"], cs)
            mh.moe_dispatch(d, c, b["x"], b["row_of"], b["xd"], None, None, cs)
            mh.moe_expert_ffn(d, c, b["xd"], None, b["w1"], None, b["w2"], None, b["offsets"], b["gu"], b["h"],
                              None, b["yd"], cs)
            mh.moe_combine(d, c, b["yd"], b["gates"], b["row_of"], b["out"], cs)
        for c in range(cfg.n_chunks):
            mh.moe_combine_bwd(d, c, b["dy"], b["yd"], b["gates"], b["row_of"], b["dyd"], b["dgates"], cs)
            mh.moe_route_bwd(d, c, b["dgates"], b["gates"], b["topk_idx"], b["x"], b["dlogits"], b["dwr_acc"],
                             b["dwr"], b["workspace"], cs)
            mh.moe_expert_ffn_bwd(d, c, b["dyd"], b["xd"], b["gu"], b["h"], b["w1"], b["w2"], b["offsets"],
                                  b["dgu"], b["dxd"], None, None, None, cs)
            mh.moe_dispatch_bwd(d, c, b["dxd"], b["row_of"], b["topk_idx"], b["dlogits"], b["w_r"], b["dx"], cs)
        mh.moe_expert_wgrad(d, b["dyd"], b["dgu"], b["xd"], b["h"], b["offsets"], b["dw1"], b["dw2"], b["workspace"],
                            cs)

    stages()
    torch.cuda.synchronize()
    mh.moe_trace_enable(True)
    for _ in range(args.steps):
        stages()
    torch.cuda.synchronize()
    mh.moe_trace_disable()
    iso = {}
    for name, _stream, ms in mh.moe_trace_entries():
        p = iso.setdefault(name, [0, 0.0])
        p[0] += 1
        p[1] += ms

    # the row kernels once more, each stage called back to back `reps` times between two events
    # on its stream: per-launch event overhead (a few us) amortised away
    def amortized_us(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cs)
        for _ in range(reps):
            fn()
        e1.record(cs)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    b = bufs
    row_stages = {
        "dispatch": lambda c: mh.moe_dispatch(d, c, b["x"], b["row_of"], b["xd"], None, None, cs),
        "combine": lambda c: mh.moe_combine(d, c, b["yd"], b["gates"], b["row_of"], b["out"], cs),
        "combine_bwd": lambda c: mh.moe_combine_bwd(d, c, b["dy"], b["yd"], b["gates"], b["row_of"], b["dyd"],
                                                    b["dgates"], cs),
        "dispatch_bwd": lambda c: mh.moe_dispatch_bwd(d, c, b["dxd"], b["row_of"], b["topk_idx"], b["dlogits"],
                                                      b["w_r"], b["dx"], cs),
    }
    amort = {name: amortized_us(lambda f=f: [f(c) for c in range(cfg.n_chunks)]) for name, f in row_stages.items()}

    # routing from x (router projection fused into the top-k) against routing from given logits,
    # all chunks per call; the second call restores the timed step's routing in the buffers
    chunks = range(cfg.n_chunks)
    rx_us = amortized_us(lambda: [mh.moe_route_x(d, c, b["x"], b["w_r"], None, b["topk_idx"], b["gates"],
                                                 b["counts"], b["offsets"], b["row_of"], b["src_token"],
                                                 b["workspace"], cs) for c in chunks])
    rl_us = amortized_us(lambda: [mh.moe_route(d, c, b["logits"], b["topk_idx"], b["gates"], b["counts"],
                                               b["offsets"], b["row_of"], b["src_token"], b["workspace"], cs)
                                  for c in chunks])
    proj_flops = 2.0 * cfg.T * cfg.E * cfg.H
    route_x_line = {"from_x_us_per_step": round(rx_us, 3), "from_logits_us_per_step": round(rl_us, 3),
                    "projection_tflops_est": round(proj_flops / ((rx_us - rl_us) * 1e-6) / 1e12, 1)
                    if rx_us > rl_us else None}

    # paged activation stash: one chunk's expert-output rows (yd) stored into a page pool under a
    # shuffled page table and loaded back, each called back to back between one event pair
    live = int(bufs["offsets"][0, cfg.E_local].item())
    rb, page_rows = cfg.H * 2, 256
    npg = -(-live // page_rows)
    g = torch.Generator().manual_seed(7)
    pages = torch.randperm(npg, generator=g).to(torch.int32).cuda()
    pool = torch.empty((npg * page_rows, rb), dtype=torch.uint8, device="cuda")
    back = torch.empty((live, rb), dtype=torch.uint8, device="cuda")
    yd0 = bufs["yd"].view(torch.uint8)
    st_us = amortized_us(lambda: mh.moe_stash_store(yd0, None, live, rb, pool, None, npg, page_rows, pages,
                                                    stream=cs))
    ld_us = amortized_us(lambda: mh.moe_stash_load(pool, None, live, rb, npg, page_rows, pages, back, stream=cs))
    moved = 2.0 * live * rb
    stash_line = {"rows": live, "row_bytes": rb, "page_rows": page_rows, "store_us": round(st_us, 3),
                  "load_us": round(ld_us, 3), "store_frac_hbm": round(moved / (st_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "load_frac_hbm": round(moved / (ld_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del pool, back

    # the same layer with one chunk (no overlap, larger per-expert GEMMs), untraced
    n1 = None
    if cfg.n_chunks > 1:
        d1 = mh.make_desc(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_local=cfg.E_local, k=cfg.k, n_chunks=1,
                          dtype=cfg.dtype, e0=cfg.e0)
        b1 = mh.allocate(d1, backward=True)
        for name in ("x", "logits", "w1", "w2", "w_r", "dy"):
            b1[name] = bufs[name]
        for _ in range(args.warmup):
            mh.moe_layer_forward_backward(d1, b1, cs, aux)
        torch.cuda.synchronize()
        n0 = time.perf_counter()
        for _ in range(args.steps):
            mh.moe_layer_forward_backward(d1, b1, cs, aux)
        torch.cuda.synchronize()
        ms1 = (time.perf_counter() - n0) * 1e3 / args.steps
        n1 = {"n_chunks": 1, "ms_per_step_untraced": round(ms1, 4), "tokens_per_s": round(cfg.T / (ms1 * 1e-3), 1)}
        del b1
        torch.cuda.empty_cache()

    imb = None if args.no_imbalanced or args.workload != "fb16k" else imbalanced_leg(args, mh, torch, np)

    # FP8 payload path, forward only (the same shapes; weights quantised per output row outside the
    # timed region): expert GEMMs on FP8 MFMA, dispatch quantises per token, combine in BF16
    fp8 = fp8_forward(args, cfg, inp, mh, torch, np)
    # FP8 input gradients in the fused step (BF16 forward, weight gradients and payload copies)
    fp8dg = fp8_dgrad(args, cfg, bufs, mh, torch, np)

    counts = bufs["counts"].cpu().numpy()
    offsets = bufs["offsets"].cpu().numpy()
    row_of = bufs["row_of"].cpu().numpy()
    touched = int(np.count_nonzero((row_of >= 0).any(axis=1)))
    work, N, Tt = algorithmic_work(cfg, counts, offsets, touched)
    # the fused step's GEMM launches: per-step work of the launch kinds the layer primitive issues
    # (the isolated stage calls keep the per-GEMM kinds of `work`)
    fused = fused_gemm_work(cfg, [int(v) for v in offsets[:, cfg.E_local]])
    work_f = dict(work)
    work_f.update({k: v[0] for k, v in fused.items()})

    per = {}
    for name, _stream, ms in entries:
        p = per.setdefault(name, [0, 0.0])
        p[0] += 1
        p[1] += ms
    kernels = {}
    gbytes = gemm_bytes(cfg, N)
    gbytes_f = dict(gbytes)
    gbytes_f.update({k: v[1] for k, v in fused.items()})
    names = list(per) + [n for n in iso if n not in per]
    for name in names:
        entry = {}
        if name in per:
            cnt, tot = per[name]
            entry = {"launches_per_step": cnt / args.steps, "avg_us": round(tot / cnt * 1e3, 3),
                     "ms_per_step": round(tot / args.steps, 4)}
        if name in per and name in work_f:
            wk, unit = work_f[name]
            rate = wk / (tot / args.steps * 1e-3)
            if unit == "flop":
                entry.update(achieved_tflops=round(rate / 1e12, 2), frac_mfma=round(rate / 1e12 / PEAK_BF16_TFLOPS, 4))
                if name in gbytes_f:
                    ai = wk / gbytes_f[name]
                    attain = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
                    entry.update(intensity_flop_per_byte=round(ai, 1), attainable_tflops=round(attain, 1),
                                 frac_attainable=round(rate / 1e12 / attain, 4))
            else:
                entry.update(achieved_gbs=round(rate / 1e9, 1), frac_hbm=round(rate / 1e9 / PEAK_HBM_GBS, 4))
        if name in amort:
            us = amort[name]  # both chunks
            entry["isolated_amortized_us"] = round(us / cfg.n_chunks, 3)
            if name in work:
                entry["isolated_amortized_frac"] = round(work[name][0] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        if name in iso:
            ic, it = iso[name]
            entry["isolated_avg_us"] = round(it / ic * 1e3, 3)
            if name in work:
                wk, unit = work[name]
                r = wk / (it / args.steps * 1e-3)
                entry["isolated_frac"] = round(r / 1e12 / PEAK_BF16_TFLOPS if unit == "flop" else r / 1e9 / PEAK_HBM_GBS, 4)
        kernels[name] = entry
    # the dominant kernel's launches timed inside the timed region
    dcnt, dtot = len(dom_ms), sum(dom_ms)
    wk, unit = work_f.get(dom, (None, None))
    if unit == "flop":
        ach = wk / (dtot / args.steps * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": committed_traffic(dom), "kernel": dom,
                "avg_launch_us": round(dtot / dcnt * 1e3, 3), "work_per_launch": wk / (dcnt / args.steps)}
    else:
        ach = wk / (dtot / args.steps * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": committed_traffic(dom), "kernel": dom,
                "avg_launch_us": round(dtot / dcnt * 1e3, 3), "work_per_launch": wk / (dcnt / args.steps)}

    iso_ms = sum(v[1] for v in iso.values()) / args.steps
    gemm_flops = sum(work_f[n][0] for n in GEMM_KERNELS if n in per)
    gemm_ms = sum(per[n][1] for n in GEMM_KERNELS if n in per) / args.steps
    value = cfg.T / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one EP8 rank's MoE layer share, BF16 fused forward+backward",
                   "tokens": cfg.T, "n_chunks": cfg.n_chunks, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "local_experts": cfg.E_local, "top_k": cfg.k,
                   "local_rows": N, "tokens_with_local_expert": Tt},
        "fwd_tokens_per_s": round(cfg.T / (ms_fwd * 1e-3), 1), "fwd_ms": round(ms_fwd, 4),
        "ms_per_step_untraced": round(ms_untraced, 4),
        "step_ms_median": round(statistics.median(per_step), 4), "step_ms_min": round(min(per_step), 4),
        "step_ms_max": round(max(per_step), 4), "steps_measured": len(per_step),
        "tokens_per_s_at_median_step": round(cfg.T / (statistics.median(per_step) * 1e-3), 1),
        "ms_per_step_traced": round(ms_traced, 4),
        "isolated_kernel_ms_sum": round(iso_ms, 4),
        "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms > 0 else None,
        "roofline": roof, "kernels": kernels,
    }
    line["one_chunk"] = n1
    if imb:
        imb["time_per_local_row_vs_balanced"] = round(
            (imb["ms_per_step_untraced"] / max(1, imb["local_rows"])) / (ms_untraced / max(1, N)), 3)
    line["imbalanced"] = imb
    line["stash"] = stash_line
    line["route_from_x"] = route_x_line
    line["fp8_fwd"] = fp8
    line["fp8_dgrad"] = fp8dg
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
