"""Seeded synthetic inputs for the MoE route / dispatch / expert / combine path.

This module is shared by the CPU oracle, the GPU tests and the benchmark, and
it holds none of the method's arithmetic: it only draws random tensors, rounds
them once to the payload dtype, and names the workload shapes.

Recipe (every tensor):
  * ``numpy.random.default_rng(seed_base + tensor_id)`` (PCG64), drawn in FP32
    with ``standard_normal`` and scaled by the tensor's standard deviation;
  * rounded once, round-to-nearest-even, to BF16 when the payload is BF16 or
    FP8 (FP8 quantisation belongs to the method and is done by each side);
  * router logits always stay FP32.
Tensor ids: x=1, logits=2, W1=3, W2=4, W_r=5, dy=6, Zipf popularity ranks=7, upstream
gate gradients for the route-backward stage alone=8, tie-heavy logits=9.

Workloads follow the token-wise ChunkedEP single-layer setting (Megatron-LM
PR 7342, "Historical single-layer OP measurements": EP8, top-k 8, two token
chunks) reduced to one GPU's share, plus a tiny FP32 case.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

TENSOR_IDS = {"x": 1, "logits": 2, "w1": 3, "w2": 4, "w_r": 5, "dy": 6, "zipf": 7, "dgates": 8,
              "tie_logits": 9}


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # logical tokens on this GPU
    H: int            # hidden size
    I: int            # expert intermediate size (SwiGLU)
    E: int            # router width (all experts)
    E_local: int      # local experts [e0, e0 + E_local)
    k: int            # top-k
    n_chunks: int
    dtype: str        # "f32" | "bf16" | "fp8"
    seed_base: int
    e0: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: Optional[float] = None   # popularity bias exponent (imbalanced routing)
    n_empty: int = 0                 # least-popular local experts forced empty
    backward: bool = False

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


# The tiny FP32 case, the BF16 one-rank share at 16K tokens (forward), the
# fused forward/backward at 32K and at 16K tokens, imbalanced (Zipf 1.2)
# routing, and the FP8 payload path at H=2048 and H=7168.
CONFIGS: Dict[str, MoeConfig] = {
    "tiny": MoeConfig("tiny", T=256, H=128, I=256, E=8, E_local=8, k=2, n_chunks=1,
                      dtype="f32", seed_base=0, x_std=0.02, backward=True),
    "fwd16k": MoeConfig("fwd16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8,
                        n_chunks=2, dtype="bf16", seed_base=100),
    "fb32k": MoeConfig("fb32k", T=32768, H=2048, I=768, E=128, E_local=16, k=8,
                       n_chunks=2, dtype="bf16", seed_base=200, backward=True),
    "fb16k": MoeConfig("fb16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8,
                       n_chunks=2, dtype="bf16", seed_base=250, backward=True),
    "zipf16k": MoeConfig("zipf16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8,
                         n_chunks=2, dtype="bf16", seed_base=300, zipf_s=1.2, n_empty=3,
                         backward=True),
    "fp8_16k": MoeConfig("fp8_16k", T=16384, H=2048, I=768, E=128, E_local=16, k=8,
                         n_chunks=2, dtype="fp8", seed_base=400),
    "fp8_16k_h7168": MoeConfig("fp8_16k_h7168", T=16384, H=7168, I=768, E=128, E_local=16,
                               k=8, n_chunks=2, dtype="fp8", seed_base=450),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(cfg: MoeConfig, name: str, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(cfg.seed_base + TENSOR_IDS[name])
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _payload(cfg: MoeConfig, a: np.ndarray) -> Dict[str, np.ndarray]:
    """FP32 draw -> payload values. Returns ``f32`` (values as FP32) and, for 16-bit payloads, ``bits``."""
    if cfg.dtype == "f32":
        return {"f32": a, "bits": None}
    bits = f32_to_bf16_bits(a)
    return {"f32": bf16_bits_to_f32(bits), "bits": bits}


def zipf_bias(cfg: MoeConfig) -> np.ndarray:
    """Per-expert logit bias giving a Zipf(s) popularity order over a seeded permutation.

    bias_e = -s * ln(rank_e), rank = a seeded permutation of 1..E; the ``n_empty``
    least popular local experts get -1e4 so that they receive no token.
    """
    rng = np.random.default_rng(cfg.seed_base + TENSOR_IDS["zipf"])
    rank = rng.permutation(cfg.E).astype(np.float64) + 1.0
    bias = -cfg.zipf_s * np.log(rank)
    if cfg.n_empty:
        local = np.arange(cfg.e0, cfg.e0 + cfg.E_local)
        least = local[np.argsort(-rank[local], kind="stable")[: cfg.n_empty]]
        bias[least] = -1e4
    return bias.astype(np.float32)


def make_inputs(cfg: MoeConfig, with_backward: Optional[bool] = None,
                parts=("x", "logits", "w1", "w2", "w_r", "dy")) -> Dict[str, np.ndarray]:
    """Draw the layer's inputs. Keys: name -> FP32 values, name+'_bits' -> uint16 BF16 patterns."""
    if with_backward is None:
        with_backward = cfg.backward
    out: Dict[str, np.ndarray] = {}
    shapes = {
        "x": ((cfg.T, cfg.H), cfg.x_std),
        "w1": ((cfg.E_local, 2 * cfg.I, cfg.H), cfg.w_std),
        "w2": ((cfg.E_local, cfg.H, cfg.I), cfg.w_std),
        "w_r": ((cfg.E, cfg.H), cfg.w_std),
        "dy": ((cfg.T, cfg.H), 1.0),
    }
    for name in parts:
        if name == "logits":
            lg = _normal(cfg, "logits", (cfg.T, cfg.E), 1.0)
            if cfg.zipf_s is not None:
                lg = (lg + zipf_bias(cfg)[None, :]).astype(np.float32)
            out["logits"] = lg
            continue
        if name == "dy" and not with_backward:
            continue
        shape, std = shapes[name]
        p = _payload(cfg, _normal(cfg, name, shape, std))
        out[name] = p["f32"]
        if p["bits"] is not None:
            out[name + "_bits"] = p["bits"]
    return out


def make_dgates(cfg: MoeConfig) -> np.ndarray:
    """Upstream gate gradients [T, k] ~ N(0, 1) in FP32, for running the route backward on its own."""
    return _normal(cfg, "dgates", (cfg.T, cfg.k), 1.0)


def make_tie_logits(cfg: MoeConfig, nan_frac: float = 0.02) -> np.ndarray:
    """Router logits [T, E] in FP32 with many exact ties: N(0, 1) rounded to multiples of 0.5, so
    that equal values, including the k-th and (k+1)-th largest of a row, are common. Zeros come
    with both signs (rounding keeps the sign of small negative draws, and half of the remaining
    zeros are negated), and a fraction ``nan_frac`` of the entries are NaN (at most
    E - k per row, so every row keeps k non-NaN entries). Row 0 is all zeros of mixed sign, row 1
    holds k - 1 finite values with -inf and NaN elsewhere (when T > 1)."""
    rng = np.random.default_rng(cfg.seed_base + TENSOR_IDS["tie_logits"])
    T, E, k = cfg.T, cfg.E, cfg.k
    lg = np.round(rng.standard_normal((T, E), dtype=np.float32) * np.float32(2.0)) * np.float32(0.5)
    zeros = lg == 0
    flip = rng.random((T, E)) < 0.5
    lg[zeros & flip] = np.float32(-0.0)
    if nan_frac > 0 and E > k:
        cand = rng.random((T, E)) < nan_frac
        # keep at most E - k NaNs per row
        over = np.cumsum(cand, axis=1) > (E - k)
        lg[cand & ~over] = np.float32(np.nan)
    if T > 0:
        lg[0] = np.where(rng.random(E) < 0.5, np.float32(0.0), np.float32(-0.0))
    if T > 1 and k >= 2:
        row = np.full(E, -np.inf, dtype=np.float32)
        row[rng.random(E) < 0.5] = np.float32(np.nan)
        pos = rng.choice(E, size=k - 1, replace=False)
        row[pos] = np.float32(1.0) + np.arange(k - 1, dtype=np.float32)
        lg[1] = row
    return lg.astype(np.float32)
