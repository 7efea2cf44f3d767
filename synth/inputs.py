"""Synthetic Q/K/V/dO generator.

Recipe (frozen draw order, one independent PCG64 stream per tensor and head so
that any head can be drawn alone):

1. ``u[Hkv, d]`` ~ N(0, 1), each row scaled to unit norm.
2. ``Q0[Hq, N, d]``, ``K0[Hkv, N, d]``, ``V[Hkv, N, d]``, ``dO[Hq, N, d]`` ~ N(0, 1).
3. Outlier key positions: ``n_out`` distinct positions drawn uniformly, shared
   by every kv head.
4. ``Q = Q0 + c * u[g(h)]``, ``K = K0 + c * u[g]``; outlier rows of K are scaled
   by ``f_out``.
5. Rotary embedding (rotate-half convention, frequency ``theta_i =
   base^(-2i/d)``, global positions 0..N-1), optionally with Yarn scaling.
6. Round to the workload dtype (fp32, or bf16 via fp32 with round-to-nearest-even).

The shared mean ``c * u`` before the rotation is what makes the rotary
expectation model of the MTraining review (page 1, section 三.1, the expectation
formula for ``E[z_{n,m}]``) non-trivial: it supplies the position-independent
constants ``A_i, B_i``, so the expected logit depends on ``n - m`` only and
peaks at ``n = m`` (the slash band). Scaled key rows give the vertical lines
(same section: outlier tokens with abnormally large key norms).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

_TAGS = {"u": 1, "q": 2, "k": 3, "v": 4, "do": 5, "outliers": 6}


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16"
    n_out: int            # number of outlier keys
    f_out: float          # outlier key scale
    c: float              # shared-mean strength (0 = literal N(0,1) inputs)
    top_p: float
    seed: int
    last_q: int = 64
    rope_base: float = 10000.0
    yarn_scale: float = 1.0   # 1 = plain RoPE
    backward: bool = False
    P: int = 1                # context-parallel ranks (ring simulation)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# Shared-mean strengths calibrated per workload so that the oracle's mean
# per-head sparsity is ~95% (python -m oracle.calibrate --config NAME).
# Sparsity depends strongly on N at fixed c, hence one value per workload.
C_STAR = {"qwen32k": 7.27, "qwen128k": 3.64, "qwen512k_cp32": 0.0, "llama256k": 0.0}

CONFIGS = {
    "tiny": WorkloadConfig("tiny", 1, 1, 2048, 64, "f32", 8, 8.0, 0.0, 0.9, 1001),
    "qwen32k": WorkloadConfig("qwen32k", 16, 2, 32768, 128, "bf16", 33, 6.0, C_STAR["qwen32k"], 0.95, 1002),
    "qwen128k": WorkloadConfig("qwen128k", 16, 2, 131072, 128, "bf16", 131, 6.0, C_STAR["qwen128k"], 0.95, 1003,
                               backward=True),
    "qwen512k_cp32": WorkloadConfig("qwen512k_cp32", 16, 2, 524288, 128, "bf16", 524, 6.0, C_STAR["qwen512k_cp32"], 0.95,
                                    1004, backward=True, P=32),
    "llama256k": WorkloadConfig("llama256k", 32, 8, 262144, 128, "bf16", 262, 6.0, C_STAR["llama256k"], 0.95, 1005,
                                yarn_scale=32.0, backward=True),
}


def config_by_name(name: str, **overrides) -> WorkloadConfig:
    return dataclasses.replace(CONFIGS[name], **overrides)


def _rng(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(_TAGS[tag], idx))
    return np.random.Generator(np.random.PCG64(ss))


def rope_frequencies(D: int, base: float, yarn_scale: float, n_orig: int) -> np.ndarray:
    """Per-pair rotation frequencies theta_i, i in [0, D/2).

    Plain RoPE: theta_i = base^(-2i/D). With Yarn (Peng et al.), frequencies
    are blended between interpolated (theta/s) and original by a linear ramp in
    r = n_orig / wavelength with alpha=1, beta=32 ("NTK-by-parts").
    """
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    if yarn_scale == 1.0:
        return theta
    s = yarn_scale
    wavelength = 2.0 * math.pi / theta
    r = n_orig / wavelength
    alpha, beta = 1.0, 32.0
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / s + gamma * theta


def apply_rope(x: np.ndarray, pos: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on x[..., N, D] (fp64) at integer positions pos[N]."""
    D = x.shape[-1]
    h = D // 2
    ang = pos[:, None].astype(np.float64) * theta[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = x1 * cos - x2 * sin
    out[..., h:] = x2 * cos + x1 * sin
    return out


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the workload dtype; returns float32 (values exactly representable)."""
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_from_bf16_bits(bf16_bits_from_f32(x32))
    raise ValueError(dtype)


def _outlier_positions(cfg: WorkloadConfig) -> np.ndarray:
    if cfg.n_out == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg.seed, "outliers").choice(cfg.N, size=cfg.n_out, replace=False))


def _mean_dirs(cfg: WorkloadConfig) -> np.ndarray:
    u = _rng(cfg.seed, "u").standard_normal((cfg.Hkv, cfg.D))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def generate(cfg: WorkloadConfig, tensors=("q", "k", "v", "do"), heads: Optional[dict] = None,
             rows: Optional[slice] = None) -> dict:
    """Draw the workload's tensors as float32 arrays holding dtype-exact values.

    ``heads`` may restrict a tensor to some heads, e.g. ``{"q": [3]}``;
    ``rows`` may restrict the sequence range (same values as the full draw).
    Returns ``{"q": [Hq', n, D], "k": [Hkv', n, D], ..., "outliers": positions}``.
    """
    heads = heads or {}
    N, D = cfg.N, cfg.D
    sl = rows if rows is not None else slice(0, N)
    pos = np.arange(N, dtype=np.int64)[sl]
    u = _mean_dirs(cfg)
    outl = _outlier_positions(cfg)
    theta = rope_frequencies(D, cfg.rope_base, cfg.yarn_scale, max(1, int(N / cfg.yarn_scale)))
    yarn_mult = (0.1 * math.log(cfg.yarn_scale) + 1.0) if cfg.yarn_scale != 1.0 else 1.0
    group = cfg.Hq // cfg.Hkv
    out = {"outliers": outl}
    for t in tensors:
        nh = cfg.Hq if t in ("q", "do") else cfg.Hkv
        hl = list(heads.get(t, range(nh)))
        arr = np.empty((len(hl), pos.shape[0], D), dtype=np.float32)
        for a, h in enumerate(hl):
            full = _rng(cfg.seed, t, h).standard_normal((N, D))
            x = full[sl]
            if t == "q":
                x = x + cfg.c * u[h // group]
            elif t == "k":
                x = x + cfg.c * u[h]
                is_out = np.isin(pos, outl)
                x[is_out] *= cfg.f_out
            if t in ("q", "k"):
                x = apply_rope(x, pos, theta) * yarn_mult
            arr[a] = round_to_dtype(x, cfg.dtype)
        out[t] = arr
    return out


def layout_permutation(kind: str, N: int, P: int, rank: int) -> np.ndarray:
    """Global positions owned by ``rank``, in local (storage) order.

    contig: rank r owns [r N/P, (r+1) N/P).
    striped: 64-token stripes dealt round-robin; rank r owns global 64-blocks
             G with G mod P == r (the balanced layout of the review, page 1,
             section 三.3).
    striped1: single positions dealt round-robin; rank r owns positions n with
             n mod P == r (the fine-grained stripes of the Ring Attention
             overview, section 3.1).
    zigzag: 2P equal chunks; rank r owns chunks r and 2P-1-r (same section).
    """
    if kind == "contig":
        n = N // P
        return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)
    if kind == "striped":
        T = N // 64
        blocks = np.arange(rank, T, P, dtype=np.int64)
        return (blocks[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    if kind == "striped1":
        return np.arange(rank, N, P, dtype=np.int64)
    if kind == "zigzag":
        c = N // (2 * P)
        a = np.arange(rank * c, (rank + 1) * c, dtype=np.int64)
        b = np.arange((2 * P - 1 - rank) * c, (2 * P - rank) * c, dtype=np.int64)
        return np.concatenate([a, b])
    raise ValueError(kind)
