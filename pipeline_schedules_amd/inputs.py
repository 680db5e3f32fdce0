"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and converts their storage format; it
holds none of the method's arithmetic.

Draw order (fixed): for every stage s in ``stages`` (ascending), for every
chunk c, for every block b: the block's weights (SwiGLU: Wg, Wu, Wd; toy: W),
then x[0..M-1] (the stage-0 input of every micro-batch), then G[0..M-1] (the
output-gradient probe).  Distributions (second parameter = std):
weights N(0, 0.02), x N(0, 1), G N(0, 0.01), gamma = 1, toy bias = 0.

Two backends:
  * ``numpy``: ``numpy.random.default_rng(seed)``, float64 draws, cast to
    float32 and, for bf16 workloads, rounded to bf16 (round-to-nearest-even).
    Used for every size the oracle runs on.
  * ``torch``: ``torch.Generator(device).manual_seed(seed)`` on the GPU,
    float32 draws cast with ``.to(torch.bfloat16)`` (RNE).  Used for the
    full-size workloads whose weights (tens of GB) are drawn in HBM.
The two backends give different numbers for the same seed.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array of the bf16 values nearest to ``a`` (ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 storage of a float32 array that already holds bf16 values."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class StageInputs:
    """Inputs of one or more stages.  Arrays are float32 (bf16-exact for bf16)."""
    params: list = field(default_factory=list)   # [stage][chunk*L + block] -> dict
    xs: list = field(default_factory=list)       # M arrays [T, d]
    Gs: list = field(default_factory=list)       # M arrays [T, d]


def _store(a, bf16):
    a = a.astype(np.float32)
    return round_to_bf16(a) if bf16 else a


def make_inputs(cfg, stages=None, gamma=None, bias=None, rng_seed=None, T=None, M=None):
    """numpy backend.  ``stages`` defaults to [cfg.k].

    ``gamma``/``bias`` may be ``"random"`` to draw gamma ~ 1 + N(0, 0.1) and
    bias ~ N(0, 0.02) after each block's weights (used by tests so that a
    mistake in those paths cannot hide behind gamma = 1 or bias = 0).
    ``T``/``M`` override the workload's tokens per micro-batch / count.
    """
    seed = cfg.seed if rng_seed is None else rng_seed
    rng = np.random.default_rng(seed)
    bf16 = cfg.dtype == "bf16"
    T = cfg.T if T is None else T
    M = cfg.M if M is None else M
    stages = [cfg.k] if stages is None else list(stages)
    out = StageInputs()
    for _s in stages:
        blocks = []
        for _c in range(cfg.v):
            for _b in range(cfg.L):
                if cfg.block == "swiglu":
                    p = {
                        "Wg": _store(rng.normal(0.0, cfg.w_std, (cfg.d, cfg.f)), bf16),
                        "Wu": _store(rng.normal(0.0, cfg.w_std, (cfg.d, cfg.f)), bf16),
                        "Wd": _store(rng.normal(0.0, cfg.w_std, (cfg.f, cfg.d)), bf16),
                    }
                    if gamma == "random":
                        p["gamma"] = _store(1.0 + rng.normal(0.0, 0.1, (cfg.d,)), False)
                    else:
                        p["gamma"] = np.ones((cfg.d,), dtype=np.float32)
                else:
                    p = {"W": _store(rng.normal(0.0, cfg.w_std, (cfg.d, cfg.d)), bf16)}
                    if bias == "random":
                        p["b"] = _store(rng.normal(0.0, cfg.w_std, (cfg.d,)), False)
                    else:
                        p["b"] = np.zeros((cfg.d,), dtype=np.float32)
                blocks.append(p)
        out.params.append(blocks)
    out.xs = [_store(rng.normal(0.0, cfg.x_std, (T, cfg.d)), bf16) for _ in range(M)]
    out.Gs = [_store(rng.normal(0.0, cfg.g_std, (T, cfg.d)), bf16) for _ in range(M)]
    return out


def make_sparse_token_inputs(cfg, rows_per_mb, rng_seed=None, T=None, M=None, gamma=None):
    """Inputs where only ``rows_per_mb`` sampled tokens of each micro-batch are
    non-zero in x and G; every other row of x and G is exactly 0.

    Returns (inputs, rows) with ``rows[i]`` the sorted non-zero row indices of
    micro-batch i (always including the last row, so a ragged tail is hit).
    """
    inp = make_inputs(cfg, rng_seed=rng_seed, T=T, M=M, gamma=gamma)
    T = cfg.T if T is None else T
    rng = np.random.default_rng((cfg.seed if rng_seed is None else rng_seed) + 7919)
    rows = []
    for i in range(len(inp.xs)):
        r = rng.choice(T - 1, size=rows_per_mb - 1, replace=False) if T > 1 else np.array([], dtype=np.int64)
        r = np.sort(np.concatenate([r, [T - 1]])).astype(np.int64)
        mask = np.zeros((T, 1), dtype=np.float32)
        mask[r] = 1.0
        inp.xs[i] = inp.xs[i] * mask
        inp.Gs[i] = inp.Gs[i] * mask
        rows.append(r)
    return inp, rows


def make_device_inputs(cfg, device, M=None, T=None, with_G=True):
    """torch backend for full-size workloads: draws in HBM with a seeded
    Philox generator.  Returns dict with ``params`` [chunk*L + block] of
    device tensors (bf16 weights, fp32 gamma), ``xs`` and ``Gs`` lists.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    T = cfg.T if T is None else T
    M = cfg.M if M is None else M

    def draw(shape, std):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(dt)

    params = []
    for _c in range(cfg.v):
        for _b in range(cfg.L):
            if cfg.block == "swiglu":
                params.append({
                    "Wg": draw((cfg.d, cfg.f), cfg.w_std),
                    "Wu": draw((cfg.d, cfg.f), cfg.w_std),
                    "Wd": draw((cfg.f, cfg.d), cfg.w_std),
                    "gamma": torch.ones((cfg.d,), device=device, dtype=torch.float32),
                })
            else:
                params.append({
                    "W": draw((cfg.d, cfg.d), cfg.w_std),
                    "b": torch.zeros((cfg.d,), device=device, dtype=torch.float32),
                })
    xs = [draw((T, cfg.d), cfg.x_std) for _ in range(M)]
    Gs = [draw((T, cfg.d), cfg.g_std) for _ in range(M)] if with_G else []
    return {"params": params, "xs": xs, "Gs": Gs}
