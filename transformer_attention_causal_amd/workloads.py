"""Seeded synthetic inputs for the attention workloads.

This module is the one thing the HIP path's tests/benchmark and the oracle
share: it draws random inputs and stores them in the dtype the kernels read.
It holds none of the attention arithmetic -- only random draws, the scaling
the workload recipe states, and rounding of the stored values to bf16.

Recipe (numpy ``Generator(PCG64(seed))``; draws in fp64, scaled, rounded to
fp32, then -- for bf16 storage -- to bf16 with round-to-nearest-even):

* Q, K, V are drawn in that order, each as one [B,H,T,d] C-order block.
* ``scale`` multiplies all three (the T=2048 softmax workload uses 1/sqrt(2)).
* ``heavy_frac`` > 0: per (b,h), in order, round(heavy_frac*T) distinct key
  positions are drawn without replacement and those K rows are multiplied by
  ``heavy_scale`` (5 % of keys with 3x norm concentrate demand).
* Learned temperatures (head dimension 128): per (b,h) a temperature
  t ~ U[tau_min, tau_max] = U[5, 10] (the clip range the focal page settles
  on) is drawn from its own stream, and the kernels get the multiplier
  tau = sqrt(d) / t.
* Decode: the initial demand D0[s,h,pos] ~ U[0, 4 (L-pos)/L] (fp64 draw,
  stored fp32); the per-step queries are N(0,1) bf16, drawn as one
  [steps,S,H,d] block from their own seed.  Caches too large to draw on the
  host are drawn on the device with torch's seeded Philox generator.

The pages measure dilution on FineWeb-Edu training and softmax/temperature on
trained LLaMA-style models; neither dataset nor any trained weights are used:
these synthetic tensors stand in for the per-layer Q/K/V of such models.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_round_bits(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even on the fp32 value); return uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs only: the carry cannot leave 32 bits
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Prefill:
    """One forward workload: shapes, storage dtype and input distribution."""

    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str  # "f32" or "bf16"
    seed: int
    scale: float = 1.0
    heavy_frac: float = 0.0
    heavy_scale: float = 3.0
    yarn_s: float = 4.0  # extension factor whose YaRN temperature the softmax run uses
    eps: float = 1e-6
    note: str = ""


@dataclass(frozen=True)
class Decode:
    """The cached-decode workload."""

    name: str
    S: int
    H: int
    L: int
    d: int
    steps: int
    seed: int
    demand_max: float = 4.0
    eps: float = 1e-6
    tau: float = 1.0
    note: str = ""


# The named workloads: the shapes the pages train and evaluate at (16K context,
# 128K evaluation, 64-dim heads; the focal models' 20 heads of 128), the
# oracle-sized fp32 case, and the 32K-key decode cache.
PREFILL = {
    "fp32_t256": Prefill("fp32_t256", 1, 2, 256, 64, "f32", seed=20261,
                         note="fp32, tau=1 and YaRN s=4, dilution eps=1e-6"),
    "softmax_t2048": Prefill("softmax_t2048", 4, 16, 2048, 64, "bf16", seed=20262,
                             scale=1.0 / math.sqrt(2.0),
                             note="tempered, bf16 I/O, tau=YaRN(s=4)"),
    "dilution_t16k": Prefill("dilution_t16k", 1, 16, 16384, 64, "bf16", seed=20263,
                             heavy_frac=0.05,
                             note="24-layer 209M decoder per-layer shape at 16K"),
    "long_t128k": Prefill("long_t128k", 1, 16, 131072, 64, "bf16", seed=20264,
                          heavy_frac=0.05, yarn_s=8.0,
                          note="8x the training context; oracle on head 0"),
    "focal_d128_t16k": Prefill("focal_d128_t16k", 1, 20, 16384, 128, "bf16", seed=20266,
                               heavy_frac=0.05,
                               note="2.7B focal model's attention shape (20 heads of 128) at "
                                    "16K, per-head learned temperatures"),
}

DECODE = {
    "decode_32k": Decode("decode_32k", 64, 16, 32768, 64, 128, seed=20265,
                         note="64 sequences x 32768-key cache, 128 steps"),
}


@dataclass
class HostInputs:
    """Host copies of one workload's inputs, exactly as the device receives them.

    For bf16 storage ``q``/``k``/``v`` hold uint16 bit patterns; for fp32 they
    hold float32 arrays.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    heavy: list = field(default_factory=list)


def draw_qkv(B: int, H: int, T: int, d: int, dtype: str, seed: int, scale: float = 1.0,
             heavy_frac: float = 0.0, heavy_scale: float = 3.0) -> HostInputs:
    """Draw Q, K, V per the recipe in the module docstring."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, T, d)
    arrs = []
    for _ in range(3):
        x = rng.standard_normal(shape)
        if scale != 1.0:
            x *= scale
        arrs.append(x.astype(np.float32))
    q, k, v = arrs
    heavy = []
    if heavy_frac > 0.0:
        n = int(round(heavy_frac * T))
        for b in range(B):
            for h in range(H):
                pos = rng.choice(T, size=n, replace=False)
                k[b, h, pos, :] *= np.float32(heavy_scale)
                heavy.append(np.sort(pos))
    if dtype == "bf16":
        q, k, v = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
    return HostInputs(q, k, v, dtype, heavy)


def learned_tau(B: int, H: int, d: int, seed: int, t_min: float = 5.0,
                t_max: float = 10.0) -> np.ndarray:
    """Per-(b,h) multipliers sqrt(d)/t with t ~ U[t_min, t_max], fp32 [B,H]
    (stream seed+37)."""
    rng = np.random.Generator(np.random.PCG64(seed + 37))
    t = rng.uniform(t_min, t_max, size=(B, H))
    return (math.sqrt(d) / t).astype(np.float32)


def draw_grad(B: int, H: int, T: int, d: int, seed: int) -> np.ndarray:
    """An incoming output gradient dO ~ N(0,1), bf16 bit patterns (stream seed+29)."""
    rng = np.random.Generator(np.random.PCG64(seed + 29))
    return bf16_round_bits(rng.standard_normal((B, H, T, d)).astype(np.float32))


def prefill_inputs(w: Prefill, T: int | None = None, H: int | None = None,
                   B: int | None = None) -> HostInputs:
    """Inputs of a named forward workload (optionally at a reduced shape)."""
    return draw_qkv(B or w.B, H or w.H, T or w.T, w.d, w.dtype, w.seed, w.scale,
                    w.heavy_frac, w.heavy_scale)


def decode_initial_demand(S: int, H: int, L: int, seed: int,
                          demand_max: float = 4.0) -> np.ndarray:
    """D0[s,h,pos] ~ U[0, demand_max * (L - pos) / L], fp32."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    u = rng.random((S, H, L))
    ramp = demand_max * (L - np.arange(L, dtype=np.float64)) / L
    return (u * ramp).astype(np.float32)


def decode_queries(steps: int, S: int, H: int, d: int, seed: int) -> np.ndarray:
    """Per-step decode queries, N(0,1), bf16 bits, shape [steps,S,H,d]."""
    rng = np.random.Generator(np.random.PCG64(seed + 11))
    return bf16_round_bits(rng.standard_normal((steps, S, H, d)))


def decode_cache_host(S: int, H: int, L: int, d: int, seed: int):
    """K and V caches, N(0,1), bf16 bits [S,H,L,d] -- for sizes the host can draw."""
    rng = np.random.Generator(np.random.PCG64(seed + 13))
    k = bf16_round_bits(rng.standard_normal((S, H, L, d)))
    v = bf16_round_bits(rng.standard_normal((S, H, L, d)))
    return k, v


def decode_cache_device(S: int, H: int, L: int, d: int, seed: int, device="cuda"):
    """K and V caches, N(0,1) bf16 [S,H,L,d], drawn on the device with torch's
    seeded Philox generator (one sequence at a time, so no fp32 copy of the
    whole cache is ever held)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed + 17)
    out = []
    for _ in range(2):
        t = torch.empty((S, H, L, d), dtype=torch.bfloat16, device=device)
        for s in range(S):
            t[s].copy_(torch.randn((H, L, d), generator=g, device=device,
                                   dtype=torch.float32))
        out.append(t)
    return out[0], out[1]
