"""Seeded synthetic workloads for jagged attention.

This module only *draws* inputs: sequence lengths, prefix-sum offsets, normal
values rounded to bf16, an additive bias table and an upstream gradient. It
holds none of the attention arithmetic, so both the fp64 CPU oracle and the
GPU path can be fed the very same bytes.

Workloads follow the five shapes the method is benchmarked on (jagged
self-attention with uniform or lognormal lengths, an asymmetric query/key-value
case with a per-head relative-position bias, and a long-tail causal case).
Lengths: uniform integers, or ``clip(rint(exp(N(mu, sigma))), lo, hi)`` for the
lognormal cases. Draw order per workload: query lengths, key/value lengths (only
for asymmetric workloads), Q, K, V, dO, bias.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

BIAS_RADIUS = 128  # bias table is [H, 2*R+1]; index clip(i-j, -R, R) + R


@dataclasses.dataclass(frozen=True)
class LengthDist:
    kind: str  # "uniform" (inclusive ints) or "lognormal"
    lo: int
    hi: int
    mu: float = 0.0
    sigma: float = 0.0

    def sample(self, rng: np.random.Generator, n: int) -> np.ndarray:
        if self.kind == "uniform":
            return rng.integers(self.lo, self.hi + 1, size=n).astype(np.int64)
        if self.kind == "lognormal":
            x = np.rint(np.exp(rng.normal(self.mu, self.sigma, size=n)))
            return np.clip(x, self.lo, self.hi).astype(np.int64)
        if self.kind == "fixed":
            return np.full(n, self.lo, dtype=np.int64)
        raise ValueError(self.kind)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    dtype: str  # "bf16" or "f32"
    causal: bool
    bias: bool
    q_len: LengthDist
    kv_len: Optional[LengthDist] = None  # None: self-attention (kv lengths = q lengths)
    seed: int = 0


# The five benchmark workloads. Seeds are 1000 + workload number.
WORKLOADS = {
    1: Workload("tiny_f32", 4, 2, 32, "f32", False, False, LengthDist("uniform", 1, 64), seed=1001),
    2: Workload("uniform1024_d64", 64, 8, 64, "bf16", False, False, LengthDist("uniform", 1, 1024), seed=1002),
    3: Workload("gem_lognormal_causal_d128", 256, 4, 128, "bf16", True, False,
                LengthDist("lognormal", 32, 4096, math.log(1500.0), 0.6), seed=1003),
    4: Workload("asym_bias_d128", 128, 8, 128, "bf16", False, True, LengthDist("uniform", 1, 64),
                LengthDist("lognormal", 64, 16384, math.log(4000.0), 0.8), seed=1004),
    5: Workload("longtail_causal_d128", 32, 4, 128, "bf16", True, False,
                LengthDist("lognormal", 16, 32768, math.log(6000.0), 1.0), seed=1005),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def offsets_from_lengths(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off.astype(np.int32)


@dataclasses.dataclass
class Batch:
    """Host copy of one synthetic batch.

    Tensors of dtype bf16 are kept as uint16 bit patterns (``*_bits``) plus their
    exact fp32 values; f32 workloads keep fp32 values only (``*_bits`` is None).
    Layout: values [T, H, D] row-major; offsets int32 [B+1]; lse-like [T, H].
    """
    wl: Workload
    q_lengths: np.ndarray
    kv_lengths: np.ndarray
    q_offsets: np.ndarray
    kv_offsets: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dout: np.ndarray
    bias: Optional[np.ndarray]
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    dout_bits: Optional[np.ndarray] = None

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_offsets[-1])


def _normal(rng: np.random.Generator, shape: Tuple[int, ...], bf16: bool):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if not bf16:
        return x, None
    bits = bf16_round(x)
    del x
    return bf16_bits_to_f32(bits), bits


def make_batch(wl: Workload, seed: Optional[int] = None, *, q_lengths=None, kv_lengths=None,
               with_dout: bool = True) -> Batch:
    """Draw one batch for workload ``wl``.

    ``q_lengths``/``kv_lengths`` override the sampled lengths (edge-case tests);
    everything else is still drawn from ``seed`` in the fixed order.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    ql = wl.q_len.sample(rng, wl.B)
    if wl.kv_len is not None:
        kl = wl.kv_len.sample(rng, wl.B)
    else:
        kl = ql
    if q_lengths is not None:
        ql = np.asarray(q_lengths, dtype=np.int64)
    if kv_lengths is not None:
        kl = np.asarray(kv_lengths, dtype=np.int64)
    elif q_lengths is not None and wl.kv_len is None:
        kl = ql
    qo, ko = offsets_from_lengths(ql), offsets_from_lengths(kl)
    Tq, Tk = int(qo[-1]), int(ko[-1])
    bf = wl.dtype == "bf16"
    q, qb = _normal(rng, (Tq, wl.H, wl.D), bf)
    k, kb = _normal(rng, (Tk, wl.H, wl.D), bf)
    v, vb = _normal(rng, (Tk, wl.H, wl.D), bf)
    if with_dout:
        do, dob = _normal(rng, (Tq, wl.H, wl.D), bf)
    else:
        do, dob = None, None
    bias = None
    if wl.bias:
        bias = (rng.standard_normal(size=(wl.H, 2 * BIAS_RADIUS + 1)) * 0.1).astype(np.float32)
    return Batch(wl, ql, kl, qo, ko, q, k, v, do, bias, qb, kb, vb, dob)


def small_workload(base: Workload, B: int, lo: int, hi: int, *, H: Optional[int] = None,
                   kv: Optional[Tuple[int, int]] = None, seed: int = 7) -> Workload:
    """A reduced copy of ``base`` (same H/D/dtype/mask/bias) with uniform lengths."""
    return dataclasses.replace(
        base, B=B, H=base.H if H is None else H, q_len=LengthDist("uniform", lo, hi),
        kv_len=None if kv is None else LengthDist("uniform", kv[0], kv[1]), seed=seed)
