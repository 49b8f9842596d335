"""Seeded synthetic inputs for jagged HSTU attention.

This module only draws random inputs: jagged lengths and offsets, int64
timestamps, Q/K/V, per-head bucket weights and an upstream gradient.  It holds
none of the method's arithmetic (no bucketing, no attention, no SiLU), so both
the float64 oracle and the HIP path can consume the same arrays without sharing
any computation.

Shapes and distributions follow the workloads described for the method:

* jagged ``values`` are token-major ``[T, H, d]`` with int64 ``offsets[B+1]``
  (the TorchRec values/offsets/max_lengths representation; Scaling Generative
  Recommendations with Context Parallelism on HSTU, §2.2 "Jagged Tensors");
* timestamps are int64, strictly increasing per sequence, with exponential gaps
  and a per-sequence start near 1.7e9 s so the int64 path is exercised;
* bucket weights are drawn from a normal distribution (same paper, §2.1,
  timestamp-bias paragraph: the learnable ``ts_weights`` table starts from
  normally distributed values); the standard deviation 0.02 is the workload's
  choice.

bf16 values are produced by round-to-nearest-even of float32 draws and are
returned both as raw uint16 bit patterns (for device upload) and as exact
float64 values (for the oracle).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TS_BASE = 1_700_000_000
TS_START_SPREAD = 10_000_000


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """A generated floating-point tensor: exact float64 values plus raw bits."""

    f64: np.ndarray          # exact values the device sees, as float64
    raw: np.ndarray          # uint16 bf16 bits, or float32 values
    dtype: str               # "bf16" or "fp32"


def make_tensor(rng: np.random.Generator, shape, dtype: str, std: float = 1.0) -> Tensor:
    x = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return from_f32(x, dtype)


def from_f32(x: np.ndarray, dtype: str) -> Tensor:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return Tensor(bf16_bits_to_f64(bits), bits, "bf16")
    if dtype == "fp32":
        return Tensor(x.astype(np.float64), x, "fp32")
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    lengths: np.ndarray
    offsets: np.ndarray      # int64 [B+1]
    ts: np.ndarray           # int64 [T]
    num_heads: int
    d_qk: int
    d_v: int
    num_buckets: int
    q: Tensor
    k: Tensor
    v: Tensor
    w: Tensor                # [H, NB]
    dout: Optional[Tensor]
    seed: int

    @property
    def num_seqs(self) -> int:
        return int(len(self.lengths))

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    @property
    def max_seq_len(self) -> int:
        return int(self.lengths.max()) if len(self.lengths) else 0


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def make_timestamps(rng: np.random.Generator, lengths, gap_mean: float) -> np.ndarray:
    """Strictly increasing int64 timestamps per sequence: start + cumsum(ceil(Exp(mean)))."""
    parts = []
    for n in np.asarray(lengths, dtype=np.int64):
        start = TS_BASE + int(rng.integers(0, TS_START_SPREAD))
        gaps = np.maximum(np.ceil(rng.exponential(gap_mean, size=int(n))), 1).astype(np.int64)
        if n:
            gaps[0] = 0
        parts.append(start + np.cumsum(gaps))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts).astype(np.int64)


def power_law_lengths(rng: np.random.Generator, n: int, alpha: float, lo: int, hi: int) -> np.ndarray:
    """Inverse-CDF draw from pdf ∝ L^-alpha truncated to [lo, hi], floored."""
    u = rng.random(n)
    a = 1.0 - alpha
    x = (lo ** a + u * (hi ** a - lo ** a)) ** (1.0 / a)
    return np.clip(np.floor(x).astype(np.int64), lo, hi)


def make_workload(name: str, lengths, *, num_heads: int, d_qk: int, d_v: int,
                  num_buckets: int, dtype: str, gap_mean: float, seed: int,
                  w_std: float = 0.02, with_dout: bool = True,
                  rng: Optional[np.random.Generator] = None) -> Workload:
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    offsets = offsets_from_lengths(lengths)
    total = int(offsets[-1])
    ts = make_timestamps(rng, lengths, gap_mean)
    q = make_tensor(rng, (total, num_heads, d_qk), dtype)
    k = make_tensor(rng, (total, num_heads, d_qk), dtype)
    v = make_tensor(rng, (total, num_heads, d_v), dtype)
    w = make_tensor(rng, (num_heads, num_buckets), dtype, std=w_std)
    dout = make_tensor(rng, (total, num_heads, d_v), dtype) if with_dout else None
    return Workload(name, dtype, lengths, offsets, ts, num_heads, d_qk, d_v,
                    num_buckets, q, k, v, w, dout, seed)


# The five workloads: (name, default seed).  Seeds 1001..1005; parity tests also
# use seed + 100.
CONFIGS = {
    "tiny_fp32": 1001,
    "bf16_fwd_u256_1024": 1002,
    "bf16_len3072": 1003,
    "cp8_rank3_len16384": 1004,
    "skewed_powerlaw": 1005,
}

CP_SIZE = 8
CP_RANK = 3


def config(name: str, seed: Optional[int] = None, *, with_dout: bool = True,
           num_seqs: Optional[int] = None) -> Workload:
    """Build one of the named workloads.  ``num_seqs`` (if given) keeps only the
    first sequences, for bounded samples of a large workload."""
    seed = CONFIGS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        lengths = rng.integers(1, 65, size=4)
        kw = dict(num_heads=2, d_qk=32, d_v=32, num_buckets=128, dtype="fp32", gap_mean=3600.0)
    elif name == "bf16_fwd_u256_1024":
        lengths = rng.integers(256, 1025, size=32)
        kw = dict(num_heads=4, d_qk=128, d_v=128, num_buckets=128, dtype="bf16", gap_mean=3600.0)
    elif name == "bf16_len3072":
        lengths = np.full(16, 3072)
        kw = dict(num_heads=4, d_qk=128, d_v=128, num_buckets=128, dtype="bf16", gap_mean=3600.0)
    elif name == "cp8_rank3_len16384":
        lengths = np.full(4, 16384)
        kw = dict(num_heads=4, d_qk=128, d_v=128, num_buckets=128, dtype="bf16", gap_mean=3600.0)
    elif name == "skewed_powerlaw":
        lengths = power_law_lengths(rng, 256, 1.2, 16, 8192)
        kw = dict(num_heads=8, d_qk=64, d_v=64, num_buckets=256, dtype="bf16", gap_mean=600.0)
    else:
        raise KeyError(name)
    if num_seqs is not None:
        lengths = lengths[:num_seqs]
    return make_workload(name, lengths, seed=seed, with_dout=with_dout, rng=rng, **kw)


def custom(lengths, *, num_heads=2, d_qk=32, d_v=32, num_buckets=128, dtype="fp32",
           gap_mean=3600.0, seed=0, w_std=0.02, with_dout=True) -> Workload:
    return make_workload("custom", lengths, num_heads=num_heads, d_qk=d_qk, d_v=d_v,
                         num_buckets=num_buckets, dtype=dtype, gap_mean=gap_mean,
                         seed=seed, w_std=w_std, with_dout=with_dout)


@dataclasses.dataclass
class LayerInputs:
    x: Tensor        # [T, d_model]
    w: Tensor        # [H (2 d_v + 2 d_qk), d_model]
    num_heads: int
    d_qk: int
    d_v: int


def layer_inputs(total_rows: int, d_model: int, num_heads: int, d_qk: int, d_v: int, *, dtype: str = "bf16",
                 seed: int = 0) -> LayerInputs:
    """Inputs of the layer steps around the attention: X ~ N(0, 1) and a
    projection weight ~ N(0, 1 / d_model) (unit-variance outputs)."""
    rng = np.random.default_rng(seed)
    x = make_tensor(rng, (total_rows, d_model), dtype)
    w = make_tensor(rng, (num_heads * (2 * d_v + 2 * d_qk), d_model), dtype, std=1.0 / np.sqrt(d_model))
    return LayerInputs(x, w, num_heads, d_qk, d_v)
