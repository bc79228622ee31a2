"""Seeded synthetic inputs for the multi-exit hot path.

This module only draws random numbers and packs them; it holds none of the
method's arithmetic.  Both the CPU oracle's callers (tests, benchmark
baseline) and the HIP path's callers take their inputs from here, so the two
sides always see the same values.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per suite, seed = 1000 +
workload index for the named workloads).  Draw order: the token sequence,
then block outputs h_1..h_M, then residual embedding tables e_1..e_M, then
head matrices W^1..W^M.

* block outputs  h_m  ~ N(0, 4^2) per element, shape [N, D_m]
  (the pages say a block's output is much larger than a fresh embedding:
  Matryoshka LM suites, main-visual explainer, panel (c));
* residual tables e_m ~ N(0, 0.02^2), shape [V, D_m - D_{m-1}], D_0 = 0
  (copyedit of Sec. 2 "Modeling": one table per block, width difference);
* heads W^m ~ N(0, 0.02^2), shape [V, D_m] (same section: W^m in R^{V x D_m});
* token ids: per batch row a sequence of L+1 tokens is drawn, ids are its
  first L entries and labels its last L (next-token structure).  Either
  uniform on [0, V) or a finite Zipf law P(k) ~ (k+1)^-s on [0, V) sampled by
  inverse CDF; the pages train on web text, which is not available here, so
  the Zipf law stands in for natural token frequencies.

Floats are drawn in float32.  For bf16 suites every float is rounded to
bfloat16 (round to nearest even) once; the arrays then hold bf16-exact values
in float32 and ``bf16_bits`` gives the 16-bit patterns the device consumes.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Suite", "WORKLOADS", "make_suite", "make_workload", "round_to_bf16",
    "bf16_bits", "bits_to_f32", "zipf_sample",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 arrays holding bf16-exact values.  Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 arrays that already hold bf16-exact values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array is not bf16-exact")
    return (u >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_sample(rng: np.random.Generator, vocab: int, s: float, size) -> np.ndarray:
    """Inverse-CDF draw from the finite law P(k) proportional to (k+1)^-s, k in [0, vocab)."""
    w = (np.arange(vocab, dtype=np.float64) + 1.0) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(size)
    k = np.searchsorted(cdf, u, side="right")
    return np.minimum(k, vocab - 1).astype(np.int32)


@dataclasses.dataclass
class Suite:
    """One batch of synthetic inputs for an M-exit suite (all host arrays)."""
    name: str
    dtype: str                 # "bf16" or "f32"
    widths: tuple              # D_1 < ... < D_M
    vocab: int
    batch: int
    seq: int
    ids: np.ndarray            # int32 [N]
    labels: np.ndarray         # int32 [N]
    h: List[np.ndarray]        # float32 [N, D_m] (bf16-exact when dtype == "bf16")
    emb: List[np.ndarray]      # float32 [V, D_m - D_{m-1}]
    w: List[np.ndarray]        # float32 [V, D_m]
    alpha: float = 0.3
    exits: Optional[tuple] = None   # subset of exits a workload runs (0-based), None = all

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq

    @property
    def n_exits(self) -> int:
        return len(self.widths)

    def device_array(self, x: np.ndarray) -> np.ndarray:
        """The array in the element encoding the device consumes."""
        return bf16_bits(x) if self.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return round_to_bf16(x) if dtype == "bf16" else x


def make_suite(widths: Sequence[int], vocab: int, batch: int, seq: int, *, dtype: str = "bf16",
               seed: int = 0, ids: str = "zipf", zipf_s: float = 1.1, h_std: float = 4.0,
               w_std: float = 0.02, alpha: float = 0.3, name: str = "custom",
               exits: Optional[tuple] = None) -> Suite:
    widths = tuple(int(d) for d in widths)
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    if ids == "zipf":
        seqs = zipf_sample(rng, vocab, zipf_s, (batch, seq + 1))
    elif ids == "uniform":
        seqs = rng.integers(0, vocab, size=(batch, seq + 1), dtype=np.int64).astype(np.int32)
    else:
        raise ValueError(ids)
    tok = np.ascontiguousarray(seqs[:, :seq].reshape(-1))
    lab = np.ascontiguousarray(seqs[:, 1:].reshape(-1))
    n = batch * seq
    h = [_normal(rng, (n, d), h_std, dtype) for d in widths]
    prev = [0] + list(widths[:-1])
    emb = [_normal(rng, (vocab, d - p), w_std, dtype) for d, p in zip(widths, prev)]
    w = [_normal(rng, (vocab, d), w_std, dtype) for d in widths]
    return Suite(name=name, dtype=dtype, widths=widths, vocab=vocab, batch=batch, seq=seq,
                 ids=tok, labels=lab, h=h, emb=emb, w=w, alpha=alpha, exits=exits)


# The five named workloads: (name, widths, V, batch, seq, dtype, ids, alpha, exits)
WORKLOADS = [
    ("tiny-3exit-f32", (64, 128, 256), 512, 2, 64, "f32", "uniform", 0.3, None),
    ("200M-proxy-3exit", (512, 768, 1024), 32768, 8, 2048, "bf16", "zipf", 0.3, None),
    ("500M-1.5B-3B-3exit", (1024, 2304, 4352), 32768, 8, 2048, "bf16", "zipf", 0.3, None),
    ("4exit", (512, 1024, 1536, 2048), 32768, 16, 2048, "bf16", "zipf", 0.3, None),
    ("spec-verify-102x7", (1024, 2304, 4352), 32768, 102, 7, "bf16", "zipf", 0.3, (0, 2)),
]


def make_workload(k: int, *, batch: Optional[int] = None, seed: Optional[int] = None) -> Suite:
    """Workload k (0..4) with seed 1000 + k; ``batch`` may shrink the batch for a
    quick run (the first rows of the full draw are NOT reproduced then)."""
    name, widths, vocab, b, seq, dtype, ids, alpha, exits = WORKLOADS[k]
    return make_suite(widths, vocab, batch or b, seq, dtype=dtype,
                      seed=(1000 + k) if seed is None else seed, ids=ids, alpha=alpha,
                      name=name, exits=exits)
