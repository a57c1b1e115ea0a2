"""Seeded synthetic inputs for the packed low-bit BitLinear workloads.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no packing, decoding, quantization or products), so the
tests can feed the same inputs to the HIP path and to the CPU oracle.

Workload shapes and value distributions (the pages print no data, so these
stand in for real checkpoints):

* ternary weights i.i.d. with P(-1) = P(+1) = 0.3, P(0) = 0.4;
* i2_s per-tensor fp32 scales ~ U(0.01, 0.1) (0.0625 for the 256x512 case);
* TQ2_0 per-block fp16 scales ~ U(0.005, 0.05), rounded to fp16 by numpy;
* binary (W1) weights derived from dense fp32 ~ N(0, 0.02), generated in
  row chunks so the 248,320-row LM head never has to exist densely;
* activations fp32 ~ N(0, 1); bf16 activations are those values rounded to
  bf16 (nearest, ties to even) when the input is produced.

Every generator takes an explicit seed; chunked generators take the chunk
index as a second seed word, so any chunk can be regenerated alone.
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 4096


def rng(seed, *words) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), *[int(w) for w in words]]))


def ternary(seed, N, K, p0=0.4, *, chunk=None) -> np.ndarray:
    """int8 [N, K] in {-1, 0, +1}, P(0) = p0, P(-1) = P(+1) = (1 - p0)/2."""
    g = rng(seed) if chunk is None else rng(seed, chunk)
    pm = (1.0 - p0) / 2.0
    return g.choice(np.array([-1, 0, 1], np.int8), size=(N, K), p=[pm, p0, pm])


def uniform_f32(seed, n, lo, hi) -> np.ndarray:
    return rng(seed).uniform(lo, hi, size=n).astype(np.float32)


def uniform_f16_bits(seed, n, lo, hi) -> np.ndarray:
    """fp16 bit patterns of U(lo, hi) draws (rounded by numpy's float16 cast)."""
    return rng(seed).uniform(lo, hi, size=n).astype(np.float16).view(np.uint16)


def normal_f32(seed, M, K, sigma=1.0) -> np.ndarray:
    return (rng(seed).standard_normal(size=(M, K)) * sigma).astype(np.float32)


def normal_bf16_bits(seed, M, K) -> np.ndarray:
    """bf16 bit patterns of N(0,1) draws, rounded to nearest-even bf16."""
    x = normal_f32(seed, M, K)
    u = x.view(np.uint32).astype(np.uint64)
    # round-to-nearest-even on the low 16 bits (no NaNs are drawn)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def dense_chunk(seed, K, chunk, rows=CHUNK_ROWS, sigma=0.02) -> np.ndarray:
    """Dense fp32 ~ N(0, sigma) rows [chunk*CHUNK_ROWS, +rows) of a K-wide matrix."""
    return (rng(seed, chunk).standard_normal(size=(rows, K)) * sigma).astype(np.float32)


def dense_rows(seed, N, K, row_ids, sigma=0.02) -> np.ndarray:
    """The given rows of the chunked dense matrix (regenerating their chunks)."""
    row_ids = np.asarray(row_ids, np.int64)
    out = np.empty((row_ids.size, K), np.float32)
    for c in np.unique(row_ids // CHUNK_ROWS):
        rows = min(CHUNK_ROWS, N - c * CHUNK_ROWS)
        d = dense_chunk(seed, K, int(c), rows, sigma)
        sel = np.nonzero(row_ids // CHUNK_ROWS == c)[0]
        out[sel] = d[row_ids[sel] - c * CHUNK_ROWS]
    return out


def sample_rows(seed, N, n) -> np.ndarray:
    """n distinct sorted row indices, always including the first and last row."""
    if n >= N:
        return np.arange(N, dtype=np.int64)
    pick = rng(seed, 7).choice(N, size=n, replace=False)
    pick = np.unique(np.concatenate([pick, [0, N - 1]]))
    return pick.astype(np.int64)
