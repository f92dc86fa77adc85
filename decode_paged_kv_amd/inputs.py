"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module draws numbers and builds block tables; it holds none of the
attention or relayout arithmetic.  Every tensor comes from its own stream
``np.random.default_rng([seed, config_id, layer, tensor_id, index])`` so any
layer or request can be regenerated alone.

* Floating-point inputs are standard normals drawn in float32, multiplied by
  the workload's scale, and (for bfloat16 workloads) rounded to bfloat16
  with round-to-nearest-even.  bfloat16 values travel as ``uint16`` bit
  patterns.
* Physical blocks come from a seeded random permutation of the pool; each
  request takes the next ``ceil(tokens / block_size)`` entries in order, as a
  block allocator handing out blocks from a shuffled free list would.
"""

from __future__ import annotations

import numpy as np

# tensor ids of the per-(config, layer) streams
T_Q, T_K, T_V, T_PERM, T_CTX = 1, 2, 3, 4, 5
T_Q_DECODE, T_K_DECODE, T_V_DECODE, T_DST_PERM = 6, 7, 8, 9


def stream(seed: int, config_id: int, layer: int, tensor_id: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, config_id, layer, tensor_id, index])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite here, so no NaN handling is needed.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, scale: float, dtype: str, gen: np.random.Generator) -> np.ndarray:
    """N(0,1)*scale in float32, then bf16 bits (dtype 'bf16') or float32 ('f32')."""
    x = gen.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Element values as float64 (exact for both element types)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def blocks_needed(tokens: int, block_size: int) -> int:
    return -(-tokens // block_size)


def assign_blocks(pool_blocks: int, token_counts, block_size: int, gen: np.random.Generator):
    """Block tables for requests holding ``token_counts`` tokens each.

    Returns (tables [R, max_blocks] int32 padded with -1, per-request block
    counts).  Blocks are consecutive entries of a permutation of the pool.
    """
    perm = gen.permutation(pool_blocks).astype(np.int32)
    counts = [blocks_needed(int(t), block_size) for t in token_counts]
    if sum(counts) > pool_blocks:
        raise ValueError(f"pool of {pool_blocks} blocks is too small for {sum(counts)}")
    width = max(counts) if counts else 0
    tables = np.full((len(counts), max(width, 1)), -1, dtype=np.int32)
    at = 0
    for r, c in enumerate(counts):
        tables[r, :c] = perm[at:at + c]
        at += c
    return tables, counts
