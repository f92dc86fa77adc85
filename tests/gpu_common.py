"""Shared helpers for the GPU parity tests.

Inputs come from ``decode_paged_kv_amd.inputs`` (seeded, host numpy).  The
GPU side fills its pools through the library (slot mapping + kv_write) and
runs the kernels through the C ABI; the oracle is fed the same logical
tensors and never sees a pool the GPU wrote.
"""

from __future__ import annotations

import numpy as np
import torch

from decode_paged_kv_amd import inputs, ops

BF16_TOL = {"max_abs": 2e-2, "rel_l2": 5e-3}
F32_TOL = {"max_abs": 1e-5, "rel_l2": 1e-5}
SENTINEL = {"bf16": 0x7FBF, "f32": 0x7FC0DEAD}   # NaN patterns: a stray read would poison the result


def tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def to_dev(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def i32(x, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(device)


def assert_close(got, ref, dtype, what=""):
    from oracle.attention import error_metrics
    m = error_metrics(got, ref)
    t = tol(dtype)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    assert m["max_abs"] <= t["max_abs"] and m["rel_l2"] <= t["rel_l2"], f"{what}: {m} vs {t}"
    return m


class Scenario:
    """Seeded logical K/V/Q for a set of requests and the GPU pool holding them."""

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, block_size, dtype, lengths, pool_blocks,
                 num_shards=1, scale=1.0, seed=0, config_id=0, layer=0, err_word=None, table_pad=0):
        self.hq, self.hkv, self.d, self.bs, self.dtype = num_q_heads, num_kv_heads, head_dim, block_size, dtype
        self.lengths = [int(x) for x in lengths]
        self.seed, self.cfg, self.layer = seed, config_id, layer
        g = lambda t, i=0: inputs.stream(seed, config_id, layer, t, i)  # noqa: E731
        self.k = [inputs.normal((n, num_kv_heads, head_dim), scale, dtype, g(inputs.T_K, r)) for r, n in enumerate(self.lengths)]
        self.v = [inputs.normal((n, num_kv_heads, head_dim), scale, dtype, g(inputs.T_V, r)) for r, n in enumerate(self.lengths)]
        self.tables, _ = inputs.assign_blocks(pool_blocks, self.lengths, block_size, g(inputs.T_PERM))
        if table_pad:
            self.tables = np.concatenate([self.tables, np.full((self.tables.shape[0], table_pad), -1, np.int32)], 1)
        self.pool = ops.PagedPool(pool_blocks, block_size, num_kv_heads, num_shards, head_dim, dtype,
                                  err_word=err_word).fill_bits(SENTINEL[dtype])
        self.bt_dev = i32(self.tables)

    def kf(self, r):
        return inputs.as_float(self.k[r], self.dtype)

    def vf(self, r):
        return inputs.as_float(self.v[r], self.dtype)

    def write_all(self, upto=None):
        """Write every request's first ``upto[r]`` tokens (default all) with one slot-mapping + kv_write."""
        upto = upto or self.lengths
        kk = np.concatenate([self.k[r][:n] for r, n in enumerate(upto)])
        vv = np.concatenate([self.v[r][:n] for r, n in enumerate(upto)])
        start = np.concatenate([[0], np.cumsum(upto)]).astype(np.int32)
        self.write_tokens(kk, vv, start, np.zeros(len(upto), np.int32))

    def write_tokens(self, kk, vv, start_loc, pos_start, tables=None):
        bt = self.bt_dev if tables is None else tables
        n = int(start_loc[-1])
        slots = ops.slot_mapping(bt, i32(start_loc), i32(pos_start), n, self.bs, self.pool.num_blocks,
                                 err_word=self.pool.err_word)
        ops.kv_write(self.pool, to_dev(kk, self.dtype), to_dev(vv, self.dtype), slots)
        return slots
