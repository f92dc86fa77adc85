"""Host model of the paged KV pool: slot mapping, write, gather, relayout.

TEST INFRASTRUCTURE ONLY (see the package header): the GPU path never
imports this module.

Everything here moves raw element bits (``uint16`` for bfloat16, ``float32``
for fp32) with plain per-token / per-head Python loops, so a result can be
checked by eye against the rules it follows:

* Slot mapping: token ``p`` of a request whose block table is ``bt`` lives
  at ``slot = bt[p // bs] * bs + p % bs``, i.e. physical block
  ``bt[p // bs]``, offset ``p % bs`` ([DISAGG] "实现", the ``admit`` step
  that builds slots before writing each layer).
* Head shards: with ``S`` shards of ``H/S`` heads, KV head ``h`` lives in
  shard ``h // (H/S)`` as local head ``h % (H/S)``.  The pages split the KV
  heads of a layer into 4 or 8 parts for TP 4 / TP 8 ([DISAGG] self-test
  answer 3 and "布局转换"); contiguous head ranges per shard are the
  reading taken here.  All shards of one instance share the request's
  block table (tensor-parallel ranks replicate block ids).
* Relayout: gather each (token, head) row through the source block table
  and shard split, and write it at the destination block table's position
  under the destination's split ([DISAGG] self-test answer 3, "实现" and
  "布局转换").  Slots past the request's ``n`` tokens are never touched.

Pool layout (the library's documented layout, one layer of one instance):
shard ``s`` holds

* ``k[s]``: ``[num_blocks, H/S, block_size, D]``  (token rows per head)
* ``v[s]``: ``[num_blocks, H/S, D, block_size]``  (V stored dim-major
  inside a block)

The pages view a layer's pool as ``[slot, kv_heads, head_dim]``; this model
stores the same logical content, and the tests compare logical
``(token, head, dim)`` values as well as raw pool bytes.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class PoolModel:
    """One layer of one instance's pool, as host numpy arrays."""

    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_shards: int
    head_dim: int
    elem: type = np.uint16          # np.uint16 = bfloat16 bits, np.float32 = fp32
    fill: int | float = 0
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)

    def __post_init__(self):
        if self.num_kv_heads % self.num_shards:
            raise ValueError("kv heads must split evenly over shards")
        hl = self.num_kv_heads // self.num_shards
        if not self.k:
            self.k = [np.full((self.num_blocks, hl, self.block_size, self.head_dim), self.fill, dtype=self.elem)
                      for _ in range(self.num_shards)]
            self.v = [np.full((self.num_blocks, hl, self.head_dim, self.block_size), self.fill, dtype=self.elem)
                      for _ in range(self.num_shards)]

    @property
    def heads_per_shard(self) -> int:
        return self.num_kv_heads // self.num_shards

    def where(self, slot: int, head: int):
        """(shard, block, offset, local head) holding ``head`` of ``slot``."""
        hl = self.heads_per_shard
        return head // hl, slot // self.block_size, slot % self.block_size, head % hl

    def copy(self) -> "PoolModel":
        return PoolModel(self.num_blocks, self.block_size, self.num_kv_heads, self.num_shards,
                         self.head_dim, self.elem, self.fill,
                         [a.copy() for a in self.k], [a.copy() for a in self.v])


def slots_for(block_table, block_size: int, positions) -> list[int]:
    """Slot of each absolute position under one request's block table."""
    return [int(block_table[p // block_size]) * block_size + p % block_size for p in positions]


def write(pool: PoolModel, k, v, slots) -> None:
    """Naive scatter of token rows: k, v are [n, H, D] in the pool's element type.

    Row ``i`` goes to ``slots[i]``; a negative slot means "skip this row".
    """
    k = np.asarray(k)
    v = np.asarray(v)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        for h in range(pool.num_kv_heads):
            s, blk, off, lh = pool.where(int(slot), h)
            pool.k[s][blk, lh, off, :] = k[i, h, :]
            pool.v[s][blk, lh, :, off] = v[i, h, :]


def read_row(pool: PoolModel, slot: int, head: int):
    """The (K row, V row) stored for ``head`` at ``slot``."""
    s, blk, off, lh = pool.where(slot, head)
    return pool.k[s][blk, lh, off, :].copy(), pool.v[s][blk, lh, :, off].copy()


def gather(pool: PoolModel, block_table, n: int):
    """Logical K/V of a request's first ``n`` tokens: two [n, H, D] arrays."""
    slots = slots_for(block_table, pool.block_size, range(n))
    k = np.empty((n, pool.num_kv_heads, pool.head_dim), dtype=pool.elem)
    v = np.empty_like(k)
    for i, slot in enumerate(slots):
        for h in range(pool.num_kv_heads):
            k[i, h, :], v[i, h, :] = read_row(pool, slot, h)
    return k, v


def relayout(src: PoolModel, src_bt, dst: PoolModel, dst_bt, n: int) -> int:
    """Naive per-(token, head) copy of one layer from ``src`` into ``dst``.

    Returns the payload bytes copied (K and V rows), for the closed-form
    byte check.
    """
    if (src.num_kv_heads, src.head_dim, src.elem) != (dst.num_kv_heads, dst.head_dim, dst.elem):
        raise ValueError("relayout keeps heads, head_dim and element type")
    src_slots = slots_for(src_bt, src.block_size, range(n))
    dst_slots = slots_for(dst_bt, dst.block_size, range(n))
    moved = 0
    for p in range(n):
        for h in range(src.num_kv_heads):
            krow, vrow = read_row(src, src_slots[p], h)
            s, blk, off, lh = dst.where(dst_slots[p], h)
            dst.k[s][blk, lh, off, :] = krow
            dst.v[s][blk, lh, :, off] = vrow
            moved += krow.nbytes + vrow.nbytes
    return moved


def allocated_untouched(pool: PoolModel, fill, used_slots) -> bool:
    """True when every (slot, head) outside ``used_slots`` still holds ``fill``."""
    used = np.zeros((pool.num_blocks, pool.block_size), dtype=bool)
    for slot in used_slots:
        used[int(slot) // pool.block_size, int(slot) % pool.block_size] = True
    fill_arr = np.array(fill, dtype=pool.elem)
    for s in range(pool.num_shards):
        k_rows = pool.k[s].transpose(0, 2, 1, 3)      # [blk, off, head, D]
        v_rows = pool.v[s].transpose(0, 3, 1, 2)      # [blk, off, head, D]
        if not (np.all(k_rows[~used] == fill_arr) and np.all(v_rows[~used] == fill_arr)):
            return False
    return True
