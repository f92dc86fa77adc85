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

from . import fp8


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


# ---------------------------------------------------------------------------
# Relayout with a change of element type and/or physical layout
# ---------------------------------------------------------------------------
#
# [DISAGG] "布局转换": besides the block size and the head split, the
# attention backend's layout (K and V fused or separate, the order of the
# head and token dimensions) and the KV element type (BF16 on one side, FP8
# on the other) may differ between the two instances.  Three destination
# layouts are modelled (per shard s, block b, offset o, local head lh, dim d):
#
# * POOL:         k[s][b, lh, o, d],  v[s][b, lh, d, o]   (the layout above)
# * TOKEN_MAJOR:  k[s][b, o, lh, d],  v[s][b, o, lh, d]   (slot-major rows:
#   a shard's tensor viewed as [slot, heads, dim] is the pages' pool view)
# * KV_FUSED:     kv[s][b, 0, o, lh, d] for K and kv[s][b, 1, o, lh, d] for V
#
# The FP8 element type is the E4M3 encoding of ``oracle.fp8`` (one scale per
# tensor); a BF16 source value x is stored as encode(fp32(x) * fp32(1/scale)).

LAYOUT_POOL, LAYOUT_TOKEN_MAJOR, LAYOUT_KV_FUSED = 0, 1, 2


@dataclass
class DestModel:
    """One layer in a destination layout; ``elem`` np.uint8 means FP8 E4M3 bits."""

    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_shards: int
    head_dim: int
    elem: type
    layout: int
    fill: int | float = 0
    scale: float = 1.0
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)

    def __post_init__(self):
        hl = self.num_kv_heads // self.num_shards
        nb, bs, d = self.num_blocks, self.block_size, self.head_dim
        if self.layout == LAYOUT_POOL:
            ks, vs = (nb, hl, bs, d), (nb, hl, d, bs)
        elif self.layout == LAYOUT_TOKEN_MAJOR:
            ks = vs = (nb, bs, hl, d)
        else:
            ks, vs = (nb, 2, bs, hl, d), None
        self.k = [np.full(ks, self.fill, dtype=self.elem) for _ in range(self.num_shards)]
        self.v = [np.full(vs, self.fill, dtype=self.elem) for _ in range(self.num_shards)] if vs else []

    def put(self, slot: int, head: int, krow, vrow) -> None:
        hl = self.num_kv_heads // self.num_shards
        s, b, o, lh = head // hl, slot // self.block_size, slot % self.block_size, head % hl
        if self.layout == LAYOUT_POOL:
            self.k[s][b, lh, o, :] = krow
            self.v[s][b, lh, :, o] = vrow
        elif self.layout == LAYOUT_TOKEN_MAJOR:
            self.k[s][b, o, lh, :] = krow
            self.v[s][b, o, lh, :] = vrow
        else:
            self.k[s][b, 0, o, lh, :] = krow
            self.k[s][b, 1, o, lh, :] = vrow


def convert_row(row, src_elem, dst_elem, scale: float):
    """One row in the destination element type: unchanged, or BF16 bits -> E4M3 bits."""
    if dst_elem == src_elem:
        return row
    if src_elem == np.uint16 and dst_elem == np.uint8:
        return fp8.quantize_bf16(row, scale)
    raise ValueError("only BF16 -> FP8 changes the element type")


def relayout_convert(src: PoolModel, src_bt, dst: DestModel, dst_bt, n: int) -> int:
    """Naive per-(token, head) copy of one layer into ``dst``'s layout and element type.

    Returns the bytes written into the destination (K and V rows).
    """
    if (src.num_kv_heads, src.head_dim) != (dst.num_kv_heads, dst.head_dim):
        raise ValueError("relayout keeps heads and head_dim")
    src_slots = slots_for(src_bt, src.block_size, range(n))
    dst_slots = slots_for(dst_bt, dst.block_size, range(n))
    written = 0
    for p in range(n):
        for h in range(src.num_kv_heads):
            krow, vrow = read_row(src, src_slots[p], h)
            krow = convert_row(krow, src.elem, dst.elem, dst.scale)
            vrow = convert_row(vrow, src.elem, dst.elem, dst.scale)
            dst.put(dst_slots[p], h, krow, vrow)
            written += krow.nbytes + vrow.nbytes
    return written
