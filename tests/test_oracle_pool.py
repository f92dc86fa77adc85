"""Pins for the pool / relayout oracle.

* the slot rule on hand-computed positions ("PD 分离与 KV 传输", section
  "实现": slot = block id * block size + offset);
* the documented pool layout on a hand-placed element;
* write-then-gather returns the logical rows; relayout keeps the logical
  rows bit for bit and never touches slots past the request;
* a 16 -> 32 -> 16 round trip through the inverse tables is the identity;
* bytes moved equal the closed form layers x 2 x heads x dim x bytes x tokens.
"""

import numpy as np
import pytest

from conftest import kv_fields, read_golden
from decode_paged_kv_amd import inputs
from oracle import accounting, fp8, pool


def test_slot_rule_hand_values():
    bt = [5, 2, 9]
    assert pool.slots_for(bt, 16, [0, 15, 16, 17, 40]) == [80, 95, 32, 33, 152]
    assert pool.slots_for([3, 0], 32, [0, 31, 32, 63]) == [96, 127, 0, 31]


def test_layout_of_one_written_row():
    pm = pool.PoolModel(num_blocks=4, block_size=16, num_kv_heads=4, num_shards=2, head_dim=8, elem=np.float32)
    k = np.arange(2 * 4 * 8, dtype=np.float32).reshape(2, 4, 8)
    v = -k
    pool.write(pm, k, v, [17, 3])          # token 0 -> slot 17 = block 1, offset 1
    # head 3 lives in shard 1 as local head 1
    assert np.array_equal(pm.k[1][1, 1, 1, :], k[0, 3])
    assert np.array_equal(pm.v[1][1, 1, :, 1], v[0, 3])
    # head 0 of token 1: shard 0, local 0, block 0, offset 3
    assert np.array_equal(pm.k[0][0, 0, 3, :], k[1, 0])
    assert np.array_equal(pm.v[0][0, 0, :, 3], v[1, 0])
    # negative slots are skipped
    pm2 = pool.PoolModel(4, 16, 4, 2, 8, np.float32)
    pool.write(pm2, k, v, [-1, -5])
    assert all(not a.any() for a in pm2.k + pm2.v)


def _filled_pool(n, bs, shards, blocks, seed, heads=8, d=16, fill=0xDEAD):
    g = inputs.stream(seed, 99, 0, inputs.T_PERM)
    bt, _ = inputs.assign_blocks(blocks, [n], bs, g)
    pm = pool.PoolModel(blocks, bs, heads, shards, d, np.uint16, fill)
    k = inputs.normal((n, heads, d), 0.5, "bf16", inputs.stream(seed, 99, 0, inputs.T_K))
    v = inputs.normal((n, heads, d), 0.5, "bf16", inputs.stream(seed, 99, 0, inputs.T_V))
    pool.write(pm, k, v, pool.slots_for(bt[0], bs, range(n)))
    return pm, bt[0], k, v


def test_write_then_gather_round_trip():
    pm, bt, k, v = _filled_pool(100, 16, 4, 16, seed=1)
    gk, gv = pool.gather(pm, bt, 100)
    assert np.array_equal(gk, k) and np.array_equal(gv, v)
    assert pool.allocated_untouched(pm, 0xDEAD, pool.slots_for(bt, 16, range(100)))


def test_relayout_bit_exact_and_untouched_tail():
    n = 150
    src, src_bt, k, v = _filled_pool(n, 16, 4, 16, seed=2)
    dst = pool.PoolModel(8, 32, 8, 8, 16, np.uint16, fill=0xBEEF)
    g = inputs.stream(2, 99, 0, inputs.T_DST_PERM)
    dst_bt, _ = inputs.assign_blocks(8, [n + 1], 32, g)   # room for the next token, as decode reserves
    moved = pool.relayout(src, src_bt, dst, dst_bt[0], n)
    gk, gv = pool.gather(dst, dst_bt[0], n)
    assert np.array_equal(gk, k) and np.array_equal(gv, v)
    assert pool.allocated_untouched(dst, 0xBEEF, pool.slots_for(dst_bt[0], 32, range(n)))
    assert moved == accounting.relayout_payload_bytes(n, 8, 16, 2)


def test_relayout_round_trip_is_identity():
    n = 96
    src, src_bt, _, _ = _filled_pool(n, 16, 4, 8, seed=3)
    mid = pool.PoolModel(4, 32, 8, 8, 16, np.uint16, fill=0)
    mid_bt = np.array([2, 0, 3], dtype=np.int32)
    pool.relayout(src, src_bt, mid, mid_bt, n)
    back = pool.PoolModel(8, 16, 8, 4, 16, np.uint16, fill=0xDEAD)
    pool.relayout(mid, mid_bt, back, src_bt, n)
    for a, b in zip(src.k + src.v, back.k + back.v):
        assert np.array_equal(a, b)


def test_relayout_bytes_match_pages_closed_form():
    rows = {r[0] + ":" + r[1]: kv_fields(r[2:]) for r in read_golden("kv_bytes.txt") if len(r) > 1}
    t = rows["transfer:llama3-70b"]
    per_token = accounting.kv_bytes_per_token(80, 8, 128, 2)
    assert per_token == int(t["per_token"])
    total = accounting.kv_bytes(int(t["tokens"]), 80, 8, 128, 2)
    assert total == 1_342_177_280
    assert round(total / 1e9, 2) == float(t["gb"])
    assert round(total / float(t["link"]) * 1e3) == int(t["ms"])
    # the relayout oracle moves exactly one layer's share per call
    assert accounting.relayout_payload_bytes(4096, 8, 128, 2) * 80 == total


# --- relayout with a change of layout / element type ([DISAGG] "布局转换") ---

def _logical_rows(dst, slots):
    """Per layout, the destination's K and V as [n, heads, dim] through a plain reshape of the shard tensors
    (heads of shard s are the s-th run of H/S heads); independent of DestModel.put's indexing."""
    if dst.layout == pool.LAYOUT_KV_FUSED:
        kk = np.concatenate([t[:, 0] for t in dst.k], axis=2)      # [blocks, bs, H, D]
        vv = np.concatenate([t[:, 1] for t in dst.k], axis=2)
    else:
        kk = np.concatenate(dst.k, axis=2)
        vv = np.concatenate(dst.v, axis=2)
    flat = lambda t: t.reshape(dst.num_blocks * dst.block_size, dst.num_kv_heads, dst.head_dim)  # noqa: E731
    return flat(kk)[slots], flat(vv)[slots]


def test_convert_hand_placed_elements():
    src = pool.PoolModel(2, 16, 4, 1, 8, np.float32)
    k = np.arange(4 * 8, dtype=np.float32).reshape(1, 4, 8) + 1
    pool.write(src, k, -k, [5])                          # position 5 of a request whose table is [0]
    for layout in (pool.LAYOUT_POOL, pool.LAYOUT_TOKEN_MAJOR, pool.LAYOUT_KV_FUSED):
        dst = pool.DestModel(4, 32, 4, 2, 8, np.float32, layout)
        pool.relayout_convert(src, [0], dst, [3], 6)     # position 5 -> block 3, offset 5; head 3 = shard 1, local 1
        if layout == pool.LAYOUT_POOL:
            got_k, got_v = dst.k[1][3, 1, 5, :], dst.v[1][3, 1, :, 5]
        elif layout == pool.LAYOUT_TOKEN_MAJOR:
            got_k, got_v = dst.k[1][3, 5, 1, :], dst.v[1][3, 5, 1, :]
        else:
            got_k, got_v = dst.k[1][3, 0, 5, 1, :], dst.k[1][3, 1, 5, 1, :]
        assert np.array_equal(got_k, k[0, 3]) and np.array_equal(got_v, -k[0, 3])
        assert sum(np.count_nonzero(t) for t in dst.k + dst.v) == 2 * 4 * 8


def test_convert_pool_layout_same_dtype_equals_relayout():
    n = 150
    src, src_bt, _, _ = _filled_pool(n, 16, 4, 16, seed=5)
    g = inputs.stream(5, 99, 0, inputs.T_DST_PERM)
    dst_bt, _ = inputs.assign_blocks(8, [n + 1], 32, g)
    ref = pool.PoolModel(8, 32, 8, 8, 16, np.uint16, fill=0xBEEF)
    pool.relayout(src, src_bt, ref, dst_bt[0], n)
    got = pool.DestModel(8, 32, 8, 8, 16, np.uint16, pool.LAYOUT_POOL, fill=0xBEEF)
    assert pool.relayout_convert(src, src_bt, got, dst_bt[0], n) == accounting.relayout_payload_bytes(n, 8, 16, 2)
    for a, b in zip(ref.k + ref.v, got.k + got.v):
        assert np.array_equal(a, b)


def test_convert_token_major_and_fused_are_the_slot_view():
    n = 137
    src, src_bt, k, v = _filled_pool(n, 16, 4, 16, seed=6)
    g = inputs.stream(6, 99, 0, inputs.T_DST_PERM)
    dst_bt, _ = inputs.assign_blocks(6, [n], 32, g)
    slots = np.array(pool.slots_for(dst_bt[0], 32, range(n)))
    for layout in (pool.LAYOUT_TOKEN_MAJOR, pool.LAYOUT_KV_FUSED):
        dst = pool.DestModel(6, 32, 8, 2, 16, np.uint16, layout, fill=0xBEEF)
        pool.relayout_convert(src, src_bt, dst, dst_bt[0], n)
        gk, gv = _logical_rows(dst, slots)
        assert np.array_equal(gk, k) and np.array_equal(gv, v)
        # every other slot keeps the fill
        rest = np.setdiff1d(np.arange(6 * 32), slots)
        rk, rv = _logical_rows(dst, rest)
        assert np.all(rk == 0xBEEF) and np.all(rv == 0xBEEF)


def test_convert_to_fp8_matches_torch_cast_and_scale():
    import torch
    n, scale = 70, 0.02
    src, src_bt, k, v = _filled_pool(n, 16, 2, 8, seed=7)
    dst_bt = np.array([1, 0, 2], np.int32)
    dst = pool.DestModel(3, 32, 8, 4, 16, np.uint8, pool.LAYOUT_TOKEN_MAJOR, fill=0x7F, scale=scale)
    assert pool.relayout_convert(src, src_bt, dst, dst_bt, n) == n * 8 * 16 * 2
    gk, gv = _logical_rows(dst, np.array(pool.slots_for(dst_bt, 32, range(n))))
    inv = np.float32(1.0) / np.float32(scale)
    for got, x in ((gk, k), (gv, v)):
        xf = (x.astype(np.uint32) << 16).view(np.float32)
        # torch's E4M3 cast rounds to nearest even but does not saturate: clamp first
        ref = torch.from_numpy(np.clip(xf * inv, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, ref)
        # decoded x scale is within half a code step of x (3 mantissa bits: relative 2^-4, or 2^-10 absolute
        # below the smallest normal 2^-6, times the scale)
        dec = fp8.dequantize(got, scale)
        step = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * scale)
        assert np.all(np.abs(dec - xf) <= step * (1 + 1e-6))


@pytest.mark.parametrize("where", ["k_row", "v_row", "k_last_dim", "v_other_shard", "unused_block"])
def test_allocated_untouched_catches_a_stray_write(where):
    # negative pin: one element outside the written slots changed (in K or V, any shard, any block) must make
    # allocated_untouched say so; a version that always answers True fails here
    pm, bt, _, _ = _filled_pool(100, 16, 4, 16, seed=4)
    used = pool.slots_for(bt, 16, range(100))
    assert pool.allocated_untouched(pm, 0xDEAD, used)
    free_slots = sorted(set(range(pm.num_blocks * 16)) - set(int(s) for s in used))
    slot = free_slots[len(free_slots) // 2]
    blk, off = slot // 16, slot % 16
    if where == "k_row":
        pm.k[0][blk, 0, off, 0] = 0x1234            # K: [block][head][offset][dim]
    elif where == "v_row":
        pm.v[0][blk, 1, 3, off] = 0x1234            # V: [block][head][dim][offset]
    elif where == "k_last_dim":
        pm.k[pm.num_shards - 1][blk, -1, off, -1] = 0x1234
    elif where == "v_other_shard":
        pm.v[pm.num_shards - 1][blk, 0, 0, off] = 0x1234
    else:
        unused = [b for b in range(pm.num_blocks) if b not in set(int(x) for x in bt[:7])]
        pm.k[0][unused[0], 0, 0, 0] = 0x1234
    assert not pool.allocated_untouched(pm, 0xDEAD, used)


def test_allocated_untouched_ignores_the_written_slots():
    # the complement: changing a written slot is not a stray write
    pm, bt, _, _ = _filled_pool(100, 16, 4, 16, seed=4)
    used = pool.slots_for(bt, 16, range(100))
    s = int(used[37])
    pm.k[1][s // 16, 0, s % 16, 5] ^= 0xFFFF
    assert pool.allocated_untouched(pm, 0xDEAD, used)
