"""GPU parity of slot mapping, kv_write and kv_relayout: bit-exact against the oracle.

The oracle's pool model (``oracle.pool``) is filled by its own naive loops
from the same logical K/V; the GPU pools are copied back and compared byte
for byte, including every slot that must stay untouched (sentinel bits).
"""

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops, workloads
from gpu_common import SENTINEL, Scenario, from_dev, i32, to_dev
from oracle import accounting, pool as opool

pytestmark = pytest.mark.gpu


def _elem(dtype):
    return np.uint16 if dtype == "bf16" else np.float32


def _oracle_pool_from(sc: Scenario, num_shards=None, lengths=None):
    pm = opool.PoolModel(sc.pool.num_blocks, sc.bs, sc.hkv, num_shards or sc.pool.num_shards, sc.d,
                         _elem(sc.dtype), fill=_fill_value(sc.dtype))
    for r, n in enumerate(lengths or sc.lengths):
        opool.write(pm, sc.k[r][:n], sc.v[r][:n], opool.slots_for(sc.tables[r], sc.bs, range(n)))
    return pm


def _fill_value(dtype):
    return SENTINEL[dtype] if dtype == "bf16" else np.array([SENTINEL[dtype]], np.uint32).view(np.float32)[0]


def _assert_pool_equal(gpu_pool: ops.PagedPool, pm: opool.PoolModel):
    for s in range(pm.num_shards):
        gk, gv = from_dev(gpu_pool.k[s], gpu_pool.dtype), from_dev(gpu_pool.v[s], gpu_pool.dtype)
        # compare raw bits (NaN sentinels compare equal this way)
        assert np.array_equal(gk.view(np.uint8), pm.k[s].view(np.uint8)), f"K shard {s}"
        assert np.array_equal(gv.view(np.uint8), pm.v[s].view(np.uint8)), f"V shard {s}"


def test_slot_mapping_matches_oracle():
    sc = Scenario(num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16, dtype="f32",
                  lengths=[37, 64, 100, 128, 1], pool_blocks=64, seed=3)
    start = np.concatenate([[0], np.cumsum(sc.lengths)]).astype(np.int32)
    # decode-style: one token per request at position L-1; prefill-style: all tokens
    pos = np.array(sc.lengths, np.int32) - 1
    slots = ops.slot_mapping(sc.bt_dev, i32(np.arange(len(sc.lengths) + 1)), i32(pos), len(sc.lengths), 16, 64)
    ref = [opool.slots_for(sc.tables[r], 16, [int(pos[r])])[0] for r in range(len(sc.lengths))]
    assert slots.cpu().tolist() == ref
    slots = ops.slot_mapping(sc.bt_dev, i32(start), i32(np.zeros(5)), int(start[-1]), 16, 64)
    ref = sum((opool.slots_for(sc.tables[r], 16, range(n)) for r, n in enumerate(sc.lengths)), [])
    assert slots.cpu().tolist() == ref


@pytest.mark.parametrize("dtype,bs,shards,hkv,d", [("f32", 16, 1, 2, 64), ("bf16", 16, 4, 8, 128),
                                                  ("bf16", 32, 8, 8, 128), ("bf16", 64, 2, 4, 64),
                                                  ("f32", 128, 2, 2, 128)])
def test_kv_write_bit_exact(dtype, bs, shards, hkv, d):
    sc = Scenario(num_q_heads=hkv, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                  lengths=[37, 130, 5], pool_blocks=24, num_shards=shards, seed=11)
    sc.write_all()
    torch.cuda.synchronize()
    _assert_pool_equal(sc.pool, _oracle_pool_from(sc))


def test_kv_write_skips_negative_slots():
    sc = Scenario(num_q_heads=2, num_kv_heads=2, head_dim=64, block_size=16, dtype="bf16", lengths=[20],
                  pool_blocks=4, seed=12)
    slots = np.array(opool.slots_for(sc.tables[0], 16, range(20)), np.int32)
    slots[::3] = -1
    ops.kv_write(sc.pool, to_dev(sc.k[0], "bf16"), to_dev(sc.v[0], "bf16"), i32(slots))
    torch.cuda.synchronize()
    pm = opool.PoolModel(4, 16, 2, 1, 64, np.uint16, fill=SENTINEL["bf16"])
    opool.write(pm, sc.k[0], sc.v[0], slots.tolist())
    _assert_pool_equal(sc.pool, pm)


def _relayout_case(dtype, n, src_bs, src_shards, src_blocks, dst_bs, dst_shards, dst_blocks, hkv, d, seed,
                   layers=1):
    out = []
    for layer in range(layers):
        sc = Scenario(num_q_heads=hkv, num_kv_heads=hkv, head_dim=d, block_size=src_bs, dtype=dtype, lengths=[n],
                      pool_blocks=src_blocks, num_shards=src_shards, seed=seed, layer=layer)
        sc.write_all()
        g = inputs.stream(seed, 0, layer, inputs.T_DST_PERM)
        dst_bt, _ = inputs.assign_blocks(dst_blocks, [n], dst_bs, g)
        dst = ops.PagedPool(dst_blocks, dst_bs, hkv, dst_shards, d, dtype).fill_bits(SENTINEL[dtype])
        out.append((sc, dst, dst_bt))
    for sc, dst, dst_bt in out:            # back to back, as layer-wise submission does
        ops.kv_relayout(sc.pool, sc.bt_dev[0], dst, i32(dst_bt[0]), n)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,n,sbs,ssh,sblk,dbs,dsh,dblk,hkv,d", [
    ("f32", 256, 16, 1, 64, 32, 2, 32, 2, 64),          # the tiny check: 1 shard x 2 heads -> 2 x 1, bs 16 -> 32
    ("bf16", 4096, 16, 4, 256, 32, 8, 128, 8, 128),     # the 70B shape, one layer at full size
    ("bf16", 1000, 32, 8, 40, 16, 4, 70, 8, 128),       # the inverse direction, ragged tail
    ("bf16", 77, 16, 2, 8, 64, 1, 4, 4, 64),
    ("f32", 300, 128, 1, 4, 16, 2, 30, 2, 128),
    ("bf16", 333, 16, 4, 24, 64, 16, 8, 16, 64),        # the most shards (16 x 1 head), block size 64
])
def test_relayout_bit_exact(dtype, n, sbs, ssh, sblk, dbs, dsh, dblk, hkv, d):
    (sc, dst, dst_bt), = _relayout_case(dtype, n, sbs, ssh, sblk, dbs, dsh, dblk, hkv, d, seed=21)
    pm_src = _oracle_pool_from(sc)
    pm_dst = opool.PoolModel(dblk, dbs, hkv, dsh, d, _elem(dtype), fill=_fill_value(dtype))
    moved = opool.relayout(pm_src, sc.tables[0], pm_dst, dst_bt[0], n)
    assert moved == accounting.relayout_payload_bytes(n, hkv, d, 2 if dtype == "bf16" else 4)
    _assert_pool_equal(dst, pm_dst)
    # logical content equals the request's K/V
    gk, gv = opool.gather(pm_dst, dst_bt[0], n)
    assert np.array_equal(gk, sc.k[0]) and np.array_equal(gv, sc.v[0])


def test_relayout_70b_layers_back_to_back():
    w = workloads.RELAYOUT_70B
    layers = 6
    cases = _relayout_case("bf16", w.prompt_len, w.block_size, w.src_shards, w.pool_blocks, w.dst_block_size,
                           w.dst_shards, w.dst_pool_blocks, w.num_kv_heads, w.head_dim, seed=w.seed, layers=layers)
    for sc, dst, dst_bt in cases:
        # logical check through the oracle's gather on a host copy of the GPU pool
        pm = opool.PoolModel(w.dst_pool_blocks, w.dst_block_size, 8, 8, 128, np.uint16)
        pm.k = [from_dev(t, "bf16") for t in dst.k]
        pm.v = [from_dev(t, "bf16") for t in dst.v]
        gk, gv = opool.gather(pm, dst_bt[0], w.prompt_len)
        assert np.array_equal(gk, sc.k[0]) and np.array_equal(gv, sc.v[0])


# --- relayout with a change of layout / element type ([DISAGG] "布局转换") ---

_DEST_ELEM = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}
_DEST_FILL = {"bf16": SENTINEL["bf16"], "f32": _fill_value("f32"), "fp8": 0x7F}
_LAYOUT = {"pool": opool.LAYOUT_POOL, "token_major": opool.LAYOUT_TOKEN_MAJOR, "kv_fused": opool.LAYOUT_KV_FUSED}


def _convert_case(dtype, ddtype, layout, n, sbs, ssh, sblk, dbs, dsh, dblk, hkv, d, seed, scale=1.0, plant=None):
    sc = Scenario(num_q_heads=hkv, num_kv_heads=hkv, head_dim=d, block_size=sbs, dtype=dtype, lengths=[n],
                  pool_blocks=sblk, num_shards=ssh, seed=seed)
    if plant is not None:
        plant(sc)
    sc.write_all()
    g = inputs.stream(seed, 0, 0, inputs.T_DST_PERM)
    dst_bt, _ = inputs.assign_blocks(dblk, [n], dbs, g)
    dst = ops.ConvertedPool(dblk, dbs, hkv, dsh, d, ddtype, layout, scale)
    fill = {"bf16": SENTINEL["bf16"], "f32": SENTINEL["f32"], "fp8": 0x7F}[ddtype]
    dst.fill_bits(fill)
    print(f"kv_relayout_convert {dtype}->{ddtype} {layout} n={n} bs {sbs}->{dbs} shards {ssh}->{dsh}", flush=True)
    ops.kv_relayout_convert(sc.pool, sc.bt_dev[0], dst, i32(dst_bt[0]), n)
    torch.cuda.synchronize()
    pm_src = _oracle_pool_from(sc)
    ref = opool.DestModel(dblk, dbs, hkv, dsh, d, _DEST_ELEM[ddtype], _LAYOUT[layout], fill=_DEST_FILL[ddtype],
                          scale=scale)
    opool.relayout_convert(pm_src, sc.tables[0], ref, dst_bt[0], n)
    got = [t.cpu().numpy() if ddtype == "fp8" else from_dev(t, ddtype) for t in dst.k + dst.v]
    return sc, dst, dst_bt, got, ref.k + ref.v


@pytest.mark.parametrize("dtype,ddtype,layout,n,sbs,ssh,sblk,dbs,dsh,dblk,hkv,d,scale", [
    # the 70B layer at full size: bs16 / 4 shards -> bs32 / 8 shards, into FP8 slot-major rows
    ("bf16", "fp8", "token_major", 4096, 16, 4, 256, 32, 8, 128, 8, 128, 0.02),
    ("bf16", "fp8", "pool", 1003, 32, 8, 40, 16, 4, 70, 8, 128, 0.05),        # ragged tail: element copies of V
    ("bf16", "fp8", "kv_fused", 517, 16, 2, 40, 128, 1, 8, 4, 64, 0.01),      # 8 source blocks per destination block
    ("bf16", "bf16", "kv_fused", 77, 16, 2, 8, 64, 1, 4, 4, 64, 1.0),
    ("bf16", "bf16", "token_major", 333, 128, 1, 4, 16, 2, 30, 2, 128, 1.0),
    ("bf16", "bf16", "pool", 250, 16, 1, 20, 128, 2, 4, 2, 64, 1.0),
    ("f32", "f32", "token_major", 300, 128, 1, 4, 16, 2, 30, 2, 128, 1.0),
    ("f32", "f32", "pool", 95, 16, 2, 8, 32, 1, 4, 2, 64, 1.0),
    ("f32", "f32", "kv_fused", 130, 32, 1, 8, 128, 2, 3, 2, 64, 1.0),
    ("bf16", "fp8", "token_major", 700, 128, 2, 8, 16, 16, 50, 16, 64, 0.125),   # 16 shards, bs 128 -> 16
])
def test_relayout_convert_bit_exact(dtype, ddtype, layout, n, sbs, ssh, sblk, dbs, dsh, dblk, hkv, d, scale):
    sc, dst, dst_bt, got, ref = _convert_case(dtype, ddtype, layout, n, sbs, ssh, sblk, dbs, dsh, dblk, hkv, d,
                                              seed=41, scale=scale)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"destination tensor {i}"
    if ddtype == dtype and layout == "pool":
        # the same bytes as kv_relayout into a pool of that shape
        same = ops.PagedPool(dblk, dbs, hkv, dsh, d, dtype).fill_bits(SENTINEL[dtype])
        ops.kv_relayout(sc.pool, sc.bt_dev[0], same, i32(dst_bt[0]), n)
        torch.cuda.synchronize()
        for a, b in zip(dst.k + dst.v, same.k + same.v):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_relayout_convert_fp8_special_values():
    """Overflow clamps to +-448, NaN stays NaN, tiny values become subnormal codes or zero."""
    special = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x4400, 0xC400, 0x43E0, 0x3A80, 0x3A00, 0x0001, 0x8000,
                        0x4380], np.uint16)   # NaN, -NaN, +-inf, +-512, 448, 2^-10 x 1.0, 2^-11, tiny, -0, 256

    def plant(sc):
        flat_k, flat_v = sc.k[0].reshape(-1), sc.v[0].reshape(-1)
        idx = np.arange(special.size) * 97
        flat_k[idx] = special
        flat_v[idx + 5] = special

    sc, dst, dst_bt, got, ref = _convert_case("bf16", "fp8", "token_major", 300, 16, 2, 24, 32, 2, 12, 4, 128,
                                              seed=42, scale=1.0, plant=plant)
    for a, b in zip(got, ref):
        nan_a = (a & 0x7F) == 0x7F
        nan_b = (b & 0x7F) == 0x7F
        bad = np.flatnonzero((nan_a != nan_b) | (~nan_a & (a != b)))
        assert bad.size == 0, [(int(i), hex(a.flat[i]), hex(b.flat[i])) for i in bad[:16]]


@pytest.mark.parametrize("convert", [False, True])
def test_relayout_bad_block_ids_are_skipped_and_flagged(convert):
    """A source or destination table entry outside its pool is never dereferenced: the tokens it covers are
    not written (their destination slots keep the sentinel), every other token is, and the error word gets the
    block-id bit."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    n, sbs, dbs, hkv, d, dblk = 200, 16, 32, 4, 128, 8
    sc = Scenario(num_q_heads=hkv, num_kv_heads=hkv, head_dim=d, block_size=sbs, dtype="bf16", lengths=[n],
                  pool_blocks=16, num_shards=2, seed=51, err_word=err)
    sc.write_all()
    torch.cuda.synchronize()
    err.zero_()
    dst_bt, _ = inputs.assign_blocks(dblk, [n], dbs, inputs.stream(51, 0, 0, inputs.T_DST_PERM))
    src_tab, dst_tab = sc.tables[0].copy(), dst_bt[0].copy()
    src_tab[3] = 16 + 5                    # source tokens 48..63: block id past the pool
    dst_tab[5] = -2                        # destination tokens 160..191: negative block id
    skipped = list(range(48, 64)) + list(range(160, 192))
    print(f"relayout with bad block ids, convert={convert}", flush=True)
    pm_src = _oracle_pool_from(sc)
    if convert:
        dst = ops.ConvertedPool(dblk, dbs, hkv, 1, d, "fp8", "token_major", 0.05).fill_bits(0x7F)
        ops.kv_relayout_convert(sc.pool, i32(src_tab), dst, i32(dst_tab), n)
        ref = opool.DestModel(dblk, dbs, hkv, 1, d, np.uint8, opool.LAYOUT_TOKEN_MAJOR, fill=0x7F, scale=0.05)
        opool.relayout_convert(pm_src, sc.tables[0], ref, dst_bt[0], n)
        fill_row = np.full(d, 0x7F, np.uint8)
        for p in skipped:                  # what the valid tables would have written there stays unwritten
            for h in range(hkv):
                ref.put(opool.slots_for(dst_bt[0], dbs, [p])[0], h, fill_row, fill_row)
        got, want = [t.cpu().numpy() for t in dst.k + dst.v], ref.k + ref.v
    else:
        dst = ops.PagedPool(dblk, dbs, hkv, 1, d, "bf16", err_word=err).fill_bits(SENTINEL["bf16"])
        ops.kv_relayout(sc.pool, i32(src_tab), dst, i32(dst_tab), n)
        ref = opool.PoolModel(dblk, dbs, hkv, 1, d, np.uint16, fill=SENTINEL["bf16"])
        opool.relayout(pm_src, sc.tables[0], ref, dst_bt[0], n)
        for p in skipped:
            for h in range(hkv):
                s, blk, off, lh = ref.where(opool.slots_for(dst_bt[0], dbs, [p])[0], h)
                ref.k[s][blk, lh, off, :] = SENTINEL["bf16"]
                ref.v[s][blk, lh, :, off] = SENTINEL["bf16"]
        got, want = [from_dev(t, "bf16") for t in dst.k + dst.v], ref.k + ref.v
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert int(err.item()) & 1
