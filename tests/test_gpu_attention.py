"""GPU parity of decode and chunked-prefill attention against the fp64 oracle.

Tolerances (written here, applied to every case): bf16 max |err| <= 2e-2
and rel-L2 <= 5e-3; fp32 max |err| <= 1e-5 and rel-L2 <= 1e-5.  The
oracle never chunks: every chunk the GPU computes is compared with rows
S..S+T-1 of the oracle's one-shot prefill ("Lecture 7" section 2.3:
chunked prefill is lossless).  Pools are filled with NaN sentinels first,
so any read of a slot that was never written would poison the output.
"""

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops, workloads
from gpu_common import SENTINEL, Scenario, assert_close, from_dev, i32, to_dev
from oracle import attention as oa

pytestmark = pytest.mark.gpu


def _q(sc, shape, tid=inputs.T_Q, idx=0, scale=1.0):
    g = inputs.stream(sc.seed, sc.cfg, sc.layer, tid, idx)
    return inputs.normal(shape, scale, sc.dtype, g)


def _tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def run_decode(sc: Scenario, q_np, max_ctx=None):
    b = len(sc.lengths)
    q = to_dev(q_np, sc.dtype)
    out = torch.empty((b, sc.hq, sc.d), dtype=_tdtype(sc.dtype), device="cuda")
    ops.attn_decode(sc.pool, q, out, sc.bt_dev, i32(sc.lengths), max_ctx or max(sc.lengths), sc.hq)
    torch.cuda.synchronize()
    return inputs.as_float(from_dev(out, sc.dtype), sc.dtype)


def oracle_decode(sc: Scenario, q_np):
    qf = inputs.as_float(q_np, sc.dtype)
    return np.stack([oa.decode(qf[r], sc.kf(r), sc.vf(r)) for r in range(len(sc.lengths))])


@pytest.mark.parametrize("dtype,hq,hkv,d,bs,shards,lengths", [
    ("f32", 4, 2, 64, 16, 1, [37, 64, 100, 128]),          # the tiny check's decode requests
    ("bf16", 32, 8, 128, 16, 1, [1, 2, 15, 16, 17, 63, 64, 65, 300, 511, 1000, 1537]),
    ("bf16", 64, 8, 128, 16, 1, [2048, 8192, 3001, 4097]),
    ("bf16", 16, 16, 128, 32, 4, [129, 700]),              # G = 1, several shards
    ("bf16", 32, 16, 64, 16, 16, [1, 47, 300]),            # the most shards (16 x 1 head)
    ("bf16", 32, 2, 64, 64, 2, [1, 333, 2000]),            # G = 16, head dim 64
    ("bf16", 8, 4, 128, 128, 1, [5, 256, 1025]),
    ("f32", 8, 2, 128, 32, 2, [1, 90, 513]),
    # 512 (request, KV head) pairs: one workgroup per pair, no partials
    ("bf16", 32, 8, 128, 16, 1, [int(x) for x in np.random.default_rng(11).integers(1, 600, 64)]),
])
def test_decode_matches_oracle(dtype, hq, hkv, d, bs, shards, lengths):
    nblk = sum(-(-n // bs) for n in lengths) + 3
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype, lengths=lengths,
                  pool_blocks=nblk, num_shards=shards, scale=0.5 if dtype == "bf16" else 1.0, seed=5)
    sc.write_all()
    q = _q(sc, (len(lengths), hq, d), scale=0.5 if dtype == "bf16" else 1.0)
    got = run_decode(sc, q)
    assert_close(got, oracle_decode(sc, q), dtype, "decode")


def test_decode_single_key_is_exact():
    # one key: the softmax weight is exactly 1, so the output is v0 itself
    for dtype in ("f32", "bf16"):
        sc = Scenario(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype=dtype, lengths=[1, 1, 1],
                      pool_blocks=8, seed=6)
        sc.write_all()
        got = run_decode(sc, _q(sc, (3, 8, 128)))
        for r in range(3):
            for h in range(8):
                assert np.array_equal(got[r, h], sc.vf(r)[0, h // 4])


def test_decode_longer_max_context_than_needed():
    # grid sized by a larger max_context_len: extra splits must be idle
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=[100, 700],
                  pool_blocks=64, scale=0.5, seed=7, table_pad=260)
    sc.write_all()
    q = _q(sc, (2, 32, 128), scale=0.5)
    got = run_decode(sc, q, max_ctx=4000)
    assert_close(got, oracle_decode(sc, q), "bf16", "decode(max_ctx 4000)")


@pytest.mark.parametrize("bs", [16, 64])
def test_decode_short_contexts_in_a_table_of_exact_width(bs):
    # 64 requests x 8 KV heads: one workgroup per pair, whose waves read the
    # table entries of their first three tiles before the context length is
    # known; with contexts of 1-100 keys and a table exactly as wide as the
    # longest needs, most of those entries lie past the context (the reads
    # are clamped to the table row and discarded)
    lengths = [int(x) for x in np.random.default_rng(41).integers(1, 101, 64)]
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=bs, dtype="bf16", lengths=lengths,
                  pool_blocks=64 * (-(-100 // bs)) + 8, scale=0.5, seed=41)
    assert sc.tables.shape[1] == -(-max(lengths) // bs)
    sc.write_all()
    q = _q(sc, (64, 32, 128), scale=0.5)
    got = run_decode(sc, q)
    assert_close(got, oracle_decode(sc, q), "bf16", f"decode(64 short contexts, bs {bs})")


def run_prefill_chunks(sc: Scenario, q_np, chunk, req=0):
    """Write + attend chunk by chunk for one request; returns the stacked GPU rows."""
    n = sc.lengths[req]
    outs = []
    for s in range(0, n, chunk):
        t = min(chunk, n - s)
        sc.write_tokens(sc.k[req][s:s + t], sc.v[req][s:s + t], np.array([0, t], np.int32), np.array([s], np.int32),
                        tables=sc.bt_dev[req:req + 1])
        q = to_dev(q_np[s:s + t], sc.dtype)
        out = torch.empty((t, sc.hq, sc.d), dtype=_tdtype(sc.dtype), device="cuda")
        ops.attn_prefill_chunk(sc.pool, q, out, sc.bt_dev[req:req + 1], i32([0, t]), i32([s]), t, sc.hq)
        outs.append(out)
    torch.cuda.synchronize()
    return np.concatenate([inputs.as_float(from_dev(o, sc.dtype), sc.dtype) for o in outs])


@pytest.mark.parametrize("dtype,hq,hkv,d,bs,n,chunk,shards", [
    ("f32", 4, 2, 64, 16, 256, 64, 1),          # the tiny check: 4 causal chunks of 64
    ("bf16", 32, 8, 128, 16, 1024, 512, 1),     # Llama-3-8B shape, 2 chunks of 512 (all rows)
    ("bf16", 32, 8, 128, 16, 1024, 1024, 1),    # same prompt one-shot
    ("bf16", 64, 8, 128, 16, 1100, 1100, 1),    # >= 512 workgroups: one key-tile group per workgroup
    ("bf16", 8, 2, 128, 16, 300, 77, 1),        # ragged chunks and tail
    ("bf16", 16, 1, 64, 32, 517, 200, 1),       # G = 16, head dim 64
    ("bf16", 4, 4, 128, 64, 130, 130, 1),       # G = 1, one chunk of 130
    ("bf16", 8, 8, 64, 128, 1, 1, 1),           # a single token
    ("f32", 4, 2, 128, 32, 70, 33, 1),
    ("bf16", 32, 16, 64, 16, 700, 300, 16),     # the most shards (16 x 1 head), G = 2
    ("bf16", 64, 8, 128, 32, 1300, 600, 4),     # Qwen3-32B heads in 4 shards of 2
])
def test_chunked_prefill_matches_one_shot_oracle(dtype, hq, hkv, d, bs, n, chunk, shards):
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype, lengths=[n],
                  pool_blocks=-(-n // bs) + 2, num_shards=shards, scale=0.5 if dtype == "bf16" else 1.0, seed=8)
    q = _q(sc, (n, hq, d), scale=0.5 if dtype == "bf16" else 1.0)
    got = run_prefill_chunks(sc, q, chunk)
    ref = oa.prefill(inputs.as_float(q, dtype), sc.kf(0), sc.vf(0))
    assert_close(got, ref, dtype, f"prefill chunk {chunk}")


def test_prefill_varlen_batch():
    # three requests with different chunk starts and lengths in one launch
    lengths = [700, 129, 1500]
    starts = [500, 0, 1024]
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=lengths,
                  pool_blocks=200, scale=0.5, seed=9)
    sc.write_all()
    qs = [_q(sc, (n - s, 32, 128), idx=r, scale=0.5) for r, (n, s) in enumerate(zip(lengths, starts))]
    tl = [n - s for n, s in zip(lengths, starts)]
    start_loc = np.concatenate([[0], np.cumsum(tl)]).astype(np.int32)
    q = to_dev(np.concatenate(qs), "bf16")
    out = torch.empty((int(start_loc[-1]), 32, 128), dtype=torch.bfloat16, device="cuda")
    ops.attn_prefill_chunk(sc.pool, q, out, sc.bt_dev, i32(start_loc), i32(starts), max(tl), 32)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    for r in range(3):
        ref = oa.prefill_chunk(inputs.as_float(qs[r], "bf16"), sc.kf(r), sc.vf(r), starts[r])
        assert_close(got[start_loc[r]:start_loc[r + 1]], ref, "bf16", f"request {r}")


def test_single_token_chunk_equals_decode():
    # a T=1 chunk at S is the decode query at L = S+1: the two kernels agree
    L = 777
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=[L],
                  pool_blocks=60, scale=0.5, seed=10)
    sc.write_all()
    q = _q(sc, (1, 32, 128), scale=0.5)
    dec = run_decode(sc, q)
    out = torch.empty((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    ops.attn_prefill_chunk(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32([0, 1]), i32([L - 1]), 1, 32)
    torch.cuda.synchronize()
    pre = inputs.as_float(from_dev(out, "bf16"), "bf16")
    ref = oracle_decode(sc, q)
    assert_close(dec, ref, "bf16", "decode")
    assert_close(pre, ref, "bf16", "prefill T=1")
    assert np.abs(dec - pre).max() <= 2e-2


def test_tiny_config_relayout_then_decode_unchanged():
    """The tiny check: prompt prefilled in 64-token chunks, decode, relayout to bs 32 (1 -> 2 shards), decode again."""
    w = workloads.TINY
    ctx = list(w.decode_context)
    lengths = [w.prompt_len] + ctx
    sc = Scenario(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  block_size=w.block_size, dtype=w.dtype, lengths=lengths, pool_blocks=w.pool_blocks,
                  num_shards=w.src_shards, scale=w.input_scale, seed=w.seed, config_id=w.config_id)
    assert sum(-(-n // 16) for n in lengths) == 38
    qp = _q(sc, (w.prompt_len, w.num_q_heads, w.head_dim))
    got = run_prefill_chunks(sc, qp, w.chunk_sizes[0], req=0)
    assert_close(got, oa.prefill(qp, sc.kf(0), sc.vf(0)), "f32", "tiny prefill")
    sc.write_all([0] + ctx)      # decode requests' K/V (the prompt is already written)
    sc_dec_lengths = sc.lengths
    qd = _q(sc, (len(ctx), w.num_q_heads, w.head_dim), tid=inputs.T_Q_DECODE)
    tables = sc.bt_dev[1:]
    out = torch.empty((len(ctx), w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ops.attn_decode(sc.pool, to_dev(qd, "f32"), out, tables, i32(ctx), max(ctx), w.num_q_heads)
    ref = np.stack([oa.decode(qd[i], sc.kf(i + 1), sc.vf(i + 1)) for i in range(len(ctx))])
    before = out.cpu().numpy().astype(np.float64)
    assert_close(before, ref, "f32", "tiny decode (bs 16)")
    # relayout every request to block size 32, 2 shards x 1 head
    g = inputs.stream(w.seed, w.config_id, 0, inputs.T_DST_PERM)
    dst_bt, _ = inputs.assign_blocks(w.dst_pool_blocks, sc_dec_lengths, w.dst_block_size, g)
    dst = ops.PagedPool(w.dst_pool_blocks, w.dst_block_size, w.num_kv_heads, w.dst_shards, w.head_dim, "f32")
    dst.fill_bits(0x7FC0DEAD)
    dst_bt_dev = i32(dst_bt)
    for r, n in enumerate(sc_dec_lengths):
        ops.kv_relayout(sc.pool, sc.bt_dev[r], dst, dst_bt_dev[r], n)
    out2 = torch.empty_like(out)
    ops.attn_decode(dst, to_dev(qd, "f32"), out2, dst_bt_dev[1:], i32(ctx), max(ctx), w.num_q_heads)
    torch.cuda.synchronize()
    after = out2.cpu().numpy().astype(np.float64)
    assert_close(after, ref, "f32", "tiny decode (bs 32, 2 shards)")
    assert np.abs(after - before).max() <= 1e-6


def test_bad_block_id_makes_its_keys_absent():
    """A block-table entry outside [0, num_blocks) is never dereferenced: its
    keys drop out of the softmax (decode and prefill alike) and the error
    word gets the block-id bit.  Reference: the oracle over the remaining keys."""
    bs, hq, hkv, d = 16, 16, 4, 128
    lengths = [300, 200]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype="bf16", lengths=lengths,
                  pool_blocks=40, scale=0.5, seed=12, err_word=err)
    sc.write_all()
    bad = {0: [3, 10], 1: [5]}                      # logical block indices made invalid
    tables = sc.tables.copy()
    for r, js in bad.items():
        for j in js:
            tables[r, j] = 40 + 7 * j               # out of range
    sc.bt_dev = i32(tables)
    f = lambda x: inputs.as_float(x, "bf16")  # noqa: E731

    def present(r, upto):
        keep = [p for p in range(upto) if p // bs not in bad[r]]
        return sc.kf(r)[keep], sc.vf(r)[keep]

    # decode: every request's last position
    q = _q(sc, (2, hq, d), scale=0.5)
    got = run_decode(sc, q)
    for r in range(2):
        k, v = present(r, lengths[r])
        assert_close(got[r], oa.decode(f(q)[r], k, v), "bf16", f"decode request {r}")
    assert int(err.item()) & 1
    # prefill: request 0, one chunk covering positions 100..299 (a bad block on each side of 100)
    err.zero_()
    s0, t = 100, 200
    qp = _q(sc, (t, hq, d), tid=inputs.T_Q, idx=1, scale=0.5)
    out = torch.empty((t, hq, d), dtype=torch.bfloat16, device="cuda")
    ops.attn_prefill_chunk(sc.pool, to_dev(qp, "bf16"), out, sc.bt_dev[0:1], i32([0, t]), i32([s0]), t, hq)
    torch.cuda.synchronize()
    got = f(from_dev(out, "bf16"))
    ref = np.stack([oa.decode(f(qp)[i], *present(0, s0 + i + 1)) for i in range(t)])
    assert_close(got, ref, "bf16", "prefill with absent keys")
    assert int(err.item()) & 1


@pytest.mark.parametrize("dtype,hq,hkv,d,bs,shards,lengths", [
    # 512 (request, KV head) pairs: one workgroup per pair, the new key in its merge
    ("bf16", 32, 8, 128, 16, 1, [int(x) for x in np.random.default_rng(13).integers(1, 600, 64)]),
    # few pairs, long contexts: the stream split (the new key in the last piece of each pair)
    ("bf16", 64, 8, 128, 16, 1, [2048, 8192, 3001, 4097, 33]),
    ("bf16", 32, 2, 64, 64, 2, [1, 333, 2000, 32, 33]),    # G = 16, head dim 64, tile-edge contexts
    ("bf16", 8, 4, 128, 128, 1, [5, 256, 1025]),
    ("f32", 8, 2, 128, 32, 2, [1, 90, 513]),               # fp32: the append kernel, then decode
])
def test_decode_append_writes_the_row_and_attends(dtype, hq, hkv, d, bs, shards, lengths):
    """attn_decode_append over contexts L whose first L-1 tokens are in the pool: out equals the oracle over all
    L keys, and the pool equals, byte for byte, the oracle's pool with all L tokens written."""
    from oracle import pool as opool
    nblk = sum(-(-n // bs) for n in lengths) + 3
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype, lengths=lengths,
                  pool_blocks=nblk, num_shards=shards, scale=0.5 if dtype == "bf16" else 1.0, seed=15)
    sc.write_all(upto=[n - 1 for n in lengths])
    kn = np.stack([sc.k[r][n - 1] for r, n in enumerate(lengths)])
    vn = np.stack([sc.v[r][n - 1] for r, n in enumerate(lengths)])
    q = _q(sc, (len(lengths), hq, d), scale=0.5 if dtype == "bf16" else 1.0)
    out = torch.empty((len(lengths), hq, d), dtype=_tdtype(dtype), device="cuda")
    print(f"attn_decode_append {dtype} hq={hq} hkv={hkv} d={d} bs={bs} lengths={lengths[:6]}", flush=True)
    ops.attn_decode_append(sc.pool, to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), out, sc.bt_dev,
                           i32(lengths), max(lengths), hq)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, dtype), dtype)
    assert_close(got, oracle_decode(sc, q), dtype, "decode append")
    elem = np.uint16 if dtype == "bf16" else np.float32
    fill = SENTINEL[dtype] if dtype == "bf16" else np.array([SENTINEL[dtype]], np.uint32).view(np.float32)[0]
    pm = opool.PoolModel(nblk, bs, hkv, shards, d, elem, fill=fill)
    for r, n in enumerate(lengths):
        opool.write(pm, sc.k[r], sc.v[r], opool.slots_for(sc.tables[r], bs, range(n)))
    for s in range(shards):
        assert np.array_equal(from_dev(sc.pool.k[s], dtype).view(np.uint8), pm.k[s].view(np.uint8)), f"K shard {s}"
        assert np.array_equal(from_dev(sc.pool.v[s], dtype).view(np.uint8), pm.v[s].view(np.uint8)), f"V shard {s}"


def test_decode_append_with_a_bad_last_block():
    """The block holding a request's new key is outside the pool: nothing is written, the whole block's keys
    (the new one included) are absent, the error word gets the block-id bit; other requests are unaffected."""
    bs, hq, hkv, d = 16, 16, 4, 128
    lengths = [300, 77]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype="bf16", lengths=lengths,
                  pool_blocks=40, scale=0.5, seed=16, err_word=err)
    sc.write_all(upto=[n - 1 for n in lengths])
    torch.cuda.synchronize()
    err.zero_()
    tables = sc.tables.copy()
    tables[0, 299 // bs] = 40 + 3                          # request 0's last block: past the pool
    sc.bt_dev = i32(tables)
    before = [from_dev(t, "bf16").copy() for t in sc.pool.k + sc.pool.v]
    kn = np.stack([sc.k[r][n - 1] for r, n in enumerate(lengths)])
    vn = np.stack([sc.v[r][n - 1] for r, n in enumerate(lengths)])
    q = _q(sc, (2, hq, d), scale=0.5)
    out = torch.empty((2, hq, d), dtype=torch.bfloat16, device="cuda")
    ops.attn_decode_append(sc.pool, to_dev(q, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"), out, sc.bt_dev,
                           i32(lengths), max(lengths), hq)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    qf = inputs.as_float(q, "bf16")
    keep = [p for p in range(300) if p // bs != 299 // bs]
    assert_close(got[0], oa.decode(qf[0], sc.kf(0)[keep], sc.vf(0)[keep]), "bf16", "request with a bad last block")
    assert_close(got[1], oa.decode(qf[1], sc.kf(1), sc.vf(1)), "bf16", "request 1")
    assert int(err.item()) & 1
    after = [from_dev(t, "bf16") for t in sc.pool.k + sc.pool.v]
    # only request 1's new row changed the pool
    changed = sum(int(np.count_nonzero(a != b)) for a, b in zip(after, before))
    assert 0 < changed <= 2 * hkv * d


def _decode_with(sc, q_np, ctx, max_ctx, workspace, err=None):
    b = len(ctx)
    out = torch.empty((b, sc.hq, sc.d), dtype=_tdtype(sc.dtype), device="cuda")
    ops.attn_decode(sc.pool, to_dev(q_np, sc.dtype), out, sc.bt_dev, i32(ctx), max_ctx, sc.hq, workspace=workspace)
    torch.cuda.synchronize()
    return inputs.as_float(from_dev(out, sc.dtype), sc.dtype)


def test_decode_stream_split_reads_only_rows_it_wrote():
    """Stream split with max_context_len far above every context: the batch has fewer 32-key tiles than the
    grid has workgroups.  The workspace starts as NaN bits and is then reused for another set of contexts, so a
    partial row that no workgroup of the current launch wrote would poison the output."""
    lengths = [2100, 700, 33]
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=lengths,
                  pool_blocks=200, scale=0.5, seed=17, table_pad=120)
    sc.write_all()
    q = _q(sc, (3, 32, 128), scale=0.5)
    qf = inputs.as_float(q, "bf16")
    max_ctx = 4000
    nbytes = ops.attn_decode_workspace_size_for(sc.pool, 3, 32, max_ctx)
    assert nbytes > 0                                   # the stream plan (24 pairs, splits needed)
    ws = torch.full((nbytes // 4,), 0x7FC00000, dtype=torch.int32, device="cuda").view(torch.uint8)
    for ctx in ([100, 700, 33], [2100, 650, 20], [40, 64, 33], [2100, 700, 33]):
        print(f"stream split contexts {ctx} max_ctx {max_ctx}", flush=True)
        got = _decode_with(sc, q, ctx, max_ctx, ws)
        ref = np.stack([oa.decode(qf[r], sc.kf(r)[:L], sc.vf(r)[:L]) for r, L in enumerate(ctx)])
        assert_close(got, ref, "bf16", f"stream split, contexts {ctx}")


@pytest.mark.parametrize("dtype,hq,hkv,lengths,max_ctx", [
    ("bf16", 32, 8, [300, 90, 250], 200),       # stream split (24 pairs, two splits at 200)
    ("f32", 8, 2, [300, 90, 250], 200),         # fp32 equal splits
    ("bf16", 32, 8, [40] * 70, 32),             # 560 pairs: one workgroup per pair
])
def test_decode_context_above_max_is_cut_and_flagged(dtype, hq, hkv, lengths, max_ctx):
    """A context above max_context_len attends to its first max_context_len keys in every plan, and sets the
    context bit of the error word."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d = 128
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=16, dtype=dtype, lengths=lengths,
                  pool_blocks=sum(-(-n // 16) for n in lengths) + 2, scale=0.5 if dtype == "bf16" else 1.0, seed=18,
                  err_word=err)
    sc.write_all()
    torch.cuda.synchronize()
    err.zero_()
    q = _q(sc, (len(lengths), hq, d), scale=0.5 if dtype == "bf16" else 1.0)
    qf = inputs.as_float(q, dtype)
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size_for(sc.pool, len(lengths), hq, max_ctx)),
                     dtype=torch.uint8, device="cuda")
    got = _decode_with(sc, q, lengths, max_ctx, ws)
    ref = np.stack([oa.decode(qf[r], sc.kf(r)[:min(L, max_ctx)], sc.vf(r)[:min(L, max_ctx)])
                    for r, L in enumerate(lengths)])
    assert_close(got, ref, dtype, "contexts cut to max_context_len")
    assert int(err.item()) & ops.ERRBIT_CONTEXT


def test_mixed_batch_decode_context_above_max_is_cut_and_flagged():
    """The mixed batch's decode part (equal splits) cuts and flags like attn_decode."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lengths = [300, 90, 250]
    sc = Scenario(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=lengths,
                  pool_blocks=50, scale=0.5, seed=19, err_word=err)
    sc.write_all()
    torch.cuda.synchronize()
    err.zero_()
    q = _q(sc, (3, 32, 128), scale=0.5)
    qf = inputs.as_float(q, "bf16")
    out = torch.empty((3, 32, 128), dtype=torch.bfloat16, device="cuda")
    ops.attn_mixed_batch(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32(lengths), 200, None, None, None, None, None,
                         0, 32)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    ref = np.stack([oa.decode(qf[r], sc.kf(r)[:min(L, 200)], sc.vf(r)[:min(L, 200)]) for r, L in enumerate(lengths)])
    assert_close(got, ref, "bf16", "mixed batch, contexts cut")
    assert int(err.item()) & ops.ERRBIT_CONTEXT


def test_prefill_chunk_past_max_total_len_is_cut_and_flagged():
    """A chunk reaching past max_total_len attends to keys [0, max_total_len) only and sets the context bit."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    n, s0, t, cap = 400, 200, 200, 330
    sc = Scenario(num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16, dtype="bf16", lengths=[n],
                  pool_blocks=30, scale=0.5, seed=20, err_word=err)
    sc.write_all()
    torch.cuda.synchronize()
    err.zero_()
    qp = _q(sc, (t, 16, 128), scale=0.5)
    out = torch.empty((t, 16, 128), dtype=torch.bfloat16, device="cuda")
    ops.attn_prefill_chunk(sc.pool, to_dev(qp, "bf16"), out, sc.bt_dev, i32([0, t]), i32([s0]), t, 16,
                           max_total_len=cap)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    qf = inputs.as_float(qp, "bf16")
    ref = np.stack([oa.decode(qf[i], sc.kf(0)[:min(s0 + i + 1, cap)], sc.vf(0)[:min(s0 + i + 1, cap)])
                    for i in range(t)])
    assert_close(got, ref, "bf16", "prefill cut at max_total_len")
    assert int(err.item()) & ops.ERRBIT_CONTEXT
