"""Pools past 4 GiB per shard tensor: block offsets beyond 2^32 bytes.

A Llama-3-8B-shaped pool (8 KV heads in 4 shards, head dim 128, bf16,
block size 16) of 540,000 blocks puts 4.42 GB in every shard tensor, so
blocks from 524,288 on start past byte 2^32 of their tensor.  The requests'
blocks are drawn from the first 200 blocks and the last 3,000, so every
request's K/V sits mostly past that boundary, and every kernel that turns a
block id into an address meets such blocks:

* slot mapping + kv_write fill the pool;
* attn_decode over contexts 40,000 / 700 / 1 / 333 (32 pairs: the stream
  split) against the oracle, every row;
* attn_prefill_chunk of two chunks (200 tokens at 500 of the 700-token
  request; 1,000 tokens at 39,000 of the 40,000-token one) against the
  oracle, sampled rows, all heads;
* kv_relayout of the 40,000-token request into a block-size-32 pool of
  270,000 blocks (4.42 GB per shard tensor, destination blocks past 2^32
  bytes too), checked bit for bit against the request's K/V;
* no error bit is set.

About 71 GB of device memory, freed at the end.
"""

import gc

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops
from gpu_common import Scenario, assert_close, from_dev, i32, to_dev
from oracle import attention as oa

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, SHARDS = 32, 8, 128, 16, 4
NB = 540_000
DST_BS, DST_NB = 32, 270_000
LENGTHS = [40_000, 700, 1, 333]


def _tables(n_blocks, lengths, bs, candidates, rng):
    need = [-(-n // bs) for n in lengths]
    pick = rng.permutation(candidates)[:sum(need)]
    width = max(need)
    tab = np.full((len(lengths), width), -1, np.int32)
    at = 0
    for r, k in enumerate(need):
        tab[r, :k] = pick[at:at + k]
        at += k
    assert tab.max() < n_blocks
    return tab


def test_pools_past_4gib_per_shard():
    shard_bytes = NB * (HKV // SHARDS) * BS * D * 2
    assert shard_bytes > 2 ** 32 and 524_288 * (HKV // SHARDS) * BS * D * 2 == 2 ** 32
    print(f"large pool: {NB} blocks, {shard_bytes / 1e9:.2f} GB per shard tensor", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = Scenario(num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_size=BS, dtype="bf16", lengths=LENGTHS,
                  pool_blocks=NB, num_shards=SHARDS, scale=0.5, seed=81, config_id=2, err_word=err)
    rng = np.random.default_rng(81)
    cand = np.concatenate([np.arange(200), np.arange(NB - 3000, NB)]).astype(np.int32)
    sc.tables = _tables(NB, LENGTHS, BS, cand, rng)
    sc.bt_dev = i32(sc.tables)
    assert (sc.tables[0] >= 524_288).mean() > 0.9
    sc.write_all()
    torch.cuda.synchronize()

    # decode, every row
    print("large pool: decode", flush=True)
    q = inputs.normal((len(LENGTHS), HQ, D), 0.5, "bf16", inputs.stream(81, 2, 0, inputs.T_Q, 0))
    out = torch.empty((len(LENGTHS), HQ, D), dtype=torch.bfloat16, device="cuda")
    ops.attn_decode(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32(LENGTHS), max(LENGTHS), HQ)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    qf = inputs.as_float(q, "bf16")
    for r in range(len(LENGTHS)):
        assert_close(got[r], oa.decode(qf[r], sc.kf(r), sc.vf(r)), "bf16", f"large-pool decode request {r}")

    # prefill chunks, sampled rows
    for r, S, T in ((1, 500, 200), (0, 39_000, 1000)):
        print(f"large pool: prefill request {r} chunk {T} at {S}", flush=True)
        qp = inputs.normal((T, HQ, D), 0.5, "bf16", inputs.stream(81, 2, 0, inputs.T_Q, 1 + r))
        op = torch.empty((T, HQ, D), dtype=torch.bfloat16, device="cuda")
        ops.attn_prefill_chunk(sc.pool, to_dev(qp, "bf16"), op, sc.bt_dev[r:r + 1], i32([0, T]), i32([S]), T, HQ)
        torch.cuda.synchronize()
        g = inputs.as_float(from_dev(op, "bf16"), "bf16")
        rows = np.unique(np.concatenate([[0, 1, 127, 128, T - 1], rng.integers(0, T, 9)]))
        ref = oa.attend(inputs.as_float(qp, "bf16")[rows], sc.kf(r)[:S + T], sc.vf(r)[:S + T], S + rows)
        assert_close(g[rows], ref, "bf16", f"large-pool prefill request {r}")

    # relayout of the long request into a second large pool
    print("large pool: relayout", flush=True)
    n = LENGTHS[0]
    dst = ops.PagedPool(DST_NB, DST_BS, HKV, SHARDS, D, "bf16", err_word=err).fill_bits(0x7FBF)
    dcand = np.concatenate([np.arange(100), np.arange(DST_NB - 1500, DST_NB)]).astype(np.int32)
    dtab = _tables(DST_NB, [n], DST_BS, dcand, rng)
    ops.kv_relayout(sc.pool, sc.bt_dev[0:1], dst, i32(dtab), n)
    torch.cuda.synchronize()
    blocks = torch.as_tensor(dtab[0].astype(np.int64), device="cuda")
    hl = HKV // SHARDS
    for s in range(SHARDS):
        kb = from_dev(dst.k[s].index_select(0, blocks).contiguous(), "bf16")   # [nblk, hl, bs, D]
        vb = from_dev(dst.v[s].index_select(0, blocks).contiguous(), "bf16")   # [nblk, hl, D, bs]
        k_log = kb.transpose(0, 2, 1, 3).reshape(-1, hl, D)[:n]               # [token, hl, D]
        v_log = vb.transpose(0, 3, 1, 2).reshape(-1, hl, D)[:n]
        assert np.array_equal(k_log, sc.k[0][:, s * hl:(s + 1) * hl]), f"relayout K, shard {s}"
        assert np.array_equal(v_log, sc.v[0][:, s * hl:(s + 1) * hl]), f"relayout V, shard {s}"
    assert int(err.item()) == 0
    del dst, sc, blocks
    gc.collect()
    torch.cuda.empty_cache()
