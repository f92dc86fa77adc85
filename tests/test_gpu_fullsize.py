"""Parity at the full sizes the benchmark times, in the launch configurations
it times.

* Decode of the Llama-3-8B-shaped step (64 requests at context 512: one
  workgroup per (request, KV head) pair) and of the Qwen3-32B-like step
  (16 requests, contexts drawn as the benchmark draws them from
  U[2048, 8192]: the stream split with its merge kernel): every output row
  against the oracle.
* Prefill of the 16384-token Qwen3-32B-like prompt: its last chunk of 2048
  (one key-tile group per workgroup) and its last chunk of 512 (two key-tile
  groups per workgroup), and every one of its 8 chunks of 2048 in order,
  with the whole prompt's K/V in the pool; a sample of rows (first, last and
  seeded picks, all 64 heads each) against the oracle computed row by row
  over keys [0, position] ("Lecture 7" section 2.3).
* One PD-multiplexing round at the multiplexing workload's shapes ("PD
  multiplexing" page, "SGLang's PD multiplexing", the main loop): the decode
  step of 128 requests at context 2048 on the decode stream of the level the
  rule picks (128 decode CUs), while one layer of the whole 32768-token
  prompt (8192 workgroups, 512 key tiles: eight periods of block ids) is
  prefilled on the complementary CUs.  Every decode row, the new token's K/V
  in the pool, and the first and last query tiles of the prompt (all heads)
  plus seeded rows are checked against the oracle.

Tolerances as everywhere for bf16: max |err| <= 2e-2, rel-L2 <= 5e-3.
"""

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops, workloads
from gpu_common import Scenario, assert_close, from_dev, i32, to_dev
from oracle import attention as oa

pytestmark = pytest.mark.gpu


def _q(sc, shape, idx=0):
    return inputs.normal(shape, 0.5, "bf16", inputs.stream(sc.seed, sc.cfg, sc.layer, inputs.T_Q, idx))


@pytest.mark.parametrize("name", ["llama3-8b", "qwen3-32b"])
def test_decode_full_step(name):
    w = {"llama3-8b": workloads.LLAMA3_8B, "qwen3-32b": workloads.QWEN3_32B}[name]
    ctx = [int(x) for x in w.decode_contexts()]
    print(f"full-size decode {name}: {len(ctx)} requests, max context {max(ctx)}", flush=True)
    nblk = sum(-(-n // w.block_size) for n in ctx) + 4
    sc = Scenario(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  block_size=w.block_size, dtype="bf16", lengths=ctx, pool_blocks=nblk, scale=w.input_scale,
                  seed=71, config_id=w.config_id)
    sc.write_all()
    q = _q(sc, (len(ctx), w.num_q_heads, w.head_dim))
    out = torch.empty((len(ctx), w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ops.attn_decode(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32(ctx), max(ctx), w.num_q_heads)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    qf = inputs.as_float(q, "bf16")
    ref = np.stack([oa.decode(qf[r], sc.kf(r), sc.vf(r)) for r in range(len(ctx))])
    assert_close(got, ref, "bf16", f"decode {name}")


@pytest.mark.parametrize("chunk", [2048, 512])
def test_prefill_last_chunk_of_16k_prompt_sampled(chunk):
    w = workloads.QWEN3_32B
    n = w.prompt_len
    S = n - chunk
    print(f"full-size prefill: chunk {chunk} at {S} of a {n}-token prompt", flush=True)
    sc = Scenario(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  block_size=w.block_size, dtype="bf16", lengths=[n], pool_blocks=n // w.block_size + 2,
                  scale=w.input_scale, seed=72, config_id=w.config_id)
    sc.write_all()
    q = _q(sc, (chunk, w.num_q_heads, w.head_dim), idx=1)
    out = torch.empty((chunk, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ops.attn_prefill_chunk(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32([0, chunk]), i32([S]), chunk,
                           w.num_q_heads)
    torch.cuda.synchronize()
    got = inputs.as_float(from_dev(out, "bf16"), "bf16")
    rng = np.random.default_rng(chunk)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, chunk - 1], rng.integers(0, chunk, 11)]))
    ref = oa.attend(inputs.as_float(q, "bf16")[rows], sc.kf(0), sc.vf(0), S + rows)
    assert_close(got[rows], ref, "bf16", f"prefill chunk {chunk} at {S}")


def test_prefill_every_2048_chunk_of_16k_prompt_sampled():
    w = workloads.QWEN3_32B
    n, chunk = w.prompt_len, 2048
    sc = Scenario(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  block_size=w.block_size, dtype="bf16", lengths=[n], pool_blocks=n // w.block_size + 2,
                  scale=w.input_scale, seed=74, config_id=w.config_id)
    sc.write_all()
    kf, vf = sc.kf(0), sc.vf(0)
    for ci, S in enumerate(range(0, n, chunk)):
        print(f"full-size prefill: chunk {ci} of 2048 at {S}", flush=True)
        q = _q(sc, (chunk, w.num_q_heads, w.head_dim), idx=10 + ci)
        out = torch.empty((chunk, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        ops.attn_prefill_chunk(sc.pool, to_dev(q, "bf16"), out, sc.bt_dev, i32([0, chunk]), i32([S]), chunk,
                               w.num_q_heads, max_total_len=n)
        torch.cuda.synchronize()
        got = inputs.as_float(from_dev(out, "bf16"), "bf16")
        rng = np.random.default_rng(1000 + ci)
        rows = np.unique(np.concatenate([[0, 63, 64, 127, 128, chunk - 1], rng.integers(0, chunk, 6)]))
        ref = oa.attend(inputs.as_float(q, "bf16")[rows], kf, vf, S + rows)
        assert_close(got[rows], ref, "bf16", f"prefill chunk {ci} at {S}")


def test_mux_round_at_full_multiplexing_shapes():
    w = workloads.PDMUX_8B
    B, ctx, N = w.decode_batch, w.decode_context[0], w.prompt_len
    hq, hkv, d, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    nblk = B * (ctx // bs) + N // bs + 8
    g = lambda t, i=0: inputs.stream(75, w.config_id, 0, t, i)  # noqa: E731
    tables, _ = inputs.assign_blocks(nblk, [ctx] * B + [N], bs, g(inputs.T_PERM))
    dec_bt, pr_bt = i32(tables[:B]), i32(tables[B:B + 1])
    print(f"full-size mux round: decode {B} x {ctx}, prompt {N}, pool {nblk} blocks", flush=True)
    pool = ops.PagedPool(nblk, bs, hkv, 1, d, "bf16").fill_bits(0x7FBF)
    # decode history: positions 0 .. ctx-2 of every request, written up front
    hk = inputs.normal((B, ctx - 1, hkv, d), 0.5, "bf16", g(inputs.T_K, 0))
    hv = inputs.normal((B, ctx - 1, hkv, d), 0.5, "bf16", g(inputs.T_V, 0))
    start = np.arange(B + 1, dtype=np.int32) * (ctx - 1)
    slots = ops.slot_mapping(dec_bt, i32(start), i32(np.zeros(B)), B * (ctx - 1), bs, nblk)
    ops.kv_write(pool, to_dev(hk.reshape(-1, hkv, d), "bf16"), to_dev(hv.reshape(-1, hkv, d), "bf16"), slots)
    kn = inputs.normal((B, hkv, d), 0.5, "bf16", g(inputs.T_K_DECODE))
    vn = inputs.normal((B, hkv, d), 0.5, "bf16", g(inputs.T_V_DECODE))
    qd = inputs.normal((B, hq, d), 0.5, "bf16", g(inputs.T_Q_DECODE))
    qp = inputs.normal((N, hq, d), 0.5, "bf16", g(inputs.T_Q, 1))
    kp = inputs.normal((N, hkv, d), 0.5, "bf16", g(inputs.T_K, 1))
    vp = inputs.normal((N, hkv, d), 0.5, "bf16", g(inputs.T_V, 1))
    dec_slots = ops.slot_mapping(dec_bt, i32(np.arange(B + 1)), i32([ctx - 1] * B), B, bs, nblk)
    pr_slots = ops.slot_mapping(pr_bt, i32([0, N]), i32([0]), N, bs, nblk)
    o_dec = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    o_pr = torch.zeros((N, hq, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size_for(pool, B, hq, ctx)), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    decode = ops.DecodeStepArgs([pool], [to_dev(qd, "bf16")], [to_dev(kn, "bf16")], [to_dev(vn, "bf16")], [o_dec],
                                dec_slots, dec_bt, i32([ctx] * B), ctx, hq, ws)
    job = ops.PrefillJobArgs([pool], [to_dev(qp, "bf16")], [to_dev(kp, "bf16")], [to_dev(vp, "bf16")], [o_pr],
                             pr_slots, pr_bt, i32([0, N]), i32([0]), N, hq)
    mux = ops.Mux(0, w.extra["cu_granularity"], w.extra["min_decode_cus"], w.extra["group_num"],
                  w.extra["decode_bs_divisor"], w.extra["token_budget"])
    try:
        groups = mux.groups()
        level = mux.choose(B, True)
        assert groups[level] == (128, 128)
        lvl, _ = mux.run_round(decode, job)
        assert lvl == level and job.done_submitting
        mux.wait_prefill()
        torch.cuda.synchronize()
    finally:
        mux.close()
    f = lambda x: inputs.as_float(x, "bf16")  # noqa: E731
    # decode: every row over the history plus the new key, written by this round
    got = f(from_dev(o_dec, "bf16"))
    qdf = f(qd)
    for r in range(B):
        k = np.concatenate([f(hk[r]), f(kn[r:r + 1])])
        v = np.concatenate([f(hv[r]), f(vn[r:r + 1])])
        assert_close(got[r], oa.decode(qdf[r], k, v), "bf16", f"mux decode request {r}")
    # the new token's row sits at position ctx-1 of each request, bit for bit
    kpool = from_dev(pool.k[0], "bf16")               # [blocks, Hkv, bs, D]
    vpool = from_dev(pool.v[0], "bf16")               # [blocks, Hkv, D, bs]
    for r in (0, 57, B - 1):
        blk = tables[r, (ctx - 1) // bs]
        off = (ctx - 1) % bs
        assert np.array_equal(kpool[blk, :, off, :], kn[r]) and np.array_equal(vpool[blk, :, :, off], vn[r])
    # prefill: first and last 128-query tiles and seeded rows, all heads, over keys [0, row]
    got = f(from_dev(o_pr, "bf16"))
    rng = np.random.default_rng(76)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(N - 128, N), rng.integers(0, N, 16)]))
    ref = oa.attend(f(qp)[rows], f(kp), f(vp), rows)
    assert_close(got[rows], ref, "bf16", "mux prefill of the 32K prompt")
