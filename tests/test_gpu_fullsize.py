"""Parity at the full sizes the benchmark times, in the launch configurations
it times.

* Decode of the Llama-3-8B-shaped step (64 requests at context 512: one
  workgroup per (request, KV head) pair) and of the Qwen3-32B-like step
  (16 requests, contexts drawn as the benchmark draws them from
  U[2048, 8192]: the stream split with its merge kernel): every output row
  against the oracle.
* Prefill of the 16384-token Qwen3-32B-like prompt: its last chunk of 2048
  (one key-tile group per workgroup) and its last chunk of 512 (two key-tile
  groups per workgroup), with the whole prompt's K/V in the pool; a sample
  of rows (first, last and seeded picks, all 64 heads each) against the
  oracle computed row by row over keys [0, position] ("Lecture 7" section
  2.3).

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
