"""Stall-free mixed batch on the GPU: attn_mixed_batch's decode rows against
the decode oracle, its prefill rows against the oracle over the chunk
([L7] sections 2.3-2.4); where the decode part runs the same plan as
attn_decode, the fused launch must give the same bits as attn_decode, and
where attn_prefill_chunk runs one key-tile group per workgroup (at least 512
query tiles x q-heads) the same bits as attn_prefill_chunk (each workgroup
runs the same code; with fewer, the standalone kernel splits the keys over
two groups and sums in another order).
"""

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops
from gpu_common import Scenario, assert_close, from_dev, i32, to_dev
from oracle import attention as oa
from oracle import policy

pytestmark = pytest.mark.gpu


def _q(sc, shape, idx, scale):
    return inputs.normal(shape, scale, sc.dtype, inputs.stream(sc.seed, sc.cfg, sc.layer, inputs.T_Q, idx))


def _tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _setup(dtype, hq, hkv, d, bs, dec_lengths, prompt, budget, seed):
    """Decode requests (K/V written through L-1) plus one prompt whose first S tokens are already cached and
    whose next chunk (the stall-free share of the budget) is written now."""
    nd = len(dec_lengths)
    S = prompt // 3
    chunk = ops.stall_free_chunk(budget, nd, prompt - S)
    assert chunk == policy.stall_free_batch(budget, nd, [prompt - S])[1][0] and chunk > 0
    lengths = list(dec_lengths) + [prompt]
    nblk = sum(-(-n // bs) for n in lengths) + 4
    sc = Scenario(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype, lengths=lengths,
                  pool_blocks=nblk, scale=0.5 if dtype == "bf16" else 1.0, seed=seed)
    sc.write_all(upto=list(dec_lengths) + [S + chunk])
    sc_scale = 0.5 if dtype == "bf16" else 1.0
    qd = _q(sc, (nd, hq, d), 0, sc_scale)
    qp = _q(sc, (chunk, hq, d), 1, sc_scale)
    return sc, S, chunk, qd, qp


def _run_mixed(sc, nd, S, chunk, qd, qp):
    dt = _tdtype(sc.dtype)
    out_d = torch.empty((nd, sc.hq, sc.d), dtype=dt, device="cuda")
    out_p = torch.empty((chunk, sc.hq, sc.d), dtype=dt, device="cuda")
    ops.attn_mixed_batch(sc.pool, to_dev(qd, sc.dtype), out_d, sc.bt_dev[:nd], i32(sc.lengths[:nd]),
                         max(sc.lengths[:nd]), to_dev(qp, sc.dtype), out_p, sc.bt_dev[nd:], i32([0, chunk]), i32([S]),
                         chunk, sc.hq)
    torch.cuda.synchronize()
    return out_d, out_p


def _run_separate(sc, nd, S, chunk, qd, qp):
    dt = _tdtype(sc.dtype)
    out_d = torch.empty((nd, sc.hq, sc.d), dtype=dt, device="cuda")
    out_p = torch.empty((chunk, sc.hq, sc.d), dtype=dt, device="cuda")
    ops.attn_decode(sc.pool, to_dev(qd, sc.dtype), out_d, sc.bt_dev[:nd], i32(sc.lengths[:nd]),
                    max(sc.lengths[:nd]), sc.hq)
    ops.attn_prefill_chunk(sc.pool, to_dev(qp, sc.dtype), out_p, sc.bt_dev[nd:], i32([0, chunk]), i32([S]), chunk,
                           sc.hq)
    torch.cuda.synchronize()
    return out_d, out_p


def _check_oracle(sc, nd, S, chunk, qd, qp, out_d, out_p):
    f = lambda t: inputs.as_float(from_dev(t, sc.dtype), sc.dtype)  # noqa: E731
    qdf, qpf = inputs.as_float(qd, sc.dtype), inputs.as_float(qp, sc.dtype)
    ref_d = np.stack([oa.decode(qdf[r], sc.kf(r), sc.vf(r)) for r in range(nd)])
    ref_p = oa.prefill_chunk(qpf, sc.kf(nd)[:S + chunk], sc.vf(nd)[:S + chunk], S)
    assert_close(f(out_d), ref_d, sc.dtype, "mixed batch: decode rows")
    assert_close(f(out_p), ref_p, sc.dtype, "mixed batch: prefill rows")


@pytest.mark.parametrize("dtype,hq,hkv,d,bs,dec_lengths,prompt,budget", [
    # 64 decodes x 8 KV heads = 512 pairs: one workgroup per pair, same plan as attn_decode
    ("bf16", 32, 8, 128, 16, [int(x) for x in np.random.default_rng(21).integers(1, 700, 64)], 3000, 512),
    # and a chunk of 2048 (16 query tiles x 32 q-heads = 512): same prefill variant as attn_prefill_chunk
    ("bf16", 32, 8, 128, 16, [int(x) for x in np.random.default_rng(22).integers(1, 700, 64)], 6000, 2112),
    # G = 8 (Qwen3-32B heads) with both parts at full size: 512 pairs and a 2048-token chunk (16 x 64 >= 512);
    # the two kinds of workgroup share one LDS allocation, so two of either fit on a CU
    ("bf16", 64, 8, 128, 16, [int(x) for x in np.random.default_rng(23).integers(1, 700, 64)], 6000, 2112),
    # few pairs, long contexts: the decode part takes equal splits and a merge kernel follows
    ("bf16", 64, 8, 128, 16, [4097, 2048, 77, 1500], 2500, 2048),
    ("bf16", 16, 1, 64, 32, [1, 333, 1024], 900, 300),      # G = 16, head dim 64
    ("f32", 8, 2, 128, 32, [1, 90, 513], 700, 200),         # fp32: the two kernels back to back
])
def test_mixed_batch_matches_oracle(dtype, hq, hkv, d, bs, dec_lengths, prompt, budget):
    sc, S, chunk, qd, qp = _setup(dtype, hq, hkv, d, bs, dec_lengths, prompt, budget, seed=31)
    nd = len(dec_lengths)
    out_d, out_p = _run_mixed(sc, nd, S, chunk, qd, qp)
    _check_oracle(sc, nd, S, chunk, qd, qp, out_d, out_p)
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t)  # noqa: E731
    sep_d, sep_p = _run_separate(sc, nd, S, chunk, qd, qp)
    if nd * hkv >= 512 or dtype == "f32":
        # same decode plan and same per-workgroup code as attn_decode: same bits
        assert torch.equal(bits(out_d), bits(sep_d))
    if -(-chunk // 128) * hq >= 512 or dtype == "f32":
        assert torch.equal(bits(out_p), bits(sep_p))


def test_mixed_batch_with_an_empty_part():
    sc, S, chunk, qd, qp = _setup("bf16", 32, 8, 128, 16, [600, 1200], 1000, 512, seed=32)
    nd = 2
    ref_d, ref_p = _run_mixed(sc, nd, S, chunk, qd, qp)
    # decode only
    out_d = torch.empty_like(ref_d)
    ops.attn_mixed_batch(sc.pool, to_dev(qd, "bf16"), out_d, sc.bt_dev[:nd], i32(sc.lengths[:nd]),
                         max(sc.lengths[:nd]), None, None, None, None, None, 0, sc.hq)
    # prefill only
    out_p = torch.empty_like(ref_p)
    ops.attn_mixed_batch(sc.pool, None, None, None, None, 0, to_dev(qp, "bf16"), out_p, sc.bt_dev[nd:],
                         i32([0, chunk]), i32([S]), chunk, sc.hq)
    torch.cuda.synchronize()
    assert torch.equal(out_d.view(torch.int16), ref_d.view(torch.int16))
    assert torch.equal(out_p.view(torch.int16), ref_p.view(torch.int16))
