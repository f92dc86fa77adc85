"""GPU tests of the single-GPU PD-multiplexing runtime.

* The split levels and the CU masks the library builds: complementary,
  the right sizes, and balanced over the 8 XCDs (mask bit i selects a CU of
  XCD i % 8).
* A multi-round run: decode steps of a small batch on the decode stream of
  the chosen level while a prompt is prefilled layer by layer on the prefill
  stream ("PD multiplexing" page, "SGLang's PD multiplexing": the main
  loop).  Every decode and prefill output is checked against the oracle,
  and the level changes only when the prefill starts and after it finishes.
* Decode on the CU-masked stream of a split level with one split per
  (request, KV head) (the whole-line kernel): head dims 64 and 128, GQA
  groups 1 to 16, block sizes 16 to 128, 1 to 8 head shards, ragged
  contexts from 1 key, plain and append steps, eager and as graphs, against
  the oracle.
"""

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import inputs, ops
from gpu_common import assert_close, from_dev, i32, to_dev
from oracle import attention as oa
from oracle import policy

pytestmark = pytest.mark.gpu


def _popcount(words):
    return sum(bin(w).count("1") for w in words)


def _bits(words):
    return [i for i in range(len(words) * 32) if (words[i // 32] >> (i % 32)) & 1]


def test_levels_and_cu_masks():
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=65536)
    try:
        groups = mux.groups()
        assert groups == policy.mi355x_stream_groups()
        assert mux.choose(128, True) == policy.choose_level(len(groups), 128, True) == 6
        assert mux.choose(5, False) == len(groups) - 1 and mux.choose(0, True) == 0
        assert mux.layers_per_round(32768, 32) == 2
        for lvl, (pcu, dcu) in enumerate(groups):
            if pcu == 0 or dcu == 0:
                continue
            pm, dm = mux.cu_mask(lvl, 0), mux.cu_mask(lvl, 1)
            assert _popcount(pm) == pcu and _popcount(dm) == dcu
            assert all((a & b) == 0 for a, b in zip(pm, dm))
            assert all((a | b) == 0xFFFFFFFF for a, b in zip(pm, dm))
            for bits, n in ((_bits(pm), pcu), (_bits(dm), dcu)):
                per_xcd = [sum(1 for b in bits if b % 8 == x) for x in range(8)]
                assert per_xcd == [n // 8] * 8
            assert mux.stream(lvl, 0) and mux.stream(lvl, 1) and mux.stream(lvl, 0) != mux.stream(lvl, 1)
    finally:
        mux.close()


class _MuxCase:
    """A few layers with a decode batch and one prompt sharing each layer's pool."""

    def __init__(self, layers=3, hq=8, hkv=2, d=128, bs=16, ctx=(100, 37, 300, 64), prompt=500, seed=31, shards=1):
        self.L, self.hq, self.hkv, self.d, self.bs = layers, hq, hkv, d, bs
        self.ctx = list(ctx)
        self.N = prompt
        B = len(ctx)
        nblk = sum(-(-c // bs) for c in ctx) + -(-prompt // bs) + 4
        g = lambda t, i=0, l=0: inputs.stream(seed, 50, l, t, i)  # noqa: E731
        tables, _ = inputs.assign_blocks(nblk, self.ctx + [prompt], bs, g(inputs.T_PERM))
        self.dec_bt, self.pr_bt = i32(tables[:B]), i32(tables[B:])
        self.pools, self.hist_k, self.hist_v = [], [], []
        self.kn, self.vn, self.qd, self.qp, self.kp, self.vp = [], [], [], [], [], []
        for l in range(layers):
            pool = ops.PagedPool(nblk, bs, hkv, shards, d, "bf16").fill_bits(0x7FBF)
            hk = [inputs.normal((c - 1, hkv, d), 0.5, "bf16", g(inputs.T_K, r, l)) for r, c in enumerate(self.ctx)]
            hv = [inputs.normal((c - 1, hkv, d), 0.5, "bf16", g(inputs.T_V, r, l)) for r, c in enumerate(self.ctx)]
            start = np.concatenate([[0], np.cumsum([c - 1 for c in self.ctx])]).astype(np.int32)
            slots = ops.slot_mapping(self.dec_bt, i32(start), i32(np.zeros(B)), int(start[-1]), bs, nblk)
            ops.kv_write(pool, to_dev(np.concatenate(hk), "bf16"), to_dev(np.concatenate(hv), "bf16"), slots)
            self.pools.append(pool)
            self.hist_k.append(hk)
            self.hist_v.append(hv)
            self.kn.append(inputs.normal((B, hkv, d), 0.5, "bf16", g(inputs.T_K_DECODE, 0, l)))
            self.vn.append(inputs.normal((B, hkv, d), 0.5, "bf16", g(inputs.T_V_DECODE, 0, l)))
            self.qd.append(inputs.normal((B, hq, d), 0.5, "bf16", g(inputs.T_Q_DECODE, 0, l)))
            self.qp.append(inputs.normal((prompt, hq, d), 0.5, "bf16", g(inputs.T_Q, 0, l)))
            self.kp.append(inputs.normal((prompt, hkv, d), 0.5, "bf16", g(inputs.T_K, 99, l)))
            self.vp.append(inputs.normal((prompt, hkv, d), 0.5, "bf16", g(inputs.T_V, 99, l)))
        self.dec_slots = ops.slot_mapping(self.dec_bt, i32(np.arange(B + 1)), i32([c - 1 for c in self.ctx]), B, bs,
                                          nblk)
        self.pr_slots = ops.slot_mapping(self.pr_bt, i32([0, prompt]), i32([0]), prompt, bs, nblk)
        torch.cuda.synchronize()
        self.o_dec = [torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
        self.o_pr = [torch.zeros((prompt, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
        self.dev = dict(qd=[to_dev(x, "bf16") for x in self.qd], kn=[to_dev(x, "bf16") for x in self.kn],
                        vn=[to_dev(x, "bf16") for x in self.vn], qp=[to_dev(x, "bf16") for x in self.qp],
                        kp=[to_dev(x, "bf16") for x in self.kp], vp=[to_dev(x, "bf16") for x in self.vp])
        ws = torch.zeros(max(16, ops.attn_decode_workspace_size(B, hq, max(self.ctx), d)), dtype=torch.uint8,
                         device="cuda")
        self.decode = ops.DecodeStepArgs(self.pools, self.dev["qd"], self.dev["kn"], self.dev["vn"], self.o_dec,
                                         self.dec_slots, self.dec_bt, i32(self.ctx), max(self.ctx), hq, ws)
        self.prefill = ops.PrefillJobArgs(self.pools, self.dev["qp"], self.dev["kp"], self.dev["vp"], self.o_pr,
                                          self.pr_slots, self.pr_bt, i32([0, prompt]), i32([0]), prompt, hq)

    def check_decode(self):
        f = lambda x: inputs.as_float(x, "bf16")  # noqa: E731
        for l in range(self.L):
            got = f(from_dev(self.o_dec[l], "bf16"))
            for r in range(len(self.ctx)):
                k = np.concatenate([f(self.hist_k[l][r]), f(self.kn[l][r:r + 1])])
                v = np.concatenate([f(self.hist_v[l][r]), f(self.vn[l][r:r + 1])])
                assert_close(got[r], oa.decode(f(self.qd[l][r]), k, v), "bf16", f"decode layer {l} request {r}")

    def check_prefill(self):
        f = lambda x: inputs.as_float(x, "bf16")  # noqa: E731
        for l in range(self.L):
            got = f(from_dev(self.o_pr[l], "bf16"))
            assert_close(got, oa.prefill(f(self.qp[l]), f(self.kp[l]), f(self.vp[l])), "bf16", f"prefill layer {l}")


def test_mux_rounds_match_oracle_and_follow_the_level_rule():
    case = _MuxCase()
    # budget 1000 with a 500-token prompt: 2 layers per round, 3 layers -> 2 rounds
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=1000)
    try:
        groups = mux.groups()
        with_prefill = policy.choose_level(len(groups), 4, True)
        decode_only = policy.choose_level(len(groups), 4, False)
        levels, done = [], False
        for _ in range(10):
            lvl, done = mux.run_round(case.decode, case.prefill)
            levels.append(lvl)
            if done:
                break
        assert case.prefill.done_submitting and done
        assert case.prefill.c.next_layer == case.L
        assert levels[0] == with_prefill and all(x == with_prefill for x in levels)
        assert len(levels) >= 2          # 2 layers per round for 3 layers
        # after the prefill finished, the next round changes level (decode only)
        lvl, done = mux.run_round(case.decode, None)
        assert lvl == decode_only and not done
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_decode()
        case.check_prefill()
    finally:
        mux.close()


def test_mux_prefill_only_and_decode_only():
    case = _MuxCase(layers=2, ctx=(40, 33), prompt=300)
    mux = ops.Mux(0, token_budget=65536)
    try:
        lvl, done = mux.run_round(None, case.prefill)       # prefill alone: group 0, whole device
        assert lvl == 0
        mux.wait_prefill()
        lvl, done = mux.run_round(None, case.prefill)       # already submitted: reports done
        assert done
        lvl, _ = mux.run_round(case.decode, None)
        assert lvl == len(mux.groups()) - 1
        torch.cuda.synchronize()
        case.check_decode()
        case.check_prefill()
    finally:
        mux.close()


def test_mux_manual_divisions_pick_the_level():
    # 4 decode requests: the divisor rule would pick level 1; thresholds
    # that start level 5 at 4 requests move the round there
    case = _MuxCase()
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=1000)
    try:
        t = [1, 2, 3, 3, 4, 50]
        mux.set_manual_divisions(t)
        want = policy.choose_level_manual(len(mux.groups()), 4, True, t)
        assert want == 5 and mux.choose(4, True) == want
        levels, done = [], False
        for _ in range(10):
            lvl, done = mux.run_round(case.decode, case.prefill)
            levels.append(lvl)
            if done:
                break
        assert done and all(x == want for x in levels)
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_decode()
        case.check_prefill()
        mux.set_manual_divisions(None)
        assert mux.choose(4, True) == policy.choose_level(len(mux.groups()), 4, True)
        with pytest.raises(Exception):
            mux.set_manual_divisions([1, 2, 3])      # one per split level
    finally:
        mux.close()


def test_mux_decode_graphs_replay_the_eager_step():
    # the decode step as a per-level HIP graph: every replay (with eager work
    # and synchronizations in between) gives the bits of the plain launches,
    # with and without a prefill on the complementary stream
    case = _MuxCase(layers=2, ctx=(100, 37, 300, 64), prompt=500)
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=1000)
    try:
        mux.run_round(case.decode, None)
        torch.cuda.synchronize()
        eager = [o.clone() for o in case.o_dec]
        case.check_decode()
        mux.set_decode_graphs(True)
        scratch = torch.ones(1 << 20, device="cuda")
        for i in range(4):
            for o in case.o_dec:
                o.zero_()
            torch.cuda.synchronize()
            mux.run_round(case.decode, None)
            scratch.mul_(1.0001)                 # eager work between replays
            torch.cuda.synchronize()
            for got, want in zip(case.o_dec, eager):
                assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {i}"
        # on a split level while a prefill runs
        done = False
        for _ in range(10):
            for o in case.o_dec:
                o.zero_()
            _, done = mux.run_round(case.decode, case.prefill)
            torch.cuda.synchronize()
            for got, want in zip(case.o_dec, eager):
                assert torch.equal(got.view(torch.int16), want.view(torch.int16))
            if done:
                break
        assert done
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_prefill()
    finally:
        mux.close()


def test_mux_decode_append_matches_the_oracle():
    # the decode step as one attn_decode_append per layer: outputs against the
    # oracle, eager and as a per-level graph, alone and beside a prefill
    case = _MuxCase(layers=2, ctx=(100, 37, 300, 64), prompt=500)
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=1000)
    try:
        mux.set_decode_append(True)
        mux.run_round(case.decode, None)
        torch.cuda.synchronize()
        case.check_decode()
        mux.set_decode_graphs(True)
        for _ in range(3):
            for o in case.o_dec:
                o.zero_()
            mux.run_round(case.decode, None)
            torch.cuda.synchronize()
            case.check_decode()
        done = False
        for _ in range(10):
            for o in case.o_dec:
                o.zero_()
            _, done = mux.run_round(case.decode, case.prefill)
            torch.cuda.synchronize()
            case.check_decode()
            if done:
                break
        assert done
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_prefill()
    finally:
        mux.close()


def _ragged_contexts(n, hi, seed):
    # every tile-edge case of a 32-key tile and a 16-key block, then random
    fixed = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128]
    rng = np.random.default_rng(seed)
    return tuple(int(c) for c in ([c for c in fixed if c <= hi] + list(rng.integers(1, hi + 1, n)))[:n])


# (q-heads, KV heads, head dim, contexts): 64 x 8 pairs take one split each;
# the smaller batches have contexts of at most 128 keys, also one split
# (q-heads, KV heads, head dim, block size, head shards, contexts); a
# 32-key tile takes two blocks at block size 16 and one block (both halves)
# above it
_LINE_CASES = [
    (32, 8, 128, 16, 1, _ragged_contexts(64, 700, 1)),
    (8, 8, 128, 16, 1, _ragged_contexts(9, 128, 2)),
    (16, 1, 128, 16, 1, _ragged_contexts(13, 128, 3)),
    (16, 2, 64, 16, 1, _ragged_contexts(13, 128, 4)),
    (4, 2, 64, 16, 1, _ragged_contexts(7, 128, 5)),
    (32, 8, 128, 32, 4, _ragged_contexts(64, 700, 6)),
    (16, 2, 64, 64, 2, _ragged_contexts(13, 128, 7)),
    (8, 8, 128, 128, 8, _ragged_contexts(9, 128, 8)),
]


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("hq,hkv,d,bs,shards,ctx", _LINE_CASES)
def test_mux_split_level_decode_matches_the_oracle(hq, hkv, d, bs, shards, ctx, append):
    print(f"split-level decode hq={hq} hkv={hkv} d={d} bs={bs} shards={shards} batch={len(ctx)} append={append}",
          flush=True)
    case = _MuxCase(layers=3, hq=hq, hkv=hkv, d=d, bs=bs, ctx=ctx, prompt=400, seed=40 + hq + d + bs, shards=shards)
    # budget 400 with a 400-token prompt: 1 layer per round, 3 rounds
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=400)
    try:
        groups = mux.groups()
        mux.set_decode_append(append)
        for i in range(3):
            mux.set_decode_graphs(i > 0)        # eager first, then the level's graph (captured, replayed)
            for o in case.o_dec:
                o.zero_()
            lvl, _ = mux.run_round(case.decode, case.prefill)
            torch.cuda.synchronize()
            pcu, dcu = groups[lvl]
            assert pcu > 0 and dcu > 0, "a split level"
            case.check_decode()
        assert case.prefill.done_submitting    # finished or not: waited for below
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_prefill()
    finally:
        mux.close()


def _random_line_case(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    bs = int(rng.choice([16, 32, 64, 128]))
    shards = int(rng.choice([s for s in (1, 2, 4, 8) if hkv % s == 0]))
    # one split per (request, KV head): 512 or more pairs, or contexts of at
    # most 128 keys
    if rng.random() < 0.5:
        batch, hi = int(-(-512 // hkv)), int(rng.integers(33, 400))
    else:
        batch, hi = int(rng.integers(1, 24)), 128
    ctx = tuple(int(c) for c in rng.integers(1, hi + 1, batch))
    return g * hkv, hkv, d, bs, shards, ctx


@pytest.mark.parametrize("seed", range(8))
def test_mux_split_level_decode_random_shapes(seed):
    hq, hkv, d, bs, shards, ctx = _random_line_case(seed)
    print(f"random split-level decode seed={seed}: hq={hq} hkv={hkv} d={d} bs={bs} shards={shards} "
          f"batch={len(ctx)} max ctx={max(ctx)}", flush=True)
    case = _MuxCase(layers=2, hq=hq, hkv=hkv, d=d, bs=bs, ctx=ctx, prompt=256, seed=500 + seed, shards=shards)
    mux = ops.Mux(0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36, token_budget=256)
    try:
        groups = mux.groups()
        mux.set_decode_append(seed % 2 == 1)
        for i in range(2):
            for o in case.o_dec:
                o.zero_()
            lvl, _ = mux.run_round(case.decode, case.prefill)
            torch.cuda.synchronize()
            assert all(x > 0 for x in groups[lvl]), "a split level"
            case.check_decode()
        mux.wait_prefill()
        torch.cuda.synchronize()
        case.check_prefill()
    finally:
        mux.close()
