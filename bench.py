"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--full]

Workloads (all synthetic, seeded, resident in HBM before timing):

* ``all`` (default): ``qwen3-32b`` (its prefill TFLOP/s is ``value``), then
  ``llama3-8b``, ``relayout-70b`` and ``pdmux``, each reported under
  ``metrics["workloads"]`` with its own value, roofline and oracle baseline.
* ``llama3-8b``: 32 layers of a Llama-3-8B-shaped attention
  (32 q-heads / 8 KV heads, head dim 128, bf16, block size 16, pool of 8192
  blocks cut into 4 head shards).  One step = the decode step of 64
  requests at context 512 (slot mapping, then per layer kv_write of the new
  token + attn_decode), the 1024-token prompt prefilled in 2 chunks of 512
  (per chunk: slot mapping, then per layer kv_write + attn_prefill_chunk),
  and the prompt's KV relayout to a block-size-32, 8-shard pool (one
  kv_relayout per layer).  ``value`` is decode-attention HBM GB/s.
* ``qwen3-32b``: 64 layers, 64/8 heads; decode of 16 requests with contexts
  uniform in [2048, 8192]; a 16384-token prompt prefilled at chunk 2048 and
  at chunk 512.  ``value`` is prefill-attention TFLOP/s.
* ``relayout-70b``: 80 layers of a 4096-token request moved from block size
  16 / 4 shards to block size 32 / 8 shards, 80 calls back to back.
  ``value`` is relayout HBM GB/s (read + write).  ``metrics`` adds the
  converting relayout of the same layers into FP8 E4M3 token-major rows and
  into a fused bf16 K/V tensor (kv_relayout_convert, timed separately), and
  the layer-wise overlap of the moves with the prompt's prefill (each
  layer's relayout released by an event as soon as that layer is computed).
* ``pdmux``: the PD-multiplexing round (see ``bench_pdmux``).  ``value`` is
  the multiplexed decode step in ms.
* ``copy-1gib``: a plain 1 GiB device copy, the known-size kernel that
  calibrates the FETCH_SIZE / WRITE_SIZE counters behind ``traffic``.
* ``mfma-peak``: the device's dense bf16 matrix-core rate (four independent
  MFMA chains per wave, two waves per SIMD) and the shader clock the waves
  ran at, measured on the box the other workloads run on.
* ``hbm-ceiling``: what HBM delivers to decode's permuted 4 KiB tile reads
  and to the relayout's permuted tile copies at those kernels' launch sizes
  (see ``bench_hbm_ceiling``).

One JSON line is printed.  Kernel times come from HIP events recorded on
the stream the kernels are launched on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_paged_kv_amd import inputs, ops, workloads  # noqa: E402

METRIC = "prefill-attn TFLOP/s, decode-attn & relayout HBM GB/s, mux decode step ms"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


# ------------------------------------------------------------- counts ----
def decode_bytes(contexts, hkv, d, hq, esize=2):
    """Algorithmic bytes of one decode launch: every K/V row once, plus q and out."""
    return int(sum(contexts)) * 2 * hkv * d * esize + 2 * len(contexts) * hq * d * esize


def prefill_flops(hq, d, t, s):
    """The pages' causal attention count for one layer and one chunk: 4*Hq*D*(T*S + T^2/2)."""
    return 4.0 * hq * d * (t * s + t * t / 2.0)


def relayout_bytes(n, hkv, d, esize=2):
    """HBM traffic of one layer's relayout: the K/V payload read once and written once."""
    return 2 * n * 2 * hkv * d * esize


# ------------------------------------------------------------ traffic ----
# HBM bytes of each roofline kernel, from two rocprofv3 --pmc runs of this
# script's own workload (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch,
# mean over the dispatches of one run), scaled by what the same counters
# read for a plain 1 GiB copy (torch copy_): FETCH_SIZE reads 0.5 GiB for
# 1 GiB fetched, WRITE_SIZE 1.0 GiB for 1 GiB written.  Each entry holds the
# SHA-256 of the sources the kernel is built from when the counters were
# taken; once they differ the figure no longer describes the kernel and
# `traffic` is reported as null.  Commands and per-kernel tables are in the
# profiles/ summaries named for each kernel and workload.
PMC_SCALE = {"fetch": 2.0, "write": 1.0}
TRAFFIC = {
    "attn_decode": {"sources": ['decode_paged_kv_amd/csrc/attn_decode.hip', 'decode_paged_kv_amd/csrc/decode_bf16.h', 'decode_paged_kv_amd/csrc/pkv_internal.h'],
                    "sha256": "d59f9903fbaf3d3ceb8d6d7f1409f324651dae4daee4c20a6b568c4fea4f6e39",
                    "fetch_kib": 65947.92, "write_kib": 512.00},
    "attn_prefill_chunk": {"sources": ['decode_paged_kv_amd/csrc/attn_prefill.hip', 'decode_paged_kv_amd/csrc/prefill_bf16.h', 'decode_paged_kv_amd/csrc/pkv_internal.h'],
                           "sha256": "f1c506b4032bde6f62eabd80daefa7ee583efb0b26015f98ebfe9a76b1e41535",
                           "fetch_kib": 28005.17, "write_kib": 15974.16},
    "kv_relayout": {"sources": ['decode_paged_kv_amd/csrc/kv_ops.hip', 'decode_paged_kv_amd/csrc/pkv_internal.h'],
                    "sha256": "2af290f6b8645156babeeffc1daaf7f7995952fecb4c047393f841a8662d15ff",
                    "fetch_kib": 8233.68, "write_kib": 16391.06},
    "attn_decode_line": {"sources": ['decode_paged_kv_amd/csrc/attn_decode.hip', 'decode_paged_kv_amd/csrc/decode_line.h', 'decode_paged_kv_amd/csrc/decode_bf16.h', 'decode_paged_kv_amd/csrc/pkv_internal.h'],
                         "sha256": "b7a4c9dad65532bbe3349a13279d35cef7b828d934c263785b782dbc108e233d",
                         "fetch_kib": 525630.24, "write_kib": 1024.00},
}


def traffic_bytes(kernel):
    """Measured HBM bytes per launch of `kernel`, or None if its sources changed since the counters were taken."""
    e = TRAFFIC.get(kernel)
    if e is None:
        return None
    h = hashlib.sha256()
    for f in e["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != e["sha256"]:
        return None
    return int(round(1024 * (e["fetch_kib"] * PMC_SCALE["fetch"] + e["write_kib"] * PMC_SCALE["write"])))


# ------------------------------------------------------------- helpers ----
class PhaseGraphs:
    """HIP graphs of the step's phases, captured once and replayed.

    The library launches every kernel on the stream it is given; under
    capture those launches become graph nodes, so a replay runs them back
    to back with no host work between kernels.  Durations come from HIP
    events recorded around each replay on the replaying stream.
    """

    def __init__(self, stream):
        self.stream = stream
        self.graphs = {}

    def capture(self, name, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            fn()                                  # eager run first (warms up code objects)
        self.stream.synchronize()
        with torch.cuda.graph(g, stream=self.stream):
            fn()
        self.graphs[name] = g

    def replay(self, name):
        with torch.cuda.stream(self.stream):
            self.graphs[name].replay()


def time_replays(pg: PhaseGraphs, names, steps, warmup):
    """Mean ms of each named graph over `steps` timed rounds (all replayed in order each round)."""
    for _ in range(warmup):
        for n in names:
            pg.replay(n)
    torch.cuda.synchronize()
    ev = {n: [] for n in names}
    for _ in range(steps):
        for n in names:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(pg.stream)
            pg.replay(n)
            b.record(pg.stream)
            ev[n].append((a, b))
    torch.cuda.synchronize()
    return {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}


def rand_bf16(shape, gen, scale=0.5):
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


def fill_pool_random(pool, gen, scale=0.5):
    for t in pool.k + pool.v:
        t.copy_(rand_bf16(t.shape, gen, scale))


def make_tables(w, counts_tokens, block_size, pool_blocks, tid=inputs.T_PERM):
    g = inputs.stream(w.seed, w.config_id, 0, tid)
    tables, _ = inputs.assign_blocks(pool_blocks, counts_tokens, block_size, g)
    return tables


def cores_used():
    try:
        from threadpoolctl import threadpool_info
        n = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        return int(n)
    except Exception:
        return len(os.sched_getaffinity(0))


# --------------------------------------------------------- llama3-8b ----
def bench_llama3_8b(args):
    w = workloads.LLAMA3_8B
    L, hq, hkv, d, bs = w.layers, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    B, ctx, N, chunk = w.decode_batch, w.decode_context[0], w.prompt_len, w.chunk_sizes[0]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    stream = torch.cuda.Stream()
    # block tables: decode requests then the prompt, from one shuffled pool
    tables = make_tables(w, [ctx] * B + [N], bs, w.pool_blocks)
    dec_bt, pr_bt = i32(tables[:B]), i32(tables[B:B + 1])
    dst_bt = i32(make_tables(w, [N], w.dst_block_size, w.dst_pool_blocks, inputs.T_DST_PERM))
    pools = [ops.PagedPool(w.pool_blocks, bs, hkv, w.src_shards, d, "bf16") for _ in range(L)]
    dsts = [ops.PagedPool(w.dst_pool_blocks, w.dst_block_size, hkv, w.dst_shards, d, "bf16") for _ in range(L)]
    for p in pools:
        fill_pool_random(p, gen)
    q_dec = [rand_bf16((B, hq, d), gen) for _ in range(L)]
    kn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    vn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    o_dec = [torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    q_pr = [rand_bf16((N, hq, d), gen) for _ in range(L)]
    k_pr = [rand_bf16((N, hkv, d), gen) for _ in range(L)]
    v_pr = [rand_bf16((N, hkv, d), gen) for _ in range(L)]
    o_pr = [torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ctx_t = i32([ctx] * B)
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size(B, hq, ctx, d)), dtype=torch.uint8, device="cuda")
    dec_start, dec_pos = i32(np.arange(B + 1)), i32([ctx - 1] * B)
    dec_slots = torch.empty(B, dtype=torch.int32, device="cuda")
    chunks = [(s, min(chunk, N - s)) for s in range(0, N, chunk)]
    ch_args = [(i32([0, t]), i32([s]), torch.empty(t, dtype=torch.int32, device="cuda")) for s, t in chunks]
    sh = stream.cuda_stream

    def decode_attn():
        for l in range(L):
            ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws, stream=sh)

    def decode_step():
        ops.slot_mapping(dec_bt, dec_start, dec_pos, B, bs, w.pool_blocks, out=dec_slots, stream=sh)
        for l in range(L):
            ops.kv_write(pools[l], kn[l], vn[l], dec_slots, stream=sh)
            ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws, stream=sh)

    def decode_step_append():
        # the same step with each layer's write and attention in one attn_decode_append launch
        for l in range(L):
            ops.attn_decode_append(pools[l], q_dec[l], kn[l], vn[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws,
                                   stream=sh)

    def prefill_attn():
        for (s, t), (sl, cs, _) in zip(chunks, ch_args):
            for l in range(L):
                ops.attn_prefill_chunk(pools[l], q_pr[l][s:s + t], o_pr[l][s:s + t], pr_bt, sl, cs, t, hq, stream=sh,
                                       max_total_len=N)

    def prefill():
        for (s, t), (sl, cs, slots) in zip(chunks, ch_args):
            ops.slot_mapping(pr_bt, sl, cs, t, bs, w.pool_blocks, out=slots, stream=sh)
            for l in range(L):
                ops.kv_write(pools[l], k_pr[l][s:s + t], v_pr[l][s:s + t], slots, stream=sh)
                ops.attn_prefill_chunk(pools[l], q_pr[l][s:s + t], o_pr[l][s:s + t], pr_bt, sl, cs, t, hq, stream=sh,
                                       max_total_len=N)

    def relayout():
        for l in range(L):
            ops.kv_relayout(pools[l], pr_bt, dsts[l], dst_bt, N, stream=sh)

    def step():
        decode_step()
        prefill()
        relayout()

    pg = PhaseGraphs(stream)
    for name, fn in (("step", step), ("decode_attn", decode_attn), ("prefill_attn", prefill_attn),
                     ("relayout", relayout), ("decode_step", decode_step), ("decode_step_append", decode_step_append)):
        pg.capture(name, fn)
    t_step = time_replays(pg, ["step"], args.steps, args.warmup)["step"]
    t = time_replays(pg, ["decode_attn", "prefill_attn", "relayout", "decode_step", "decode_step_append"], args.steps,
                     args.warmup)

    dec_launch_ms = t["decode_attn"] / L
    dbytes = decode_bytes([ctx] * B, hkv, d, hq)
    dec_gbps = dbytes / (dec_launch_ms * 1e-3) / 1e9
    pf_flops = L * sum(prefill_flops(hq, d, tt, s) for s, tt in chunks)
    pf_tflops = pf_flops / (t["prefill_attn"] * 1e-3) / 1e12
    rl_ms = t["relayout"] / L
    rl_gbps = relayout_bytes(N, hkv, d) / (rl_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-attn: 32 layers, 32/8 heads, d128, bs16; decode 64x512 + prompt 1024 "
                               "in 2 chunks of 512 + relayout 1024 tokens bs16/4 shards -> bs32/8 shards",
                   "layers": L, "decode_batch": B, "decode_context": ctx, "prompt": N, "chunk": chunk,
                   "timing": "each phase captured once as a HIP graph and replayed; HIP events around replays",
                   "value_is": "attn_decode HBM GB/s (algorithmic K/V + q/out bytes per launch / mean launch time "
                               "over 32 back-to-back launches)"},
        "roofline": {"kernel": "attn_decode", "bound": "hbm", "achieved": round(dec_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_bytes("attn_decode"), "bytes_per_launch": dbytes,
                     "launch_ms": round(dec_launch_ms, 5)},
        "metrics": {
            "decode_attn_gbps": round(dec_gbps, 1),
            "decode_step_ms": round(t["decode_step"], 4),
            "decode_step_append_ms": round(t["decode_step_append"], 4),
            "prefill_attn_tflops": round(pf_tflops, 2),
            "prefill_attn_frac_bf16_peak": round(pf_tflops / BF16_PEAK_TFLOPS, 4),
            "prefill_attn_ms_per_layer": round(t["prefill_attn"] / L, 5),
            "relayout_gbps": round(rl_gbps, 1),
            "relayout_layer_ms": round(rl_ms, 5),
        },
    }
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(w, seconds=args.cpu_seconds)
    return result


def cpu_baseline_decode(w, nreq=16, seconds=10.0):
    """The oracle's decode on a bounded sample of the same workload, timed on the host."""
    from oracle import attention as oa
    hq, hkv, d, ctx = w.num_q_heads, w.num_kv_heads, w.head_dim, w.decode_context[0]
    g = lambda t, i: inputs.stream(w.seed, w.config_id, 0, t, i)  # noqa: E731
    ks = [inputs.as_float(inputs.normal((ctx, hkv, d), 0.5, "bf16", g(inputs.T_K, r)), "bf16") for r in range(nreq)]
    vs = [inputs.as_float(inputs.normal((ctx, hkv, d), 0.5, "bf16", g(inputs.T_V, r)), "bf16") for r in range(nreq)]
    q = inputs.as_float(inputs.normal((nreq, hq, d), 0.5, "bf16", g(inputs.T_Q, 0)), "bf16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oa.decode_batch(q, ks, vs)
        reps += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = decode_bytes([ctx] * nreq, hkv, d, hq) * reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores_used(), "kind": "oracle",
            "sample": f"oracle decode of {nreq} requests x {ctx} keys x {hq}/{hkv} heads (one layer of the same "
                      f"workload), repeated {reps} times in {dt:.1f} s; bf16 K/V/q/out bytes / wall time"}


# --------------------------------------------------------- qwen3-32b ----
def bench_qwen3_32b(args):
    w = workloads.QWEN3_32B
    L, hq, hkv, d, bs = w.layers, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    ctxs = [int(x) for x in w.decode_contexts()]
    B, N = len(ctxs), w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    tables = make_tables(w, ctxs + [N], bs, w.pool_blocks)
    dec_bt, pr_bt = i32(tables[:B]), i32(tables[B:B + 1])
    pools = [ops.PagedPool(w.pool_blocks, bs, hkv, 1, d, "bf16") for _ in range(L)]
    for p in pools:
        fill_pool_random(p, gen)
    maxc = max(ctxs)
    q_dec = [rand_bf16((B, hq, d), gen) for _ in range(L)]
    kn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    vn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    o_dec = [torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    q_pr = [rand_bf16((N, hq, d), gen) for _ in range(L)]
    k_pr = [rand_bf16((N, hkv, d), gen) for _ in range(L)]
    v_pr = [rand_bf16((N, hkv, d), gen) for _ in range(L)]
    o_pr = [torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ctx_t = i32(ctxs)
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size(B, hq, maxc, d)), dtype=torch.uint8, device="cuda")
    dec_start, dec_pos = i32(np.arange(B + 1)), i32([c - 1 for c in ctxs])
    dec_slots = torch.empty(B, dtype=torch.int32, device="cuda")
    plans = {}
    for c in w.chunk_sizes:
        chunks = [(s, min(c, N - s)) for s in range(0, N, c)]
        plans[c] = [(s, t, i32([0, t]), i32([s]), torch.empty(t, dtype=torch.int32, device="cuda")) for s, t in chunks]

    def decode_attn():
        for l in range(L):
            ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, maxc, hq, workspace=ws, stream=sh)

    def decode_step():
        ops.slot_mapping(dec_bt, dec_start, dec_pos, B, bs, w.pool_blocks, out=dec_slots, stream=sh)
        for l in range(L):
            ops.kv_write(pools[l], kn[l], vn[l], dec_slots, stream=sh)
            ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, maxc, hq, workspace=ws, stream=sh)

    def prefill(c, with_write=True):
        def run():
            for s, t, sl, cs, slots in plans[c]:
                if with_write:
                    ops.slot_mapping(pr_bt, sl, cs, t, bs, w.pool_blocks, out=slots, stream=sh)
                for l in range(L):
                    if with_write:
                        ops.kv_write(pools[l], k_pr[l][s:s + t], v_pr[l][s:s + t], slots, stream=sh)
                    ops.attn_prefill_chunk(pools[l], q_pr[l][s:s + t], o_pr[l][s:s + t], pr_bt, sl, cs, t, hq,
                                           stream=sh, max_total_len=N)
        return run

    pg = PhaseGraphs(stream)
    pg.capture("decode_step", decode_step)
    pg.capture("decode_attn", decode_attn)
    for c in plans:
        pg.capture(f"prefill_c{c}", prefill(c))          # writes the prompt's K/V too
    for c in plans:
        pg.capture(f"prefill_attn_c{c}", prefill(c, with_write=False))
    names = ["decode_step"] + [f"prefill_c{c}" for c in plans]
    t_step = time_replays(pg, names, args.steps, args.warmup)
    step_ms = sum(t_step.values())
    t = time_replays(pg, ["decode_attn"] + [f"prefill_attn_c{c}" for c in plans], args.steps, args.warmup)
    dec_ms = t["decode_attn"] / L
    dbytes = decode_bytes(ctxs, hkv, d, hq)
    dec_gbps = dbytes / (dec_ms * 1e-3) / 1e9
    per = {}
    tot_flops = tot_ms = 0.0
    for c, plan in plans.items():
        fl = L * sum(prefill_flops(hq, d, tt, s) for s, tt, *_ in plan)
        ms = t[f"prefill_attn_c{c}"]
        per[c] = (fl, ms)
        tot_flops += fl
        tot_ms += ms
    tflops = tot_flops / (tot_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-32b-attn: 64 layers, 64/8 heads, d128, bs16; decode 16 x U[2048,8192]; "
                               "prompt 16384 prefilled at chunk 2048 and at chunk 512 (slot mapping + kv_write + "
                               "attn_prefill_chunk per chunk and layer)",
                   "decode_contexts": ctxs, "prompt": N, "chunks": list(w.chunk_sizes),
                   "timing": "each phase captured once as a HIP graph and replayed; HIP events around replays",
                   "value_is": "attn_prefill_chunk TFLOP/s over both chunkings (pages' flop count / time of the "
                               "back-to-back prefill launches)"},
        "roofline": {"kernel": "attn_prefill_chunk", "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_bytes("attn_prefill_chunk"), "flops_per_step": tot_flops,
                     "launch_ms": round(tot_ms / sum(L * len(p) for p in plans.values()), 5)},
        "metrics": {
            "decode_attn_gbps": round(dec_gbps, 1), "decode_attn_frac_hbm": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "decode_launch_ms": round(dec_ms, 5), "decode_step_ms": round(t_step["decode_step"], 3),
            **{f"prefill_c{c}_tflops": round(fl / (ms * 1e-3) / 1e12, 2) for c, (fl, ms) in per.items()},
            **{f"prefill_c{c}_attn_ms": round(ms, 3) for c, (fl, ms) in per.items()},
            **{f"prefill_c{c}_with_writes_ms": round(t_step[f"prefill_c{c}"], 3) for c in plans},
        },
    }
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(w, seconds=max(args.cpu_seconds, 10.0))
    return result


def bench_stall_free_qwen(args):
    """One stall-free step of the Qwen3-32B-like batch (G = 8): the 16 decodes and what they leave of a
    2048-token budget for the 16K prompt at position 8192, every layer's attention as one attn_mixed_batch
    launch against attn_decode + attn_prefill_chunk.  16 layers (own pools), per-layer times."""
    w = workloads.QWEN3_32B
    L, hq, hkv, d, bs = 16, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    ctxs = [int(x) for x in w.decode_contexts()]
    B, N = len(ctxs), w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    tables = make_tables(w, ctxs + [N], bs, w.pool_blocks)
    dec_bt, pr_bt = i32(tables[:B]), i32(tables[B:B + 1])
    pools = [ops.PagedPool(w.pool_blocks, bs, hkv, 1, d, "bf16") for _ in range(L)]
    for p in pools:
        fill_pool_random(p, gen)
    maxc = max(ctxs)
    s0 = N // 2
    t = ops.stall_free_chunk(2048, B, N - s0)
    q_dec = [rand_bf16((B, hq, d), gen) for _ in range(L)]
    o_dec = [torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    q_pr = [rand_bf16((t, hq, d), gen) for _ in range(L)]
    o_pr = [torch.empty((t, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ctx_t, sl, cs = i32(ctxs), i32([0, t]), i32([s0])
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size(B, hq, maxc, d)), dtype=torch.uint8, device="cuda")

    def step(fused):
        def run():
            for l in range(L):
                if fused:
                    ops.attn_mixed_batch(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, maxc, q_pr[l], o_pr[l], pr_bt,
                                         sl, cs, t, hq, workspace=ws, stream=sh, max_total_len=N)
                else:
                    ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, maxc, hq, workspace=ws, stream=sh)
                    ops.attn_prefill_chunk(pools[l], q_pr[l], o_pr[l], pr_bt, sl, cs, t, hq, stream=sh,
                                           max_total_len=N)
        return run

    pg = PhaseGraphs(stream)
    pg.capture("fused", step(True))
    pg.capture("two_launches", step(False))
    tm = time_replays(pg, ["fused", "two_launches"], args.steps, args.warmup)
    fused, two = tm["fused"] / L, tm["two_launches"] / L
    return {"metric": "stall-free step attention, ms per layer", "value": round(fused, 4), "unit": "ms",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tm["fused"], 3),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"stall-free step, Qwen3-32B-like heads (64/8, d128, bs16): decode 16 x "
                                   f"U[2048,8192] + a {t}-token chunk of the 16K prompt at {s0} (budget 2048); "
                                   f"{L} layers, own pools"},
            "metrics": {"fused_ms_per_layer": round(fused, 4), "two_launches_ms_per_layer": round(two, 4),
                        "fused_over_two_launches": round(fused / two, 4), "chunk": t, "chunk_start": s0}}


def cpu_baseline_prefill(w, seconds=10.0):
    from oracle import attention as oa
    hq, hkv, d, N = w.num_q_heads, w.num_kv_heads, w.head_dim, w.prompt_len
    t, s = 512, N - 512
    g = lambda tid: inputs.stream(w.seed, w.config_id, 0, tid)  # noqa: E731
    k = inputs.as_float(inputs.normal((N, hkv, d), 0.5, "bf16", g(inputs.T_K)), "bf16")
    v = inputs.as_float(inputs.normal((N, hkv, d), 0.5, "bf16", g(inputs.T_V)), "bf16")
    q = inputs.as_float(inputs.normal((t, hq, d), 0.5, "bf16", g(inputs.T_Q)), "bf16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oa.prefill_chunk(q, k, v, s)
        reps += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    fl = prefill_flops(hq, d, t, s) * reps
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores_used(), "kind": "oracle",
            "sample": f"oracle prefill of the last 512-token chunk (S={s}) of one layer, {hq}/{hkv} heads, repeated "
                      f"{reps} times in {dt:.1f} s; pages' flop count / wall time"}


# ------------------------------------------------------ relayout-70b ----
def bench_relayout_70b(args):
    w = workloads.RELAYOUT_70B
    L, hkv, d, N = w.layers, w.num_kv_heads, w.head_dim, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    src_bt = i32(make_tables(w, [N], w.block_size, w.pool_blocks))
    dst_bt = i32(make_tables(w, [N], w.dst_block_size, w.dst_pool_blocks, inputs.T_DST_PERM))
    srcs = [ops.PagedPool(w.pool_blocks, w.block_size, hkv, w.src_shards, d, "bf16") for _ in range(L)]
    dsts = [ops.PagedPool(w.dst_pool_blocks, w.dst_block_size, hkv, w.dst_shards, d, "bf16") for _ in range(L)]
    for p in srcs:
        fill_pool_random(p, gen)

    def relayout_all():
        for l in range(L):
            ops.kv_relayout(srcs[l], src_bt, dsts[l], dst_bt, N, stream=sh)

    pg = PhaseGraphs(stream)
    pg.capture("relayout", relayout_all)
    # the converting variant ([DISAGG] "布局转换"): into FP8 slot-major rows, and into a fused bf16 K/V tensor
    conv = {"fp8_token_major": ("fp8", "token_major"), "bf16_kv_fused": ("bf16", "kv_fused")}
    for name, (ddt, lay) in conv.items():
        cdst = [ops.ConvertedPool(w.dst_pool_blocks, w.dst_block_size, hkv, w.dst_shards, d, ddt, lay, 0.02)
                for _ in range(L)]

        def convert_all(cdst=cdst):
            for l in range(L):
                ops.kv_relayout_convert(srcs[l], src_bt, cdst[l], dst_bt, N, stream=sh)
        pg.capture(name, convert_all)
    step_ms = time_replays(pg, ["relayout"], args.steps, args.warmup)["relayout"]
    t = time_replays(pg, list(conv), args.steps, args.warmup)
    per_layer = relayout_bytes(N, hkv, d)
    conv_metrics = {}
    for name, (ddt, _) in conv.items():
        nbytes = per_layer // 2 * (1 + (0.5 if ddt == "fp8" else 1))   # bf16 read + destination write
        ms = t[name] / L
        conv_metrics[f"convert_{name}_gbps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        conv_metrics[f"convert_{name}_launch_ms"] = round(ms, 5)
    launch_ms = step_ms / L
    gbps = per_layer / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "relayout-llama3-70b: 80 layers x one 4096-token request, 8 kv heads, d128; "
                               "bs16 / 4 shards x 2 heads -> bs32 / 8 shards x 1 head; 80 kv_relayout calls back to "
                               "back", "payload_bytes": per_layer // 2 * L,
                   "timing": "the 80 calls captured once as a HIP graph and replayed; HIP events around replays",
                   "value_is": "relayout HBM GB/s = 2 x payload / time of the 80 back-to-back calls"},
        "roofline": {"kernel": "kv_relayout", "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_bytes("kv_relayout"), "bytes_per_launch": per_layer,
                     "launch_ms": round(launch_ms, 5)},
        "metrics": {"relayout_gbps": round(gbps, 1), "relayout_frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                    "relayout_launch_ms": round(launch_ms, 5), **conv_metrics},
    }
    result["metrics"]["layerwise_overlap"] = layerwise_overlap(w, srcs, dsts, src_bt, dst_bt, args.steps, args.warmup)
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_relayout(w, seconds=args.cpu_seconds)
    return result


def layerwise_overlap(w, srcs, dsts, src_bt, dst_bt, steps, warmup):
    """[DISAGG] "流程": a layer's KV moves as soon as that layer is computed.  The prompt's prefill (per layer:
    kv_write of its 4096 tokens + attn_prefill_chunk from position 0) runs on a compute stream; after each layer
    an event releases that layer's kv_relayout on a second stream, so the move overlaps the next layers'
    prefill.  Compared with the prefill alone and with prefill + relayout in one stream."""
    L, hq, hkv, d, N = w.layers, w.num_q_heads, w.num_kv_heads, w.head_dim, w.prompt_len
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 1)
    q = rand_bf16((N, hq, d), gen)
    out = torch.empty_like(q)
    k, v = rand_bf16((N, hkv, d), gen), rand_bf16((N, hkv, d), gen)
    start, pos0 = i32([0, N]), i32([0])
    slots = ops.slot_mapping(src_bt, start, pos0, N, w.block_size, w.pool_blocks)
    torch.cuda.synchronize()
    comp, xfer = torch.cuda.Stream(), torch.cuda.Stream()
    cs, xs = comp.cuda_stream, xfer.cuda_stream

    def prefill_layer(l):
        ops.kv_write(srcs[l], k, v, slots, stream=cs)
        ops.attn_prefill_chunk(srcs[l], q, out, src_bt, start, pos0, N, hq, stream=cs)

    def run(mode):
        for l in range(L):
            prefill_layer(l)
            if mode == "serial":
                ops.kv_relayout(srcs[l], src_bt, dsts[l], dst_bt, N, stream=cs)
            elif mode == "overlap":
                ev = torch.cuda.Event()
                ev.record(comp)
                xfer.wait_event(ev)
                ops.kv_relayout(srcs[l], src_bt, dsts[l], dst_bt, N, stream=xs)
        comp.wait_stream(xfer)

    def timed(mode):
        for _ in range(warmup):
            run(mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        for _ in range(steps):
            run(mode)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t = {m: timed(m) for m in ("prefill", "serial", "overlap")}
    added_serial = t["serial"] - t["prefill"]
    return {"prefill_ms": round(t["prefill"], 3), "prefill_then_relayout_ms": round(t["serial"], 3),
            "overlapped_ms": round(t["overlap"], 3),
            "relayout_hidden_frac": round((t["serial"] - t["overlap"]) / added_serial, 3) if added_serial > 0 else None}


def cpu_baseline_relayout(w, seconds=10.0):
    from oracle import pool as opool
    hkv, d, N = w.num_kv_heads, w.head_dim, w.prompt_len
    g = lambda tid: inputs.stream(w.seed, w.config_id, 0, tid)  # noqa: E731
    src_bt, _ = inputs.assign_blocks(w.pool_blocks, [N], w.block_size, g(inputs.T_PERM))
    dst_bt, _ = inputs.assign_blocks(w.dst_pool_blocks, [N], w.dst_block_size, g(inputs.T_DST_PERM))
    src = opool.PoolModel(w.pool_blocks, w.block_size, hkv, w.src_shards, d, np.uint16)
    for a in src.k + src.v:
        a[...] = inputs.normal(a.shape, 0.5, "bf16", g(inputs.T_K))
    t0 = time.perf_counter()
    reps = 0
    while True:
        dst = opool.PoolModel(w.dst_pool_blocks, w.dst_block_size, hkv, w.dst_shards, d, np.uint16)
        opool.relayout(src, src_bt[0], dst, dst_bt[0], N)
        reps += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(relayout_bytes(N, hkv, d) * reps / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"oracle naive relayout of one layer (4096 tokens x 8 heads), repeated {reps} "
                                         f"times in {dt:.1f} s; 2 x payload / wall time"}


# ------------------------------------------------------------- pdmux ----
def bench_pdmux(args):
    """PD multiplexing on one GPU, Llama-3-8B attention shape, 32 layers, bf16, block size 16.

    Decode batch 128 at context 2048 (slot of the new token rewritten each
    step, so every step does the same work).  Arms:
      A  solo decode: rounds with no prefill (whole device);
      B  multiplexed: rounds of decode on the CU-masked decode stream while a
         prompt (32768 tokens, 2 layers per round, and a 16384-token variant,
         4 layers per round) is prefilled layer by layer on the complementary
         CUs; the level comes from the batch-size rule (128 : 128 CUs), and a
         sweep fixes each level 1..6 for the 16K prompt;
      C  chunked prefill on the whole device: each step runs the decode step
         and then one chunk (2048 or 512 tokens) through all layers, on one
         stream;
      D  prefill alone on the whole device (one stream);
      A, B with the decode step captured as one HIP graph per level and
         replayed (metrics "decode_graphs"), and with each decode layer as
         one attn_decode_append launch (metrics "decode_append");
      E  stall-free batches on the whole device: each step takes every decode
         request and the prompt's share of a token budget (2048 and 512, the
         pages' loose and strict settings), per layer one attn_mixed_batch
         launch, and for comparison the same chunks as attn_decode then
         attn_prefill_chunk.
    A decode step's time is the host wall time of one round, which blocks on
    the decode stream (the inter-token interval a serving loop would see).
    """
    w = workloads.PDMUX_8B
    L, hq, hkv, d, bs = w.layers, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    B, ctx = w.decode_batch, w.decode_context[0]
    prompts = {"32k": w.prompt_len, "16k": w.extra["prompt_variant"]}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    tables = make_tables(w, [ctx] * B + [w.prompt_len], bs, w.pool_blocks)
    dec_bt, pr_bt = i32(tables[:B]), i32(tables[B:B + 1])
    pools = [ops.PagedPool(w.pool_blocks, bs, hkv, 1, d, "bf16") for _ in range(L)]
    for p in pools:
        fill_pool_random(p, gen)
    q_dec = [rand_bf16((B, hq, d), gen) for _ in range(L)]
    kn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    vn = [rand_bf16((B, hkv, d), gen) for _ in range(L)]
    o_dec = [torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    Nmax = w.prompt_len
    q_pr = [rand_bf16((Nmax, hq, d), gen) for _ in range(L)]
    k_pr = [rand_bf16((Nmax, hkv, d), gen) for _ in range(L)]
    v_pr = [rand_bf16((Nmax, hkv, d), gen) for _ in range(L)]
    o_pr = [torch.empty((Nmax, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ctx_t = i32([ctx] * B)
    ws = torch.zeros(max(16, ops.attn_decode_workspace_size(B, hq, ctx, d)), dtype=torch.uint8, device="cuda")
    dec_slots = ops.slot_mapping(dec_bt, i32(np.arange(B + 1)), i32([ctx - 1] * B), B, bs, w.pool_blocks)
    decode = ops.DecodeStepArgs(pools, q_dec, kn, vn, o_dec, dec_slots, dec_bt, ctx_t, ctx, hq, ws)
    pr_slots = {k: ops.slot_mapping(pr_bt, i32([0, n]), i32([0]), n, bs, w.pool_blocks) for k, n in prompts.items()}
    torch.cuda.synchronize()
    mux = ops.Mux(0, w.extra["cu_granularity"], w.extra["min_decode_cus"], w.extra["group_num"],
                  w.extra["decode_bs_divisor"], w.extra["token_budget"])
    groups = mux.groups()

    def job(key):
        n = prompts[key]
        return ops.PrefillJobArgs(pools, [t[:n] for t in q_pr], [t[:n] for t in k_pr], [t[:n] for t in v_pr],
                                  [t[:n] for t in o_pr], pr_slots[key], pr_bt, i32([0, n]), i32([0]), n, hq)

    def solo(rounds):
        ts = []
        for _ in range(rounds):
            t0 = time.perf_counter()
            mux.run_round(decode, None)
            ts.append((time.perf_counter() - t0) * 1e3)
        return ts

    def muxed(key, level=-1):
        mux.set_level_override(level)
        j = job(key)
        ts, levels = [], []
        t_start = time.perf_counter()
        done = False
        while not done:
            t0 = time.perf_counter()
            lvl, done = mux.run_round(decode, j)
            ts.append((time.perf_counter() - t0) * 1e3)
            levels.append(lvl)
            if len(ts) > 5000:
                raise RuntimeError("prefill did not finish")
        mux.wait_prefill()
        t_pf = (time.perf_counter() - t_start) * 1e3
        mux.run_round(decode, None)           # the level returns to decode-only
        mux.set_level_override(-1)
        return ts, t_pf, sorted(set(levels))

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def chunked(key, c):
        n = prompts[key]
        chunks = [(s0, min(c, n - s0)) for s0 in range(0, n, c)]
        args_ = [(i32([0, t]), i32([s0]), ops.slot_mapping(pr_bt, i32([0, t]), i32([s0]), t, bs, w.pool_blocks))
                 for s0, t in chunks]
        torch.cuda.synchronize()
        ts = []
        t_start = time.perf_counter()
        for (s0, t), (sl, cs, slots) in zip(chunks, args_):
            t0 = time.perf_counter()
            for l in range(L):
                ops.kv_write(pools[l], kn[l], vn[l], dec_slots, stream=sh)
                ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws, stream=sh)
            for l in range(L):
                ops.kv_write(pools[l], k_pr[l][s0:s0 + t], v_pr[l][s0:s0 + t], slots, stream=sh)
                ops.attn_prefill_chunk(pools[l], q_pr[l][s0:s0 + t], o_pr[l][s0:s0 + t], pr_bt, sl, cs, t, hq,
                                       stream=sh)
            stream.synchronize()
            ts.append((time.perf_counter() - t0) * 1e3)
        return ts, (time.perf_counter() - t_start) * 1e3

    def stall_free(key, budget, fused=True):
        """Stall-free steps: every decode request plus the prompt's share of the token budget, per layer one
        attn_mixed_batch launch (fused) or attn_decode then attn_prefill_chunk (same chunks, two launches)."""
        n = prompts[key]
        steps, s0 = [], 0
        while s0 < n:
            t = ops.stall_free_chunk(budget, B, n - s0)
            if t <= 0:
                raise RuntimeError("the decode requests fill the whole token budget")
            steps.append((s0, t))
            s0 += t
        args_ = [(i32([0, t]), i32([s0]), ops.slot_mapping(pr_bt, i32([0, t]), i32([s0]), t, bs, w.pool_blocks))
                 for s0, t in steps]
        torch.cuda.synchronize()
        ts = []
        t_start = time.perf_counter()
        for (s0, t), (sl, cs, slots) in zip(steps, args_):
            t0 = time.perf_counter()
            for l in range(L):
                ops.kv_write(pools[l], kn[l], vn[l], dec_slots, stream=sh)
                ops.kv_write(pools[l], k_pr[l][s0:s0 + t], v_pr[l][s0:s0 + t], slots, stream=sh)
                if fused:
                    ops.attn_mixed_batch(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, q_pr[l][s0:s0 + t],
                                         o_pr[l][s0:s0 + t], pr_bt, sl, cs, t, hq, workspace=ws, stream=sh)
                else:
                    ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws, stream=sh)
                    ops.attn_prefill_chunk(pools[l], q_pr[l][s0:s0 + t], o_pr[l][s0:s0 + t], pr_bt, sl, cs, t, hq,
                                           stream=sh)
            stream.synchronize()
            ts.append((time.perf_counter() - t0) * 1e3)
        return ts, (time.perf_counter() - t_start) * 1e3

    def prefill_alone(key):
        n = prompts[key]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            ops.kv_write(pools[l], k_pr[l][:n], v_pr[l][:n], pr_slots[key], stream=sh)
            ops.attn_prefill_chunk(pools[l], q_pr[l][:n], o_pr[l][:n], pr_bt, i32([0, n]), i32([0]), n, hq, stream=sh)
        stream.synchronize()
        return (time.perf_counter() - t0) * 1e3

    def stats(ts):
        a = np.array(ts)
        return {"median_ms": round(float(np.median(a)), 3), "p99_ms": round(float(np.percentile(a, 99)), 3),
                "max_ms": round(float(a.max()), 3), "n": int(a.size)}

    def muxed_reps(key, min_rounds=30):
        """Multiplexed runs of the prompt back to back until at least min_rounds decode steps are timed."""
        ts, pfs, lv = [], [], set()
        while len(ts) < min_rounds:
            t, pf, levels = muxed(key)
            ts += t
            pfs.append(pf)
            lv |= set(levels)
        return ts, float(np.median(pfs)), sorted(lv)

    # warm-up: code objects, the whole-device stream, and the CU-masked
    # streams of the level the rule picks (created by one untimed
    # multiplexed run, so no timed round pays for their creation)
    solo(max(2, args.warmup))
    prefill_alone("16k")
    muxed("16k")
    A = solo(max(30, args.steps))
    B16, pf16, lv16 = muxed_reps("16k")
    B32, pf32, lv32 = muxed_reps("32k")
    extra = {}
    if args.full:
        # the same with the decode step as a per-level HIP graph
        mux.set_decode_graphs(True)
        Ag = solo(max(30, args.steps))
        B16g, pf16g, _ = muxed_reps("16k")
        mux.set_decode_graphs(False)
        # the same with each decode layer as one attn_decode_append (write + attention)
        mux.set_decode_append(True)
        Aa = solo(max(30, args.steps))
        B16a, pf16a, _ = muxed_reps("16k")
        mux.set_decode_append(False)
        sweep = {}
        for lvl in range(1, len(groups) - 1):
            ts, pf, _ = muxed("16k", lvl)
            sweep[f"{groups[lvl][0]}:{groups[lvl][1]}"] = {"decode_median_ms": round(float(np.median(ts)), 3),
                                                            "prefill_ms": round(pf, 2)}
        extra = {"decode_graphs": {"solo_decode": stats(Ag), "mux_16k_decode": stats(B16g),
                                   "mux_16k_prefill_ms": round(pf16g, 2),
                                   "mux_over_solo_16k": round(float(np.median(B16g)) / float(np.median(Ag)), 3)},
                 "decode_append": {"solo_decode": stats(Aa), "mux_16k_decode": stats(B16a),
                                   "mux_16k_prefill_ms": round(pf16a, 2),
                                   "mux_over_solo_16k": round(float(np.median(B16a)) / float(np.median(Aa)), 3)},
                 "level_sweep_16k": sweep}
    C = {}
    for key in ("16k", "32k"):
        for c in w.chunk_sizes:
            ts, tot = chunked(key, c)
            C[f"{key}_c{c}"] = {**stats(ts), "prefill_ms": round(tot, 2)}
    E = {}
    for key in ("16k", "32k"):
        for budget in w.extra["stall_free_budgets"]:
            for fused in ((True, False) if args.full else (True,)):
                ts, tot = stall_free(key, budget, fused)
                E[f"{key}_b{budget}_{'fused' if fused else 'two_launches'}"] = {
                    **stats(ts), "chunk": ops.stall_free_chunk(budget, B, prompts[key]), "prefill_ms": round(tot, 2)}
    D = {key: round(prefill_alone(key), 2) for key in prompts}
    mux.close()
    solo_med = float(np.median(A))
    mux_med = float(np.median(B16))
    dstep_bytes = decode_bytes([ctx] * B, hkv, d, hq) * L
    line_traffic = traffic_bytes("attn_decode_line")
    result = {
        "metric": METRIC, "value": round(mux_med, 3), "unit": "ms", "n_gpus": 1, "steps": len(B16),
        "warmup": args.warmup, "ms_per_step": round(mux_med, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "pdmux-llama3-8b: 32 layers, 32/8 heads, d128, bs16; decode 128 x 2048 on a CU-masked "
                               "stream while a 16384-token prompt is prefilled layer-wise on the complementary CUs",
                   "groups": [f"{p}:{q}" for p, q in groups], "level_16k": [f"{groups[x][0]}:{groups[x][1]}" for x in lv16],
                   "level_32k": [f"{groups[x][0]}:{groups[x][1]}" for x in lv32],
                   "value_is": "median decode step (32 layers: kv_write + attn_decode) wall time per round while the "
                               "16K prefill runs"},
        "roofline": {"kernel": "attn_decode (decode step under multiplexing: the whole-line K kernel on the "
                               "CU-masked stream)", "bound": "hbm",
                     "achieved": round(dstep_bytes / (mux_med * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dstep_bytes / (mux_med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": L * line_traffic if line_traffic else None,
                     "bytes_per_step": dstep_bytes,
                     "note": "decode K/V + q/out bytes of the 32-layer step over its median wall time (host "
                             "clock around each round, kv_write launches included); traffic: the counters' bytes "
                             "of the step's 32 decode launches"},
        "metrics": {
            "solo_decode": stats(A),
            "mux_16k_decode": stats(B16), "mux_16k_prefill_ms": round(pf16, 2),
            "mux_32k_decode": stats(B32), "mux_32k_prefill_ms": round(pf32, 2),
            "mux_over_solo_16k": round(mux_med / solo_med, 3),
            "mux_over_solo_32k": round(float(np.median(B32)) / solo_med, 3),
            "mux_p99_over_solo_median_16k": round(float(np.percentile(B16, 99)) / solo_med, 3),
            "mux_p99_over_solo_median_32k": round(float(np.percentile(B32, 99)) / solo_med, 3),
            **extra,
            "chunked_whole_gpu": C,
            "stall_free_whole_gpu": E,
            "prefill_alone_ms": D,
            "decode_bytes_per_step": decode_bytes([ctx] * B, hkv, d, hq) * L,
        },
    }
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(w, nreq=8, seconds=args.cpu_seconds)
    return result


# --------------------------------------------------------- copy-1gib ----
def bench_copy_1gib(args):
    """A plain device copy of 1 GiB (torch copy_), the reference kernel for reading the
    FETCH_SIZE / WRITE_SIZE counters: its bytes read and written are known exactly."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(1, args.warmup)):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    gbps = 2 * n / (ms * 1e-3) / 1e9
    return {"metric": "device copy GB/s (read + write)", "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "copy-1gib: torch copy_ of 1 GiB, the calibration kernel for the HBM counters"},
            "roofline": {"kernel": "copy", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": 2 * n}}


# ------------------------------------------------------- mfma-peak ----
def bench_mfma_peak(args):
    """The device's dense bf16 matrix-core rate and its shader clock while the matrix cores are busy: 512
    workgroups of 4 waves (two per CU, two waves per SIMD), each wave running four independent chains of
    32x32x16 bf16 MFMAs, timed with HIP events on the launching stream; every wave also reads the shader clock
    counter and the 100 MHz reference counter around its loop (kernel in decode_paged_kv_amd/calib).  The value
    is with constant operands; metrics.random_operands is the same stream with operands that change from one
    MFMA to the next."""
    lib = _calib_lib()
    blocks, iters = 512, 4096
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(blocks * 4 * 2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.Stream()
    flops = blocks * 4 * iters * 4 * 32 * 32 * 16 * 2

    def run(fn, name):
        def launch():
            rc = fn(iters, blocks, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"{name}: HIP error {rc}")

        for _ in range(max(1, args.warmup)):
            launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(3, args.steps)):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            e.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(e))
        ck = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        return times, ck[:, 0] / (ck[:, 1] / 100e6) / 1e9

    # operands that change from one MFMA to the next (as in attention), then
    # the constant operands of the headline calibration (last, so the
    # kernel trace of this workload ends with it)
    rtimes, rghz = run(lib.pkv_calib_mfma_random, "pkv_calib_mfma_random")
    rms = float(np.median(rtimes))
    times, ghz = run(lib.pkv_calib_mfma, "pkv_calib_mfma")
    ms = float(np.median(times))
    tflops = flops / (ms * 1e-3) / 1e12
    clk = float(np.median(ghz))
    # the rate the same MFMA stream would reach at the nominal 2.4 GHz, and the peak at the measured clock
    peak_at_clock = BF16_PEAK_TFLOPS * clk / 2.4
    return {"metric": "dense bf16 MFMA TFLOP/s (calibration)", "value": round(tflops, 1), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": len(times), "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "mfma-peak: 512 workgroups x 4 waves, 4 independent chains of "
                                   "v_mfma_f32_32x32x16_bf16 per wave, 4096 rounds"},
            "roofline": {"kernel": "mfma_chain_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": None},
            "metrics": {"shader_clock_ghz_median": round(clk, 3), "shader_clock_ghz_min": round(float(ghz.min()), 3),
                        "shader_clock_ghz_max": round(float(ghz.max()), 3),
                        "peak_at_measured_clock_tflops": round(peak_at_clock, 1),
                        "frac_of_peak_at_measured_clock": round(tflops / peak_at_clock, 4),
                        "random_operands": {"tflops": round(flops / (rms * 1e-3) / 1e12, 1),
                                            "ms_per_launch": round(rms, 4),
                                            "shader_clock_ghz_median": round(float(np.median(rghz)), 3),
                                            "note": "eight pseudo-random bf16 operand pairs cycled through by "
                                                    "consecutive MFMAs"}}}


# ----------------------------------------------------- hbm-ceiling ----
def _calib_lib():
    import ctypes as C
    from decode_paged_kv_amd import build as b
    if not os.path.exists(b.CALIB_LIB):
        raise RuntimeError(f"{b.CALIB_LIB} is not built (python -m decode_paged_kv_amd.build)")
    lib = C.CDLL(b.CALIB_LIB)
    lib.pkv_calib_mfma.restype = C.c_int
    lib.pkv_calib_mfma.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.pkv_calib_mfma_random.restype = C.c_int
    lib.pkv_calib_mfma_random.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.pkv_calib_tiled_read.restype = C.c_int
    lib.pkv_calib_tiled_read.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    lib.pkv_calib_tiled_copy.restype = C.c_int
    lib.pkv_calib_tiled_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                         C.c_void_p]
    lib.pkv_calib_copy.restype = C.c_int
    lib.pkv_calib_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    return lib


def bench_hbm_ceiling(args):
    """What HBM delivers to the library's own access patterns, measured like the kernels they bound (HIP graph
    of back-to-back launches, HIP events on the replaying stream; kernels in decode_paged_kv_amd/calib):

    * decode's reads: 512 workgroups, each reading the 64 permuted 4 KiB tiles of one (request, KV head) pair
      (the Llama-3-8B-shaped decode launch: 134,217,728 B), 32 launches over 32 pools; and 150 tiles per
      workgroup (314,572,800 B, the size of the Qwen3-32B-like decode launch), 16 launches over 16 pools;
    * the relayout's copies: 80 layers of 4096 permuted 4 KiB source tiles (16.8 MB) to permuted destination
      tiles, 1024 workgroups of 4 tiles (all loads before the stores, as kv_relayout), and a contiguous copy of
      the same bytes.

    ``value`` is the decode-shaped read rate (best of the unroll depths tried)."""
    lib = _calib_lib()
    stream = torch.cuda.Stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    res = {}

    def timed(name, launch, n_launch, nbytes, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            launch()
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            launch()
        for _ in range(max(1, args.warmup)):
            with torch.cuda.stream(stream):
                g.replay()
        stream.synchronize()
        ts = []
        for _ in range(reps):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                a.record(stream)
                g.replay()
                e.record(stream)
            stream.synchronize()
            ts.append(a.elapsed_time(e))
        us = float(np.median(ts)) * 1e3 / n_launch
        res[name] = {"us_per_launch": round(us, 3), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del g

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: HIP error {rc}")

    reps = max(3, args.steps)
    # decode-shaped reads
    for label, tpw, nl in (("read_134mb", 64, 32), ("read_315mb", 150, 16)):
        wgs = 512
        ntile = wgs * tpw
        pools = [torch.empty(ntile * 4096, dtype=torch.uint8, device="cuda") for _ in range(nl)]
        ids = [torch.randperm(ntile, generator=gen, device="cuda").to(torch.int32) for _ in range(nl)]
        sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
        for u in (4, 8, 16):
            def launch(u=u):
                for l in range(nl):
                    check(lib.pkv_calib_tiled_read(pools[l].data_ptr(), ids[l].data_ptr(), wgs, tpw, u,
                                                   sink.data_ptr(), stream.cuda_stream), "pkv_calib_tiled_read")
            timed(f"{label}_unroll{u}", launch, nl, ntile * 4096, reps)
        del pools, ids, sink
        _free_device()
    # relayout-shaped copies: 80 layers of 16.8 MB read + 16.8 MB written
    L, ntile = 80, 4096
    src = [torch.empty(ntile * 4096, dtype=torch.uint8, device="cuda") for _ in range(L)]
    dst = [torch.empty(ntile * 4096, dtype=torch.uint8, device="cuda") for _ in range(L)]
    sids = [torch.randperm(ntile, generator=gen, device="cuda").to(torch.int32) for _ in range(L)]
    dids = [torch.randperm(ntile, generator=gen, device="cuda").to(torch.int32) for _ in range(L)]
    for u in (2, 4):
        def launch(u=u):
            for l in range(L):
                check(lib.pkv_calib_tiled_copy(src[l].data_ptr(), sids[l].data_ptr(), dst[l].data_ptr(),
                                               dids[l].data_ptr(), 1024, 4, u, stream.cuda_stream),
                      "pkv_calib_tiled_copy")
        timed(f"copy_tiled_16.8mb_unroll{u}", launch, L, 2 * ntile * 4096, reps)
    for wgs in (1024, 2048):
        def launch(wgs=wgs):
            for l in range(L):
                check(lib.pkv_calib_copy(src[l].data_ptr(), dst[l].data_ptr(), ntile * 4096, wgs, stream.cuda_stream),
                      "pkv_calib_copy")
        timed(f"copy_contiguous_16.8mb_wgs{wgs}", launch, L, 2 * ntile * 4096, reps)
    del src, dst, sids, dids
    _free_device()
    best_read = max(v["gbps"] for k, v in res.items() if k.startswith("read_134mb"))
    return {"metric": "HBM GB/s at the library's access patterns (calibration)", "value": best_read, "unit": "GB/s",
            "n_gpus": 1, "steps": reps, "warmup": args.warmup,
            "ms_per_step": min(v["us_per_launch"] for k, v in res.items() if k.startswith("read_134mb")) / 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "hbm-ceiling: permuted 4 KiB tile reads of decode's launch sizes (134 MB, "
                                   "315 MB) and permuted tile copies / contiguous copies of the 70B relayout's "
                                   "layer (16.8 MB read + 16.8 MB written)"},
            "roofline": {"kernel": "tiled_read_kernel", "bound": "hbm", "achieved": best_read, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(best_read / HBM_PEAK_GBPS, 4), "traffic": None},
            "metrics": res}


# ---------------------------------------------------------------- all ----
def _free_device():
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bench_all(args):
    """The headline workload (Qwen3-32B-like 16K prompt at chunks 2048 and 512: prefill TFLOP/s is ``value``),
    the matrix-core calibration of the same box (``metrics["mfma_calibration"]``), under
    ``metrics["workloads"]`` the Llama-3-8B-shaped step (decode GB/s), the 70B relayout (GB/s) and the
    PD-multiplexing round (decode step ms), each with its own roofline, traffic and oracle baseline, and the HBM
    calibration at the decode's and the relayout's access patterns (``metrics["hbm_calibration"]``).  The
    workloads run one after the other; each frees its device memory before the next."""
    t0 = time.perf_counter()
    res = bench_qwen3_32b(args)
    _free_device()
    # the dense bf16 rate this machine sustains on a pure MFMA stream, with
    # constant operands and with operands that change from one MFMA to the
    # next (the headline's roofline peak stays the published figure)
    cal = bench_mfma_peak(args)
    rnd = cal["metrics"]["random_operands"]
    res["metrics"]["mfma_calibration"] = {
        "constant_operands_tflops": cal["value"], "constant_operands_clock_ghz": cal["metrics"]["shader_clock_ghz_median"],
        "random_operands_tflops": rnd["tflops"], "random_operands_clock_ghz": rnd["shader_clock_ghz_median"],
        "prefill_value_over_random_operands_rate": round(res["value"] / rnd["tflops"], 4)}
    sub = {}
    for name, fn in (("llama3_8b", bench_llama3_8b), ("relayout_70b", bench_relayout_70b), ("pdmux", bench_pdmux)):
        t1 = time.perf_counter()
        r = fn(args)
        _free_device()
        sub[name] = {k: r[k] for k in ("metric", "value", "unit", "higher_is_better", "ms_per_step", "config",
                                       "roofline", "metrics", "cpu_baseline") if k in r}
        sub[name]["wall_s"] = round(time.perf_counter() - t1, 1)
    res["metrics"]["workloads"] = sub
    # the fused stall-free launch at G = 8 (the mixed-batch kernel)
    sf = bench_stall_free_qwen(args)
    _free_device()
    res["metrics"]["stall_free_qwen3_32b"] = {**sf["metrics"], "layers": 16}
    # what HBM delivers on this machine to the decode's and the relayout's own
    # access patterns (the rooflines' peak stays the published 8 TB/s)
    hb = bench_hbm_ceiling(args)["metrics"]
    _free_device()
    best = lambda prefix: max(v["gbps"] for k, v in hb.items() if k.startswith(prefix))  # noqa: E731
    r134, r315, ct = best("read_134mb"), best("read_315mb"), best("copy_tiled")
    res["metrics"]["hbm_calibration"] = {
        "tiled_read_134mb_gbps": r134, "tiled_read_315mb_gbps": r315, "tiled_copy_16.8mb_gbps": ct,
        "contiguous_copy_16.8mb_gbps": best("copy_contiguous"),
        "llama_decode_over_tiled_read": round(sub["llama3_8b"]["value"] / r134, 4),
        "qwen_decode_over_tiled_read": round(res["metrics"]["decode_attn_gbps"] / r315, 4),
        "relayout_over_tiled_copy": round(sub["relayout_70b"]["value"] / ct, 4)}
    res["metrics"]["wall_s"] = round(time.perf_counter() - t0, 1)
    return res


# --------------------------------------------------------------- main ----
BENCHES = {"all": bench_all, "llama3-8b": bench_llama3_8b, "qwen3-32b": bench_qwen3_32b,
           "relayout-70b": bench_relayout_70b, "pdmux": bench_pdmux, "copy-1gib": bench_copy_1gib,
           "mfma-peak": bench_mfma_peak, "hbm-ceiling": bench_hbm_ceiling,
           "stall-free-qwen3-32b": bench_stall_free_qwen}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="all", choices=sorted(BENCHES))
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="host time per oracle baseline of the secondary workloads (the headline's takes >= 10 s)")
    ap.add_argument("--full", action="store_true",
                    help="pdmux: also the per-level graph and append arms, the level sweep, the two-launch "
                         "stall-free arm")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path runs on one MI355X's share of the work (decode and prefill "
              "attention shard by request or KV head with no exchange; relayout sends each head to the "
              "destination shard that owns it) and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    res = BENCHES[args.workload](args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
