"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workloads (all synthetic, seeded, resident in HBM before timing):

* ``llama3-8b`` (default): 32 layers of a Llama-3-8B-shaped attention
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
  ``value`` is relayout HBM GB/s (read + write).
* ``pdmux``: the PD-multiplexing round (see ``bench_pdmux``).  ``value`` is
  the multiplexed decode step in ms.

One JSON line is printed.  Kernel times come from HIP events recorded on
the stream the kernels are launched on.
"""

from __future__ import annotations

import argparse
import json
import math
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


# ------------------------------------------------------------- helpers ----
class Timer:
    """Pairs of HIP events on one stream; durations in ms after a sync."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = {}

    def start(self, key):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.setdefault(key, []).append([e, None])

    def stop(self, key):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[key][-1][1] = e

    def ms(self, key):
        return [a.elapsed_time(b) for a, b in self.pairs.get(key, [])]

    def reset(self):
        self.pairs = {}


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
    ws = torch.empty(max(16, ops.attn_decode_workspace_size(B, hq, ctx, d)), dtype=torch.uint8, device="cuda")
    dec_start, dec_pos = i32(np.arange(B + 1)), i32([ctx - 1] * B)
    dec_slots = torch.empty(B, dtype=torch.int32, device="cuda")
    chunks = [(s, min(chunk, N - s)) for s in range(0, N, chunk)]
    ch_args = [(i32([0, t]), i32([s]), torch.empty(t, dtype=torch.int32, device="cuda")) for s, t in chunks]
    timer = Timer(stream)

    def step(timed):
        tk = timer if timed else None
        with torch.cuda.stream(stream):
            if tk: tk.start("step")
            if tk: tk.start("decode_step")
            ops.slot_mapping(dec_bt, dec_start, dec_pos, B, bs, w.pool_blocks, out=dec_slots, stream=stream)
            for l in range(L):
                ops.kv_write(pools[l], kn[l], vn[l], dec_slots, stream=stream)
                if tk: tk.start("attn_decode")
                ops.attn_decode(pools[l], q_dec[l], o_dec[l], dec_bt, ctx_t, ctx, hq, workspace=ws, stream=stream)
                if tk: tk.stop("attn_decode")
            if tk: tk.stop("decode_step")
            if tk: tk.start("prefill")
            for (s, t), (sl, cs, slots) in zip(chunks, ch_args):
                ops.slot_mapping(pr_bt, sl, cs, t, bs, w.pool_blocks, out=slots, stream=stream)
                for l in range(L):
                    ops.kv_write(pools[l], k_pr[l][s:s + t], v_pr[l][s:s + t], slots, stream=stream)
                    if tk: tk.start(f"attn_prefill_{s}")
                    ops.attn_prefill_chunk(pools[l], q_pr[l][s:s + t], o_pr[l][s:s + t], pr_bt, sl, cs, t, hq,
                                           stream=stream)
                    if tk: tk.stop(f"attn_prefill_{s}")
            if tk: tk.stop("prefill")
            if tk: tk.start("relayout")
            for l in range(L):
                ops.kv_relayout(pools[l], pr_bt, dsts[l], dst_bt, N, stream=stream)
            if tk: tk.stop("relayout")
            if tk: tk.stop("step")

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / args.steps

    step_ms = float(np.mean(timer.ms("step")))
    dec_launch_ms = float(np.mean(timer.ms("attn_decode")))
    dbytes = decode_bytes([ctx] * B, hkv, d, hq)
    dec_gbps = dbytes / (dec_launch_ms * 1e-3) / 1e9
    pf_flops = sum(prefill_flops(hq, d, t, s) for s, t in chunks)
    pf_ms = sum(float(np.mean(timer.ms(f"attn_prefill_{s}"))) for s, _ in chunks)   # per layer, both chunks
    pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12
    rl_ms = float(np.mean(timer.ms("relayout"))) / L
    rl_gbps = relayout_bytes(N, hkv, d) / (rl_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-attn: 32 layers, 32/8 heads, d128, bs16; decode 64x512 + prompt 1024 "
                               "in 2 chunks of 512 + relayout 1024 tokens bs16/4 shards -> bs32/8 shards",
                   "layers": L, "decode_batch": B, "decode_context": ctx, "prompt": N, "chunk": chunk,
                   "value_is": "attn_decode HBM GB/s (algorithmic K/V + q/out bytes per launch / mean launch time)"},
        "roofline": {"kernel": "attn_decode (split + merge)", "bound": "hbm", "achieved": round(dec_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": dbytes, "launch_ms": round(dec_launch_ms, 5)},
        "metrics": {
            "decode_attn_gbps": round(dec_gbps, 1),
            "decode_step_ms": round(float(np.mean(timer.ms("decode_step"))), 4),
            "prefill_attn_tflops": round(pf_tflops, 2),
            "prefill_attn_frac_bf16_peak": round(pf_tflops / BF16_PEAK_TFLOPS, 4),
            "prefill_layer_ms": round(pf_ms, 5),
            "relayout_gbps": round(rl_gbps, 1),
            "relayout_layer_ms": round(rl_ms, 5),
            "wall_ms_per_step": round(wall, 3),
        },
    }
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(w)
    return result


def cpu_baseline_decode(w):
    """The oracle's decode on a bounded sample of the same workload, timed on the host."""
    from oracle import attention as oa
    hq, hkv, d, ctx = w.num_q_heads, w.num_kv_heads, w.head_dim, w.decode_context[0]
    nreq = 16
    g = lambda t, i: inputs.stream(w.seed, w.config_id, 0, t, i)  # noqa: E731
    ks = [inputs.as_float(inputs.normal((ctx, hkv, d), 0.5, "bf16", g(inputs.T_K, r)), "bf16") for r in range(nreq)]
    vs = [inputs.as_float(inputs.normal((ctx, hkv, d), 0.5, "bf16", g(inputs.T_V, r)), "bf16") for r in range(nreq)]
    q = inputs.as_float(inputs.normal((nreq, hq, d), 0.5, "bf16", g(inputs.T_Q, 0)), "bf16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oa.decode_batch(q, ks, vs)
        reps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = time.perf_counter() - t0
    nbytes = decode_bytes([ctx] * nreq, hkv, d, hq) * reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores_used(), "kind": "oracle",
            "sample": f"oracle decode of {nreq} requests x {ctx} keys x {hq}/{hkv} heads (one layer of the same "
                      f"workload), repeated {reps} times in {dt:.1f} s; bf16 K/V/q/out bytes / wall time"}


# --------------------------------------------------------------- main ----
BENCHES = {"llama3-8b": bench_llama3_8b}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3-8b", choices=sorted(BENCHES))
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path runs on one MI355X's share of the work and has no multi-GPU "
              "mode (how it would shard is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    res = BENCHES[args.workload](args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
