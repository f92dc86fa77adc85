"""Pins for the policy rules and the closed-form counts.

The policy must reproduce, value for value, the split tables, level picks
and layers-per-round printed in "PD multiplexing: splitting prefill and
decode by SM on one GPU" (section "SGLang's PD multiplexing" and its
exercises).  The prefill flop count must reproduce that chapter's estimate
table (section "Is it worth it: an estimate") when plugged into the page's
model.  KV byte counts and the chunked re-read ratio must match the numbers
printed in "PD 分离与 KV 传输", "Lecture 7" and "推理 INFRA 方法论（6）".
"""

import math

from conftest import kv_fields, read_golden
from oracle import accounting, policy


def _pairs(fields):
    return [tuple(int(x) for x in f.split(":")) for f in fields]


def test_split_tables_match_pages():
    for rec in read_golden("mux_policy_demo.txt"):
        if rec[0] == "groups":
            _, _name, sms, cc = rec[:4]
            assert policy.nvidia_stream_groups(int(sms), int(cc)) == _pairs(rec[4:])


def test_level_choice_and_layers_match_pages():
    groups = policy.nvidia_stream_groups(132, 9)
    seen = 0
    for rec in read_golden("mux_policy_demo.txt"):
        if rec[0] == "choose":
            bs, has_prefill, idx = int(rec[1]), bool(int(rec[2])), int(rec[3])
            k = policy.choose_level(len(groups), bs, has_prefill)
            assert k == idx and groups[k] == _pairs([rec[4]])[0]
            seen += 1
        elif rec[0] == "layers":
            assert policy.layers_per_round(int(rec[1]), int(rec[2])) == int(rec[3])
            seen += 1
    assert seen == 14


def test_exercises():
    recs = {r[0]: r for r in read_golden("mux_policy_demo.txt")}
    lv = recs["levels"]
    g = policy.nvidia_stream_groups(78, 9)
    assert len(g) - 2 == int(lv[2]) and len(g) == int(lv[3])
    first_at, divisor, first_at_new = (int(x) for x in recs["first_last_level"][1:])
    h100 = policy.nvidia_stream_groups(132, 9)
    last = len(h100) - 2
    assert min(b for b in range(1, 200) if policy.choose_level(8, b, True) == last) == first_at
    assert min(b for b in range(1, 200) if policy.choose_level(8, b, True, divisor) == last) == first_at_new


def test_mi355x_cu_levels():
    g = policy.mi355x_stream_groups()
    assert g == [(256, 0), (208, 48), (192, 64), (176, 80), (160, 96), (144, 112), (128, 128), (0, 256)]
    # decode >= 16 gives the same table: the 32-CU floor does not bind
    assert policy.stream_groups(256, 8, 8, 16) == g
    k = policy.choose_level(len(g), 128, True)
    assert k == 6 and g[k] == (128, 128)
    assert policy.layers_per_round(32768, 32) == 2 and policy.layers_per_round(16384, 32) == 4


def test_estimate_table_pins_attention_flop_count():
    c = kv_fields(read_golden("mux_estimate.txt")[0][1:])
    sms, layers, hidden = int(c["sms"]), int(c["layers"]), int(c["hidden"])
    bw = float(c["bw"]) * float(c["bw_frac"])
    flops = float(c["flops"]) * float(c["mfu"])
    kvh, ffn, vocab = int(c["kv_hidden"]), int(c["ffn"]), int(c["vocab"])
    dbs, ctx, prompt = int(c["decode_bs"]), int(c["context"]), int(c["prompt"])
    # the page's model: linear-layer parameters, KV bytes per token
    linear = layers * (2 * hidden * hidden + 2 * hidden * kvh + 3 * hidden * ffn) + hidden * vocab
    kv_per_token = accounting.kv_bytes_per_token(layers, kvh // 128, 128, 2)

    def decode_step(units, s_sat):
        return (2 * linear + dbs * ctx * kv_per_token) / (bw * min(1.0, units / s_sat))

    def prefill_flops(tokens, start=0):
        # attention term from the oracle: per layer, 32 q-heads x 128 dims = 4096
        return 2 * linear * tokens + layers * accounting.prefill_attention_flops(32, 128, tokens, start)

    rows = {r[1]: r[2:] for r in read_golden("mux_estimate.txt") if r[0] == "row"}
    base = decode_step(sms, 66)
    assert round(base * 1e3) == int(rows["decode_only"][0])
    t = prefill_flops(prompt) / flops
    assert round((t + base) * 1e3) == int(rows["prefill_first"][0]) and round(t * 1e3) == int(rows["prefill_first"][2])
    for chunk in (2048, 512):
        steps = [max((prefill_flops(chunk, s) + 2 * linear * dbs) / flops, base) for s in range(0, prompt, chunk)]
        itl, nsteps, total, _ = rows[f"chunked_{chunk}"]
        assert round(sum(steps) / len(steps) * 1e3) == int(itl)
        assert len(steps) == int(nsteps) and round(sum(steps) * 1e3) == int(total)
    groups = policy.nvidia_stream_groups(sms, 9)
    p_units, d_units = groups[policy.choose_level(len(groups), dbs, True)]
    assert (p_units, d_units) == (80, 52)
    t = prefill_flops(prompt) / (flops * p_units / sms)
    for s_sat in (44, 66, 88):
        itl_ms, _, pf_ms, toks = rows[f"pdmux_80_52_ssat{s_sat}"]
        itl = decode_step(d_units, s_sat)
        assert round(itl * 1e3) == int(itl_ms) and round(t * 1e3) == int(pf_ms) and round(t / itl) == int(toks)


def test_flop_count_against_brute_force_pair_count():
    # the page's count is 4*Hq*D*(pairs - T/2), pairs = visible (query, key) pairs
    for t, s in ((1, 0), (5, 0), (16, 32), (64, 192)):
        pairs = sum(s + i + 1 for i in range(t))
        assert accounting.prefill_attention_flops(3, 8, t, s) == 4 * 3 * 8 * (pairs - t / 2)


def test_kv_byte_figures_from_pages():
    recs = read_golden("kv_bytes.txt")
    for r in recs:
        f = kv_fields(r[1:]) if r[0] != "transfer" else kv_fields(r[2:])
        if r[0] == "transfer":
            total = int(f["per_token"]) * int(f["tokens"])
            assert round(total / 1e9, 2) == float(f["gb"])
            assert round(total / float(f["link"]) * 1e3) == int(f["ms"])
        elif r[0] == "pd_demo":
            # Qwen3-0.6B's KV shape (28 layers, 8 KV heads, head dim 128) is its
            # published model config, not stated on the page
            assert accounting.kv_bytes(int(f["tokens"]), 28, 8, 128, 2) == int(f["kib"]) * 1024
        elif r[0] == "per_token":
            f = kv_fields(r[2:])
            assert accounting.kv_bytes_per_token(int(f["layers"]), int(f["kv_heads"]), int(f["head_dim"])) == int(f["kib"]) * 1024
        elif r[0] == "rate":
            f = kv_fields(r[2:])
            rate = int(f["rps"]) * int(f["tokens"]) * int(f["per_token"])
            assert round(rate / 1e9, 1) == float(f["gbps"])
        elif r[0] == "reread":
            assert accounting.chunked_reread_ratio(int(f["n"]), int(f["chunk"])) == float(f["ratio"])


def test_chunked_reads_closed_form():
    for n, c in ((192, 16), (16384, 2048), (16384, 512), (1000, 64)):
        m = math.ceil(n / c)
        if n % c == 0:
            assert accounting.chunked_kv_reads(n, c) == c * m * (m + 1) // 2
        # brute force: chunk k reads keys [0, end_k)
        assert accounting.chunked_kv_reads(n, c) == sum(min(n, (k + 1) * c) for k in range(m))


def test_decode_bytes():
    assert accounting.decode_attention_bytes([512] * 64, 8, 128) == 134_217_728
    assert accounting.decode_attention_bytes([2048] * 128, 8, 128) == 1_073_741_824
