"""Closed forms for the bytes and flops the path must move or compute.

TEST INFRASTRUCTURE ONLY (see the package header): the GPU path never
imports this module.  ``bench.py`` has its own copy of the per-launch
counts it reports, and the tests check that copy against these.

* KV bytes per token: layers x 2 (K and V) x KV heads x head dim x element
  bytes ([L7] section 10, exercise 5; [DISAGG] "传输的代价"; the estimate
  model in [MUX] "Is it worth it: an estimate").  Transfer size is that
  times the prompt length ([DISAGG] summary).
* Chunked-prefill KV reads: chunk k (1-based) of size c reads the k*c keys
  before and inside it, so the total over n/c chunks is c*m*(m+1)/2 with
  m = n/c, about n^2/(2c); the ratio to a one-shot prefill is m/2 + 1/2
  ([L7] section 2.3 and section 10, exercise 2).
* Causal attention flops of one layer for a chunk of T tokens starting at
  S: 4 * Hq * D * (T*S + T^2/2).  This is the attention term of the
  prefill cost in [MUX] "Is it worth it: an estimate" (there written for
  36 layers with Hq*D = 4096).  The T^2/2 term counts half of the diagonal
  block, as on the page.
* Decode attention bytes of one layer: every request reads its whole K and
  V once: sum over requests of L_b * 2 * Hkv * D * element bytes ([L7]
  section 1.1: decode reads all of the KV; each KV head's rows are read
  once for all of its q-heads).
"""

from __future__ import annotations


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return num_layers * 2 * num_kv_heads * head_dim * elem_bytes


def kv_bytes(tokens: int, num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return tokens * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)


def chunked_kv_reads(n: int, chunk: int) -> int:
    """Keys read (K or V rows, one head) over all chunks of an n-token prefill."""
    total = 0
    start = 0
    while start < n:
        end = min(n, start + chunk)
        total += end            # this chunk reads keys [0, end)
        start = end
    return total


def chunked_reread_ratio(n: int, chunk: int) -> float:
    return chunked_kv_reads(n, chunk) / n


def prefill_attention_flops(num_q_heads: int, head_dim: int, chunk_len: int, chunk_start: int) -> float:
    """Causal attention flops of one layer for one chunk (the pages' count)."""
    t, s = chunk_len, chunk_start
    return 4.0 * num_q_heads * head_dim * (t * s + t * t / 2.0)


def decode_attention_bytes(context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """K and V bytes one layer of decode must read (algorithmic, once each)."""
    return int(sum(int(l) for l in context_lens)) * 2 * num_kv_heads * head_dim * elem_bytes


def relayout_payload_bytes(tokens: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """K and V payload of one layer of one request; HBM traffic is twice this (read + write)."""
    return tokens * 2 * num_kv_heads * head_dim * elem_bytes
