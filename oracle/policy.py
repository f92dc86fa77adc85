"""PD-multiplexing policy rules, as plain integer arithmetic.

TEST INFRASTRUCTURE ONLY (see the package header): the GPU path never
imports this module.

Rules, restated from [MUX] section "SGLang's PD multiplexing" (the split and
selection rules and the demo output printed under them) and its exercises:

* Split candidates.  A split gives ``x`` compute units to prefill and
  ``total - x`` to decode.  ``x`` runs over a grid: it starts at the
  minimum part size and steps by the granularity up to ``total - min_part``.
  A candidate must give prefill at least half (``2x >= total``) and decode
  at least ``min_decode`` units.  When there are at least ``levels``
  candidates, keep every ``(count // levels)``-th one (at least every one)
  starting from the smallest, and then only the first ``levels`` of those.
  Splits are listed with the largest prefill share first.
* Groups.  Group 0 gives the whole device to prefill, the split levels
  follow, and the last group gives the whole device to decode; the number of
  split levels is ``sm_group_num - 2``.
* Level choice.  With ``n`` groups: when both decode requests and a prefill
  are present, the level is ``decode_bs * (n - 2) // divisor`` clamped to
  ``[1, n - 2]``; with decode only, the last group; otherwise group 0.  The
  default divisor is 36.
* Layers per round.  A prefill of ``tokens`` tokens advances
  ``budget // tokens`` layers per round, at least 1 and at most the model's
  layer count; the default budget is 65536.

On the pages the unit is an NVIDIA SM, with (minimum part, granularity) of
(2, 2) for compute capability 7, (4, 2) for 8 and (8, 8) for 9 and later.
The MI355X reading uses compute units: 256 CUs, granularity 8, minimum part
8 and decode of at least 32 CUs.
"""

from __future__ import annotations

# (minimum part, granularity) per compute-capability major, as listed in
# [MUX] "SGLang's PD multiplexing".
NVIDIA_SPLIT_GRID = {6: (1, 1), 7: (2, 2), 8: (4, 2), 9: (8, 8)}


def split_levels(total: int, min_part: int, granularity: int, min_decode: int, levels: int) -> list[tuple[int, int]]:
    """(prefill units, decode units) for each split level, largest prefill first."""
    candidates = []
    x = min_part
    while x <= total - min_part:
        if 2 * x >= total and total - x >= min_decode:
            candidates.append(x)
        x += granularity
    if len(candidates) >= levels:
        stride = max(1, len(candidates) // levels)
        candidates = candidates[::stride][:levels]
    return [(x, total - x) for x in sorted(candidates, reverse=True)]


def stream_groups(total: int, min_part: int, granularity: int, min_decode: int, group_num: int = 8) -> list[tuple[int, int]]:
    """All-prefill group, then the split levels, then the all-decode group."""
    return [(total, 0)] + split_levels(total, min_part, granularity, min_decode, group_num - 2) + [(0, total)]


def nvidia_stream_groups(sms: int, cc_major: int, group_num: int = 8) -> list[tuple[int, int]]:
    """The pages' SM version: decode keeps at least 16 SMs."""
    min_part, granularity = NVIDIA_SPLIT_GRID[cc_major]
    return stream_groups(sms, min_part, granularity, 16, group_num)


def mi355x_stream_groups(total_cus: int = 256, granularity: int = 8, min_decode: int = 32, group_num: int = 8):
    """The CU version used on MI355X (256 CUs, steps of 8, decode >= 32)."""
    return stream_groups(total_cus, granularity, granularity, min_decode, group_num)


def choose_level(num_groups: int, decode_bs: int, has_prefill: bool, divisor: int = 36) -> int:
    """Index of the group to run, from the decode batch size."""
    if decode_bs > 0 and has_prefill:
        return min(num_groups - 2, max(1, decode_bs * (num_groups - 2) // divisor))
    if decode_bs > 0:
        return num_groups - 1
    return 0


def layers_per_round(prefill_tokens: int, num_layers: int, budget: int = 65536) -> int:
    """Layers of prefill submitted per multiplexing round."""
    return min(num_layers, max(1, budget // prefill_tokens))


def stall_free_batch(token_budget: int, num_decode: int, prompts_remaining: list[int]) -> tuple[int, list[int]]:
    """One step of a stall-free batch, following [L7] section 2.4.

    Every decoding request joins the step first, one token each; then each
    unfinished prompt, in order, takes at most what is left of the token
    budget.  Returns (decode tokens, chunk per prompt).  Decode requests are
    never dropped, so a budget at or below the decode count leaves the
    prompts nothing.
    """
    left = max(0, token_budget - num_decode)
    chunks = []
    for rem in prompts_remaining:
        take = min(rem, left)
        chunks.append(take)
        left -= take
    return num_decode, chunks


def choose_level_manual(num_groups: int, decode_bs: int, has_prefill: bool, thresholds: list[int]) -> int:
    """Level choice with manual divisions ([MUX] "SGLang's PD multiplexing", level choice and its exercise).

    ``thresholds[i-1]`` is the decode batch size from which split level ``i``
    is used (one per split level, non-decreasing); below the first threshold
    the first split level.  Decode only and prefill only keep the whole device.
    """
    assert len(thresholds) == num_groups - 2
    if decode_bs > 0 and has_prefill:
        level = 1
        for i, t in enumerate(thresholds, start=1):
            if decode_bs >= t:
                level = i
        return level
    if decode_bs > 0:
        return num_groups - 1
    return 0
