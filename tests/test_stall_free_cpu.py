"""Stall-free batch rule ([L7] section 2.4): the oracle's reading pinned by
what the page states, and the library's pkv_stall_free_chunk against it."""

import itertools

import pytest

from oracle import policy


def test_decode_first_and_budget_bound():
    # decode requests always join the step; the prompt gets what is left
    assert policy.stall_free_batch(512, 32, [8192]) == (32, [480])
    # the step never exceeds the budget once decode fits in it
    for budget, nd, rem in itertools.product((128, 512, 2048), (0, 1, 100, 127, 128, 300), (0, 1, 384, 5000)):
        d, (c,) = policy.stall_free_batch(budget, nd, [rem])
        assert d == nd and 0 <= c <= rem
        assert d + c <= max(budget, nd)
        # the budget is filled as far as the prompt allows
        assert c == min(rem, max(0, budget - nd))


def test_small_budget_starves_prefill():
    # the page's warning: at budget 128 with a hundred or more decoding
    # requests the prompt barely (or never) gets in
    assert policy.stall_free_batch(128, 100, [7059]) == (100, [28])
    assert policy.stall_free_batch(128, 128, [7059]) == (128, [0])
    assert policy.stall_free_batch(128, 300, [7059]) == (300, [0])


def test_unbounded_budget_is_the_mixed_batch():
    # with a budget that no step reaches, the whole prompt goes in at once
    # (the page's check that chunking with an unbounded budget equals the
    # mixed batch)
    assert policy.stall_free_batch(10 ** 9, 64, [1730, 7059]) == (64, [1730, 7059])


def test_prompts_in_order_share_what_is_left():
    assert policy.stall_free_batch(2048, 128, [1000, 1000, 1000]) == (128, [1000, 920, 0])


def test_library_rule_matches_oracle():
    from decode_paged_kv_amd import _lib, ops
    try:
        _lib.load()
    except Exception as e:  # noqa: BLE001
        pytest.skip(f"libpkv not built: {e}")
    for budget, nd, rem in itertools.product((0, 1, 128, 512, 2048, 65536), (0, 1, 127, 128, 129, 4096),
                                             (0, 1, 383, 384, 16384)):
        assert ops.stall_free_chunk(budget, nd, rem) == policy.stall_free_batch(budget, nd, [rem])[1][0]
    with pytest.raises(_lib.PkvError):
        ops.stall_free_chunk(-1, 0, 0)
