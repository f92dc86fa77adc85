"""Stall-free batch rule ([L7] section 2.4): the oracle's reading pinned by
what the page states, and the library's pkv_stall_free_chunk against it."""

import itertools

import pytest

from conftest import read_golden
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


def test_budget_exercise_golden_values(golden):
    # "Lecture 7" section 10, exercise 3: values the page prints
    recs = golden("stall_free_budget.txt")
    assert len(recs) == 3
    for _, budget, nd, left in recs:
        budget, nd, left = int(budget), int(nd), int(left)
        # a prompt longer than any budget: its chunk is exactly what the decodes leave
        d, (c,) = policy.stall_free_batch(budget, nd, [10 ** 6])
        assert (d, c) == (nd, left)


def test_budget_golden_values_fail_a_planted_mistake(golden):
    # a rule that lets decodes past the budget push prefill negative, or that forgets to reserve the decode
    # tokens, disagrees with the page's numbers
    def forgets_decodes(budget, nd, rems):
        return nd, [min(rems[0], budget)]

    def clamps_late(budget, nd, rems):
        return nd, [min(rems[0], budget - nd)]

    for mutant in (forgets_decodes, clamps_late):
        bad = 0
        for _, budget, nd, left in golden("stall_free_budget.txt"):
            if mutant(int(budget), int(nd), [10 ** 6])[1][0] != int(left):
                bad += 1
        assert bad > 0, mutant.__name__


def test_ongoing_prefills_before_new_requests():
    # section 2.4 steps 3-4: unfinished prefills take the leftover budget first, new requests are cut to what
    # remains after them; the caller lists ongoing prompts first
    assert policy.stall_free_batch(512, 300, [100, 5000]) == (300, [100, 112])
    assert policy.stall_free_batch(512, 300, [500, 5000]) == (300, [212, 0])


def test_library_multi_prompt_rule_matches_oracle():
    from decode_paged_kv_amd import _lib, ops
    try:
        _lib.load()
    except Exception as e:  # noqa: BLE001
        pytest.skip(f"libpkv not built: {e}")
    for budget, nd in itertools.product((0, 128, 256, 512, 2048), (0, 1, 127, 128, 300)):
        for rems in ([], [0], [5000], [100, 5000], [1000, 1000, 1000], [7, 0, 9, 10 ** 6]):
            d, chunks = policy.stall_free_batch(budget, nd, rems)
            assert ops.stall_free_batch(budget, nd, rems) == chunks
    for _, budget, nd, left in read_golden("stall_free_budget.txt"):
        assert ops.stall_free_batch(int(budget), int(nd), [10 ** 6]) == [int(left)]
    with pytest.raises(_lib.PkvError):
        ops.stall_free_batch(512, 3, [10, -1])
