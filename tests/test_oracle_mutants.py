"""Planted mistakes in the oracle must be caught by the pins.

Each mutant below is the oracle with one plausible slip planted in it, on
the CPU: an exclusive causal edge, a wrong GQA head map, a missing softmax
scale, a sign error in the scores, keys and values swapped, a dropped
normalisation.  For every mutant at least one of the independent pins (the
brute force, the library SDPA, the closed forms) must fail.
"""

import math

import numpy as np
import pytest

from oracle import attention as oa
from test_oracle_attention import _sdpa, brute_force


def _exclusive_edge(q, k, v, pos, scale=None):
    pos = np.maximum(np.asarray(pos) - 1, 0)
    return oa.attend(q, k, v, pos, scale)


def _modulo_head_map(q, k, v, pos, scale=None):
    # h % Hkv instead of h // G: reorder q-heads so the oracle's map becomes modulo
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    order = [(h % hkv) * g + h // hkv for h in range(hq)]
    inv = np.argsort(order)
    return oa.attend(q[:, order], k, v, pos, scale)[:, inv]


def _no_scale(q, k, v, pos, scale=None):
    return oa.attend(q, k, v, pos, 1.0)


def _score_sign(q, k, v, pos, scale=None):
    return oa.attend(-np.asarray(q), k, v, pos, scale)


def _kv_swapped(q, k, v, pos, scale=None):
    return oa.attend(q, v, k, pos, scale)


def _unnormalised(q, k, v, pos, scale=None):
    out = oa.attend(q, k, v, pos, scale)
    return out * (np.asarray(pos)[:, None, None] + 1)


MUTANTS = [_exclusive_edge, _modulo_head_map, _no_scale, _score_sign, _kv_swapped, _unnormalised]


def _pins_pass(fn):
    rng = np.random.default_rng(123)
    n, hq, hkv, d = 12, 4, 2, 8
    q, k, v = (rng.standard_normal(s) for s in ((n, hq, d), (n, hkv, d), (n, hkv, d)))
    pos = np.arange(n)
    got = fn(q, k, v, pos)
    ok_brute = np.abs(got - brute_force(q, k, v, list(pos), 1 / math.sqrt(d))).max() <= 1e-12
    ok_sdpa = np.abs(got - _sdpa(q, k, v, pos)).max() <= 1e-12
    # closed form: two keys with weights 1:3
    q1 = np.array([[[1.0]]])
    k1 = np.array([[[0.0]], [[math.log(3.0)]]])
    v1 = np.array([[[0.0]], [[4.0]]])
    ok_closed = abs(fn(q1, k1, v1, np.array([1]), 1.0)[0, 0, 0] - 3.0) <= 1e-15
    return ok_brute and ok_sdpa and ok_closed


def test_unmutated_oracle_passes_the_pins():
    assert _pins_pass(oa.attend)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_each_planted_mistake_fails_a_pin(mutant):
    assert not _pins_pass(mutant)
