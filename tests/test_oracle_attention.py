"""Pins for the attention oracle, independent of the oracle's own code.

Each check is something the pages or the mathematics fix, chosen so that a
plausible slip in the oracle (a wrong sign, an off-by-one causal edge, a
wrong GQA head map, a missing scale, a transposed operand) fails at least
one of them:

* brute force on tiny inputs: pure-Python loops with ``math.fsum`` and no
  max-subtraction (a different evaluation order from the oracle's GEMMs);
* a library routine: ``torch.nn.functional.scaled_dot_product_attention``
  on the CPU in float64 (GQA via ``enable_gqa``, whose documented head map
  repeats each KV head over consecutive q-heads);
* closed forms: one key gives that key's value; a zero query or identical
  keys give the mean of the visible values; a 2-key example whose weights
  are exactly 1:3;
* invariants: chunked prefill equals one-shot prefill ("Lecture 7" section
  2.3: chunking is lossless); a decode query at L-1 equals prefill row L-1;
  rows never depend on keys after their position; a shift of every key by
  the same vector leaves the output unchanged.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, positions, scale):
    """Direct definition with Python loops and exact-sum accumulation."""
    m_rows, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((m_rows, hq, d))
    for m in range(m_rows):
        for h in range(hq):
            kvh = h // g
            w = []
            for j in range(positions[m] + 1):
                s = math.fsum(float(q[m, h, t]) * float(k[j, kvh, t]) for t in range(d)) * scale
                w.append(math.exp(s))
            den = math.fsum(w)
            for t in range(d):
                out[m, h, t] = math.fsum(w[j] * float(v[j, kvh, t]) for j in range(len(w))) / den
    return out


@pytest.mark.parametrize("n,hq,hkv,d", [(1, 4, 2, 8), (7, 4, 2, 16), (32, 4, 2, 16), (20, 2, 2, 4), (17, 6, 1, 8)])
def test_brute_force_tiny(n, hq, hkv, d):
    q, k, v = _rand((n, hq, d), 1), _rand((n, hkv, d), 2), _rand((n, hkv, d), 3)
    scale = 1.0 / math.sqrt(d)
    got = oa.prefill(q, k, v)
    ref = brute_force(q, k, v, list(range(n)), scale)
    assert np.abs(got - ref).max() <= 1e-12


def test_brute_force_chunk_and_decode_positions():
    n, hq, hkv, d = 24, 4, 2, 8
    q, k, v = _rand((n, hq, d), 4), _rand((n, hkv, d), 5), _rand((n, hkv, d), 6)
    s, t = 9, 11
    got = oa.prefill_chunk(q[s:s + t], k, v, s)
    ref = brute_force(q[s:s + t], k, v, list(range(s, s + t)), 1.0 / math.sqrt(d))
    assert np.abs(got - ref).max() <= 1e-12
    got_d = oa.decode(q[5], k[:13], v[:13])
    ref_d = brute_force(q[5][None], k[:13], v[:13], [12], 1.0 / math.sqrt(d))[0]
    assert np.abs(got_d - ref_d).max() <= 1e-12


def _sdpa(q, k, v, positions):
    """torch SDPA (CPU, float64) with a boolean mask 'key j visible to row m'."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]   # [1, Hq, M, D]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    visible = torch.arange(k.shape[0])[None, :] <= torch.from_numpy(np.asarray(positions))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=visible, enable_gqa=q.shape[1] != k.shape[1])
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("n,hq,hkv,d", [(64, 4, 2, 64), (130, 8, 8, 32), (96, 8, 1, 16), (200, 32, 8, 128)])
def test_matches_torch_sdpa(n, hq, hkv, d):
    q, k, v = _rand((n, hq, d), 7), _rand((n, hkv, d), 8), _rand((n, hkv, d), 9)
    got = oa.prefill(q, k, v)
    ref = _sdpa(q, k, v, np.arange(n))
    assert np.abs(got - ref).max() <= 1e-12


def test_sdpa_is_causal_flag_agrees_for_square_case():
    # the square case can also use SDPA's own causal flag (no mask of ours)
    n, hq, d = 50, 4, 16
    q, k, v = _rand((n, hq, d), 10), _rand((n, hq, d), 11), _rand((n, hq, d), 12)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2).copy())[None], torch.from_numpy(k.transpose(1, 0, 2).copy())[None],
        torch.from_numpy(v.transpose(1, 0, 2).copy())[None], is_causal=True)
    ref = o[0].numpy().transpose(1, 0, 2)
    assert np.abs(oa.prefill(q, k, v) - ref).max() <= 1e-12


def test_single_key_returns_its_value_exactly():
    q, k, v = _rand((1, 4, 8), 13), _rand((1, 2, 8), 14), _rand((1, 2, 8), 15)
    out = oa.decode(q[0], k, v)
    assert np.array_equal(out[:2], np.broadcast_to(v[0, 0], (2, 8)))
    assert np.array_equal(out[2:], np.broadcast_to(v[0, 1], (2, 8)))


def test_zero_query_and_equal_keys_give_mean_of_visible_values():
    n, hq, hkv, d = 40, 4, 2, 16
    v = _rand((n, hkv, d), 16)
    k = _rand((n, hkv, d), 17)
    q0 = np.zeros((n, hq, d))
    out = oa.prefill(q0, k, v)
    for p in (0, 1, 17, n - 1):
        for h in range(hq):
            assert np.allclose(out[p, h], v[:p + 1, h // 2].mean(axis=0), rtol=0, atol=1e-14)
    k_same = np.broadcast_to(_rand((1, hkv, d), 18), (n, hkv, d)).copy()
    q = _rand((n, hq, d), 19)
    out = oa.prefill(q, k_same, v)
    assert np.allclose(out[n - 1, 3], v[:, 1].mean(axis=0), rtol=0, atol=1e-14)


def test_two_key_weights_are_one_to_three():
    # D=1, scale 1: scores 0 and ln 3 -> weights 1 and 3 -> (1*0 + 3*4)/4 = 3
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[0.0]], [[4.0]]])
    assert abs(oa.decode(q[0], k, v, scale=1.0)[0, 0] - 3.0) <= 1e-15
    # the first position sees only key 0
    assert oa.attend(q, k, v, np.array([0]), scale=1.0)[0, 0, 0] == 0.0


def test_gqa_head_map_is_contiguous_groups():
    n, d = 5, 4
    k = _rand((n, 2, d), 20)
    v = np.empty((n, 2, d))
    v[:, 0] = -7.0
    v[:, 1] = 7.0
    out = oa.decode(_rand((4, d), 21), k, v)
    assert np.allclose(out[:2], -7.0) and np.allclose(out[2:], 7.0)


def test_chunked_equals_one_shot():
    n, hq, hkv, d = 256, 4, 2, 64
    q, k, v = _rand((n, hq, d), 22), _rand((n, hkv, d), 23), _rand((n, hkv, d), 24)
    full = oa.prefill(q, k, v)
    for c in (64, 100, 256):
        parts = [oa.prefill_chunk(q[s:s + c], k, v, s) for s in range(0, n, c)]
        assert np.abs(np.concatenate(parts) - full).max() <= 1e-13


def test_decode_equals_last_prefill_row():
    n, hq, hkv, d = 77, 8, 2, 32
    q, k, v = _rand((n, hq, d), 25), _rand((n, hkv, d), 26), _rand((n, hkv, d), 27)
    full = oa.prefill(q, k, v)
    for length in (1, 13, 77):
        assert np.abs(oa.decode(q[length - 1], k[:length], v[:length]) - full[length - 1]).max() <= 1e-13


def test_rows_ignore_later_keys():
    n, hq, hkv, d = 60, 4, 2, 16
    q, k, v = _rand((n, hq, d), 28), _rand((n, hkv, d), 29), _rand((n, hkv, d), 30)
    base = oa.prefill(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[31:] += 100.0
    v2[31:] -= 50.0
    changed = oa.prefill(q, k2, v2)
    assert np.array_equal(base[:31], changed[:31])
    assert np.abs(base[31:] - changed[31:]).max() > 1.0


def test_shift_of_all_keys_leaves_output_unchanged():
    n, hq, hkv, d = 48, 4, 2, 16
    q, k, v = _rand((n, hq, d), 31), _rand((n, hkv, d), 32), _rand((n, hkv, d), 33)
    c = _rand((1, hkv, d), 34)
    assert np.abs(oa.prefill(q, k + c, v) - oa.prefill(q, k, v)).max() <= 1e-12


def test_scale_argument_scales_scores():
    n, hq, hkv, d = 30, 4, 2, 16
    q, k, v = _rand((n, hq, d), 35), _rand((n, hkv, d), 36), _rand((n, hkv, d), 37)
    a = oa.prefill(q * 2.5, k, v)
    b = oa.attend(q, k, v, np.arange(n), scale=2.5 / math.sqrt(d))
    assert np.abs(a - b).max() <= 1e-13


def test_error_metrics():
    m = oa.error_metrics(np.array([1.0, 2.0, 2.0]), np.array([1.0, 2.0, 3.0]))
    assert m["max_abs"] == 1.0
    assert abs(m["rel_l2"] - 1.0 / math.sqrt(14.0)) < 1e-15
