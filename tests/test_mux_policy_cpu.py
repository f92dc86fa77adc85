"""The library's multiplexing policy (pure host functions) against the oracle.

The oracle's rules are themselves pinned to the tables printed on the PD
multiplexing page ("SGLang's PD multiplexing": split levels for H100, A100
and H20, the level picked per decode batch size, layers per round); here
the C implementation must reproduce the same tables and agree with the
oracle over a sweep of device sizes, grids and batch sizes.
"""

import ctypes as C
import os

import pytest

from conftest import read_golden
from oracle import policy

lib_mod = pytest.importorskip("decode_paged_kv_amd._lib")


def _lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libpkv.so not built")
    return lib_mod.load()


def _groups(lib, total, min_part, grid, min_decode, group_num=8):
    p, d, n = (C.c_int32 * 64)(), (C.c_int32 * 64)(), C.c_int32()
    assert lib.pkv_mux_policy_groups_grid(total, min_part, grid, min_decode, group_num, p, d, 64, C.byref(n)) == 0
    return [(p[i], d[i]) for i in range(n.value)]


def test_pages_tables_from_the_library():
    lib = _lib()
    grids = {9: (8, 8), 8: (4, 2)}
    for rec in read_golden("mux_policy_demo.txt"):
        if rec[0] == "groups":
            sms, cc = int(rec[2]), int(rec[3])
            mp, g = grids[cc]
            got = _groups(lib, sms, mp, g, 16)
            assert got == [tuple(int(x) for x in f.split(":")) for f in rec[4:]]
        elif rec[0] == "choose":
            assert lib.pkv_mux_policy_choose(8, int(rec[1]), int(rec[2]), 36) == int(rec[3])
        elif rec[0] == "layers":
            assert lib.pkv_mux_policy_layers_per_round(int(rec[1]), int(rec[2]), 65536) == int(rec[3])


def test_mi355x_levels():
    lib = _lib()
    g = _groups(lib, 256, 8, 8, 32)
    assert g == policy.mi355x_stream_groups()
    assert g[lib.pkv_mux_policy_choose(len(g), 128, 1, 36)] == (128, 128)
    assert lib.pkv_mux_policy_layers_per_round(32768, 32, 65536) == 2
    assert lib.pkv_mux_policy_layers_per_round(16384, 32, 65536) == 4


@pytest.mark.parametrize("total", [64, 78, 108, 132, 192, 256, 304])
@pytest.mark.parametrize("grid", [2, 4, 8, 16])
@pytest.mark.parametrize("min_decode", [8, 16, 32])
@pytest.mark.parametrize("group_num", [3, 5, 8, 10])
def test_sweep_matches_oracle(total, grid, min_decode, group_num):
    lib = _lib()
    assert _groups(lib, total, grid, grid, min_decode, group_num) == \
        policy.stream_groups(total, grid, grid, min_decode, group_num)


def test_choose_and_layers_sweep():
    lib = _lib()
    for n in (3, 5, 8, 12):
        for bs in range(0, 300, 7):
            for hp in (0, 1):
                for div in (12, 24, 36, 50):
                    assert lib.pkv_mux_policy_choose(n, bs, hp, div) == policy.choose_level(n, bs, bool(hp), div)
    for tokens in (1, 100, 512, 4096, 16384, 32768, 65536, 100000, 131072):
        for layers in (1, 32, 36, 64, 80):
            for budget in (2048, 65536):
                assert lib.pkv_mux_policy_layers_per_round(tokens, layers, budget) == \
                    policy.layers_per_round(tokens, layers, budget)


def test_policy_rejects_bad_arguments():
    lib = _lib()
    n = C.c_int32()
    assert lib.pkv_mux_policy_groups_grid(0, 8, 8, 32, 8, None, None, 0, C.byref(n)) == -1
    assert lib.pkv_mux_policy_choose(2, 1, 1, 36) == -1
    assert lib.pkv_mux_policy_layers_per_round(0, 32, 65536) == -1


def test_manual_divisions_pins_and_library():
    lib = _lib()
    arr = lambda t: (C.c_int32 * len(t))(*t)  # noqa: E731
    # the page's exercise: thresholds that make 24 decode requests pick the
    # last of 6 split levels, as decode_bs_divisor = 24 does
    t24 = [4, 8, 12, 16, 20, 24]
    assert policy.choose_level_manual(8, 24, True, t24) == 6
    assert policy.choose_level(8, 24, True, 24) == 6
    # thresholds ceil(i * divisor / levels) reproduce the divisor rule at every batch size
    for div in (24, 36, 100):
        t = [-(-i * div // 6) for i in range(1, 7)]
        for bs in range(0, 300):
            for hp in (False, True):
                assert policy.choose_level_manual(8, bs, hp, t) == policy.choose_level(8, bs, hp, div)
    # below the first threshold: the first split level; decode only / prefill only: the whole device
    assert policy.choose_level_manual(8, 1, True, [10, 20, 30, 40, 50, 60]) == 1
    assert policy.choose_level_manual(8, 5, False, t24) == 7
    assert policy.choose_level_manual(8, 0, True, t24) == 0
    # library against the oracle, on uneven thresholds too
    for t in (t24, [1, 1, 5, 9, 9, 200], [3, 6, 64, 65, 128, 129]):
        for bs in range(0, 260, 3):
            for hp in (0, 1):
                assert lib.pkv_mux_policy_choose_manual(8, bs, hp, arr(t)) == policy.choose_level_manual(8, bs, bool(hp), t)
    assert lib.pkv_mux_policy_choose_manual(8, 5, 1, arr([4, 3, 5, 6, 7, 8])) == -1     # decreasing
    assert lib.pkv_mux_policy_choose_manual(8, 5, 1, arr([0, 3, 5, 6, 7, 8])) == -1     # below 1
