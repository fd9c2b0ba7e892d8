"""Pins of the exemplar selector's oracle (oracle/select.py) against values
worked by hand from its definition (include/moegg.h, after the padding page's
"Adapt kernels without adding a CPU stall"), special cases and invariants."""
import json
import random

import pytest

import moe_grouped_gemm_sizes_amd as mg
from oracle import select as sel


@pytest.mark.parametrize("U,expect", [
    (0, 0), (1, 0), (2, 4), (3, 6), (4, 8), (5, 9), (6, 10), (7, 11), (8, 12),
    (132, 28 + 0),          # 128 + 4: bits after the leading one are 00
    (8048, 48 + 3),         # 4096 <= 8048 < 8192, 8048 = 0b1 11 1101110000
    (32768, 60), (49152, 62),
])
def test_size_class_by_hand(U, expect):
    assert sel.size_class(U) == expect


def test_lorenz_worked_examples():
    # the padding page's two eight-expert histograms (U = 132)
    assert sel.lorenz([17, 17, 17, 17, 16, 16, 16, 16]) == [
        17 * 65536 // 132, 34 * 65536 // 132, 51 * 65536 // 132, 68 * 65536 // 132,
        84 * 65536 // 132, 100 * 65536 // 132, 116 * 65536 // 132, 65536]
    assert sel.lorenz([100, 32, 0, 0, 0, 0, 0, 0]) == [100 * 65536 // 132] + [65536] * 7


def test_lorenz_special_cases():
    assert sel.lorenz([0, 0, 0]) == [0] * 8                   # nothing routed
    assert sel.lorenz([0, 9, 0, 0]) == [65536] * 8            # one hot expert
    assert sel.lorenz([5] * 64) == [65536 * (i + 1) // 8 for i in range(8)]   # uniform
    # G = 5: k_i = ceil(5 (i + 1) / 8) = 1, 2, 2, 3, 4, 4, 5, 5
    c = [1, 2, 3, 4, 10]
    tops = [10, 14, 14, 17, 19, 19, 20, 20]
    assert sel.lorenz(c) == [t * 65536 // 20 for t in tops]


def test_lorenz_is_permutation_invariant_and_monotone():
    rng = random.Random(3)
    for _ in range(50):
        c = [rng.choice([0, 1, 7, 64, 300, 2000]) for _ in range(rng.randint(1, 80))]
        c2 = list(c)
        rng.shuffle(c2)
        L = sel.lorenz(c)
        assert L == sel.lorenz(c2)
        assert all(a <= b for a, b in zip(L, L[1:]))
        if sum(c):
            # the largest k counts hold at least k / G of the rows
            G = len(c)
            assert L[-1] == 65536
            assert all(L[i] >= 65536 * -(-G * (i + 1) // 8) // G for i in range(8))


def test_distance_and_choice():
    table = [[28, *sel.lorenz([17, 17, 17, 17, 16, 16, 16, 16]), 64],
             [28, *sel.lorenz([100, 32, 0, 0, 0, 0, 0, 0]), 256],
             [60, *sel.lorenz([4096] * 8), mg.BLOCK_M_PER_EXPERT]]
    # each exemplar's own histogram is at distance 0 and picks it
    assert sel.select([17, 17, 17, 17, 16, 16, 16, 16], table) == (0, 0)
    assert sel.select([32, 0, 100, 0, 0, 0, 0, 0], table) == (1, 0)
    assert sel.select([4096] * 8, table) == (2, 0)
    # size only: one quarter-octave step costs 8192
    assert sel.distance(sel.descriptor([8] * 8), [sel.size_class(64) + 1, *sel.lorenz([1] * 8), 64]) == 8192
    # ties go to the lower index
    assert sel.select([1] * 8, [table[0], table[0]]) == (0, sel.distance(sel.descriptor([1] * 8), table[0]))


def test_hysteresis_keeps_the_previous_choice_within_the_margin():
    table = [[40, *sel.lorenz([1] * 8), 64], [40, *sel.lorenz([3, 1, 1, 1, 1, 1, 1, 1]), 128]]
    h = [2, 1, 1, 1, 1, 1, 1, 1]                  # between the two exemplars
    d0 = sel.distance(sel.descriptor(h), table[0])
    d1 = sel.distance(sel.descriptor(h), table[1])
    assert d1 < d0                                 # nearest is exemplar 1
    assert sel.select(h, table, hysteresis=0, prev=0) == (1, d1)
    assert sel.select(h, table, hysteresis=d0 - d1, prev=0) == (0, d0)        # kept: within the margin
    assert sel.select(h, table, hysteresis=d0 - d1 - 1, prev=0) == (1, d1)    # switched: one unit past it
    assert sel.select(h, table, hysteresis=10 ** 9, prev=None) == (1, d1)     # fresh workspace
    assert sel.select(h, table, hysteresis=10 ** 9, prev=7) == (1, d1)        # out-of-range previous


def test_planted_mistake_in_the_oracle_fails_a_pin():
    """floor instead of ceil for k_i changes the G = 5 value pinned above."""
    c = [1, 2, 3, 4, 10]
    desc = sorted(c, reverse=True)
    wrong = [sum(desc[:5 * (i + 1) // 8]) * 65536 // 20 for i in range(8)]
    assert wrong != sel.lorenz(c)


@pytest.mark.parametrize("dtype", sorted(mg.EXEMPLAR_TABLE_PATHS))
def test_shipped_exemplar_table_is_well_formed(dtype):
    with open(mg.EXEMPLAR_TABLE_PATHS[dtype]) as f:
        t = json.load(f)
    rows = t["exemplars"]
    assert 1 <= len(rows) <= 256
    for r in rows:
        assert r["block_m"] in (64, 128, 256, mg.BLOCK_M_PER_EXPERT)
        assert len(r["lorenz"]) == 8 and all(0 <= v <= 65536 for v in r["lorenz"])
        assert r["lorenz"] == sorted(r["lorenz"])
        # the stored descriptor is the one of the stored histogram
        assert (r["size_class"], r["lorenz"]) == (sel.size_class(sum(r["counts"])), sel.lorenz(r["counts"]))
        assert r["block_m"] == int(min(r["times_ms"], key=r["times_ms"].get))


def test_exemplar_table_per_dtype():
    """One table per operand type; the device tensor has one moegg_exemplar_t row per entry."""
    for dtype, path in mg.EXEMPLAR_TABLE_PATHS.items():
        with open(path) as f:
            n = len(json.load(f)["exemplars"])
        assert tuple(mg.exemplar_table(device="cpu", dtype=dtype).shape) == (n, mg.EXEMPLAR_FIELDS)
    with pytest.raises(ValueError):
        mg.exemplar_table(device="cpu", dtype="fp16")
