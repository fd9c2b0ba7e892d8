"""The tile-height rule the device applies for block_m = 0, as the oracle
writes it out (oracle/choice.py), on the five workloads and on cases worked by
hand.  The GPU tests check the device's choice against the same function;
these pin what it picks, so a change to the rule shows up on the CPU as well."""
import pytest

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle.choice import PER_EXPERT, choose as choice_rule


def test_per_expert_value_is_the_librarys():
    assert PER_EXPERT == mg.BLOCK_M_PER_EXPERT


def test_hand_worked_costs():
    from oracle import choice as oc
    # [17]*4 + [16]*4, one column tile: 8 tiles at every height, one round each
    h = [17, 17, 17, 17, 16, 16, 16, 16]
    assert [oc.cost_uniform(h, q, 1) for q in (64, 128, 256)] == [128, 192, 320]
    # per expert: every last tile holds <= 64 rows -> 8 tiles of 64 rows, one round of 128
    assert oc.cost_per_expert(h, 1) == 128
    assert choice_rule(h, 1) == 64                  # per-expert only ties: the uniform choice stays
    # 300 rows, 16 column tiles: 64 -> 5 tiles x 16 = 80 items, 1 round x 128; per expert: one 256 tile +
    # a 44-row tail -> 16 + 16 items, 1 round x 320 + 1 round x 128 = 448
    assert oc.cost_uniform([300], 64, 16) == 128 and oc.cost_per_expert([300], 16) == 448


@pytest.mark.parametrize("n, expected", [(1, 64), (2, 128), (3, mg.BLOCK_M_PER_EXPERT)])
def test_workload_choices(n, expected):
    w = wl.workload(n)
    assert choice_rule(w.counts, w.N // 256) == expected


def test_uniform_ties_go_to_the_larger_height():
    # 256 rows, one column tile: every height is one round of tiles, (q + 64) decides: 64 wins outright
    assert choice_rule([256], 1) == 64
    # 64 experts x 256 rows, 16 column tiles: 64 -> 1024 items (4 rounds x 128) = 512, 128 -> 512 items
    # (2 rounds x 192) = 384, 256 -> 256 items (1 round x 320) = 320
    assert choice_rule([256] * 64, 16) == 256


def test_per_expert_needs_a_strictly_lower_cost():
    # all remainders full: per-expert heights are the 256 list itself and tie with it
    assert choice_rule([512] * 8, 16) == 256
    # one long expert plus short ones: per-expert puts the remainders on 64-row tiles
    counts = [256 * 30 + 20] + [20] * 40
    assert choice_rule(counts, 16) == mg.BLOCK_M_PER_EXPERT


def test_empty_histogram():
    assert choice_rule([0, 0, 0], 16) == 256
