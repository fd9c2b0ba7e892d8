"""The tile-height rule the device applies for block_m = 0, restated in Python
(tests.parity.choice_rule), on the five workloads and on hand-made cases.  The
GPU tests check the device's choice against the same restatement; these pin
what it picks, so a change to the rule shows up on the CPU as well."""
import pytest

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from tests.parity import choice_rule


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
