"""Pins for the oracle's integer accounting (CPU only).

The oracle is checked against four things:
- the pages' printed worked examples (tests/golden/);
- closed forms;
- invariants that hold for every histogram;
- brute-force enumeration of rows and tiles on small histograms.
"""
import json
import os
from decimal import ROUND_HALF_EVEN, Decimal
from fractions import Fraction

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import accounting as acc

QS = (1, 2, 3, 8, 16, 32, 64, 128, 256)


def _pct(fr: Fraction, digits: str) -> str:
    """Format a fraction as a percentage with as many decimals as `digits` shows."""
    places = len(digits.split(".")[1]) if "." in digits else 0
    q = Decimal(1).scaleb(-places)
    v = (Decimal(fr.numerator) * 100 / Decimal(fr.denominator)).quantize(q, rounding=ROUND_HALF_EVEN)
    return str(v)


def golden_failures(golden_dir, mod=acc):
    """Every mismatch between `mod` and the pages' printed values."""
    with open(os.path.join(golden_dir, "padding_examples.json")) as f:
        g = json.load(f)
    bad = []
    for ex in g["examples"]:
        c = ex["counts"]
        if mod.useful_rows(c) != ex["U"]:
            bad.append(("U", ex["cite"]))
        if "active" in ex and mod.active_experts(c) != ex["active"]:
            bad.append(("active", ex["cite"]))
        for row in ex["per_q"]:
            q = row["q"]
            for t, r in row["rounded"].items():
                if mod.padded_rows([int(t)], q) != r:
                    bad.append(("rounded", q, t))
            if mod.padded_rows(c, q) != row["P"]:
                bad.append(("P", q, ex["cite"]))
            if "padding" in row and mod.padding_rows(c, q) != row["padding"]:
                bad.append(("padding", q))
            if _pct(mod.padding_fraction(c, q), row["fraction_pct"]) != row["fraction_pct"]:
                bad.append(("fraction", q, ex["cite"]))
        for q, share in ex.get("useful_share_pct", {}).items():
            if _pct(mod.useful_share(c, int(q)), share) != share:
                bad.append(("share", q))
    e = g["effective_experts"]
    nu = float(mod.effective_experts(g["examples"][0]["counts"]))
    if not (e["near_uniform_above"] < nu < e["near_uniform_below"]):
        bad.append(("eff near-uniform", nu))
    conc = mod.effective_experts(g["examples"][1]["counts"])
    if _pct(conc / 100, e["concentrated_2dp"]) != e["concentrated_2dp"]:
        bad.append(("eff concentrated", float(conc)))
    return bad


def test_pages_worked_examples(golden_dir):
    assert golden_failures(golden_dir) == []


def test_issue_histogram_total(golden_dir):
    with open(os.path.join(golden_dir, "issue_histogram.json")) as f:
        g = json.load(f)
    assert len(g["counts"]) == g["experts"]
    assert acc.useful_rows(g["counts"]) == g["U"]
    # the issue's point: big tiles waste a large share on this histogram
    assert acc.padding_fraction(g["counts"], 256) > Fraction(1, 3)
    assert acc.padding_fraction(g["counts"], 16) < Fraction(1, 20)


class _Mutant:
    """The accounting module with one plausible mistake planted in it."""

    def __init__(self, **overrides):
        self.__dict__.update({k: getattr(acc, k) for k in dir(acc) if not k.startswith("__")})
        self.__dict__.update(overrides)


def _p_floor(counts, q):
    return sum(q * (int(t) // q) for t in counts)


def _p_count_inactive(counts, q):
    return sum(q * max(1, acc.ceil_div(int(t), q)) for t in counts)


def _frac_over_u(counts, q):
    u = acc.useful_rows(counts)
    return Fraction(acc.padded_rows(counts, q) - u, u)


def _eff_wrong_power(counts):
    return Fraction(acc.useful_rows(counts) ** 2, sum(int(t) for t in counts) or 1)


def _eff_sq_over_u(counts):
    return Fraction(acc.sum_squares(counts), acc.useful_rows(counts))


@pytest.mark.parametrize("mutant", [
    dict(padded_rows=_p_floor),
    dict(padded_rows=_p_count_inactive),
    dict(padding_fraction=_frac_over_u),
    dict(effective_experts=_eff_wrong_power),
    dict(effective_experts=_eff_sq_over_u),
])
def test_pins_catch_planted_mistakes(golden_dir, mutant):
    m = _Mutant(**mutant)
    if "padded_rows" in mutant:
        # derived quantities follow the mutated P
        m.padding_rows = lambda c, q: m.padded_rows(c, q) - acc.useful_rows(c)
        m.padding_fraction = lambda c, q: Fraction(m.padded_rows(c, q) - acc.useful_rows(c),
                                                   max(1, m.padded_rows(c, q)))
        m.useful_share = lambda c, q: Fraction(acc.useful_rows(c), max(1, m.padded_rows(c, q)))
    assert golden_failures(golden_dir, m) != []


# ------------------------------------------------------------- brute force


def brute_padded_rows(counts, q):
    """Enumerate every row, collect the distinct tiles it lands in, count q rows per tile."""
    tiles = set()
    for e, t in enumerate(counts):
        for r in range(t):
            tiles.add((e, r // q))
    return q * len(tiles)


hist = st.lists(st.integers(min_value=0, max_value=300), min_size=1, max_size=12)


@settings(max_examples=300, deadline=None)
@given(hist, st.sampled_from(QS))
def test_padded_rows_brute_force(counts, q):
    assert acc.padded_rows(counts, q) == brute_padded_rows(counts, q)
    assert acc.tiles_for(counts, q) == brute_padded_rows(counts, q) // q


@settings(max_examples=300, deadline=None)
@given(hist, st.sampled_from(QS), st.sampled_from((1, 4, 16, 128)))
def test_tile_list_covers_each_row_once(counts, q, align):
    tiles = acc.tile_list(counts, q, align)
    offs = acc.segment_offsets(counts, align)
    covered = []
    for e, i, start, valid in tiles:
        assert 1 <= valid <= q and counts[e] > 0
        assert start == offs[e] + i * q
        covered.extend(range(start, start + valid))
    expect = [offs[e] + r for e, t in enumerate(counts) for r in range(t)]
    assert covered == expect                        # canonical order, no gaps, no repeats
    assert sum(v for *_, v in tiles) == acc.useful_rows(counts)
    assert len(tiles) == acc.tiles_for(counts, q)
    assert [t[:2] for t in tiles] == sorted(t[:2] for t in tiles)


@settings(max_examples=300, deadline=None)
@given(hist, st.sampled_from(QS))
def test_invariants(counts, q):
    U, P = acc.useful_rows(counts), acc.padded_rows(counts, q)
    assert P >= U and P % q == 0
    assert P - U <= (q - 1) * acc.active_experts(counts)
    assert acc.padded_rows(counts, 2 * q) >= P
    assert acc.padded_rows(counts, 1) == U
    f = acc.padding_fraction(counts, q)
    assert 0 <= f < 1
    if U:
        eff = acc.effective_experts(counts)
        assert 1 <= eff <= acc.active_experts(counts)          # Cauchy-Schwarz


@settings(max_examples=100, deadline=None)
@given(st.integers(1, 64), st.integers(1, 500), st.sampled_from(QS))
def test_uniform_closed_forms(active, m, q):
    counts = [m] * active + [0] * 3
    assert acc.padded_rows(counts, q) == active * q * acc.ceil_div(m, q)
    assert acc.effective_experts(counts) == active


def test_single_expert_and_empty():
    assert acc.effective_experts([0, 57, 0]) == 1
    assert acc.effective_experts([0, 0]) == 0
    assert acc.padded_rows([0, 0], 16) == 0
    assert acc.padding_fraction([0, 0], 16) == 0
    assert acc.tile_list([0, 0, 0], 32) == []


def test_m_occupancy_issue_formula():
    # tiles = ceil(M/B_M), needed = M/B_M, occupancy = needed/tiles
    assert acc.m_occupancy(256, 128) == 1
    assert acc.m_occupancy(100, 128) == Fraction(100, 128)
    assert acc.m_occupancy(129, 128) == Fraction(129, 256)
    assert acc.m_occupancy(0, 128) is None
    counts = [4, 1026, 1799, 0, 16]
    num = sum(acc.m_occupancy(t, 64) * acc.ceil_div(t, 64) for t in counts if t)
    assert num / acc.tiles_for(counts, 64) == Fraction(acc.useful_rows(counts), acc.padded_rows(counts, 64))


def test_average_assignments():
    assert acc.average_assignments(4096, 8, 256) == 128


@settings(max_examples=300, deadline=None)
@given(hist, st.sampled_from((1, 4, 16, 128)))
def test_per_expert_tile_list(counts, align):
    """Per-expert heights: every row of every expert in exactly one tile, each
    tile's height class non-increasing along the list, expert order inside a
    class, and each expert's tiles all full (256) except its last."""
    tl = acc.tile_list_per_expert(counts, align)
    offs = acc.segment_offsets(counts, align)
    covered = {}
    for e, i, r0, rv in tl:
        assert 1 <= rv <= 256 and r0 == offs[e] + 256 * i
        for r in range(r0, r0 + rv):
            assert r not in covered
            covered[r] = e
        if i < acc.ceil_div(counts[e], 256) - 1:
            assert rv == 256
    assert len(covered) == sum(counts)
    assert sorted(tl) == sorted(acc.tile_list(counts, 256, align))
    cls = [0 if rv > 128 else (1 if rv > 64 else 2) for _, _, _, rv in tl]
    assert cls == sorted(cls)
    for c in (0, 1, 2):
        keys = [(e, i) for (e, i, _, _), k in zip(tl, cls) if k == c]
        assert keys == sorted(keys)


def test_per_expert_tile_list_example():
    """Counts [300, 0, 70, 513, 10]: full tiles first, then the 65..128-row
    remainders (70 of expert 2), then the 1..64-row ones (44, 1, 10)."""
    tl = acc.tile_list_per_expert([300, 0, 70, 513, 10])
    assert tl == [(0, 0, 0, 256), (3, 0, 370, 256), (3, 1, 626, 256),
                  (2, 0, 300, 70),
                  (0, 1, 256, 44), (3, 2, 882, 1), (4, 0, 883, 10)]
