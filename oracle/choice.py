"""The tile-height rule for block_m = 0, written out plainly (test
infrastructure only).

"MoE GroupGEMM padding under expert skew", section "Padding is not the whole
cost model", says padding alone does not pick the kernel and the candidates
must be measured; section "Adapt kernels without adding a CPU stall" asks for
the choice on the GPU.  The library's rule (include/moegg.h, documented there
and in the design notes) is an integer planning model; this module computes it
from its definition, in Python integers, from the exact tile counts of the
accounting module:

    rounds(tiles)  = ceil(tiles * n_col_tiles / 256)      (256 CUs, one tile each)
    cost(q)        = rounds(tiles(q)) * (q + 64)           q in {64, 128, 256}
    uniform        = the q of least cost, ties to the larger q
    per-expert     = rounds(n_256) * 320 + rounds(n_128) * 192 + rounds(n_64) * 128
                     where n_128 / n_64 count the experts whose last 256-row tile
                     holds 65..128 / 1..64 rows and n_256 the other 256-row tiles
    choice         = per-expert heights if strictly cheaper than the uniform
                     choice, else the uniform choice.

Whether the choice is the fastest is a measurement, not a definition: its
optimality is parity unpinned.  What is pinned is that the device takes exactly
this decision (tests/test_gpu_parity.py) and what it picks on hand-worked cases
(tests/test_choice_rule.py).
"""
from __future__ import annotations

from typing import Sequence

from . import accounting as acc

PER_EXPERT = -1            # the library's value for per-expert tile heights


def rounds(tiles: int, n_col_tiles: int) -> int:
    return acc.ceil_div(tiles * n_col_tiles, 256)


def cost_uniform(counts: Sequence[int], q: int, n_col_tiles: int) -> int:
    return rounds(acc.tiles_for(counts, q), n_col_tiles) * (q + 64)


def cost_per_expert(counts: Sequence[int], n_col_tiles: int) -> int:
    last = [m - (acc.ceil_div(m, 256) - 1) * 256 for m in counts if m > 0]   # rows of each last tile
    n128 = sum(1 for r in last if 64 < r <= 128)
    n64 = sum(1 for r in last if r <= 64)
    n256 = acc.tiles_for(counts, 256) - n128 - n64
    return (rounds(n256, n_col_tiles) * (256 + 64) + rounds(n128, n_col_tiles) * (128 + 64)
            + rounds(n64, n_col_tiles) * (64 + 64))


def choose(counts: Sequence[int], n_col_tiles: int) -> int:
    costs = {q: cost_uniform(counts, q, n_col_tiles) for q in (64, 128, 256)}
    best = min(costs.values())
    uniform = max(q for q, c in costs.items() if c == best)
    return PER_EXPERT if cost_per_expert(counts, n_col_tiles) < best else uniform
