"""Distribution-aware tile-height selection by exemplar matching, written out
plainly (test infrastructure only).

Follows "MoE GroupGEMM padding under expert skew", section "Adapt kernels
without adding a CPU stall": the per-expert counts are sorted and normalized,
matched against exemplars tuned offline, and a guard keeps neighbouring
histograms from switching the kernel.  The library's exemplar call states the
exact descriptor, distance and hysteresis rule (include/moegg.h); this module
computes the same quantities from their definitions, in Python integers:

    size class   4 * floor(log2 U) + the two bits of U after its leading one
                 (0 for U = 0), i.e. floor(4 * U / 2^floor(log2 U)) - 4 added
                 to 4 * floor(log2 U);
    lorenz[i]    floor(65536 * (sum of the k_i largest counts) / U),
                 k_i = ceil(G * (i + 1) / 8), i = 0..7 (all 0 when U = 0);
    distance     sum_i |lorenz[i] - ex.lorenz[i]| + 8192 * |size - ex.size|;
    choice       nearest exemplar, ties to the lower index; the previous
                 choice is kept while its distance <= nearest + hysteresis.

Which exemplar is *best* for speed is a measurement, not a definition: the
optimality of a choice is parity unpinned.  What is pinned is that the device
takes exactly this decision from the same table.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

SIZE_WEIGHT = 8192
LORENZ_POINTS = 8
ONE = 1 << 16


def size_class(U: int) -> int:
    if U <= 0:
        return 0
    e = U.bit_length() - 1                 # floor(log2 U)
    return 4 * e + (4 * U) // (1 << e) - 4


def lorenz(counts: Sequence[int]) -> List[int]:
    m = [max(0, int(c)) for c in counts]
    U = sum(m)
    if U == 0:
        return [0] * LORENZ_POINTS
    G = len(m)
    desc = sorted(m, reverse=True)
    out = []
    for i in range(LORENZ_POINTS):
        k = -(-G * (i + 1) // LORENZ_POINTS)   # ceil
        out.append(sum(desc[:k]) * ONE // U)
    return out


def descriptor(counts: Sequence[int]) -> Tuple[int, List[int]]:
    U = sum(max(0, int(c)) for c in counts)
    return size_class(U), lorenz(counts)


def distance(desc: Tuple[int, List[int]], ex: Sequence[int]) -> int:
    """ex: one table row (size_class, lorenz[0..7], block_m)."""
    sc, lor = desc
    return SIZE_WEIGHT * abs(sc - ex[0]) + sum(abs(a - b) for a, b in zip(lor, ex[1:9]))


def select(counts: Sequence[int], table: Sequence[Sequence[int]], hysteresis: int = 0,
           prev: Optional[int] = None) -> Tuple[int, int]:
    """(chosen exemplar index, its distance) for one call; prev is the index the
    previous call on the same workspace chose (None for a fresh workspace)."""
    desc = descriptor(counts)
    dists = [distance(desc, ex) for ex in table]
    best = min(range(len(table)), key=lambda x: (dists[x], x))
    if prev is not None and 0 <= prev < len(table) and dists[prev] <= dists[best] + hysteresis:
        return prev, dists[prev]
    return best, dists[best]
