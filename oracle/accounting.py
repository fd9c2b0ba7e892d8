"""Exact integer padding accounting and tile lists (test infrastructure only).

Every quantity here is a Python int or a fractions.Fraction, so nothing is
rounded.

Sources:
- "MoE GroupGEMM padding under expert skew", section "Calculate padded token
  columns": P, U, the padding count and the padding fraction.  Its token
  tile width q is the tile height B_M here, because tokens are rows.
- Same page, section "Summarize skew without losing the histogram": effective
  experts, and the average assignments per expert.
- Same page, section "Grouped execution does not require padded experts": the
  work list built from each expert's actual count.  Zero-sized experts get no
  work; the last tile of an expert covers only its remaining rows.
- DeepGEMM issue "Query on performance-modeling of MoE Grouped GEMM",
  "Background": M-occupancy of one GEMM problem.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

CANDIDATE_Q = (8, 16, 32, 64, 128, 256)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def useful_rows(counts: Sequence[int]) -> int:
    """U: the sum of the unrounded per-expert counts."""
    return sum(int(t) for t in counts)


def padded_rows(counts: Sequence[int], q: int) -> int:
    """P(q): each active expert's count rounded up to a multiple of q, summed.

    An inactive expert (count 0) contributes zero.
    """
    if q < 1:
        raise ValueError("tile height must be >= 1")
    total = 0
    for t in counts:
        t = int(t)
        if t > 0:
            total += q * ceil_div(t, q)
    return total


def padding_rows(counts: Sequence[int], q: int) -> int:
    """P - U."""
    return padded_rows(counts, q) - useful_rows(counts)


def padding_fraction(counts: Sequence[int], q: int) -> Fraction:
    """(P - U) / P; 0 when nothing is routed (P = 0)."""
    p = padded_rows(counts, q)
    return Fraction(0) if p == 0 else Fraction(p - useful_rows(counts), p)


def useful_share(counts: Sequence[int], q: int) -> Fraction:
    """U / P, the useful share of executed rows (1 when P = 0)."""
    p = padded_rows(counts, q)
    return Fraction(1) if p == 0 else Fraction(useful_rows(counts), p)


def active_experts(counts: Sequence[int]) -> int:
    return sum(1 for t in counts if int(t) > 0)


def sum_squares(counts: Sequence[int]) -> int:
    return sum(int(t) * int(t) for t in counts)


def effective_experts(counts: Sequence[int]) -> Fraction:
    """U^2 / sum_e t_e^2; 0 when nothing is routed."""
    s2 = sum_squares(counts)
    return Fraction(0) if s2 == 0 else Fraction(useful_rows(counts) ** 2, s2)


def average_assignments(concurrency: int, top_k: int, experts: int) -> Fraction:
    """Mean routed rows per expert: tokens in flight, each routed to top_k experts,
    spread over the experts (the padding page's companion average)."""
    return Fraction(concurrency * top_k, experts)


def m_occupancy(M: int, block_m: int) -> Optional[Fraction]:
    """One GEMM problem's M-occupancy: (M / B_M) / ceil(M / B_M).

    M = 0 uses no tile and has no occupancy (None).
    """
    tiles = ceil_div(M, block_m)
    if tiles == 0:
        return None
    return Fraction(M, block_m) / tiles


def tiles_for(counts: Sequence[int], q: int) -> int:
    return sum(ceil_div(int(t), q) for t in counts if int(t) > 0)


def segment_offsets(counts: Sequence[int], seg_align: int) -> List[int]:
    """Start row of each expert's segment in the contiguous layout, plus the end.

    offsets[e] = sum over j < e of align_up(count_j, seg_align).
    """
    offs = [0]
    for t in counts:
        offs.append(offs[-1] + ceil_div(int(t), seg_align) * seg_align)
    return offs


def tile_list(counts: Sequence[int], block_m: int, seg_align: int = 1,
              base_rows: Optional[Sequence[int]] = None) -> List[Tuple[int, int, int, int]]:
    """The flat work list: (expert, tile index in expert, first row, valid rows).

    The order is expert ascending, then tile index ascending.  Experts with
    zero rows emit nothing.  base_rows overrides the segment starts; the masked
    layout uses e * cap.
    """
    starts = segment_offsets(counts, seg_align) if base_rows is None else list(base_rows)
    out = []
    for e, t in enumerate(counts):
        t = int(t)
        for i in range(ceil_div(t, block_m) if t > 0 else 0):
            out.append((e, i, starts[e] + i * block_m, min(block_m, t - i * block_m)))
    return out


def tile_list_per_expert(counts: Sequence[int], seg_align: int = 1) -> List[Tuple[int, int, int, int]]:
    """Per-expert tile heights: the 256-row tile list, regrouped by the height of
    the smallest tile in {64, 128, 256} that holds each tile's valid rows --
    first the tiles with more than 128 valid rows, then those with 65..128,
    then 1..64, each group keeping the (expert, tile) order.

    Only an expert's last tile can hold fewer than 129 rows, so every expert
    keeps its full tiles and gets one remainder tile sized to its remainder (the
    padding page, "Calculate padded token columns": the padding of an expert is
    set by its own count and the tile height it runs with).
    """
    full = tile_list(counts, 256, seg_align)
    return ([t for t in full if t[3] > 128] + [t for t in full if 64 < t[3] <= 128]
            + [t for t in full if t[3] <= 64])


def summary(counts: Sequence[int], qs: Sequence[int] = CANDIDATE_Q) -> Dict:
    """Every accounting quantity for one histogram, exactly."""
    return {
        "U": useful_rows(counts),
        "P": {q: padded_rows(counts, q) for q in qs},
        "tiles": {q: tiles_for(counts, q) for q in qs},
        "active": active_experts(counts),
        "sum_sq": sum_squares(counts),
        "effective_experts": effective_experts(counts),
    }
