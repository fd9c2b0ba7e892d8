"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same bits, compare.

Bars:
- integer work (stats, tile lists): bit-exact;
- bf16 inputs: ||C - C_ref||_F / ||C_ref||_F <= 2e-3;
- fp8 e4m3 inputs with fp32 group scales: <= 2e-2;
- fp32 outputs (K-grouped dW): <= 1e-4.
And, for every element of every compared row (check_gemm):
- bf16 output of one GEMM:  |C - C_ref| <= 2^-8 |C_ref| + 2^-10 rms(row)
  (the one round-to-nearest-even to bf16 moves a value by at most half an ulp,
  2^-8 of its magnitude; the rms term holds the fp32 accumulation error, about
  1e-5 of the row's rms at K = 7168, with a wide margin);
- fp32 output:              |C - C_ref| <= 2^-20 |C_ref| + 2^-12 rms(row);
- fp32 output from e4m3 operands (K-grouped dW): the same plus 2^-13 S, where
  S = sum over the reduction of |x * y * scales| (the oracle on the operands'
  magnitudes).  The fp8 MFMA sums a group's 128 products at less than fp32
  precision: on MI355X a one-group dW element came out 3.8e-5 S (2^-14.7) from
  its exact value, about 40 times what an fp32 sum of those 66 terms could be
  off, and that error grows with S, not with the row's rms;
- second GEMM of the expert MLP, whose input H was rounded once more:
  bf16 H: |y - y_ref| <= 2^-8 |y_ref| + 2^-5 rms(row);
  e4m3 H (y_ref from the oracle's own codes, about 0.15 % of which sit one
  e4m3 step, up to 2^-3 of the value, from the GPU's): 2^-8 |y_ref| + 2^-4 rms(row).
Measured on CPU emulations of the same arithmetic (fp32 accumulation, one
final rounding) at K = 7168: the largest element uses 0.96, 0.94 and 0.38 of
the first three; on MI355X the single GEMMs reach 0.94 of theirs and the e4m3
chain at full size 0.60 of its own.  One wrong 16 x 16 MFMA block, or one K step of it missing,
moves its elements by a sizeable fraction of the row's rms and fails them.
"""
from __future__ import annotations

import random
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import accounting as acc
from oracle import choice as ochoice
from oracle import gemm as og

TOL = {"bf16": 2e-3, "fp8": 2e-2, "fp32": 1e-4}
ELEM = {"bf16": (2.0 ** -8, 2.0 ** -10), "fp32": (2.0 ** -20, 2.0 ** -12), "chain": (2.0 ** -8, 2.0 ** -5),
        "chain_e4m3": (2.0 ** -8, 2.0 ** -4)}
ABS_SUM_FP8 = 2.0 ** -13        # coefficient of S for fp32 outputs from e4m3 operands
SENTINEL_BITS = 0x7BAD          # a finite bf16 pattern the kernels never produce here by chance


def elementwise_ratio(got: np.ndarray, ref: np.ndarray, bound: str = "bf16",
                      abs_sum: Optional[np.ndarray] = None) -> float:
    """Largest |got - ref| / (rel * |ref| + frac * rms(row) [+ ABS_SUM_FP8 * abs_sum])
    over all elements (0 where both sides are 0)."""
    rel, frac = ELEM[bound]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    lim = rel * np.abs(ref) + frac * rms
    if abs_sum is not None:
        lim = lim + ABS_SUM_FP8 * np.asarray(abs_sum, dtype=np.float64)
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(diff == 0, 0.0, diff / lim)
    return float(np.max(r)) if r.size else 0.0


def check_gemm(got: np.ndarray, ref: np.ndarray, dtype: str, bound: str = "bf16", what: str = "",
               abs_sum: Optional[np.ndarray] = None) -> float:
    """Every compared element finite, the rel. Frobenius bar of `dtype`, and the
    per-element bound `bound` (see the module doc; abs_sum: S for e4m3 operands
    into fp32).  Returns the Frobenius error."""
    assert np.isfinite(got).all(), what
    err = og.rel_frobenius(got, ref)
    worst = elementwise_ratio(got, ref, bound, abs_sum)
    print(f"{what} rows={len(got)} rel_frobenius={err:.3e} element/bound={worst:.3f}", flush=True)
    assert err <= TOL[dtype], (what, err)
    assert worst <= 1.0, (what, worst)
    return err


def rows_every_block(counts: Sequence[int], seg_align: int, seed: int) -> List[int]:
    """One row from every 16-row block of every expert segment, counted from the
    segment start, plus each segment's first and last row.  Tiles of every height
    (64, 128, 256, per expert) start at multiples of 16 rows of their segment, so
    this visits every 16-row MFMA block of every tile; compared as whole rows it
    covers every column tile too."""
    offs = acc.segment_offsets(counts, seg_align)
    rng = random.Random(seed)
    rows = set()
    for e, m in enumerate(counts):
        if m <= 0:
            continue
        s = offs[e]
        rows.update({s, s + m - 1})
        for b in range(0, m, 16):
            rows.add(s + b + rng.randrange(min(16, m - b)))
    return sorted(rows)


_REF_CACHE: Dict = {}


def cached(key, compute):
    """The oracle's answer for `key`, computed once per test session (the full-size
    inputs are seeded, so every test that draws them sees the same bits)."""
    if key not in _REF_CACHE:
        _REF_CACHE[key] = compute()
    return _REF_CACHE[key]


def cpu(t: Optional[torch.Tensor]):
    return None if t is None else t.detach().cpu().contiguous()


def sentinel_like(shape, device="cuda") -> torch.Tensor:
    return torch.full(shape, SENTINEL_BITS, dtype=torch.int16, device=device).view(torch.bfloat16)


def sample_rows_contiguous(counts: Sequence[int], seg_align: int, block_m: int, extra: int, seed: int) -> List[int]:
    """First, last and tail-tile rows of every active expert, plus random valid rows."""
    offs = acc.segment_offsets(counts, seg_align)
    rows = set()
    valid = []
    for e, m in enumerate(counts):
        if m <= 0:
            continue
        s = offs[e]
        rows.update({s, s + m - 1, s + (m - 1) // block_m * block_m, s + m // 2})
        valid.append((s, m))
    rng = random.Random(seed)
    for _ in range(extra):
        s, m = rng.choice(valid)
        rows.add(s + rng.randrange(m))
    return sorted(rows)


def run_contiguous(w: wl.Workload, inp: Dict, block_m: int = 0, b_layout: int = mg.B_KN, scale_km: bool = False):
    """scale_km: hand the fp32 activation scales over transposed, [K/128, rows]."""
    A, B = inp["A"], inp["B"]
    if b_layout == mg.B_NK:
        B = B.transpose(1, 2).contiguous()
    C = sentinel_like((w.rows_total, w.N))
    ws = mg.workspace(w.G, w.rows_total)
    a_scale = inp.get("A_scale")
    if scale_km:
        a_scale = a_scale.t().contiguous()
    mg.grouped_gemm_contiguous(A, B, C, inp["counts"], ws, A_scale=a_scale, B_scale=inp.get("B_scale"),
                               seg_align=w.seg_align, block_m=block_m, b_layout=b_layout, scale_km=scale_km)
    torch.cuda.synchronize()
    return C, ws


def oracle_contiguous_rows(w: wl.Workload, inp_cpu: Dict, rows: Sequence[int]) -> np.ndarray:
    return og.contiguous(inp_cpu["A"], inp_cpu["B"], w.counts, rows, seg_align=w.seg_align,
                         A_scale=inp_cpu.get("A_scale"), B_scale=inp_cpu.get("B_scale"))


def check_stats(stats: mg.Stats, counts: Sequence[int], block_m: Optional[int] = None):
    """Device accounting equals the oracle's exact integers."""
    s = acc.summary(counts)
    assert stats.U == s["U"]
    assert stats.active == s["active"]
    assert stats.sum_sq == s["sum_sq"]
    assert stats.P_at == s["P"]
    assert stats.P_exec == s["P"][16]
    assert stats.error_flags == 0
    if block_m is not None:
        assert stats.block_m == block_m
        assert stats.tiles == acc.tiles_for(counts, 256 if block_m == mg.BLOCK_M_PER_EXPERT else block_m)


def rows_as_float(C: torch.Tensor, rows: Sequence[int]) -> np.ndarray:
    return C[torch.tensor(list(rows), device=C.device)].float().cpu().double().numpy()


def untouched_rows_ok(C: torch.Tensor, counts: Sequence[int], seg_align: int) -> bool:
    """Rows that belong to no expert still hold the sentinel."""
    mask = torch.ones(C.shape[0], dtype=torch.bool)
    offs = acc.segment_offsets(counts, seg_align)
    for e, m in enumerate(counts):
        mask[offs[e]:offs[e] + m] = False
    idx = mask.nonzero().flatten().to(C.device)
    if idx.numel() == 0:
        return True
    return bool((C[idx].view(torch.int16) == SENTINEL_BITS).all())


def choice_rule(counts, n_col_tiles):
    """The documented tile-height rule, from the oracle (oracle/choice.py)."""
    return ochoice.choose(counts, n_col_tiles)
