"""Seeded synthetic inputs for the MoE grouped GEMM.

This module is shared test and benchmark infrastructure.  It feeds the same
bits to both sides of every parity check: the HIP library and the CPU oracle.
It draws per-expert count histograms and operand values, then stores the
operands in the formats the GEMM consumes:

- bf16, rounded to nearest-even from fp32;
- OCP e4m3fn codes with fp32 scales, one per 1x128 row group of the
  activations and one per 128x128 block of the weights;
- the same codes with power-of-two scales, handed out twice: as fp32 values
  and as E8M0 exponent bytes (2^(b - 127)), activation bytes transposed to
  [K/128, rows];
- OCP E2M1 (fp4) weight codes with power-of-two 128x128 block scales, packed
  two per byte along K ([G, N, K/2], element 2i in the low nibble).

It holds none of the grouped GEMM's own arithmetic: no tiling, no padding
accounting, no products or sums over K.

The histograms follow the pages:

- the near-uniform and concentrated eight-expert examples of "MoE GroupGEMM
  padding under expert skew" (sections "Work a near-uniform routing example"
  and "Contrast a concentrated histogram");
- the 32-expert histogram printed in the "Background" of the DeepGEMM issue
  "Query on performance-modeling of MoE Grouped GEMM".

Where the pages give only a shape, seeded draws with the stated
distributions stand in for real routing traces (none ship with the pages):

- a Zipf(s=1.2) skew over 64 experts with some experts zeroed;
- Poisson(24) decode counts capped at the capacity;
- a Dirichlet(0.3) split of 65536 rows.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0
# E2M1 magnitude -> code (sign in bit 3)
_E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
SCALE_GROUP = 128

# ---------------------------------------------------------------- histograms


def hist_near_uniform() -> List[int]:
    """Eight experts, 132 assignments: the near-uniform worked example."""
    return [17, 17, 17, 17, 16, 16, 16, 16]


def hist_concentrated() -> List[int]:
    """Eight experts, 132 assignments, two active: the concentrated example."""
    return [100, 32, 0, 0, 0, 0, 0, 0]


def hist_issue_32() -> List[int]:
    """The 32-expert per-expert M histogram printed in the DeepGEMM issue."""
    return [4, 1026, 1799, 166, 694, 753, 0, 16, 0, 240, 1119, 19, 6, 0, 46, 659,
            10, 0, 112, 808, 181, 0, 28, 22, 90, 0, 176, 0, 37, 5, 10, 22]


def hist_zipf(seed: int, experts: int = 64, total: int = 32768, s: float = 1.2,
              p_zero: float = 0.2) -> List[int]:
    """Zipf-skewed routing over `experts`, with some experts receiving nothing.

    Draw order: a permutation that assigns Zipf ranks to experts, then a
    Bernoulli(p_zero) mask that zeroes experts, then the multinomial split of
    `total` rows over the surviving weights r^-s.
    """
    rng = np.random.default_rng(seed)
    perm = rng.permutation(experts)
    w = np.empty(experts, dtype=np.float64)
    w[perm] = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    zero = rng.random(experts) < p_zero
    if zero.all():
        zero[perm[0]] = False
    w[zero] = 0.0
    return [int(x) for x in rng.multinomial(total, w / w.sum())]


def hist_poisson_masked(seed: int, experts: int = 32, cap: int = 256, mean: float = 24.0,
                        p_zero: float = 0.2) -> List[int]:
    """Decode-time valid-row counts: Poisson(mean) clipped to [0, cap], some forced to 0."""
    rng = np.random.default_rng(seed)
    m = np.clip(rng.poisson(mean, experts), 0, cap)
    m[rng.random(experts) < p_zero] = 0
    return [int(x) for x in m]


def hist_dirichlet(seed: int, experts: int = 16, total: int = 65536, alpha: float = 0.3) -> List[int]:
    """Rows per expert for the weight-gradient case: a Dirichlet(alpha) split of `total`."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(experts, alpha))
    return [int(x) for x in rng.multinomial(total, p)]


# ---------------------------------------------------------------- operand values


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def fp32_uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    x = torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.mul_(hi - lo).add_(lo)


def fp32_normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.mul_(std)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round to bf16, nearest-even (torch's conversion)."""
    return x.to(torch.bfloat16)


def _to_e4m3(x: torch.Tensor) -> torch.Tensor:
    # torch's cast does not saturate (values past 448 become NaN): clamp first.
    return x.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)


def _scale_for(amax: torch.Tensor, pow2: bool) -> torch.Tensor:
    """amax/448, or with pow2 the smallest power of two >= amax/448 (so every
    scaled value still fits e4m3); 1 for an all-zero group."""
    s = amax / E4M3_MAX
    if pow2:
        s = torch.exp2(torch.ceil(torch.log2(s.clamp_min(2.0 ** -126))))
    return torch.where(amax > 0, s, torch.ones_like(amax))


def e8m0_bytes(s: torch.Tensor) -> torch.Tensor:
    """Power-of-two fp32 scales -> E8M0 exponent bytes (2^(b - 127)); NaN -> 255."""
    e = torch.round(torch.log2(s.nan_to_num(1.0))).to(torch.int32) + 127
    e = torch.where(torch.isnan(s), torch.full_like(e, 255), e)
    return e.clamp_(0, 255).to(torch.uint8)


def to_e2m1_codes(x: torch.Tensor) -> torch.Tensor:
    """Round (already scaled) values to the nearest E2M1 value, ties to the even
    code, clamped to +-6; returns codes 0..15 (uint8, sign in bit 3).  The grid
    spacing is 0.5 below 2, 1 on [2, 4) and 2 on [4, 6]; torch.round rounds half
    to even, and an even multiple of the spacing is an even code."""
    a = x.abs().clamp(max=E2M1_MAX)
    q = torch.where(a < 2, torch.round(a * 2) / 2, torch.where(a < 4, torch.round(a), torch.round(a / 2) * 2))
    mag = torch.zeros_like(q, dtype=torch.uint8)
    for v, c in _E2M1_CODE.items():
        mag[q == v] = c
    return mag | ((x < 0).to(torch.uint8) << 3)


def quantize_blocks_e2m1(w: torch.Tensor):
    """Weights [G, K, N] -> (packed E2M1 codes [G, N, K/2], fp32 scales [G, K/128, N/128]).

    One power-of-two scale per 128x128 block of (K, N): the smallest 2^j with
    amax / 2^j <= 6 (1 for an all-zero block).  Codes are stored K-contiguous,
    two per byte, element 2i in the low nibble."""
    G, K, N = w.shape
    assert K % SCALE_GROUP == 0 and N % SCALE_GROUP == 0
    kb, nb = K // SCALE_GROUP, N // SCALE_GROUP
    packed = torch.empty((G, N, K // 2), dtype=torch.uint8, device=w.device)
    s = torch.empty((G, kb, nb), dtype=torch.float32, device=w.device)
    for e in range(G):
        blk = w[e].float().reshape(kb, SCALE_GROUP, nb, SCALE_GROUP)
        amax = blk.abs().amax(dim=(1, 3), keepdim=True)
        se = amax / E2M1_MAX
        se = torch.exp2(torch.ceil(torch.log2(se.clamp_min(2.0 ** -126))))
        se = torch.where(amax > 0, se, torch.ones_like(amax))
        codes = to_e2m1_codes(blk / se).reshape(K, N).t().contiguous()      # [N, K]
        packed[e] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        s[e] = se.reshape(kb, nb)
    return packed, s


def quantize_rows_e4m3(x: torch.Tensor, pow2: bool = False):
    """Activations [..., K] -> (e4m3 codes [..., K], fp32 scales [..., K/128]).

    One scale per 1x128 group along K: s = amax/448 (s = 1 for an all-zero
    group), or the power of two at or above it with pow2; code = e4m3(x / s).
    """
    *lead, k = x.shape
    assert k % SCALE_GROUP == 0
    g = x.float().reshape(*lead, k // SCALE_GROUP, SCALE_GROUP)
    amax = g.abs().amax(dim=-1, keepdim=True)
    s = _scale_for(amax, pow2)
    q = _to_e4m3(g / s).reshape(*lead, k)
    return q, s.squeeze(-1).contiguous()


def quantize_blocks_e4m3(w: torch.Tensor, pow2: bool = False):
    """Weights [G, K, N] -> (e4m3 codes [G, K, N], fp32 scales [G, K/128, N/128]).

    One scale per 128x128 block of (K, N): s = amax/448 (1 if all zero), or
    the power of two at or above it with pow2.
    Done one expert at a time to bound temporary memory.
    """
    G, K, N = w.shape
    assert K % SCALE_GROUP == 0 and N % SCALE_GROUP == 0
    kb, nb = K // SCALE_GROUP, N // SCALE_GROUP
    q = torch.empty((G, K, N), dtype=torch.float8_e4m3fn, device=w.device)
    s = torch.empty((G, kb, nb), dtype=torch.float32, device=w.device)
    for e in range(G):
        blk = w[e].float().reshape(kb, SCALE_GROUP, nb, SCALE_GROUP)
        amax = blk.abs().amax(dim=(1, 3), keepdim=True)
        se = _scale_for(amax, pow2)
        q[e] = _to_e4m3(blk / se).reshape(K, N)
        s[e] = se.reshape(kb, nb)
    return q, s


def k_group_starts(counts: Sequence[int]) -> List[int]:
    """First scale group of each expert's segment along the token axis, and the
    total: groups are 128 consecutive rows of one segment, counted from the
    segment start, so expert e starts at sum over j < e of ceil(t_j / 128)."""
    starts = [0]
    for t in counts:
        starts.append(starts[-1] + (max(int(t), 0) + SCALE_GROUP - 1) // SCALE_GROUP)
    return starts


def quantize_k_groups_e4m3(x: torch.Tensor, counts: Sequence[int], pow2: bool = False):
    """Operand [T, M] of the K-grouped weight gradient, rows grouped by expert ->
    (e4m3 codes [T, M], fp32 scales [n_groups, M]).

    Each scale covers one column over a group of up to 128 consecutive rows of
    one expert's segment (groups restart at every segment start; the last group
    of a segment may be short): s = amax / 448 (with pow2 the smallest power of
    two at or above it), 1 for an all-zero group."""
    T, M = x.shape
    starts = k_group_starts(counts)
    q = torch.empty((T, M), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.ones((max(starts[-1], 1), M), dtype=torch.float32, device=x.device)
    off = 0
    for e, t in enumerate(counts):
        for gi in range(starts[e + 1] - starts[e]):
            r0, r1 = off + gi * SCALE_GROUP, min(off + (gi + 1) * SCALE_GROUP, off + t)
            blk = x[r0:r1].float()
            amax = blk.abs().amax(dim=0, keepdim=True)
            sg = _scale_for(amax, pow2)
            q[r0:r1] = _to_e4m3(blk / sg)
            s[starts[e] + gi] = sg.squeeze(0)
        off += t
    return q, s


# ---------------------------------------------------------------- workloads


@dataclass
class Workload:
    """One grouped-GEMM problem: layout, sizes, histogram and value recipe."""
    name: str
    layout: str                 # "contiguous" | "masked" | "k_grouped"
    dtype: str                  # "bf16" | "fp8"
    counts: List[int]           # m_sizes / masked_m / t_sizes
    K: int = 0                  # shared inner width (contiguous / masked)
    N: int = 0                  # shared output width (contiguous / masked)
    seg_align: int = 1          # contiguous only
    cap: int = 0                # masked only
    Mw: int = 0                 # k_grouped: dW rows
    Nw: int = 0                 # k_grouped: dW cols
    values: str = "normal"      # "uniform" | "normal" | "normal_unit"
    scales: str = "fp32"        # fp8 block scales: "fp32" | "e8m0" (powers of two)
    weights: str = "e4m3"       # fp8 workloads' weight codes: "e4m3" | "e2m1" (fp4, needs e8m0 scales)
    seed: int = 0
    extra: Dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return len(self.counts)

    @property
    def rows_total(self) -> int:
        """Rows of the contiguous A buffer: every segment padded to seg_align."""
        a = self.seg_align
        return sum((c + a - 1) // a * a for c in self.counts)

    @property
    def useful_rows(self) -> int:
        return sum(self.counts)

    def useful_flops(self) -> int:
        if self.layout == "k_grouped":
            return 2 * self.Mw * self.Nw * sum(self.counts)
        return 2 * sum(self.counts) * self.K * self.N


FIXTURE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                            "histograms.json")


def fixture_counts(name: str) -> List[int]:
    """Counts of a seeded histogram as frozen in tests/golden/histograms.json
    (written by tests/golden/make_histograms.py from the generators above)."""
    with open(FIXTURE_PATH) as f:
        return [int(c) for c in json.load(f)[name]["counts"]]


def workload(n: int) -> Workload:
    """The five benchmark problems, by number 1..5.  Workloads 3-5 take their
    histograms from the frozen fixture."""
    if n == 1:
        return Workload("near-uniform 8 experts bf16 contiguous", "contiguous", "bf16",
                        hist_near_uniform(), K=512, N=256, values="uniform", seed=1)
    if n == 2:
        return Workload("issue histogram 32 experts bf16 contiguous aligned", "contiguous", "bf16",
                        hist_issue_32(), K=7168, N=4096, seg_align=128, values="normal", seed=2)
    if n == 3:
        return Workload("zipf 64 experts fp8 contiguous", "contiguous", "fp8",
                        fixture_counts("zipf64"), K=7168, N=4096, values="normal", seed=3)
    if n == 4:
        return Workload("masked decode 32 experts bf16", "masked", "bf16",
                        fixture_counts("poisson32"), K=2048, N=7168, cap=256, values="normal", seed=4)
    if n == 5:
        return Workload("k-grouped weight gradient 16 experts bf16", "k_grouped", "bf16",
                        fixture_counts("dirichlet16"), Mw=2048, Nw=7168, values="normal_unit", seed=5)
    raise ValueError(f"no workload {n}")


def _values(shape, wl: Workload, inner: int, seed: int, device) -> torch.Tensor:
    if wl.values == "uniform":
        return fp32_uniform(shape, -1.0, 1.0, seed, device)
    if wl.values == "normal":
        return fp32_normal(shape, 1.0 / float(np.sqrt(inner)), seed, device)
    return fp32_normal(shape, 1.0, seed, device)


def materialize(wl: Workload, device="cpu", nan_padding: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the operands of `wl` on `device`.

    contiguous: A [rows_total, K], B [G, K, N], counts int32 [G]
    masked:     A [G, cap, K],     B [G, K, N], counts int32 [G]
    k_grouped:  X [T, Mw], dY [T, Nw],          counts int32 [G]
                (fp8: X_scale [n_groups, Mw], dY_scale [n_groups, Nw] fp32; with
                scales == "e8m0" powers of two, and X_scale_e8m0 / dY_scale_e8m0
                the same as exponent bytes)
    fp8 adds A_scale [..., K/128] and B_scale [G, K/128, N/128] (fp32).  With
    scales == "e8m0" those are powers of two, and A_scale_e8m0 [K/128, rows]
    (contiguous layout) and B_scale_e8m0 [G, K/128, N/128] hold the same
    scales as E8M0 bytes.
    Rows that belong to no expert (segment alignment gaps, capacity rows
    beyond the valid count) hold NaN when nan_padding is set, so that any
    leak of padding into a valid output shows.
    """
    out: Dict[str, Optional[torch.Tensor]] = {
        "counts": torch.tensor(wl.counts, dtype=torch.int32, device=device)}
    s = wl.seed * 1000
    if wl.layout == "k_grouped":
        T = sum(wl.counts)
        x = _values((T, wl.Mw), wl, T, s + 1, device)
        dy = _values((T, wl.Nw), wl, T, s + 2, device)
        if wl.dtype == "fp8":
            # e4m3 with fp32 scales per 128-row group of each expert's segment; with
            # scales == "e8m0" powers of two, also as exponent bytes [n_groups, M]
            pow2 = wl.scales == "e8m0"
            out["X"], out["X_scale"] = quantize_k_groups_e4m3(x, wl.counts, pow2)
            out["dY"], out["dY_scale"] = quantize_k_groups_e4m3(dy, wl.counts, pow2)
            if pow2:
                out["X_scale_e8m0"] = e8m0_bytes(out["X_scale"])
                out["dY_scale_e8m0"] = e8m0_bytes(out["dY_scale"])
        else:
            out["X"], out["dY"] = to_bf16(x), to_bf16(dy)
        return out
    if wl.layout == "contiguous":
        a_shape = (wl.rows_total, wl.K)
    else:
        a_shape = (wl.G, wl.cap, wl.K)
    a = _values(a_shape, wl, wl.K, s + 1, device)
    if nan_padding:
        valid = _valid_row_mask(wl, device)
        a[~valid.reshape(a_shape[:-1])] = float("nan")
    b = _values((wl.G, wl.K, wl.N), wl, wl.K, s + 2, device)
    if wl.dtype == "bf16":
        out["A"], out["A_scale"] = to_bf16(a), None
        out["B"], out["B_scale"] = to_bf16(b), None
    else:
        a_nan = torch.isnan(a)
        a = a.nan_to_num(0.0)
        pow2 = wl.scales == "e8m0"
        qa, sa = quantize_rows_e4m3(a, pow2)
        # keep padding rows poisoned: e4m3fn NaN code plus a NaN scale
        qa.view(torch.uint8)[a_nan] = 0x7F
        sa[a_nan.reshape(*a_nan.shape[:-1], -1, SCALE_GROUP).any(-1)] = float("nan")
        del a
        if wl.weights == "e2m1":
            assert pow2, "fp4 weights come with power-of-two (E8M0) scales"
            qb, sb = quantize_blocks_e2m1(b)
        else:
            qb, sb = quantize_blocks_e4m3(b, pow2)
        out["A"], out["A_scale"], out["B"], out["B_scale"] = qa, sa, qb, sb
        if pow2:
            out["A_scale_e8m0"] = e8m0_bytes(sa.reshape(-1, sa.shape[-1]).t().contiguous())
            out["B_scale_e8m0"] = e8m0_bytes(sb)
    return out


def _valid_row_mask(wl: Workload, device) -> torch.Tensor:
    """True for rows that belong to some expert's valid segment."""
    if wl.layout == "masked":
        r = torch.arange(wl.cap, device=device)
        m = torch.tensor(wl.counts, device=device).clamp(0, wl.cap)
        return (r[None, :] < m[:, None]).reshape(-1)
    mask = torch.zeros(wl.rows_total, dtype=torch.bool, device=device)
    off = 0
    for c in wl.counts:
        mask[off:off + c] = True
        off += (c + wl.seg_align - 1) // wl.seg_align * wl.seg_align
    return mask


def materialize_mlp(counts: Sequence[int], K: int, I: int, N2: int, dtype: str = "bf16", seed: int = 6,
                    device="cpu", l2: str = "bf16", w1_format: str = "e4m3") -> Dict[str, Optional[torch.Tensor]]:
    """Operands of an expert MLP (L1 -> SwiGLU -> L2), contiguous layout, packed segments.

    A [rows, K] ~ N(0, 1); gate and up weights [G, I, K] ~ N(0, 1)/sqrt(K),
    stored together as W1 [G, 2I, K] with row 32q + w = gate row 16q + w and
    row 32q + 16 + w = up row 16q + w (w < 16); W2 [G, N2, I] ~ N(0, 1)/sqrt(I).
    dtype "bf16": A, W1 bf16.  "fp8": A e4m3 with fp32 1x128 scales, W1 e4m3
    with fp32 scales per 128x128 block of the interleaved rows.  W2 is bf16,
    or with l2 = "fp8" e4m3 with fp32 scales W2_scale [G, I/128, N2/128].
    dtype "fp8" with w1_format = "e2m1": A with power-of-two 1x128 scales (also as
    E8M0 bytes A_scale_e8m0 [K/128, rows]) and W1 packed E2M1 [G, 2I, K/2]
    with power-of-two 128x128 block scales (W1_scale fp32, W1_scale_e8m0).
    Also returns the plain gate / up weights (W_gate, W_up, as W1's dtype
    before quantization: bf16 or fp32) for checks of the interleave."""
    G, R = len(counts), sum(counts)
    s = seed * 1000
    a = fp32_normal((R, K), 1.0, s + 1, device)
    wg = fp32_normal((G, I, K), 1.0 / float(np.sqrt(K)), s + 2, device)
    wu = fp32_normal((G, I, K), 1.0 / float(np.sqrt(K)), s + 3, device)
    w1 = torch.stack([wg.reshape(G, I // 16, 16, K), wu.reshape(G, I // 16, 16, K)], dim=2).reshape(G, 2 * I, K)
    w2 = fp32_normal((G, N2, I), 1.0 / float(np.sqrt(I)), s + 4, device)
    out = {"counts": torch.tensor(list(counts), dtype=torch.int32, device=device), "W2_scale": None}
    if l2 == "fp8":
        q2, s2 = quantize_blocks_e4m3(w2.transpose(1, 2).contiguous())
        out["W2"], out["W2_scale"] = q2.transpose(1, 2).contiguous(), s2
    else:
        out["W2"] = to_bf16(w2)
    del w2
    if dtype == "bf16":
        out.update({"A": to_bf16(a), "A_scale": None, "W1": to_bf16(w1), "W1_scale": None,
                    "W_gate": to_bf16(wg), "W_up": to_bf16(wu)})
    elif w1_format == "e2m1":
        qa, sa = quantize_rows_e4m3(a, pow2=True)
        qw, sw = quantize_blocks_e2m1(w1.transpose(1, 2).contiguous())         # packed [G, 2I, K/2]
        out.update({"A": qa, "A_scale": sa, "W1": qw, "W1_scale": sw, "W_gate": wg, "W_up": wu,
                    "A_scale_e8m0": e8m0_bytes(sa.t().contiguous()), "W1_scale_e8m0": e8m0_bytes(sw)})
    else:
        qa, sa = quantize_rows_e4m3(a)
        qw, sw = quantize_blocks_e4m3(w1.transpose(1, 2).contiguous())
        out.update({"A": qa, "A_scale": sa, "W1": qw.transpose(1, 2).contiguous(), "W1_scale": sw,
                    "W_gate": wg, "W_up": wu})
    return out
