"""Pins for the fp64 oracle of the K-grouped weight gradient on e4m3 operands
with fp32 scales per 128-row group of each expert's segment (CPU only).

The reading (DeepGEMM record, "Workarounds": K-grouped MoE weight backward,
FP8 with per-group scaling): the reduction axis is the token axis, so one scale
covers one column of X or dY over up to 128 consecutive rows of one expert's
segment.  Groups restart at every segment start and are numbered across experts
in order.

Each pin comes from outside the oracle:
- exact rational brute force that walks each segment in 128-row chunks (no
  division-based group index), on ragged segments whose groups all have
  distinct scales;
- the pin is sharp: the two nearby misreadings (groups on the global row index;
  groups not restarting at segment starts) differ from it far beyond rounding;
- integer codes with power-of-two scales give exact sums (numpy int64);
- with unit scales the result equals the bf16 K-grouped oracle on the same
  values (every e4m3 value is exact in bf16): an independent route;
- one expert with its scales dequantized by torch equals numpy's float64
  X^T dY;
- the input quantizer: in every group and column with a nonzero entry, the
  largest code magnitude is 448, so its groups follow the segment layout.
"""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import gemm as og


@pytest.fixture(scope="module", autouse=True)
def _built():
    og.build()
    og._lib = None
    og.lib()


def _chunks(counts):
    """(first row, end row) of every scale group, walking each segment in 128-row chunks."""
    groups, pos = [], 0
    for t in counts:
        start, end = pos, pos + t
        while start < end:
            groups.append((start, min(start + 128, end)))
            start += 128
        pos = end
    return groups


def _case(counts, Mw, Nw, seed):
    T = sum(counts)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, Mw, generator=g)
    dy = torch.randn(T, Nw, generator=g)
    qx, sx = wl.quantize_k_groups_e4m3(x, counts)
    qy, sy = wl.quantize_k_groups_e4m3(dy, counts)
    # distinct scales in every group, so that a wrong group index changes the sum
    r = random.Random(seed)
    sx = torch.tensor([[r.uniform(0.5, 4.0) for _ in range(Mw)] for _ in range(sx.shape[0])], dtype=torch.float32)
    sy = torch.tensor([[r.uniform(0.5, 4.0) for _ in range(Nw)] for _ in range(sy.shape[0])], dtype=torch.float32)
    return qx, sx, qy, sy


def _frac(t):
    return np.vectorize(Fraction, otypes=[object])(t.to(torch.float64).numpy())


def _brute(qx, sx, qy, sy, counts, group_of=None):
    """dW[e] by exact rationals; group_of(row) -> scale row (default: the chunk walk)."""
    x, y, fsx, fsy = _frac(qx.float()), _frac(qy.float()), _frac(sx), _frac(sy)
    T, Mw = x.shape
    Nw = y.shape[1]
    if group_of is None:
        row_group = {}
        for gi, (a, b) in enumerate(_chunks(counts)):
            for rr in range(a, b):
                row_group[rr] = gi
        group_of = row_group.__getitem__
    out, pos = [], 0
    for t in counts:
        dw = np.full((Mw, Nw), Fraction(0), dtype=object)
        for rr in range(pos, pos + t):
            gi = group_of(rr)
            for i in range(Mw):
                xi = x[rr, i] * fsx[gi, i]
                for j in range(Nw):
                    dw[i, j] += xi * (y[rr, j] * fsy[gi, j])
        out.append(dw)
        pos += t
    return out


def _oracle_all(qx, sx, qy, sy, counts):
    Mw = qx.shape[1]
    reqs = [(e, i) for e in range(len(counts)) for i in range(Mw)]
    got = og.k_grouped_fp8(qx, sx, qy, sy, counts, [e for e, _ in reqs], [i for _, i in reqs])
    return got.reshape(len(counts), Mw, -1)


COUNTS = [130, 0, 5, 129, 1, 256]


def test_exact_rational_brute_force():
    qx, sx, qy, sy = _case(COUNTS, 3, 4, seed=1)
    got = _oracle_all(qx, sx, qy, sy, COUNTS)
    ref = _brute(qx, sx, qy, sy, COUNTS)
    for e in range(len(COUNTS)):
        r = np.vectorize(float)(ref[e]).astype(np.float64)
        assert np.allclose(got[e], r, rtol=1e-13, atol=1e-13), e
    assert not got[1].any()                                  # t_e = 0: the empty sum


def test_pin_rejects_nearby_readings():
    """The brute-force pin tells apart the readings a mistake would produce."""
    qx, sx, qy, sy = _case(COUNTS, 3, 4, seed=2)
    ref = np.stack([np.vectorize(float)(d) for d in _brute(qx, sx, qy, sy, COUNTS)])
    scale = np.abs(ref).max()
    n_groups = sx.shape[0]
    # groups on the global row index (t // 128), ignoring segment starts
    glob = np.stack([np.vectorize(float)(d) for d in
                     _brute(qx, sx, qy, sy, COUNTS, group_of=lambda r: min(r // 128, n_groups - 1))])
    assert np.abs(glob - ref).max() > 1e-3 * scale
    # one running row counter over all segments (groups never restart)
    run = np.stack([np.vectorize(float)(d) for d in
                    _brute(qx, sx, qy, sy, COUNTS,
                           group_of=lambda r: min(r // 128, n_groups - 1) if r < 130 else
                           min((r - 130) // 128 + 2, n_groups - 1))])
    assert np.abs(run - ref).max() > 1e-3 * scale


def test_integer_codes_power_of_two_scales_exact():
    counts = [200, 3, 0, 77]
    T, Mw, Nw = sum(counts), 8, 16
    g = torch.Generator().manual_seed(3)
    cx = torch.randint(-1, 2, (T, Mw), generator=g)
    cy = torch.randint(-1, 2, (T, Nw), generator=g)
    n_groups = wl.k_group_starts(counts)[-1]
    ex = torch.randint(-3, 4, (n_groups, Mw), generator=g)
    ey = torch.randint(-3, 4, (n_groups, Nw), generator=g)
    sx, sy = torch.exp2(ex.float()), torch.exp2(ey.float())
    got = _oracle_all(cx.float().to(torch.float8_e4m3fn), sx, cy.float().to(torch.float8_e4m3fn), sy, counts)
    # exact: scale everything by 2^6 into integers
    gr = [gi for gi, (a, b) in enumerate(_chunks(counts)) for _ in range(a, b)]
    xi = cx.numpy().astype(np.int64) * (2 ** (ex.numpy()[gr] + 3))
    yi = cy.numpy().astype(np.int64) * (2 ** (ey.numpy()[gr] + 3))
    pos = 0
    for e, t in enumerate(counts):
        ref = xi[pos:pos + t].T @ yi[pos:pos + t]
        assert np.array_equal(got[e] * 64.0, ref.astype(np.float64)), e
        pos += t


def test_unit_scales_equal_bf16_route():
    counts = [64, 0, 300, 1]
    qx, _, qy, _ = _case(counts, 5, 7, seed=4)
    ones_x = torch.ones(wl.k_group_starts(counts)[-1], 5)
    ones_y = torch.ones(wl.k_group_starts(counts)[-1], 7)
    got = _oracle_all(qx, ones_x, qy, ones_y, counts)
    bx, by = qx.float().to(torch.bfloat16), qy.float().to(torch.bfloat16)
    assert torch.equal(bx.float(), qx.float()) and torch.equal(by.float(), qy.float())
    reqs = [(e, i) for e in range(len(counts)) for i in range(5)]
    ref = og.k_grouped(bx, by, counts, [e for e, _ in reqs], [i for _, i in reqs]).reshape(len(counts), 5, 7)
    assert np.array_equal(got, ref)


def test_one_expert_is_dequantized_textbook_product():
    counts = [333]
    qx, sx, qy, sy = _case(counts, 16, 24, seed=5)
    rows_group = [gi for gi, (a, b) in enumerate(_chunks(counts)) for _ in range(a, b)]
    x = qx.to(torch.float64) * sx.to(torch.float64)[rows_group]
    y = qy.to(torch.float64) * sy.to(torch.float64)[rows_group]
    ref = x.numpy().T @ y.numpy()
    got = _oracle_all(qx, sx, qy, sy, counts)[0]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_quantizer_groups_follow_segments():
    counts = [130, 0, 5, 129, 1, 256]
    T = sum(counts)
    x = torch.randn(T, 6, generator=torch.Generator().manual_seed(6))
    q, s = wl.quantize_k_groups_e4m3(x, counts)
    chunks = _chunks(counts)
    assert s.shape[0] == len(chunks) == wl.k_group_starts(counts)[-1]
    for gi, (a, b) in enumerate(chunks):
        mags = q[a:b].float().abs().amax(dim=0)
        assert torch.all(mags == 448.0), (gi, mags)
        deq = q[a:b].float() * s[gi]
        assert torch.all((deq - x[a:b]).abs() <= x[a:b].abs().amax(dim=0) * 2.0 ** -4 + 1e-30)
