"""The per-element bound for fp32 outputs from e4m3 operands (tests/parity.py)
still fails a localized mistake: the oracle computes both the exact dW rows and
rows with one planted fault (one 128-row group missing from a 16 x 16 block, one
group's scale off by a factor of two in one column), and the bound, with its
term proportional to S = sum |x * y * scales|, rejects each on a 2000-row
reduction, where S is about 35 times the row's rms."""
import numpy as np
import torch

import workloads as wl
from oracle import gemm as og
from tests import parity as P

T, MW, NW = 2000, 32, 64


def _case():
    g = torch.Generator().manual_seed(31)
    X, sx = wl.quantize_k_groups_e4m3(torch.randn(T, MW, generator=g), [T])
    dY, sy = wl.quantize_k_groups_e4m3(torch.randn(T, NW, generator=g), [T])
    return X, sx, dY, sy


def _rows(X, sx, dY, sy):
    return og.k_grouped_fp8(X, sx, dY, sy, [T], [0] * MW, list(range(MW)))


def _abs(x):
    return x.float().abs().to(torch.float8_e4m3fn)


def test_exact_rows_pass_and_abs_sum_is_large():
    X, sx, dY, sy = _case()
    ref, S = _rows(X, sx, dY, sy), _rows(_abs(X), sx, _abs(dY), sy)
    assert P.elementwise_ratio(ref, ref, "fp32", S) == 0.0
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    assert np.median(S / rms) > 20


def test_missing_group_in_one_block_fails():
    X, sx, dY, sy = _case()
    ref, S = _rows(X, sx, dY, sy), _rows(_abs(X), sx, _abs(dY), sy)
    X2 = X.float().clone()
    X2[128:256, 0:16] = 0
    bad = _rows(X2.to(torch.float8_e4m3fn), sx, dY, sy)
    got = ref.copy()
    got[0:16, 16:32] = bad[0:16, 16:32]
    assert P.elementwise_ratio(got, ref, "fp32", S) > 1.0


def test_one_scale_off_by_two_fails():
    X, sx, dY, sy = _case()
    ref, S = _rows(X, sx, dY, sy), _rows(_abs(X), sx, _abs(dY), sy)
    sx2 = sx.clone()
    sx2[7, 3] *= 2
    bad = _rows(X, sx2, dY, sy)
    got = ref.copy()
    got[3] = bad[3]
    assert P.elementwise_ratio(got, ref, "fp32", S) > 1.0
