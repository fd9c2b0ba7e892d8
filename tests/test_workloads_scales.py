"""The E8M0 inputs: the generator hands the same power-of-two scales out as
fp32 values (for the oracle) and as E8M0 bytes (for the kernels).  These pin
that the two agree, that every scaled value fits e4m3, and the byte encoding
against its definition (value 2^(b - 127), 255 = NaN)."""
import math

import numpy as np
import torch

import workloads as wl


def test_e8m0_bytes_definition():
    s = torch.tensor([1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127, float("nan")])
    assert wl.e8m0_bytes(s).tolist() == [127, 128, 126, 0, 254, 255]


def test_pow2_scales_and_bytes_agree():
    w = wl.Workload("e8", "contiguous", "fp8", [70, 0, 300, 6, 129, 3], K=512, N=512, values="normal", seed=9,
                    scales="e8m0")
    inp = wl.materialize(w, "cpu")
    sa, sb = inp["A_scale"], inp["B_scale"]
    ba, bb = inp["A_scale_e8m0"], inp["B_scale_e8m0"]
    assert ba.shape == (w.K // 128, w.rows_total) and bb.shape == sb.shape
    dec = lambda b: torch.where(b == 255, torch.tensor(float("nan")), torch.exp2(b.double() - 127))
    assert torch.equal(dec(ba).t().float().nan_to_num(-1), sa.nan_to_num(-1))
    assert torch.equal(dec(bb).float(), sb)
    # powers of two, at or above amax / 448 (so every quantized value is finite)
    fin = sa[torch.isfinite(sa)]
    assert bool((torch.log2(fin) == torch.round(torch.log2(fin))).all())
    codes = inp["A"].float()
    valid = torch.isfinite(codes).all(dim=1)
    assert float(codes[valid].abs().max()) <= 448.0
    assert float(inp["B"].float().abs().max()) <= 448.0


def test_pow2_scale_is_the_next_power_of_two():
    x = torch.zeros(1, 128)
    x[0, 0] = 448.0 * 3.0                    # amax/448 = 3 -> 4
    q, s = wl.quantize_rows_e4m3(x, pow2=True)
    assert float(s[0, 0]) == 4.0 and float(q.float()[0, 0]) == 320.0   # 1344 / 4 = 336: a tie, to even
    x[0, 0] = 448.0 * 4.0                    # exactly a power of two stays
    q, s = wl.quantize_rows_e4m3(x, pow2=True)
    assert float(s[0, 0]) == 4.0 and float(q.float()[0, 0]) == 448.0
    _, s = wl.quantize_rows_e4m3(torch.zeros(1, 128), pow2=True)
    assert float(s[0, 0]) == 1.0


def test_k_grouped_pow2_scales_and_bytes_agree():
    """K-grouped operands with E8M0 scales: one byte per (group, column), decoding
    to the fp32 power-of-two scale of that group; scaled codes fit e4m3."""
    t = [100, 0, 37, 200, 129]
    w = wl.Workload("kg e8", "k_grouped", "fp8", t, Mw=256, Nw=512, values="normal_unit", seed=5, scales="e8m0")
    inp = wl.materialize(w, "cpu")
    S = wl.k_group_starts(t)[-1]
    for name, M in (("X", 256), ("dY", 512)):
        s, b = inp[name + "_scale"], inp[name + "_scale_e8m0"]
        assert s.shape == b.shape == (S, M) and b.dtype == torch.uint8
        assert torch.equal(torch.exp2(b.double() - 127).float(), s)
        assert bool((torch.log2(s) == torch.round(torch.log2(s))).all())
        assert float(inp[name].float().abs().max()) <= 448.0
    # without e8m0 the scales are amax / 448 and no bytes are drawn
    w.scales = "fp32"
    inp = wl.materialize(w, "cpu")
    assert "X_scale_e8m0" not in inp and not bool((torch.log2(inp["X_scale"]) ==
                                                   torch.round(torch.log2(inp["X_scale"]))).all())
