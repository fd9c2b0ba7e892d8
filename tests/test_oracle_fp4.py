"""Pins of the fp8 x fp4 oracle (oracle/fp4.py) and the E2M1 inputs.

- The E2M1 decoder against the OCP definition, listed by hand.
- The packing order (element 2i in the low nibble).
- The oracle against an independent route: every E2M1 value is exact in
  e4m3, so the same weights re-encoded as e4m3 go through the fp8 C oracle
  (oracle/gemm.py) and must give the same result.
- Brute force in plain Python on a tiny case.
- The quantizer's rounding (nearest, ties to the even code, clamp at 6)."""
import numpy as np
import torch

import workloads as wl
from oracle import fp4
from oracle import gemm as og


def test_e2m1_table_is_the_ocp_definition():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(fp4.E2M1[:8]) == pos
    assert list(fp4.E2M1[8:]) == [-v for v in pos]


def test_packing_order():
    b = np.array([[0x72, 0x0F]], dtype=np.uint8)       # codes 2, 7, 15, 0
    assert fp4.dec_e2m1_packed(b).tolist() == [[1.0, 6.0, -6.0, 0.0]]


def test_quantizer_rounding():
    x = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.3, -5.9, 0.0, 1.26])
    got = [float(fp4.E2M1[c]) for c in wl.to_e2m1_codes(x).tolist()]
    assert got == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -0.5, -6.0, 0.0, 1.5]


def _case():
    w = wl.Workload("f4", "contiguous", "fp8", [40, 0, 100, 7, 9], K=256, N=256, values="normal", seed=21,
                    scales="e8m0", weights="e2m1")
    return w, wl.materialize(w, "cpu")


def test_fp4_oracle_matches_fp8_oracle_on_reencoded_weights():
    w, inp = _case()
    rows = list(range(w.rows_total))
    got = fp4.contiguous_fp8_fp4(inp["A"], inp["A_scale"], inp["B"], inp["B_scale"], w.counts, rows)
    # same weights as e4m3 codes [G, K, N]: E2M1 values are exact in e4m3
    vals = torch.from_numpy(fp4.dec_e2m1_packed(inp["B"].numpy())).float()        # [G, N, K]
    b8 = vals.transpose(1, 2).contiguous().to(torch.float8_e4m3fn)
    assert torch.equal(b8.float(), vals.transpose(1, 2))
    ref = og.contiguous(inp["A"], b8, w.counts, rows, A_scale=inp["A_scale"], B_scale=inp["B_scale"])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_fp4_oracle_brute_force_tiny():
    w = wl.Workload("f4", "contiguous", "fp8", [3, 0, 2], K=128, N=128, values="normal", seed=5,
                    scales="e8m0", weights="e2m1")
    inp = wl.materialize(w, "cpu")
    rows = list(range(w.rows_total))
    got = fp4.contiguous_fp8_fp4(inp["A"], inp["A_scale"], inp["B"], inp["B_scale"], w.counts, rows)
    a = inp["A"].view(torch.uint8).tolist()
    packed = inp["B"].tolist()
    expert = [0, 0, 0, 2, 2]
    for i, r in enumerate(rows):
        e = expert[r]
        for n in (0, 1, 77, 127):
            s = 0.0
            for k in range(128):
                byte = packed[e][n][k // 2]
                code = byte & 0xF if k % 2 == 0 else byte >> 4
                s += og.dec_e4m3(a[r][k]) * float(inp["A_scale"][r, 0]) * fp4.e2m1_value(code) * \
                    float(inp["B_scale"][e, 0, 0])
            assert abs(got[i, n] - s) <= 1e-12 * max(1.0, abs(s)), (r, n, got[i, n], s)


def test_e2m1_weights_fit_and_scales_are_powers_of_two():
    w, inp = _case()
    vals = fp4.dec_e2m1_packed(inp["B"].numpy())
    assert np.abs(vals).max() <= 6.0
    sb = inp["B_scale"]
    assert bool((torch.log2(sb) == torch.round(torch.log2(sb))).all())
    assert torch.equal(inp["B_scale_e8m0"].int() - 127, torch.log2(sb).round().int())


def test_masked_oracle_matches_the_contiguous_one():
    """The masked fp8 x fp4 sum equals the contiguous one on the same rows laid out back to back."""
    masked, cap = [5, 0, 8], 8
    w = wl.Workload("m4", "masked", "fp8", masked, K=256, N=256, cap=cap, values="normal", seed=3, scales="e8m0",
                    weights="e2m1")
    inp = wl.materialize(w, "cpu", nan_padding=False)
    pairs = [(e, r) for e in range(3) for r in range(masked[e])]
    got = fp4.masked_fp8_fp4(inp["A"], inp["A_scale"], inp["B"],
                                                                   inp["B_scale"], masked, pairs)
    rows = [e * cap + r for e, r in pairs]
    A = inp["A"].reshape(3 * cap, -1)[rows].contiguous()
    As = inp["A_scale"].reshape(3 * cap, -1)[rows].contiguous()
    ref = fp4.contiguous_fp8_fp4(A, As, inp["B"], inp["B_scale"], masked, list(range(len(rows))))
    assert np.array_equal(got, ref)
