"""Pins of the expert-MLP oracle (oracle/mlp.py): SiLU against closed forms,
the gate/up column order against its definition (and the binding's and the
generator's interleave against it), and the whole L1 -> SwiGLU -> L2 chain
against plain-Python brute force on a tiny case."""
import math

import numpy as np
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import mlp


def test_silu_closed_forms():
    x = np.array([0.0, 1.0, -1.0, 2.0, 40.0, -40.0, -800.0])
    got = mlp.silu(x)
    assert got[0] == 0.0
    assert abs(got[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(got[2] + 1.0 / (1.0 + math.e)) < 1e-16          # silu(-1) = -1 / (1 + e)
    assert abs(got[1] - got[2] - 1.0) < 1e-15                  # silu(x) - silu(-x) = x
    assert abs(got[3] - 2.0 * (1.0 - 1.0 / (1.0 + math.exp(2.0)))) < 1e-15
    assert abs(got[4] - 40.0) < 1e-15 and abs(got[5]) < 1e-15 and got[6] == 0.0


def test_gate_up_order_is_the_documented_one():
    I = 48
    c = np.arange(2 * I, dtype=np.float64)[None, :]            # column index as value
    g, u = mlp.split_gate_up(c)
    for col in range(I):
        assert g[0, col] == 32 * (col // 16) + col % 16
        assert u[0, col] == 32 * (col // 16) + 16 + col % 16


def test_binding_and_generator_interleave_agree_with_the_split():
    G, I, K = 2, 32, 8
    wg = torch.randn(G, I, K)
    wu = torch.randn(G, I, K)
    w1 = mg.interleave_gate_up(wg, wu)                          # [G, 2I, K]
    g, u = mlp.split_gate_up(w1.transpose(1, 2).numpy())        # split along the 2I axis
    assert np.array_equal(g, wg.transpose(1, 2).numpy()) and np.array_equal(u, wu.transpose(1, 2).numpy())
    inp = wl.materialize_mlp([3, 0, 2], K=128, I=32, N2=64, dtype="bf16", seed=2)
    w1 = inp["W1"].float()
    g, u = mlp.split_gate_up(w1.transpose(1, 2).numpy())
    assert np.array_equal(g, inp["W_gate"].float().transpose(1, 2).numpy())
    assert np.array_equal(u, inp["W_up"].float().transpose(1, 2).numpy())


def test_chain_against_brute_force():
    counts = [3, 0, 2]
    K, I, N2 = 128, 32, 64
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="bf16", seed=4)
    rows = list(range(sum(counts)))
    h = mlp.swiglu_rows(inp["A"], inp["W1"], counts, rows)
    y = mlp.down_rows(h, inp["W2"], counts, rows)
    A = inp["A"].float().tolist()
    Wg = inp["W_gate"].float().tolist()
    Wu = inp["W_up"].float().tolist()
    W2 = inp["W2"].float().tolist()
    expert = [0, 0, 0, 2, 2]
    for i, r in enumerate(rows):
        e = expert[r]
        hh = []
        for c in range(I):
            gs = sum(A[r][k] * Wg[e][c][k] for k in range(K))
            us = sum(A[r][k] * Wu[e][c][k] for k in range(K))
            hh.append(gs / (1.0 + math.exp(-gs)) * us)
            assert abs(h[i, c] - hh[-1]) <= 1e-12 * max(1.0, abs(hh[-1]))
        for n in (0, 17, N2 - 1):
            yy = sum(hh[c] * W2[e][n][c] for c in range(I))
            assert abs(y[i, n] - yy) <= 1e-12 * max(1.0, abs(yy))


def test_fp8_chain_uses_the_dequantized_interleaved_weights():
    """fp8 W1: the oracle's h equals SwiGLU of the dequantized gate / up codes
    (scales per 128x128 block of the interleaved rows), recomputed here with
    numpy from the codes."""
    counts = [2, 3]
    K, I = 256, 128
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=64, dtype="fp8", seed=8)
    rows = list(range(5))
    h = mlp.swiglu_rows(inp["A"], inp["W1"], counts, rows, A_scale=inp["A_scale"], W1_scale=inp["W1_scale"])
    a = inp["A"].float().double().numpy() * np.repeat(inp["A_scale"].double().numpy(), 128, axis=1)
    w = inp["W1"].float().double().numpy()                                   # [G, 2I, K]
    sw = inp["W1_scale"].double().numpy()                                    # [G, K/128, 2I/128]
    w = w * np.repeat(np.repeat(sw, 128, axis=1), 128, axis=2).transpose(0, 2, 1)
    for i, r in enumerate(rows):
        e = 0 if r < 2 else 1
        c = w[e] @ a[r]
        g, u = mlp.split_gate_up(c)
        assert np.allclose(h[i], g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-14)


def test_e4m3_rne_matches_the_library_cast():
    """The oracle's own e4m3 rounding against torch's float8_e4m3fn cast
    (round to nearest even) on values spread over the whole range, ties included."""
    g = torch.Generator().manual_seed(5)
    x = torch.cat([(torch.rand(20000, generator=g) * 2 - 1) * 448,
                   torch.randn(20000, generator=g) * 0.01,
                   torch.tensor([0.0, 1.0625, 1.1875, -1.0625, 0.0078125 * 1.5, 240.0, 232.0, 448.0, -448.0])])
    x = x.double()
    ours = mlp.e4m3_rne(x.numpy())
    ref = x.float().to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, ref)


def test_quantize_groups_definition():
    h = np.zeros((2, 256))
    h[0, :128] = np.linspace(-3.0, 5.0, 128)          # amax 5 -> s = 5/448
    h[1, 128] = -0.25                                  # one nonzero value in the second group
    q, s = mlp.quantize_groups(h)
    assert s.shape == (2, 2)
    assert s[0, 0] == 5.0 / 448.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0 and s[1, 1] == 0.25 / 448.0
    assert q[0, 127] == 448.0 and q[1, 128] == -448.0  # the group's amax maps to the largest code
    assert np.all(np.abs(q[0, :128] * s[0, 0] - h[0, :128]) <= np.abs(h[0, :128]) / 16 + 1e-12)
    assert not q[0, 128:].any()


def test_fp4_swiglu_oracle_matches_the_e4m3_route():
    """fp4 gate/up weights: every E2M1 value is exact in e4m3, so the same
    weights re-encoded as e4m3 through the C-oracle route give the same h."""
    from oracle import fp4
    counts = [3, 0, 2]
    inp = wl.materialize_mlp(counts, K=256, I=64, N2=64, dtype="fp8", seed=2, w1_format="e2m1")
    rows = list(range(5))
    h4 = mlp.swiglu_rows_fp4(inp["A"], inp["A_scale"], inp["W1"], inp["W1_scale"], counts, rows)
    w1_vals = torch.from_numpy(fp4.dec_e2m1_packed(inp["W1"].numpy())).float()       # [G, 2I, K]
    w1_e4m3 = w1_vals.to(torch.float8_e4m3fn)
    assert torch.equal(w1_e4m3.float(), w1_vals)
    h8 = mlp.swiglu_rows(inp["A"], w1_e4m3, counts, rows, A_scale=inp["A_scale"], W1_scale=inp["W1_scale"])
    assert np.allclose(h4, h8, rtol=1e-12, atol=1e-14)
