"""GPU parity of the transposed fp32 activation-scale layout
(MOEGG_FP8_E4M3_SCALE_KM: A_scale [K/128, rows] instead of [rows, K/128]).

The layout changes only where the kernel fetches a scale, not the
arithmetic: every case is checked against the oracle and, bit for bit,
against the same call with the scales stored [rows, K/128].
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import gemm as og
from oracle import mlp as omlp
from tests import parity as P
from tests import test_gpu_parity as T

pytestmark = pytest.mark.gpu

FP8_SMALL = [c for c in T.SMALL if c[4] == "fp8"]


def same_bits(x: torch.Tensor, y: torch.Tensor) -> bool:
    return torch.equal(x.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("case", FP8_SMALL, ids=[c[0] for c in FP8_SMALL])
@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_contiguous_scale_km(case, block_m, b_layout):
    name, counts, K, N, dtype, align = case
    T.announce("contiguous scale_km", name, counts, K, N, align, block_m, b_layout)
    w, inp = T.small_contig(counts, K, N, dtype, align)
    C_rows, _ = P.run_contiguous(w, inp, block_m=block_m, b_layout=b_layout)
    C, ws = P.run_contiguous(w, inp, block_m=block_m, b_layout=b_layout, scale_km=True)
    P.check_stats(mg.stats_read(ws), counts, block_m if block_m else None)
    inp_cpu = {k: P.cpu(v) for k, v in inp.items()}
    rows = list(range(w.rows_total))
    ref = P.oracle_contiguous_rows(w, inp_cpu, rows)
    valid = ~np.isnan(ref[:, 0])
    got = P.rows_as_float(C, rows)
    P.check_gemm(got[valid], ref[valid], dtype, what=f"scale_km {name} block_m={block_m} layout={b_layout}")
    assert P.untouched_rows_ok(C, counts, align)
    assert same_bits(C, C_rows)


def test_contiguous_scale_km_full_size():
    """The Zipf 64-expert fp8 workload at full size (K 7168, N 4096), per-expert
    tile heights, K-contiguous weights: the launch the benchmark times."""
    w = wl.workload(3)
    T.announce("contiguous scale_km full size", w.name)
    inp = wl.materialize(w, "cuda")
    C_rows, _ = P.run_contiguous(w, inp, block_m=mg.BLOCK_M_PER_EXPERT, b_layout=mg.B_NK)
    C, ws = P.run_contiguous(w, inp, block_m=mg.BLOCK_M_PER_EXPERT, b_layout=mg.B_NK, scale_km=True)
    assert same_bits(C, C_rows)
    # and against the oracle: one row from every 16-row block of every expert segment
    rows = T.full_size_rows(w)
    ref = T.full_size_ref(w, inp, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what="scale_km full size")


@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_masked_scale_km(b_layout):
    counts = [3, 0, 64, 65, 130, 1]
    T.announce("masked scale_km", b_layout, counts)
    w, inp = T.masked_case(counts, 160, 512, 256, "fp8")
    B = inp["B"] if b_layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    ws = mg.workspace(w.G, w.G * w.cap)
    C_rows = P.sentinel_like((w.G, w.cap, w.N))
    mg.grouped_gemm_masked(inp["A"], B, C_rows, inp["counts"], ws, inp["A_scale"], inp["B_scale"], b_layout)
    C = P.sentinel_like((w.G, w.cap, w.N))
    a_scale = inp["A_scale"].reshape(w.G * w.cap, -1).t().contiguous()
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, a_scale, inp["B_scale"], b_layout, scale_km=True)
    torch.cuda.synchronize()
    T.check_masked(w, inp, C, counts)
    assert same_bits(C, C_rows)


@pytest.mark.parametrize("block_m", [0, 128, mg.BLOCK_M_PER_EXPERT])
def test_swiglu_e4m3_scale_km(block_m):
    """L1 with the e4m3 H epilogue writes H_scale as [I/128, rows]; L2 takes it
    as its transposed activation scales."""
    counts = [70, 0, 300, 6, 129, 3]
    K, I, N2 = 256, 256, 512
    G, R = len(counts), sum(counts)
    T.announce("expert MLP fp8 H scale_km", counts, "block_m", block_m)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=16, device="cuda", l2="fp8")
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=block_m, N=2 * I)
    out = {}
    for km in (False, True):
        H = torch.empty((R, I), dtype=torch.float8_e4m3fn, device="cuda")
        Hs = torch.full((I // 128, R) if km else (R, I // 128), float("nan"), device="cuda")
        Y = P.sentinel_like((R, N2))
        a_scale = inp["A_scale"].t().contiguous() if km else inp["A_scale"]
        mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, a_scale, inp["W1_scale"],
                                         block_m=block_m, H_scale=Hs, scale_km=km)
        mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], block_m=block_m,
                                             b_layout=mg.B_NK, scale_km=km)
        torch.cuda.synchronize()
        out[km] = (H, Hs, Y)
    (H0, Hs0, Y0), (H1, Hs1, Y1) = out[False], out[True]
    assert same_bits(H1, H0)
    assert torch.equal(Hs1, Hs0.t())
    assert same_bits(Y1, Y0)
    rows = list(range(R))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    T.check_fp8_h(H1, Hs1.t().contiguous(), h, rows)
