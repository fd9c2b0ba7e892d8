"""GPU parity at the row counts where the staged epilogues change pass.

Every output tile is written to LDS and stored as whole rows, a pass of
THREADS * 16 bytes at a time (16 rows of a 256-column bf16 tile, 32 rows of
the masked 128-column tile, 64 rows of e4m3 H).  Valid-row counts just below,
at and just above those boundaries, and at each tile height, check that every
valid row is written and that no row past them is.
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

# per expert: 1 row, pass boundaries of 16 and 32 rows, tile heights 64 / 128 / 256, and one row past each
COUNTS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_m", [64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_epilogue_row_counts(dtype, block_m):
    T.announce("epilogue row counts contiguous", dtype, block_m, COUNTS)
    w, inp = T.small_contig(COUNTS, 256, 512, dtype, seed=21)
    C, ws = P.run_contiguous(w, inp, block_m=block_m, b_layout=mg.B_NK)
    P.check_stats(mg.stats_read(ws), COUNTS, block_m)
    rows = list(range(w.rows_total))
    ref = P.oracle_contiguous_rows(w, {k: P.cpu(v) for k, v in inp.items()}, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, dtype, what=f"epilogue rows {dtype} block_m={block_m}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_masked_epilogue_row_counts(dtype):
    counts = [1, 31, 32, 33, 63, 64, 65, 0, 96, 128, 129, 161, 255, 256, 257, 289]
    T.announce("epilogue row counts masked", dtype, counts)
    w, inp = T.masked_case(counts, 320, 256, 256, dtype, seed=22)
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"], ws, inp.get("A_scale"), inp.get("B_scale"),
                           mg.B_KN)
    torch.cuda.synchronize()
    T.check_masked(w, inp, C, counts)


@pytest.mark.parametrize("block_m", [64, 128, 256])
def test_swiglu_e4m3_epilogue_row_counts(block_m):
    """e4m3 H rows are 128 bytes: passes of 64 rows.  H rows of other experts'
    alignment gaps do not exist here (packed segments); every row is valid."""
    counts = [1, 63, 64, 65, 127, 128, 129, 200]
    K, I, N2 = 256, 128, 256
    G, R = len(counts), sum(counts)
    T.announce("epilogue row counts swiglu e4m3", counts, "block_m", block_m)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=23, device="cuda", l2="fp8")
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=block_m, N=2 * I)
    H = torch.full((R, I), float("nan"), device="cuda").to(torch.float8_e4m3fn)
    Hs = torch.full((R, I // 128), float("nan"), device="cuda")
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, inp["A_scale"], inp["W1_scale"],
                                     block_m=block_m, H_scale=Hs)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Hs).all())
    rows = list(range(R))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    T.check_fp8_h(H, Hs, h, rows)
