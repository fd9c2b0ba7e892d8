"""moegg_grouped_gemm_contiguous_noalloc against moegg_grouped_gemm_contiguous.

The allocation-free variant runs the same scheduler and GEMM kernels with the
library's fixed per-GPU scratch array as their workspace, so its output must
equal the workspace call's bit for bit (and meet the oracle's bar).  Two calls
in a row, the second on a smaller problem with fewer experts, check that what
the first left in the shared array does not leak into the second.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import accounting as acc
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [  # (name, counts, K, N, dtype, seg_align, block_m); the second is the smaller problem
    ("zipf 64 experts fp8", wl.hist_zipf(31, experts=64, total=6000), 1024, 1024, "fp8", 1, 0),
    ("near-uniform 8 experts bf16", wl.hist_near_uniform(), 256, 256, "bf16", 1, 0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()


def test_noalloc_matches_the_workspace_call_twice():
    for name, counts, K, N, dtype, align, block_m in CASES:
        print("CASE noalloc", name, "K", K, "N", N, "rows", sum(counts), flush=True)
        w = wl.Workload(name, "contiguous", dtype, counts, K=K, N=N, seg_align=align, values="normal", seed=31)
        inp = wl.materialize(w, "cuda")
        C_ws, _ = P.run_contiguous(w, inp, block_m=block_m, b_layout=mg.B_NK)
        B = inp["B"].transpose(1, 2).contiguous()
        C_na = P.sentinel_like((w.rows_total, w.N))
        mg.grouped_gemm_contiguous_noalloc(inp["A"], B, C_na, inp["counts"], inp.get("A_scale"), inp.get("B_scale"),
                                           seg_align=align, block_m=block_m, b_layout=mg.B_NK)
        torch.cuda.synchronize()
        assert torch.equal(C_na.view(torch.int16), C_ws.view(torch.int16)), name
        offs = acc.segment_offsets(counts, align)
        rows = [r for e, m in enumerate(counts) for r in range(offs[e], offs[e] + m)]
        ref = P.oracle_contiguous_rows(w, {k: P.cpu(v) for k, v in inp.items()}, rows)
        P.check_gemm(P.rows_as_float(C_na, rows), ref, dtype, what=f"noalloc {name}")
        assert P.untouched_rows_ok(C_na, counts, align)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    """A problem whose workspace exceeds the fixed array is refused before anything runs."""
    G, rows = 64, 8 << 20                      # about 2 MiB of tile list
    assert mg.workspace_bytes(G, rows) > mg.NOALLOC_SCRATCH_BYTES
    fake = 0x100000
    st = mg.lib().moegg_grouped_gemm_contiguous_noalloc(fake, None, fake, None, fake, fake, G, rows, 256, 256, 1,
                                                        mg.BF16, mg.B_NK, 0, None)
    assert st == mg.ERR_WORKSPACE
