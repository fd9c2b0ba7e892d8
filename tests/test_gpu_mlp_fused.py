"""GPU parity of the expert MLP in one launch (moegg_expert_mlp_fused).

The fused kernel runs the same tile code as the two-launch chain (scheduler at
block_m = 256, the SwiGLU call with the e4m3 H epilogue, the fp8 contiguous
call on H), so H, its scales and Y must equal the chain's bit for bit; the
chain itself is held to the oracle in test_gpu_parity.py, and Y is checked
against the oracle here too.  Every case prints its name before touching the GPU.
"""
import random
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import accounting as acc
from oracle import gemm as og
from oracle import mlp as omlp
from tests import parity as P
from tests.test_gpu_parity import check_fp8_h

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()
    og.lib()


def operands(counts, K, I, N2, seed, b_layout, scale_km):
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=seed, device="cuda", l2="fp8")
    for k in ("W_gate", "W_up"):
        inp.pop(k)
    inp["A_scale_op"] = inp["A_scale"].t().contiguous() if scale_km else inp["A_scale"]
    if b_layout == mg.B_NK_PANEL:
        # pack_panels takes [G, K, N]
        inp["W1_op"] = mg.pack_panels(inp["W1"].transpose(1, 2).contiguous(), mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
        inp["W2_op"] = mg.pack_panels(inp["W2"].transpose(1, 2).contiguous(), mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
    else:
        inp["W1_op"], inp["W2_op"] = inp["W1"], inp["W2"]
    return inp


def h_buffers(R, I, scale_km):
    H = torch.full((R, I), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    Hs = torch.full((I // 128, R) if scale_km else (R, I // 128), float("nan"), device="cuda")
    return H, Hs


def run_fused(inp, counts, I, N2, b_layout, scale_km):
    G, R = len(counts), sum(counts)
    ws = mg.workspace(G, R)
    H, Hs = h_buffers(R, I, scale_km)
    Y = P.sentinel_like((R, N2))
    mg.expert_mlp_fused(inp["A"], inp["W1_op"], inp["W2_op"], H, Y, inp["counts"], ws, inp["A_scale_op"],
                        inp["W1_scale"], inp["W2_scale"], Hs, b_layout=b_layout, scale_km=scale_km)
    torch.cuda.synchronize()
    return H, Hs, Y, ws


def run_chain(inp, counts, I, N2, b_layout, scale_km):
    G, R = len(counts), sum(counts)
    ws = mg.workspace(G, R)
    H, Hs = h_buffers(R, I, scale_km)
    Y = P.sentinel_like((R, N2))
    mg.schedule(inp["counts"], R, ws, block_m=256, N=2 * I)
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1_op"], H, G, ws, inp["A_scale_op"], inp["W1_scale"],
                                     block_m=256, H_scale=Hs, scale_km=scale_km, b_layout=b_layout)
    mg.grouped_gemm_contiguous_scheduled(H, inp["W2_op"], Y, G, ws, Hs, inp["W2_scale"], block_m=256,
                                         b_layout=b_layout, scale_km=scale_km)
    torch.cuda.synchronize()
    return H, Hs, Y


def same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    va = a.contiguous().view(torch.uint8)
    vb = b.contiguous().view(torch.uint8)
    diff = int((va != vb).sum())
    assert diff == 0, f"{what}: {diff} bytes differ"


def check_against_chain(inp, counts, I, N2, b_layout, scale_km):
    R = sum(counts)
    H, Hs, Y, ws = run_fused(inp, counts, I, N2, b_layout, scale_km)
    st = mg.stats_read(ws)
    assert st.error_flags & mg.FLAG_SYNC_TIMEOUT == 0
    P.check_stats(st, counts, block_m=256)
    H2, Hs2, Y2 = run_chain(inp, counts, I, N2, b_layout, scale_km)
    if R:
        same_bits(H, H2, "H")
        same_bits(Hs, Hs2, "H_scale")
        same_bits(Y, Y2, "Y")
    return H, Hs, Y


def oracle_y(cpu, q, s, counts, rows, N2):
    """Y rows from the oracle's own e4m3 H codes q and scales s (one expert per row)."""
    offs = acc.segment_offsets(counts, 1)
    ex = [next(e for e in range(len(counts)) if offs[e] <= r < offs[e] + counts[e]) for r in rows]
    y = np.empty((len(rows), N2))
    for e in sorted(set(ex)):
        idx = [i for i, x in enumerate(ex) if x == e]
        w2e = cpu["W2"][e].float().double().numpy() * np.repeat(
            np.repeat(cpu["W2_scale"][e].double().numpy(), 128, 0), 128, 1).T
        y[idx] = (q[idx] * np.repeat(s[idx], 128, axis=1)) @ w2e.T
    return y


@pytest.mark.parametrize("b_layout,scale_km", [(mg.B_NK, False), (mg.B_NK, True), (mg.B_NK_PANEL, False),
                                               (mg.B_NK_PANEL, True)])
def test_fused_mlp_small(b_layout, scale_km):
    """Ragged experts (empty, 3 rows, a 256-row tile plus 44): bit for bit against
    the chain, H and Y on every valid row against the oracle."""
    counts = [70, 0, 300, 6, 129, 3]
    K, I, N2 = 256, 256, 512
    announce("fused expert MLP small", counts, "b_layout", b_layout, "scale_km", scale_km)
    inp = operands(counts, K, I, N2, 41, b_layout, scale_km)
    H, Hs, Y = check_against_chain(inp, counts, I, N2, b_layout, scale_km)
    rows = list(range(sum(counts)))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    q, s = check_fp8_h(H, Hs.t().contiguous() if scale_km else Hs, h, rows)
    P.check_gemm(P.rows_as_float(Y, rows), oracle_y(cpu, q, s, counts, rows, N2), "fp8", bound="chain_e4m3",
                 what="fused mlp small y")


@pytest.mark.parametrize("seed", [0, 1])
def test_fused_mlp_many_row_tiles(seed):
    """Enough 256-row tiles that each phase of the grid spans several runs of
    256 workgroups, with ragged tails in each expert: bit for bit against the
    chain."""
    rng = random.Random(900 + seed)
    counts = [rng.choice([0, 1, 77, 255, 256, 257, 600, 1500]) for _ in range(24)]
    K, I, N2 = 512, 512, 768
    announce("fused expert MLP many tiles", "seed", seed, "rows", sum(counts))
    inp = operands(counts, K, I, N2, 42 + seed, mg.B_NK, False)
    check_against_chain(inp, counts, I, N2, mg.B_NK, False)


def test_fused_mlp_tiny_and_single_expert():
    K, I, N2 = 128, 128, 256
    for counts in ([0, 5, 0], [513]):
        announce("fused expert MLP", counts)
        inp = operands(counts, K, I, N2, 43, mg.B_NK, False)
        check_against_chain(inp, counts, I, N2, mg.B_NK, False)


def test_fused_mlp_one_column_tile_each():
    """I = 128 and N2 = 256: one SwiGLU item and one down-projection item per
    row tile, so the two phases of the grid hold the same number of items."""
    counts = [300, 5, 0, 700, 1]
    K, I, N2 = 128, 128, 256
    announce("fused expert MLP one column tile each", counts)
    inp = operands(counts, K, I, N2, 47, mg.B_NK, False)
    check_against_chain(inp, counts, I, N2, mg.B_NK, False)


def test_fused_mlp_many_small_experts():
    """300 experts of 0..300 rows: most row tiles are an expert's only tile
    (their weight panels stream in both phases), and the grid's L1 part alone
    spans several runs of 256 workgroups: bit for bit against the chain."""
    rng = random.Random(951)
    counts = [rng.choice([0, 1, 40, 129, 255, 256, 300]) for _ in range(300)]
    K, I, N2 = 128, 256, 512
    announce("fused expert MLP many small experts", "rows", sum(counts))
    inp = operands(counts, K, I, N2, 48, mg.B_NK_PANEL, False)
    check_against_chain(inp, counts, I, N2, mg.B_NK_PANEL, False)


def test_fused_mlp_aligned_segments():
    """seg_align = 128: each expert's segment starts on a multiple of 128 rows,
    with unused rows (holding junk codes) between segments.  One launch against
    the chain scheduled with the same alignment, bit for bit on H, its scales
    and Y; the rows between segments keep the sentinel in Y; H and Y on every
    valid row against the oracle."""
    counts = [70, 0, 300, 6, 129, 1]
    K, I, N2, align = 256, 256, 512, 128
    announce("fused expert MLP aligned segments", counts, "seg_align", align)
    inp = operands(counts, K, I, N2, 49, mg.B_NK, False)
    packed, offs = acc.segment_offsets(counts, 1), acc.segment_offsets(counts, align)
    R, G = offs[-1], len(counts)
    A = torch.full((R, K), 0x3C, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    As = torch.full((R, K // 128), 3.0, device="cuda")
    for e, m in enumerate(counts):
        A[offs[e]:offs[e] + m] = inp["A"][packed[e]:packed[e] + m]
        As[offs[e]:offs[e] + m] = inp["A_scale_op"][packed[e]:packed[e] + m]
    outs = []
    for fused in (True, False):
        ws = mg.workspace(G, R)
        H, Hs = h_buffers(R, I, False)
        Y = P.sentinel_like((R, N2))
        if fused:
            mg.expert_mlp_fused(A, inp["W1_op"], inp["W2_op"], H, Y, inp["counts"], ws, As, inp["W1_scale"],
                                inp["W2_scale"], Hs, seg_align=align)
        else:
            mg.schedule(inp["counts"], R, ws, seg_align=align, block_m=256, N=2 * I)
            mg.grouped_gemm_swiglu_scheduled(A, inp["W1_op"], H, G, ws, As, inp["W1_scale"], block_m=256,
                                             H_scale=Hs, b_layout=mg.B_NK)
            mg.grouped_gemm_contiguous_scheduled(H, inp["W2_op"], Y, G, ws, Hs, inp["W2_scale"], block_m=256,
                                                 b_layout=mg.B_NK)
        torch.cuda.synchronize()
        st = mg.stats_read(ws)
        assert st.error_flags == 0
        outs.append((H, Hs, Y))
    valid = torch.tensor([r for e, m in enumerate(counts) for r in range(offs[e], offs[e] + m)], device="cuda")
    for name, a, b in zip(("H", "H_scale", "Y"), outs[0], outs[1]):
        same_bits(a[valid], b[valid], name)
    assert P.untouched_rows_ok(outs[0][2], counts, align)
    # and against the oracle, on the packed operands the aligned ones were copied from
    H, Hs, Y = (t[valid] for t in outs[0])
    rows = list(range(sum(counts)))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    q, s = check_fp8_h(H, Hs, h, rows)
    P.check_gemm(Y.float().cpu().double().numpy(), oracle_y(cpu, q, s, counts, rows, N2), "fp8",
                 bound="chain_e4m3", what="fused mlp aligned y")


def test_fused_mlp_all_experts_empty():
    """Every count 0 on a 4-row buffer: no tile, nothing written, no wait."""
    K, I, N2, G, R = 128, 128, 256, 3, 4
    announce("fused expert MLP all empty")
    e4m3 = torch.float8_e4m3fn
    A = torch.zeros(R, K, device="cuda").to(e4m3)
    As = torch.ones(R, K // 128, device="cuda")
    W1 = torch.zeros(G, 2 * I, K, device="cuda").to(e4m3)
    W1s = torch.ones(G, K // 128, 2 * I // 128, device="cuda")
    W2 = torch.zeros(G, N2, I, device="cuda").to(e4m3)
    W2s = torch.ones(G, I // 128, N2 // 128, device="cuda")
    H, Hs = h_buffers(R, I, False)
    Y = P.sentinel_like((R, N2))
    ws = mg.workspace(G, R)
    mg.expert_mlp_fused(A, W1, W2, H, Y, torch.zeros(G, dtype=torch.int32, device="cuda"), ws, As, W1s, W2s, Hs)
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    assert st.U == 0 and st.tiles == 0 and st.error_flags == 0
    assert bool((Y.view(torch.int16) == P.SENTINEL_BITS).all())
    assert bool(torch.isnan(Hs).all())


def test_fused_mlp_graph_replay():
    """Captured in a HIP graph and replayed: the completion counters are cleared
    by the call's scheduler kernel (no memset node), so every replay equals the
    eager run."""
    counts = [300, 0, 513, 40]
    K, I, N2 = 256, 256, 512
    G, R = len(counts), sum(counts)
    announce("fused expert MLP graph replay", counts)
    inp = operands(counts, K, I, N2, 44, mg.B_NK, False)
    H0, Hs0, Y0, _ = run_fused(inp, counts, I, N2, mg.B_NK, False)
    ws = mg.workspace(G, R)
    H, Hs = h_buffers(R, I, False)
    Y = P.sentinel_like((R, N2))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mg.expert_mlp_fused(inp["A"], inp["W1_op"], inp["W2_op"], H, Y, inp["counts"], ws, inp["A_scale_op"],
                            inp["W1_scale"], inp["W2_scale"], Hs, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.expert_mlp_fused(inp["A"], inp["W1_op"], inp["W2_op"], H, Y, inp["counts"], ws, inp["A_scale_op"],
                            inp["W1_scale"], inp["W2_scale"], Hs)
    for i in range(3):
        Y.view(torch.int16).fill_(P.SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same_bits(Y, Y0, f"replay {i} Y")
        same_bits(H, H0, f"replay {i} H")
        assert mg.stats_read(ws).error_flags == 0


def test_fused_mlp_full_size():
    """The DeepSeek-V3 expert shape on the Zipf histogram (64 experts, 32768 rows):
    bit for bit against the chain on every row; sampled rows against the oracle."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    announce("fused expert MLP full size")
    inp = operands(counts, K, I, N2, 45, mg.B_NK, False)
    H, Hs, Y = check_against_chain(inp, counts, I, N2, mg.B_NK, False)
    rows = P.sample_rows_contiguous(counts, 1, 256, extra=8, seed=46)
    got_y = P.rows_as_float(Y, rows)
    cpu = {k: P.cpu(v) for k, v in inp.items() if not k.endswith("_op")}
    del inp
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    q, s = check_fp8_h(H, Hs, h, rows)
    P.check_gemm(got_y, oracle_y(cpu, q, s, counts, rows, N2), "fp8", bound="chain_e4m3",
                 what="fused mlp full size y")


def test_fused_mlp_full_size_transposed_scales_and_panels():
    """The configuration bench.py --mlp --mlp-fused times (activation and H scales
    [K/128, rows]), and with the weights in column panels: bit for bit against the
    three launches on every row of the Zipf histogram at the DeepSeek-V3 shape."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    for b_layout in (mg.B_NK, mg.B_NK_PANEL):
        announce("fused expert MLP full size, scales [K/128, rows]", "b_layout", b_layout)
        inp = operands(counts, K, I, N2, 48, b_layout, True)
        check_against_chain(inp, counts, I, N2, b_layout, True)
        del inp
        torch.cuda.empty_cache()
