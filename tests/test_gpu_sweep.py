"""A seeded random sweep of small problems through every GEMM call: random
expert counts (empty experts, one-row experts, tails of every size), shapes,
segment alignments, tile heights, operand types and weight layouts, each case
compared on every valid row (every dW row) against the oracle with the bars of
tests/parity.py, the stats against the oracle's integers, and the rows that
belong to no expert against the sentinel.  The cases are drawn once, from a
fixed seed, so a failure names a case that reproduces."""
import random

import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import fp4
from tests import parity as P
from tests import test_gpu_parity as T

pytestmark = pytest.mark.gpu

HEIGHTS = [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT]


def _counts(rng, G, hi):
    """Counts with the edge cases mixed in: zeros, single rows, tile boundaries."""
    special = [0, 1, 15, 16, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    return [rng.choice(special) if rng.random() < 0.4 else rng.randrange(0, hi) for _ in range(G)]


def _contiguous_cases(n=60, seed=2027):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kind = ["bf16", "fp8", "fp8_km", "e8m0", "fp4"][i % 5]
        G = rng.randrange(1, 33)
        counts = _counts(rng, G, 400)
        if kind in ("e8m0", "fp4"):
            seg = rng.choice([4, 8, 64, 128])                 # E8M0 activation-scale rows come in fours
            N = rng.choice([512, 1024])
        else:
            seg = rng.choice([1, 1, 8, 64, 128])
            N = rng.choice([256, 512, 768, 1024])
        K = rng.choice([128, 256, 384, 640]) if kind != "bf16" else rng.choice([64, 192, 256, 448])
        layouts = [mg.B_NK, mg.B_NK_PANEL] if kind == "fp4" else [mg.B_KN, mg.B_NK, mg.B_KN_PANEL, mg.B_NK_PANEL]
        cases.append((i, kind, counts, seg, K, N, rng.choice(layouts), rng.choice(HEIGHTS)))
    return cases


@pytest.mark.parametrize("case", _contiguous_cases(), ids=lambda c: f"c{c[0]}-{c[1]}")
def test_sweep_contiguous(case):
    i, kind, counts, seg, K, N, layout, block_m = case
    T.announce("sweep contiguous", case)
    dtype = "bf16" if kind == "bf16" else "fp8"
    w = wl.Workload(f"sweep{i}", "contiguous", dtype, counts, K=K, N=N, seg_align=seg, values="normal", seed=100 + i,
                    scales="e8m0" if kind in ("e8m0", "fp4") else "fp32", weights="e2m1" if kind == "fp4" else "e4m3")
    if w.rows_total == 0:
        pytest.skip("no rows")
    inp = wl.materialize(w, "cuda")
    if kind == "fp4":
        B = inp["B"] if layout == mg.B_NK else mg.pack_panels(inp["B"], layout, mg.PANEL_CONTIGUOUS)
    elif layout in (mg.B_KN_PANEL, mg.B_NK_PANEL):
        B = mg.pack_panels(inp["B"], layout, mg.PANEL_CONTIGUOUS)
    else:
        B = inp["B"] if layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    a_s, b_s = inp.get("A_scale"), inp.get("B_scale")
    if kind in ("e8m0", "fp4"):
        a_s, b_s = inp["A_scale_e8m0"], inp["B_scale_e8m0"]
    elif kind == "fp8_km":
        a_s = a_s.t().contiguous()
    C = P.sentinel_like((w.rows_total, N))
    ws = mg.workspace(w.G, w.rows_total)
    mg.grouped_gemm_contiguous(inp["A"], B, C, inp["counts"], ws, A_scale=a_s, B_scale=b_s, seg_align=seg,
                               block_m=block_m, b_layout=layout, scale_km=kind == "fp8_km")
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    P.check_stats(st, counts)
    rows = [r for e, s0 in enumerate(T.acc.segment_offsets(counts, seg)[:-1]) for r in range(s0, s0 + counts[e])]
    if rows:
        cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}
        if kind == "fp4":
            ref = fp4.contiguous_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], counts, rows,
                                         seg_align=seg)
        else:
            ref = P.oracle_contiguous_rows(w, cpu, rows)
        P.check_gemm(P.rows_as_float(C, rows), ref, dtype, what=f"sweep contiguous {case}")
    assert P.untouched_rows_ok(C, counts, seg)


def _masked_cases(n=32, seed=2028):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kind = ["bf16", "fp8", "e8m0", "fp4"][i % 4]
        G = rng.randrange(1, 17)
        cap = rng.choice([64, 128, 160, 260, 320])
        if kind in ("e8m0", "fp4") and (G * cap) % 4:
            cap += 4 - (G * cap) % 4
        counts = [min(c, cap + 5) if rng.random() < 0.9 else rng.choice([-3, cap + 40])
                  for c in _counts(rng, G, cap + 1)]
        N = rng.choice([512, 1024]) if kind in ("e8m0", "fp4") else rng.choice([128, 256, 384, 512])
        K = rng.choice([128, 256, 512]) if kind != "bf16" else rng.choice([64, 192, 256])
        layouts = [mg.B_NK, mg.B_NK_PANEL] if kind == "fp4" else [mg.B_KN, mg.B_NK, mg.B_KN_PANEL, mg.B_NK_PANEL]
        cases.append((i, kind, counts, cap, K, N, rng.choice(layouts)))
    return cases


@pytest.mark.parametrize("case", _masked_cases(), ids=lambda c: f"m{c[0]}-{c[1]}")
def test_sweep_masked(case):
    i, kind, counts, cap, K, N, layout = case
    T.announce("sweep masked", case)
    dtype = "bf16" if kind == "bf16" else "fp8"
    clamped = [min(max(c, 0), cap) for c in counts]
    w = wl.Workload(f"msweep{i}", "masked", dtype, clamped, K=K, N=N, cap=cap, values="normal", seed=200 + i,
                    scales="e8m0" if kind in ("e8m0", "fp4") else "fp32", weights="e2m1" if kind == "fp4" else "e4m3")
    inp = wl.materialize(w, "cuda")
    if kind == "fp4":
        B = inp["B"] if layout == mg.B_NK else mg.pack_panels(inp["B"], layout, mg.PANEL_MASKED)
    elif layout in (mg.B_KN_PANEL, mg.B_NK_PANEL):
        B = mg.pack_panels(inp["B"], layout, mg.PANEL_MASKED)
    else:
        B = inp["B"] if layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    a_s, b_s = inp.get("A_scale"), inp.get("B_scale")
    if kind in ("e8m0", "fp4"):
        a_s, b_s = inp["A_scale_e8m0"], inp["B_scale_e8m0"]
    mm = torch.tensor(counts, dtype=torch.int32, device="cuda")      # the unclamped counts, as a router writes them
    C = P.sentinel_like((w.G, cap, N))
    ws = mg.workspace(w.G, w.G * cap)
    mg.grouped_gemm_masked(inp["A"], B, C, mm, ws, a_s, b_s, layout)
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    ref_stats = T.acc.summary(clamped)
    assert (st.U, st.active, st.sum_sq, st.P_at) == (ref_stats["U"], ref_stats["active"], ref_stats["sum_sq"],
                                                     ref_stats["P"])
    flags = (mg.FLAG_NEGATIVE_COUNT if min(counts) < 0 else 0) | (mg.FLAG_COUNT_OVER_CAP if max(counts) > cap else 0)
    assert st.error_flags == flags
    if kind == "fp4":
        T.check_masked_fp4(w, inp, C, clamped)
        inval = torch.tensor([e * cap + r for e in range(w.G) for r in range(cap) if r >= clamped[e]],
                             device="cuda")
        if inval.numel():
            assert bool((C.reshape(w.G * cap, -1)[inval].view(torch.int16) == P.SENTINEL_BITS).all())
    else:
        T.check_masked(w, {k: v for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}, C, clamped)


def _k_grouped_cases(n=24, seed=2029):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kind = ["bf16", "fp8", "e8m0"][i % 3]
        G = rng.randrange(1, 9)
        t = _counts(rng, G, 700)
        cases.append((i, kind, t, rng.choice([256, 512]), rng.choice([256, 512, 768])))
    return cases


@pytest.mark.parametrize("case", _k_grouped_cases(), ids=lambda c: f"k{c[0]}-{c[1]}")
def test_sweep_k_grouped(case):
    i, kind, t, Mw, Nw = case
    T.announce("sweep k-grouped", case)
    dtype = "bf16" if kind == "bf16" else "fp8"
    w, inp, dW, ws = T.run_k_grouped(t, Mw, Nw, seed=300 + i, dtype=dtype,
                                     scales="e8m0" if kind == "e8m0" else "fp32")
    st = mg.stats_read(ws)
    assert st.U == sum(t) and st.active == sum(1 for x in t if x > 0) and st.error_flags == 0
    pairs = [(e, r) for e in range(w.G) for r in range(Mw) if t[e] > 0]
    if pairs:
        T.check_k_grouped(w, inp, dW, pairs)
    for e, x in enumerate(t):
        if x == 0:
            assert not dW[e].any()
