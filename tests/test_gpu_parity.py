"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name, sizes and seed before touching the GPU, so a
failing run names its case.
"""
import random
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg
import workloads as wl
from oracle import accounting as acc
from oracle import fp4
from oracle import gemm as og
from oracle import mlp as omlp
from oracle import select as oselect
from tests import parity as P

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


# ----------------------------------------------------------------- scheduler


SCHED_HISTS = {
    "near_uniform": wl.hist_near_uniform(),
    "concentrated": wl.hist_concentrated(),
    "issue32": wl.hist_issue_32(),
    "zipf64": wl.hist_zipf(3),
    "poisson32": wl.hist_poisson_masked(4),
    "dirichlet16": wl.hist_dirichlet(5),
    "all_empty": [0] * 7,
    "single": [1],
    "boundaries": [63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 1],
}


@pytest.mark.parametrize("name", sorted(SCHED_HISTS))
@pytest.mark.parametrize("block_m", [64, 128, 256])
@pytest.mark.parametrize("seg_align", [1, 128])
def test_schedule_bit_exact(name, block_m, seg_align):
    counts = SCHED_HISTS[name]
    announce("schedule", name, block_m, seg_align)
    rows_total = sum(acc.ceil_div(c, seg_align) * seg_align for c in counts)
    m = torch.tensor(counts, dtype=torch.int32, device="cuda")
    ws = mg.workspace(len(counts), rows_total)
    mg.schedule(m, rows_total, ws, seg_align=seg_align, block_m=block_m)
    st = mg.stats_read(ws)
    P.check_stats(st, counts, block_m)
    tiles = mg.tile_list_read(ws, acc.tiles_for(counts, 64) + 5)
    assert tiles == acc.tile_list(counts, block_m, seg_align)
    assert st.capacity_rows == rows_total - sum(counts)


@pytest.mark.parametrize("name", sorted(SCHED_HISTS))
@pytest.mark.parametrize("seg_align", [1, 128])
def test_schedule_per_expert_bit_exact(name, seg_align):
    """Per-expert heights: the device's tile list equals the oracle's regrouped
    256-row list, entry for entry."""
    counts = SCHED_HISTS[name]
    announce("schedule per expert", name, seg_align)
    rows_total = sum(acc.ceil_div(c, seg_align) * seg_align for c in counts)
    m = torch.tensor(counts, dtype=torch.int32, device="cuda")
    ws = mg.workspace(len(counts), rows_total)
    mg.schedule(m, rows_total, ws, seg_align=seg_align, block_m=mg.BLOCK_M_PER_EXPERT)
    st = mg.stats_read(ws)
    P.check_stats(st, counts, mg.BLOCK_M_PER_EXPERT)
    assert mg.tile_list_read(ws, st.tiles + 5) == acc.tile_list_per_expert(counts, seg_align)


def test_schedule_random_histograms():
    rng = random.Random(7)
    for it in range(200):
        G = rng.randint(1, 300)
        counts = [0 if rng.random() < 0.3 else rng.randint(0, 700) for _ in range(G)]
        align = rng.choice([1, 8, 64, 128])
        bm = rng.choice([64, 128, 256])
        rows_total = sum(acc.ceil_div(c, align) * align for c in counts)
        m = torch.tensor(counts, dtype=torch.int32, device="cuda")
        ws = mg.workspace(G, rows_total)
        mg.schedule(m, rows_total, ws, seg_align=align, block_m=bm)
        st = mg.stats_read(ws)
        P.check_stats(st, counts, bm)
        assert mg.tile_list_read(ws, st.tiles) == acc.tile_list(counts, bm, align), (it, counts, align, bm)


def test_schedule_clamps_bad_counts():
    announce("schedule clamps")
    counts = [5, -3, 200, 7]
    m = torch.tensor(counts, dtype=torch.int32, device="cuda")
    ws = mg.workspace(4, 100)
    mg.schedule(m, 100, ws, seg_align=1, block_m=64)
    st = mg.stats_read(ws)
    assert st.error_flags & mg.FLAG_NEGATIVE_COUNT
    assert st.error_flags & mg.FLAG_ROWS_OVERFLOW
    # clamped reading: [5, 0, 95, 0] (segment 2 truncated at row 100, segment 3 starts past the end)
    assert st.U == 100
    assert mg.tile_list_read(ws, 10) == acc.tile_list([5, 0, 95, 0], 64, 1)


def expected_tiles(counts, block_m, seg_align):
    if block_m == mg.BLOCK_M_PER_EXPERT:
        return acc.tile_list_per_expert(counts, seg_align)
    return acc.tile_list(counts, block_m, seg_align)


@pytest.mark.parametrize("name", sorted(SCHED_HISTS))
def test_schedule_device_choice_matches_rule(name):
    """block_m = 0: the device's choice equals the documented rule (one column tile)."""
    counts = SCHED_HISTS[name]
    announce("choice", name)
    rows_total = sum(counts)
    m = torch.tensor(counts, dtype=torch.int32, device="cuda")
    ws = mg.workspace(len(counts), rows_total)
    mg.schedule(m, rows_total, ws, seg_align=1, block_m=0, N=256)
    st = mg.stats_read(ws)
    assert st.block_m == P.choice_rule(counts, 1)
    assert mg.tile_list_read(ws, st.tiles) == expected_tiles(counts, st.block_m, 1)


# ----------------------------------------------------------------- contiguous, small


def small_contig(counts, K, N, dtype, seg_align=1, seed=11, values="normal"):
    w = wl.Workload("small", "contiguous", dtype, counts, K=K, N=N, seg_align=seg_align, values=values, seed=seed)
    return w, wl.materialize(w, "cuda")


SMALL = [
    ("ragged_bf16", [300, 0, 17, 513, 64, 1], 512, 512, "bf16", 1),
    ("aligned_bf16", [100, 0, 250, 3], 256, 256, "bf16", 128),
    ("ragged_fp8", [300, 0, 17, 513, 64, 1], 512, 512, "fp8", 1),
    ("aligned_fp8", [129, 0, 0, 256, 40], 1024, 256, "fp8", 64),
    ("one_expert_bf16", [700], 192, 768, "bf16", 1),
    ("one_row_fp8", [1], 128, 256, "fp8", 1),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_contiguous_small_full_compare(case, block_m, b_layout):
    name, counts, K, N, dtype, align = case
    announce("contiguous small", name, counts, K, N, dtype, align, block_m, b_layout)
    w, inp = small_contig(counts, K, N, dtype, align)
    C, ws = P.run_contiguous(w, inp, block_m=block_m, b_layout=b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, counts, block_m if block_m else None)
    inp_cpu = {k: P.cpu(v) for k, v in inp.items()}
    rows = [r for r in range(w.rows_total)]
    ref = P.oracle_contiguous_rows(w, inp_cpu, rows)
    valid = ~np.isnan(ref[:, 0])
    got = P.rows_as_float(C, rows)
    P.check_gemm(got[valid], ref[valid], dtype, what=f"small {name} block_m={block_m} layout={b_layout}")
    assert P.untouched_rows_ok(C, counts, align)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("height", [64, 128])
def test_contiguous_one_launch_long_list(dtype, height):
    """The one-launch kernel (block_m = 0) on a list the scheduler cut at 64
    or 128 rows: a 66000-row expert and a few small ones, one column tile, so
    1037 work items at 64 rows and 520 at 128 run through the launch that
    reads the height from the control block.  Every valid row is written (no
    sentinel left) and every 7th row, plus all rows of the small experts, is
    checked against the oracle."""
    counts, K, N = [66000, 3, 130, 0, 64], 128, 256
    announce("one launch long list", dtype, height, counts)
    w, inp = small_contig(counts, K, N, dtype, seed=21)
    ws = mg.workspace(w.G, w.rows_total)
    mg.schedule(inp["counts"], w.rows_total, ws, seg_align=1, block_m=height, N=N)
    C = P.sentinel_like((w.rows_total, N))
    mg.grouped_gemm_contiguous_scheduled(inp["A"], inp["B"], C, w.G, ws, inp.get("A_scale"), inp.get("B_scale"),
                                         block_m=0, b_layout=mg.B_KN)
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    P.check_stats(st, counts, height)
    assert not bool((C[:sum(counts)].view(torch.int16) == P.SENTINEL_BITS).any())
    rows = sorted(set(range(0, 66000, 7)) | set(range(65990, sum(counts))))
    inp_cpu = {k: P.cpu(v) for k, v in inp.items()}
    ref = P.oracle_contiguous_rows(w, inp_cpu, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, dtype, what=f"one launch long list {dtype} {height}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("seg_align", [3, 7, 100])
@pytest.mark.parametrize("block_m", [0, 64, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_odd_segment_alignment(dtype, seg_align, block_m):
    """Segment starts on multiples of 3, 7 or 100 rows, so tiles start at rows
    that no power of two divides: every valid row against the oracle, the
    rows between segments keep the sentinel, the stats exact."""
    counts = [70, 0, 300, 6, 129, 1, 257]
    announce("odd alignment", dtype, seg_align, block_m)
    w, inp = small_contig(counts, 256, 512, dtype, seg_align, seed=71)
    C, ws = P.run_contiguous(w, inp, block_m=block_m, b_layout=mg.B_NK)
    st = mg.stats_read(ws)
    P.check_stats(st, counts, block_m if block_m else None)
    offs = acc.segment_offsets(counts, seg_align)
    rows = [r for e, m in enumerate(counts) for r in range(offs[e], offs[e] + m)]
    ref = P.oracle_contiguous_rows(w, {k: P.cpu(v) for k, v in inp.items()}, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, dtype, what=f"odd alignment {seg_align} {block_m}")
    assert P.untouched_rows_ok(C, counts, seg_align)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_contiguous_integer_exact(dtype):
    """Inputs in {-1, 0, 1}, K <= 256, unit scales: every result is an integer
    of magnitude <= 256, exact in bf16, so GPU == oracle bit for bit."""
    announce("integer exact", dtype)
    counts, K, N = [37, 0, 200, 5], 256, 512
    g = torch.Generator().manual_seed(3)
    A = torch.randint(-1, 2, (sum(counts), K), generator=g).float()
    Bw = torch.randint(-1, 2, (len(counts), K, N), generator=g).float()
    if dtype == "bf16":
        inp = {"A": A.to(torch.bfloat16), "B": Bw.to(torch.bfloat16), "A_scale": None, "B_scale": None}
    else:
        inp = {"A": A.to(torch.float8_e4m3fn), "B": Bw.to(torch.float8_e4m3fn),
               "A_scale": torch.ones(sum(counts), K // 128), "B_scale": torch.ones(len(counts), K // 128, N // 128)}
    w = wl.Workload("int", "contiguous", dtype, counts, K=K, N=N)
    inp_gpu = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    inp_gpu["counts"] = torch.tensor(counts, dtype=torch.int32, device="cuda")
    for bl in (mg.B_KN, mg.B_NK):
        C, _ = P.run_contiguous(w, inp_gpu, b_layout=bl)
        ref = og.contiguous(inp["A"], inp["B"], counts, range(w.rows_total), A_scale=inp["A_scale"],
                            B_scale=inp["B_scale"])
        got = C.float().cpu().double().numpy()
        assert np.array_equal(got, ref)


def test_contiguous_maximum_expert_count():
    """G = 4096 (the library's maximum) with tiny ragged counts, a third empty:
    accounting, tile list and every valid row."""
    rng = random.Random(41)
    counts = [0 if rng.random() < 0.33 else rng.randint(1, 5) for _ in range(4096)]
    announce("contiguous G=4096", sum(counts))
    w, inp = small_contig(counts, 128, 256, "bf16")
    C, ws = P.run_contiguous(w, inp, block_m=64)
    st = mg.stats_read(ws)
    P.check_stats(st, counts, 64)
    assert mg.tile_list_read(ws, st.tiles + 4) == acc.tile_list(counts, 64, 1)
    rows = list(range(w.rows_total))
    ref = P.oracle_contiguous_rows(w, {k: P.cpu(v) for k, v in inp.items()}, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "bf16", what="G=4096")


def _rows_against_oracle(A, B, picks):
    """Rows A[r] @ B[e] for picks [(r, e)], expert by expert: the oracle runs on
    the picked rows gathered into a small contiguous problem (the full operand
    is several GiB), which gives exactly those rows."""
    picks = sorted(picks, key=lambda p: p[1])
    G = B.shape[0]
    counts = [sum(1 for _, e in picks if e == g) for g in range(G)]
    idx = torch.tensor([r for r, _ in picks], device=A.device)
    A_sub = A.reshape(-1, A.shape[-1])[idx].cpu()
    ref = og.contiguous(A_sub, B.cpu(), counts, list(range(len(picks))))
    return picks, ref


def test_contiguous_activations_past_4gib():
    """Activations of 4.4 GB (bf16 [271000, 8192]): the second expert's rows and
    rows around the 2 GiB and 4 GiB byte offsets of the first, against the
    oracle; every tile's buffer starts at a 64-bit offset."""
    counts, K, N = [263000, 8000], 8192, 256
    announce("contiguous activations past 4 GiB", counts, K, N)
    w = wl.Workload("big", "contiguous", "bf16", counts, K=K, N=N, values="normal", seed=43)
    inp = wl.materialize(w, "cuda")
    assert inp["A"].numel() * 2 > 1 << 32
    C, ws = P.run_contiguous(w, inp, block_m=0)
    P.check_stats(mg.stats_read(ws), counts)
    row_2g, row_4g = (1 << 31) // (K * 2), (1 << 32) // (K * 2)
    first = [0, 1] + list(range(row_2g - 20, row_2g + 20)) + list(range(row_4g - 300, counts[0]))
    second = sorted({counts[0] + b + random.Random(b).randrange(16) for b in range(0, counts[1] - 15, 16)}
                    | {counts[0], sum(counts) - 1})
    picks, ref = _rows_against_oracle(inp["A"], inp["B"], [(r, 0) for r in first] + [(r, 1) for r in second])
    P.check_gemm(P.rows_as_float(C, [r for r, _ in picks]), ref, "bf16", what="activations past 4 GiB")


def test_masked_capacity_buffer_past_4gib():
    """A masked capacity buffer of 4.4 GB (bf16 [32, 8448, 8192]) with the valid
    rows in experts around the 2 GiB and 4 GiB offsets and in the last one."""
    G, cap, K, N = 32, 8448, 8192, 256
    counts = [0] * G
    for e, m in ((0, 5), (15, 300), (16, 130), (30, 64), (31, 1000)):
        counts[e] = m
    announce("masked capacity buffer past 4 GiB", counts)
    w = wl.Workload("bigm", "masked", "bf16", counts, K=K, N=N, cap=cap, values="normal", seed=44)
    inp = wl.materialize(w, "cuda")
    assert inp["A"].numel() * 2 > 1 << 32
    C = P.sentinel_like((G, cap, N))
    mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"])
    torch.cuda.synchronize()
    pairs = [(e, r) for e in range(G) for r in range(counts[e])]
    picks, ref = _rows_against_oracle(inp["A"], inp["B"], [(e * cap + r, e) for e, r in pairs])
    got = C.reshape(G * cap, N)[torch.tensor([r for r, _ in picks], device="cuda")].float().cpu().double().numpy()
    P.check_gemm(got, ref, "bf16", what="masked past 4 GiB")
    inval = C.reshape(G * cap, N)[torch.tensor([e * cap + r for e in (15, 16, 31) for r in (counts[e], cap - 1)],
                                               device="cuda")]
    assert bool((inval.view(torch.int16) == P.SENTINEL_BITS).all())


def test_contiguous_e8m0_widest_output():
    """E8M0 scales at their widest supported output, N = 32768 (N / 128 = 256
    scale bytes per row), on a small ragged histogram; sampled rows."""
    counts = [40, 0, 200, 4]                              # 244 rows: a multiple of 4
    announce("contiguous e8m0 N=32768", counts)
    w = wl.Workload("e8w", "contiguous", "fp8", counts, K=256, N=32768, values="normal", seed=23, scales="e8m0")
    inp = wl.materialize(w, "cuda")
    C, ws = run_contiguous_e8m0(w, inp, 0, mg.B_NK)
    P.check_stats(mg.stats_read(ws), counts)
    rows = P.sample_rows_contiguous(counts, 1, 64, extra=16, seed=3)
    cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}
    ref = P.oracle_contiguous_rows(w, cpu, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what="e8m0 N=32768")


def test_contiguous_deterministic_and_empty():
    announce("determinism + all-empty")
    w, inp = small_contig([300, 0, 17, 513], 512, 512, "fp8")
    C1, _ = P.run_contiguous(w, inp)
    C2, _ = P.run_contiguous(w, inp)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    # every expert empty: nothing written, accounting all zero
    w0 = wl.Workload("empty", "contiguous", "bf16", [0, 0, 0], K=256, N=256)
    A = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(3, 256, 256, dtype=torch.bfloat16, device="cuda")
    C = P.sentinel_like((4, 256))
    ws = mg.workspace(3, 4)
    mg.grouped_gemm_contiguous(A, B, C, torch.zeros(3, dtype=torch.int32, device="cuda"), ws)
    st = mg.stats_read(ws)
    assert st.U == 0 and st.tiles == 0 and all(v == 0 for v in st.P_at.values())
    assert bool((C.view(torch.int16) == P.SENTINEL_BITS).all())
    del w0


# ----------------------------------------------------------------- contiguous, full-size configs


def full_size_rows(w):
    """Rows compared at full size: one per 16-row block of every expert segment
    (every MFMA row block of every tile at every height), whole rows."""
    return list(range(w.rows_total)) if w.rows_total <= 512 else P.rows_every_block(w.counts, w.seg_align, w.seed)


def full_size_ref(w, inp, rows, tag=""):
    """The oracle's rows for a full-size seeded workload, computed once per session."""
    def compute():
        cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}
        return P.oracle_contiguous_rows(w, cpu, rows)
    return P.cached((w.name, w.scales, w.weights, tag, tuple(rows)), compute)


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_contiguous_config_full_size(n, b_layout):
    w = wl.workload(n)
    announce("contiguous config", n, w.name, "G", w.G, "K", w.K, "N", w.N, "seed", w.seed, "layout", b_layout)
    inp = wl.materialize(w, "cuda")
    C, ws = P.run_contiguous(w, inp, block_m=0, b_layout=b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, w.counts)
    assert st.block_m == P.choice_rule(w.counts, w.N // 256)
    if n == 1:
        assert [st.P_at[q] for q in (8, 16, 32)] == [160, 192, 256]
    rows = full_size_rows(w)
    ref = full_size_ref(w, inp, rows)
    del inp
    P.check_gemm(P.rows_as_float(C, rows), ref, w.dtype, what=f"config {n} block_m={st.block_m} layout={b_layout}")
    assert P.untouched_rows_ok(C, w.counts, w.seg_align)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
@pytest.mark.parametrize("block_m", [64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_every_tile_height_long_k(dtype, b_layout, block_m):
    """Every tile height and weight layout over a long reduction (56 to 112 K
    steps), where each stage of the load ring is reused many times.  A read that
    runs ahead of the barrier publishing its part of a stage shows up here as
    sporadic wrong blocks.  Issue histogram, aligned segments, N = 1024."""
    w = wl.Workload("long K", "contiguous", dtype, wl.hist_issue_32(), K=7168, N=1024, seg_align=128,
                    values="normal", seed=2)
    announce("long K", dtype, "layout", b_layout, "block_m", block_m)
    inp = wl.materialize(w, "cuda")
    C, ws = P.run_contiguous(w, inp, block_m=block_m, b_layout=b_layout)
    rows = P.sample_rows_contiguous(w.counts, w.seg_align, 256 if block_m < 0 else block_m, extra=16, seed=1)
    inp_cpu = {k: P.cpu(v) for k, v in inp.items()}
    del inp
    ref = P.oracle_contiguous_rows(w, inp_cpu, rows)
    got = P.rows_as_float(C, rows)
    P.check_gemm(got, ref, dtype, what=f"long K {dtype} layout={b_layout} block_m={block_m}")


@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_contiguous_per_expert_full_size(n, b_layout):
    """Per-expert tile heights on the full-size issue-histogram and zipf problems."""
    w = wl.workload(n)
    announce("per-expert full size", n, w.name, "layout", b_layout)
    inp = wl.materialize(w, "cuda")
    C, ws = P.run_contiguous(w, inp, block_m=mg.BLOCK_M_PER_EXPERT, b_layout=b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, w.counts, mg.BLOCK_M_PER_EXPERT)
    assert mg.tile_list_read(ws, st.tiles) == acc.tile_list_per_expert(w.counts, w.seg_align)
    rows = full_size_rows(w)
    ref = full_size_ref(w, inp, rows)
    del inp
    P.check_gemm(P.rows_as_float(C, rows), ref, w.dtype, what=f"per-expert config {n} layout={b_layout}")
    assert P.untouched_rows_ok(C, w.counts, w.seg_align)


# ----------------------------------------------------------------- masked


def masked_case(counts, cap, K, N, dtype, seed=4):
    w = wl.Workload("masked", "masked", dtype, counts, K=K, N=N, cap=cap, seed=seed)
    return w, wl.materialize(w, "cuda")


def check_masked(w, inp, C, counts):
    inp_cpu = {k: P.cpu(v) for k, v in inp.items()}
    reqs = [(e, r) for e in range(w.G) for r in range(min(max(counts[e], 0), w.cap))]
    if not reqs:
        return
    ref = og.masked(inp_cpu["A"], inp_cpu["B"], counts, [e for e, _ in reqs], [r for _, r in reqs],
                    A_scale=inp_cpu.get("A_scale"), B_scale=inp_cpu.get("B_scale"))
    idx = torch.tensor([e * w.cap + r for e, r in reqs], device="cuda")
    got = C.reshape(w.G * w.cap, -1)[idx].float().cpu().double().numpy()
    P.check_gemm(got, ref, w.dtype, what=f"masked G={w.G} cap={w.cap} K={w.K} N={w.N}")
    # rows past masked_m keep the sentinel
    inval = torch.tensor([e * w.cap + r for e in range(w.G) for r in range(w.cap)
                          if r >= min(max(counts[e], 0), w.cap)], device="cuda")
    if inval.numel():
        assert bool((C.reshape(w.G * w.cap, -1)[inval].view(torch.int16) == P.SENTINEL_BITS).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_masked_small(dtype, b_layout):
    counts = [3, 0, 64, 65, 130, 1]
    announce("masked small", dtype, b_layout, counts)
    w, inp = masked_case(counts, 160, 512, 256, dtype)
    B = inp["B"] if b_layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, inp.get("A_scale"), inp.get("B_scale"), b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, counts)
    check_masked(w, inp, C, counts)


def run_masked_low_precision(counts, cap, K, N, weights, b_layout, seed):
    """Masked layout with fp8 activations and E8M0 scales, e4m3 or packed E2M1 weights."""
    w = wl.Workload("masked-lp", "masked", "fp8", counts, K=K, N=N, cap=cap, seed=seed, scales="e8m0",
                    weights=weights)
    inp = wl.materialize(w, "cuda")
    B = inp["B"] if (b_layout == mg.B_KN or weights == "e2m1") else inp["B"].transpose(1, 2).contiguous()
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, inp["A_scale_e8m0"], inp["B_scale_e8m0"], b_layout)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), counts)
    return w, inp, C


def check_masked_fp4(w, inp, C, counts, pairs=None):
    cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}
    pairs = pairs or [(e, r) for e in range(w.G) for r in range(min(counts[e], w.cap))]
    ref = fp4.masked_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], counts, pairs)
    idx = torch.tensor([e * w.cap + r for e, r in pairs], device="cuda")
    got = C.reshape(w.G * w.cap, -1)[idx].float().cpu().double().numpy()
    P.check_gemm(got, ref, "fp8", what=f"masked fp8 x fp4 G={w.G} cap={w.cap}")


@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_masked_fp8_e8m0(b_layout):
    counts = [3, 0, 64, 65, 130, 1]
    announce("masked fp8 e8m0", b_layout, counts)
    w, inp, C = run_masked_low_precision(counts, 160, 512, 512, "e4m3", b_layout, seed=24)
    w.scales = "e8m0"
    check_masked(w, {k: v for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}, C, counts)


def test_masked_fp8_fp4():
    counts = [3, 0, 64, 65, 130, 1]
    announce("masked fp8 x fp4", counts)
    w, inp, C = run_masked_low_precision(counts, 160, 512, 512, "e2m1", mg.B_NK, seed=25)
    check_masked_fp4(w, inp, C, counts)
    inval = torch.tensor([e * w.cap + r for e in range(w.G) for r in range(w.cap) if r >= counts[e]], device="cuda")
    assert bool((C.reshape(w.G * w.cap, -1)[inval].view(torch.int16) == P.SENTINEL_BITS).all())


# per expert: one tile of each height (1, 64 | 65, 128 rows), then several
# 128-row tiles with a last one of each height
MASKED_HEIGHT_COUNTS = [1, 64, 65, 128, 129, 192, 0, 193, 256, 257, 385, 512]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK, mg.B_KN_PANEL, mg.B_NK_PANEL])
def test_masked_per_expert_heights(dtype, b_layout):
    """The masked kernel's row tiles around each height it picks (64 and 128,
    and several 128-row tiles before a last one of each): every valid row, the
    rows past masked_m untouched, and the stats' tile count."""
    counts = MASKED_HEIGHT_COUNTS
    announce("masked per-expert heights", dtype, b_layout, counts)
    w, inp = masked_case(counts, 512, 512, 256, dtype, seed=26)
    B = inp["B"]
    if b_layout in (mg.B_NK, mg.B_NK_PANEL):
        B = B.transpose(1, 2).contiguous()
    if b_layout in (mg.B_KN_PANEL, mg.B_NK_PANEL):
        B = mg.pack_panels(inp["B"], b_layout, mg.PANEL_MASKED)
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, inp.get("A_scale"), inp.get("B_scale"), b_layout)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), counts, 128)
    check_masked(w, inp, C, counts)


@pytest.mark.parametrize("weights", ["e4m3", "e2m1"])
def test_masked_per_expert_heights_low_precision(weights):
    """E8M0 scales with e4m3 or fp4 weights at the same row counts."""
    counts = MASKED_HEIGHT_COUNTS
    announce("masked per-expert heights", weights, counts)
    w, inp, C = run_masked_low_precision(counts, 512, 512, 512, weights, mg.B_NK, seed=27)
    if weights == "e2m1":
        check_masked_fp4(w, inp, C, counts)
        inval = torch.tensor([e * w.cap + r for e in range(w.G) for r in range(w.cap) if r >= counts[e]],
                             device="cuda")
        assert bool((C.reshape(w.G * w.cap, -1)[inval].view(torch.int16) == P.SENTINEL_BITS).all())
    else:
        w.scales = "e8m0"
        check_masked(w, {k: v for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}, C, counts)


def test_masked_fp8_fp4_full_size():
    """The masked decode workload (32 experts, cap 256, K 2048, N 7168) with fp8
    activations and fp4 weights; sampled rows."""
    w0 = wl.workload(4)
    announce("masked fp8 x fp4 full size", w0.name)
    w, inp, C = run_masked_low_precision(w0.counts, w0.cap, w0.K, w0.N, "e2m1", mg.B_NK, seed=w0.seed)
    rng = random.Random(7)
    pairs = sorted({(e, r) for e in range(w.G) for r in range(w0.counts[e]) if r in (0, w0.counts[e] - 1)
                    or rng.random() < 0.1})
    check_masked_fp4(w, inp, C, w0.counts, pairs)


@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_masked_config_full_size(b_layout):
    w = wl.workload(4)
    announce("masked config 4", w.counts, "layout", b_layout)
    inp = wl.materialize(w, "cuda")
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    B = inp["B"] if b_layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, b_layout=b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, w.counts)
    check_masked(w, inp, C, w.counts)


def test_masked_counts_out_of_range_are_clamped():
    """masked_m above cap reads as cap and below 0 as 0: the stats carry both
    flags and the clamped accounting, the kernel writes exactly the clamped
    rows (every row of an over-cap expert, none of a negative one), and nothing
    is read or written past the capacity buffer."""
    counts = [300, -5, 40, 256, 0, 257, -1, 1]
    cap = 256
    clamped = [min(max(c, 0), cap) for c in counts]
    announce("masked clamp", counts, "cap", cap)
    w, inp = masked_case(counts, cap, 256, 256, "bf16")
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"], ws)
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    assert st.error_flags == mg.FLAG_NEGATIVE_COUNT | mg.FLAG_COUNT_OVER_CAP, hex(st.error_flags)
    ref = acc.summary(clamped)
    assert (st.U, st.active, st.sum_sq, st.P_at) == (ref["U"], ref["active"], ref["sum_sq"], ref["P"])
    assert st.capacity_rows == w.G * cap - ref["U"]
    check_masked(w, inp, C, counts)          # valid rows = the clamped counts; the rest keep the sentinel
    # without a workspace (no stats) the kernel clamps the same way
    C2 = P.sentinel_like((w.G, w.cap, w.N))
    mg.grouped_gemm_masked(inp["A"], inp["B"], C2, inp["counts"])
    torch.cuda.synchronize()
    assert torch.equal(C2.view(torch.int16), C.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("cap", [1, 3, 17])
def test_masked_tiny_capacity(dtype, cap):
    """Capacity buffers smaller than one MFMA row block: a tile's rows past
    masked_m read zeros from the expert's bounded buffer range, not the next
    expert's rows.  Counts at, over and under the capacity: flags, clamped
    stats, every valid row against the oracle, the rest keep the sentinel."""
    counts = [cap, 0, cap + 5, -2, 1, cap, min(2, cap)]
    clamped = [min(max(c, 0), cap) for c in counts]
    announce("masked tiny capacity", dtype, cap, counts)
    w, inp = masked_case(counts, cap, 256, 256, dtype, seed=61)
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"], ws, inp.get("A_scale"), inp.get("B_scale"))
    torch.cuda.synchronize()
    st = mg.stats_read(ws)
    assert st.error_flags == mg.FLAG_NEGATIVE_COUNT | mg.FLAG_COUNT_OVER_CAP, hex(st.error_flags)
    ref = acc.summary(clamped)
    assert (st.U, st.active, st.sum_sq, st.P_at) == (ref["U"], ref["active"], ref["sum_sq"], ref["P"])
    check_masked(w, inp, C, counts)


@pytest.mark.parametrize("scale_km", [False, True])
def test_masked_fp8_fp32_scales_full_size(scale_km):
    """The masked decode workload's shape (32 experts, cap 256, K 2048, N 7168,
    Poisson(24) counts) with e4m3 operands and fp32 scales, activation scales
    [G, cap, K/128] or transposed [K/128, G * cap]: every valid row."""
    w0 = wl.workload(4)
    announce("masked fp8 fp32 scales full size", "scale_km", scale_km)
    w = wl.Workload("masked fp8", "masked", "fp8", w0.counts, K=w0.K, N=w0.N, cap=w0.cap, seed=w0.seed)
    inp = wl.materialize(w, "cuda")
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    a_scale = inp["A_scale"].reshape(w.G * w.cap, -1).t().contiguous() if scale_km else inp["A_scale"]
    mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"], ws, a_scale, inp["B_scale"], mg.B_KN,
                           scale_km=scale_km)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), w.counts)
    check_masked(w, inp, C, w.counts)


def test_masked_graph_replay():
    """Capture once; rewrite masked_m in place between replays (no host sync
    in the capture); every replay matches the oracle."""
    counts0 = [5, 0, 40, 17]
    announce("masked graph replay")
    w, inp = masked_case(counts0, 64, 256, 256, "bf16")
    C = P.sentinel_like((w.G, w.cap, w.N))
    mm = inp["counts"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mg.grouped_gemm_masked(inp["A"], inp["B"], C, mm)        # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.grouped_gemm_masked(inp["A"], inp["B"], C, mm)
    for counts in ([5, 0, 40, 17], [0, 0, 0, 0], [64, 64, 64, 64], [1, 63, 0, 2], [5, 0, 40, 17]):
        # the capture buffer's invalid rows must be NaN for rows that become valid: refill A
        fresh = wl.materialize(wl.Workload("m", "masked", "bf16", counts, K=256, N=256, cap=64, seed=4), "cuda")
        inp["A"].copy_(fresh["A"])
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        C.view(torch.int16).fill_(P.SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        w.counts = counts
        check_masked(w, inp, C, counts)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_masked_graph_replay_across_heights(dtype):
    """The masked kernel picks its row-tile height from masked_m on the device:
    one captured graph replayed with counts that move every expert across the 64-
    and 128-row heights and the multi-tile walk (and to empty and to cap), stats
    included, each replay against the oracle."""
    cap, K, N = 300, 256, 256
    seqs = ([3, 0, 64, 65, 130], [128, 129, 0, 300, 1], [0, 0, 0, 0, 0], [257, 64, 65, 1, 200],
            [300, 300, 300, 300, 300], [3, 0, 64, 65, 130])
    announce("masked graph replay across heights", dtype)
    w, inp = masked_case(seqs[0], cap, K, N, dtype, seed=33)
    C = P.sentinel_like((w.G, cap, N))
    ws = mg.workspace(w.G, w.G * cap)
    mm = inp["counts"]
    call = lambda: mg.grouped_gemm_masked(inp["A"], inp["B"], C, mm, ws, inp.get("A_scale"), inp.get("B_scale"),
                                          mg.B_KN)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for counts in seqs:
        fresh = wl.materialize(wl.Workload("m", "masked", dtype, counts, K=K, N=N, cap=cap, seed=33), "cuda")
        for k in ("A", "A_scale"):
            if fresh.get(k) is not None:
                inp[k].copy_(fresh[k])
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        C.view(torch.int16).fill_(P.SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        P.check_stats(mg.stats_read(ws), counts, 128)
        w.counts = counts
        check_masked(w, inp, C, counts)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_contiguous_graph_replay(dtype):
    """Scheduler and contiguous GEMM captured together in one graph (block_m = 0:
    the device picks the height, every candidate kernel is in the graph).  The
    counts are rewritten in place between replays, with no host round trip
    inside the capture; each replay matches the oracle on every valid row,
    leaves the other rows alone, and lists the tiles the oracle lists."""
    rows_total = 400
    hists = ([70, 0, 300, 5], [0, 0, 0, 0], [100, 100, 100, 100], [1, 0, 398, 1], [256, 129, 15, 0], [70, 0, 300, 5])
    announce("contiguous graph replay", dtype)
    w = wl.Workload("g", "contiguous", dtype, [rows_total, 0, 0, 0], K=256, N=256, values="normal", seed=7)
    inp = wl.materialize(w, "cuda")
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    m = inp["counts"]
    C = P.sentinel_like((rows_total, w.N))
    ws = mg.workspace(w.G, rows_total)

    def step():
        mg.schedule(m, rows_total, ws, seg_align=1, block_m=0, N=w.N)
        mg.grouped_gemm_contiguous_scheduled(inp["A"], inp["B"], C, w.G, ws, inp.get("A_scale"), inp.get("B_scale"),
                                             block_m=0)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for counts in hists:
        m.copy_(torch.tensor(counts, dtype=torch.int32))
        C.view(torch.int16).fill_(P.SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        st = mg.stats_read(ws)
        P.check_stats(st, counts)
        assert st.block_m == P.choice_rule(counts, 1)
        assert mg.tile_list_read(ws, st.tiles) == expected_tiles(counts, st.block_m, 1)
        wc = wl.Workload("g", "contiguous", dtype, counts, K=256, N=256, values="normal", seed=7)
        rows = [r for e, s0 in enumerate(acc.segment_offsets(counts, 1)[:-1]) for r in range(s0, s0 + counts[e])]
        if rows:
            ref = P.oracle_contiguous_rows(wc, cpu, rows)
            P.check_gemm(P.rows_as_float(C, rows), ref, dtype, what=f"graph replay {counts}")
        assert P.untouched_rows_ok(C, counts, 1), counts


# ----------------------------------------------------------------- fp8 with E8M0 scales


def run_contiguous_e8m0(w, inp, block_m, b_layout):
    B = inp["B"] if b_layout == mg.B_KN else inp["B"].transpose(1, 2).contiguous()
    C = P.sentinel_like((w.rows_total, w.N))
    ws = mg.workspace(w.G, w.rows_total)
    mg.grouped_gemm_contiguous(inp["A"], B, C, inp["counts"], ws, A_scale=inp["A_scale_e8m0"],
                               B_scale=inp["B_scale_e8m0"], seg_align=w.seg_align, block_m=block_m,
                               b_layout=b_layout)
    torch.cuda.synchronize()
    return C, ws


@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
@pytest.mark.parametrize("b_layout", [mg.B_KN, mg.B_NK])
def test_contiguous_fp8_e8m0(block_m, b_layout):
    """fp8 with power-of-two block scales given as E8M0 bytes (the MFMA applies
    them): every valid row against the oracle run on the same scales as fp32."""
    counts = [70, 0, 300, 6, 129, 3]                     # 508 rows: a multiple of 4, ragged tails
    announce("contiguous fp8 e8m0", counts, "block_m", block_m, "layout", b_layout)
    w = wl.Workload("e8", "contiguous", "fp8", counts, K=512, N=512, values="normal", seed=9, scales="e8m0")
    inp = wl.materialize(w, "cuda")
    C, ws = run_contiguous_e8m0(w, inp, block_m, b_layout)
    st = mg.stats_read(ws)
    P.check_stats(st, counts)
    rows = list(range(w.rows_total))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    ref = P.oracle_contiguous_rows(w, cpu, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what=f"e8m0 block_m={st.block_m} layout={b_layout}")


def test_contiguous_fp8_e8m0_full_size():
    """The Zipf fp8 workload with E8M0 scales, K-contiguous weights, device-chosen height."""
    w = wl.workload(3)
    w.scales = "e8m0"
    announce("contiguous fp8 e8m0 full size", w.name)
    inp = wl.materialize(w, "cuda")
    C, ws = run_contiguous_e8m0(w, inp, 0, mg.B_NK)
    st = mg.stats_read(ws)
    P.check_stats(st, w.counts)
    rows = full_size_rows(w)
    ref = full_size_ref(w, inp, rows)
    del inp
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what=f"e8m0 full size block_m={st.block_m}")
    assert P.untouched_rows_ok(C, w.counts, w.seg_align)


# ----------------------------------------------------------------- fp8 x fp4 (E2M1 weights)


def run_contiguous_fp4(w, inp, block_m, b_layout=mg.B_NK):
    """b_layout B_NK_PANEL: the packed weights cut into 256-row panels first."""
    C = P.sentinel_like((w.rows_total, w.N))
    ws = mg.workspace(w.G, w.rows_total)
    B = inp["B"] if b_layout == mg.B_NK else mg.pack_panels(inp["B"], mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
    mg.grouped_gemm_contiguous(inp["A"], B, C, inp["counts"], ws, A_scale=inp["A_scale_e8m0"],
                               B_scale=inp["B_scale_e8m0"], seg_align=w.seg_align, block_m=block_m,
                               b_layout=b_layout)
    torch.cuda.synchronize()
    return C, ws


@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_fp8_fp4(block_m):
    """fp8 activations x packed E2M1 weights, both with E8M0 block scales:
    every valid row against the fp8 x fp4 oracle."""
    counts = [70, 0, 300, 6, 129, 3]                     # 508 rows: a multiple of 4, ragged tails
    announce("contiguous fp8 x fp4", counts, "block_m", block_m)
    w = wl.Workload("f4", "contiguous", "fp8", counts, K=512, N=512, values="normal", seed=9, scales="e8m0",
                    weights="e2m1")
    inp = wl.materialize(w, "cuda")
    assert mg._operands(w.rows_total, w.K, inp["A"], inp["A_scale_e8m0"], inp["B"], inp["B_scale_e8m0"], w.G,
                        mg.B_NK, False)[0] == mg.FP8_E4M3_FP4_E2M1
    C, ws = run_contiguous_fp4(w, inp, block_m)
    st = mg.stats_read(ws)
    P.check_stats(st, counts)
    rows = list(range(w.rows_total))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    ref = fp4.contiguous_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], counts, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what=f"fp4 block_m={st.block_m}")
    assert P.untouched_rows_ok(C, counts, 1)


@pytest.mark.parametrize("block_m", [64, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_fp8_fp4_integer_exact(block_m):
    """Activations in {-1, 0, 1}, weights in {0, +-0.5, +-1}, unit scales,
    K = 128: every result is a multiple of 0.5 of magnitude <= 128, exact in
    bf16, so GPU == oracle bit for bit.  Pins the fp4 operand's nibble order
    and K slots against the fp8 operand's."""
    announce("fp8 x fp4 integer exact", block_m)
    counts, K, N = [37, 0, 200, 7], 128, 512
    G, rows_total = len(counts), sum(counts)
    g = torch.Generator().manual_seed(7)
    A = torch.randint(-1, 2, (rows_total, K), generator=g).float().to(torch.float8_e4m3fn)
    codes = torch.tensor([0, 1, 2, 9, 10], dtype=torch.uint8)[torch.randint(0, 5, (G, N, K), generator=g)]
    B = codes[..., 0::2] | (codes[..., 1::2] << 4)
    A_s8 = torch.full((K // 128, rows_total), 127, dtype=torch.uint8)
    B_s8 = torch.full((G, K // 128, N // 128), 127, dtype=torch.uint8)
    w = wl.Workload("int4", "contiguous", "fp8", counts, K=K, N=N, scales="e8m0", weights="e2m1")
    inp = {"A": A.cuda(), "B": B.contiguous().cuda(), "A_scale_e8m0": A_s8.cuda(), "B_scale_e8m0": B_s8.cuda(),
           "counts": torch.tensor(counts, dtype=torch.int32, device="cuda")}
    C, _ = run_contiguous_fp4(w, inp, block_m)
    ref = fp4.contiguous_fp8_fp4(A, torch.ones(rows_total, K // 128), B.contiguous(), torch.ones(G, K // 128, N // 128),
                                 counts, range(rows_total))
    got = C.float().cpu().double().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_fp4_panels_bit_exact(block_m):
    """fp4 weights in 256-row panels (one K step of a panel = 16 KB of whole
    lines) give the same bits as [G, N, K/2] at every height."""
    counts = [70, 0, 300, 6, 129, 3]
    announce("contiguous fp4 panels", counts, "block_m", block_m)
    w = wl.Workload("f4p", "contiguous", "fp8", counts, K=512, N=512, values="normal", seed=29, scales="e8m0",
                    weights="e2m1")
    inp = wl.materialize(w, "cuda")
    C0, _ = run_contiguous_fp4(w, inp, block_m)
    C1, _ = run_contiguous_fp4(w, inp, block_m, mg.B_NK_PANEL)
    assert torch.equal(C0.view(torch.int16), C1.view(torch.int16))


def test_masked_fp4_panels_bit_exact():
    """The masked call with fp4 weights in 128-row panels: the same bits as
    [G, N, K/2], with experts of one and of several row tiles."""
    counts = [3, 0, 64, 65, 130, 1, 257]
    announce("masked fp4 panels", counts)
    w, inp, C0 = run_masked_low_precision(counts, 320, 512, 512, "e2m1", mg.B_NK, seed=30)
    C1 = P.sentinel_like((w.G, w.cap, w.N))
    mg.grouped_gemm_masked(inp["A"], mg.pack_panels(inp["B"], mg.B_NK_PANEL, mg.PANEL_MASKED), C1, inp["counts"],
                           None, inp["A_scale_e8m0"], inp["B_scale_e8m0"], mg.B_NK_PANEL)
    torch.cuda.synchronize()
    assert torch.equal(C0.view(torch.int16), C1.view(torch.int16))
    check_masked_fp4(w, inp, C1, counts)


def test_contiguous_fp8_fp4_aligned_segments():
    """fp4 weights with segments aligned to 64 rows (gaps between experts stay untouched)."""
    counts = [70, 0, 300, 6, 129, 3]
    announce("contiguous fp8 x fp4 aligned", counts)
    w = wl.Workload("f4a", "contiguous", "fp8", counts, K=256, N=512, seg_align=64, values="normal", seed=19,
                    scales="e8m0", weights="e2m1")
    inp = wl.materialize(w, "cuda")
    C, ws = run_contiguous_fp4(w, inp, 0)
    P.check_stats(mg.stats_read(ws), counts)
    rows = [r for e, s0 in enumerate(acc.segment_offsets(counts, 64)[:-1]) for r in range(s0, s0 + counts[e])]
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    ref = fp4.contiguous_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], counts, rows, seg_align=64)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what="fp4 aligned 64")
    assert P.untouched_rows_ok(C, counts, 64)


def test_contiguous_fp8_fp4_full_size():
    """The Zipf workload (64 experts, 32768 rows, K = 7168, N = 4096) with fp4
    weights, device-chosen height, on sampled rows."""
    w = wl.workload(3)
    w.scales, w.weights = "e8m0", "e2m1"
    announce("contiguous fp8 x fp4 full size", w.name)
    inp = wl.materialize(w, "cuda")
    C, ws = run_contiguous_fp4(w, inp, 0)
    st = mg.stats_read(ws)
    P.check_stats(st, w.counts)
    rows = full_size_rows(w)
    cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("A_scale_e8m0", "B_scale_e8m0")}
    del inp
    ref = fp4.contiguous_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], w.counts, rows)
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what=f"fp4 full size block_m={st.block_m}")
    assert P.untouched_rows_ok(C, w.counts, w.seg_align)
    # the paneled weights the benchmark streams: every element, bit for bit
    inp = wl.materialize(w, "cuda")
    C1, _ = run_contiguous_fp4(w, inp, 0, mg.B_NK_PANEL)
    assert torch.equal(C.view(torch.int16), C1.view(torch.int16))


# ----------------------------------------------------------------- exemplar selection


SELECT_HISTS = dict(SCHED_HISTS, **{
    f"zipf{s_}_{u}": wl.hist_zipf(seed=77 + u, experts=64, total=u, s=s_)
    for u in (300, 3000, 30000) for s_ in (0.0, 1.0, 1.6)})


def run_selection(counts, table, ws, hysteresis=0, N=4096):
    ct = torch.tensor(counts, dtype=torch.int32, device="cuda")
    rows = max(1, sum(counts))
    mg.schedule_exemplar(ct, rows, ws, table, hysteresis=hysteresis, N=N)
    return mg.selection_read(ws), mg.stats_read(ws)


def check_selection(counts, table_rows, got, st, expect_idx, expect_d):
    assert got.exemplar == expect_idx
    assert got.distance == expect_d
    assert (got.size_class, list(got.lorenz)) == oselect.descriptor(counts)
    bm = table_rows[expect_idx][-1]
    assert st.block_m == bm
    P.check_stats(st, counts)


@pytest.mark.parametrize("dtype", sorted(mg.EXEMPLAR_TABLE_PATHS))
@pytest.mark.parametrize("name", sorted(SELECT_HISTS))
def test_exemplar_selection_matches_oracle(name, dtype):
    """Descriptor, nearest exemplar, distance and the resulting tile list,
    bit-exact against the oracle, with each shipped MI355X table."""
    counts = SELECT_HISTS[name]
    announce("exemplar selection", name, len(counts), dtype)
    table = mg.exemplar_table(dtype=dtype)
    rows = table.cpu().tolist()
    rows_total = max(1, sum(counts))
    ws = torch.zeros(mg.workspace_bytes(len(counts), rows_total), dtype=torch.uint8, device="cuda")
    got, st = run_selection(counts, table, ws)
    idx, d = oselect.select(counts, rows)
    check_selection(counts, rows, got, st, idx, d)
    bm = rows[idx][-1]
    if bm == mg.BLOCK_M_PER_EXPERT:
        expect = acc.tile_list_per_expert(counts, 1)
    else:
        expect = acc.tile_list(counts, bm, 1)
    assert mg.tile_list_read(ws, len(expect) + 4) == expect


@pytest.mark.parametrize("G", [255, 1000, 4096])
def test_exemplar_descriptor_large_expert_counts(G):
    """The device sort covers up to 4096 experts (padded to a power of two):
    descriptor and choice against the oracle on random skewed histograms."""
    rng = random.Random(G)
    counts = [0 if rng.random() < 0.3 else int(rng.paretovariate(1.1) * 3) for _ in range(G)]
    announce("exemplar large G", G, sum(counts))
    table = mg.exemplar_table()
    rows = table.cpu().tolist()
    ws = torch.zeros(mg.workspace_bytes(G, max(1, sum(counts))), dtype=torch.uint8, device="cuda")
    got, st = run_selection(counts, table, ws)
    idx, d = oselect.select(counts, rows)
    check_selection(counts, rows, got, st, idx, d)


def test_exemplar_hysteresis_sequence():
    """One workspace through a drifting sequence of histograms: the device
    keeps or switches exemplars exactly as the oracle's state machine does."""
    table_rows = [[sel_sc, *oselect.lorenz(h), bm] for sel_sc, h, bm in (
        (oselect.size_class(4096), [64] * 64, 64),
        (oselect.size_class(4096), [1024, 1024] + [32] * 62, 256),
        (oselect.size_class(4096), [3000] + [17] * 63, mg.BLOCK_M_PER_EXPERT))]
    table = torch.tensor(table_rows, dtype=torch.int32, device="cuda")
    rng = random.Random(9)
    ws = torch.zeros(mg.workspace_bytes(64, 8192), dtype=torch.uint8, device="cuda")
    prev = None
    H = 20000
    switches = 0
    for step in range(40):
        hot = rng.choice([0, 300, 600, 900, 1200, 2000, 3000])
        counts = [hot] + [max(0, (4096 - hot) // 63 + rng.randint(-3, 3)) for _ in range(63)]
        announce("hysteresis step", step, hot)
        got, st = run_selection(counts, table, ws, hysteresis=H)
        idx, d = oselect.select(counts, table_rows, hysteresis=H, prev=prev)
        check_selection(counts, table_rows, got, st, idx, d)
        switches += prev is not None and idx != prev
        prev = idx
    assert switches > 0


def test_exemplar_invalid_block_m_falls_back_to_the_cost_rule():
    counts = wl.hist_issue_32()
    table = torch.tensor([[0] * 9 + [96]], dtype=torch.int32, device="cuda")
    ws = torch.zeros(mg.workspace_bytes(32, sum(counts)), dtype=torch.uint8, device="cuda")
    announce("exemplar fallback")
    ct = torch.tensor(counts, dtype=torch.int32, device="cuda")
    mg.schedule_exemplar(ct, sum(counts), ws, table, N=4096)
    st = mg.stats_read(ws)
    assert st.error_flags == mg.FLAG_BAD_EXEMPLAR
    assert st.block_m == P.choice_rule(counts, 4096 // 256)


def test_exemplar_selection_in_a_graph():
    """Selection and GEMM captured once, replayed with new counts written in
    place: each replay's choice, tile list and output rows match the oracle,
    and the remembered choice carries from replay to replay."""
    G, K, N, R = 16, 256, 512, 2048
    w = wl.Workload("sel-graph", "contiguous", "bf16", [128] * G, K=K, N=N, values="normal", seed=31)
    inp = wl.materialize(w, "cuda", nan_padding=False)
    table_rows = [[oselect.size_class(R), *oselect.lorenz([128] * G), 64],
                  [oselect.size_class(R), *oselect.lorenz([1800] + [16] * (G - 1)), 256]]
    table = torch.tensor(table_rows, dtype=torch.int32, device="cuda")
    counts_t = torch.tensor([128] * G, dtype=torch.int32, device="cuda")
    ws = torch.zeros(mg.workspace_bytes(G, R), dtype=torch.uint8, device="cuda")
    C = torch.zeros((R, N), dtype=torch.bfloat16, device="cuda")
    announce("exemplar graph capture")

    def step():
        mg.schedule_exemplar(counts_t, R, ws, table, hysteresis=1000, N=N)
        mg.grouped_gemm_contiguous_scheduled(inp["A"], inp["B"], C, G, ws, block_m=0)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ws.zero_()                                          # no remembered choice before the first replay
    torch.cuda.synchronize()
    prev = None
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    for counts in ([128] * G, [1800] + [16] * (G - 1), [1700] + [20] * (G - 2) + [48], [100] * G):
        announce("graph replay", counts[:3])
        counts_t.copy_(torch.tensor(counts, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, st = mg.selection_read(ws), mg.stats_read(ws)
        idx, d = oselect.select(counts, table_rows, hysteresis=1000, prev=prev)
        check_selection(counts, table_rows, got, st, idx, d)
        prev = idx
        rows = P.sample_rows_contiguous(counts, 1, 64, extra=16, seed=5)
        ref = og.contiguous(cpu["A"], cpu["B"], counts, rows)
        P.check_gemm(P.rows_as_float(C, rows), ref, "bf16", what=f"exemplar graph {counts}")


# ----------------------------------------------------------------- expert MLP: L1 -> SwiGLU -> L2

# y goes through two bf16 roundings in sequence (h, then y), each about 1.7e-3 of
# rel. Frobenius error on this data; in quadrature about 2.4e-3
TOL_MLP_BF16 = 3e-3


def run_mlp(counts, inp, block_m, N2):
    G, R = len(counts), sum(counts)
    I = inp["W1"].shape[1] // 2
    ws = mg.workspace(G, R)
    H = P.sentinel_like((R, I))
    Y = P.sentinel_like((R, N2))
    mg.schedule(inp["counts"], R, ws, block_m=block_m, N=2 * I)
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, inp["A_scale"], inp["W1_scale"],
                                     block_m=block_m)
    mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, block_m=block_m, b_layout=mg.B_NK)
    torch.cuda.synchronize()
    return H, Y, ws


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_swiglu_and_down_projection(dtype, block_m):
    """L1 with the fused SwiGLU epilogue, then L2 on H from the same schedule:
    H and y on every valid row against the fp64 chain."""
    counts = [70, 0, 300, 6, 129, 3]
    K, I, N2 = 256, 256, 512
    announce("expert MLP", dtype, counts, "block_m", block_m)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype=dtype, seed=12, device="cuda")
    H, Y, ws = run_mlp(counts, inp, block_m, N2)
    P.check_stats(mg.stats_read(ws), counts)
    rows = list(range(sum(counts)))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    y = omlp.down_rows(h, cpu["W2"], counts, rows)
    got_h, got_y = P.rows_as_float(H, rows), P.rows_as_float(Y, rows)
    P.check_gemm(got_h, h, dtype, what=f"mlp {dtype} block_m={block_m} h")
    ey = og.rel_frobenius(got_y, y)
    assert ey <= (TOL_MLP_BF16 if dtype == "bf16" else P.TOL["fp8"]), ey
    assert P.elementwise_ratio(got_y, y, "chain") <= 1.0


def dequant_h(H, Hs):
    return (H.float().double() * Hs.double().repeat_interleave(128, dim=1)).cpu().numpy()


def e4m3_ordinal(v: np.ndarray) -> np.ndarray:
    """Signed position of each e4m3 value on the code line (adjacent values differ by 1)."""
    c = torch.from_numpy(v).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_fp8_h(H, Hs, h_ref, rows):
    """GPU e4m3 H against the oracle's quantization of its fp64 h: dequantized
    values within the fp8 bar; codes equal except where the GPU's fp32 h and the
    fp64 h fall on opposite sides of a rounding boundary (measured about 0.15 %
    of codes)."""
    q, s = omlp.quantize_groups(h_ref)
    idx = torch.tensor(list(rows), device=H.device)
    got = dequant_h(H[idx], Hs[idx])
    err = og.rel_frobenius(got, q * np.repeat(s, 128, axis=1))
    gq = H[idx].float().cpu().double().numpy()
    step = np.abs(e4m3_ordinal(gq) - e4m3_ordinal(q))
    # the GPU's h carries an absolute error of about 1e-5 of the group's amax (measured:
    # two-step differences at |h / s| ~ 0.05); once |h / s| >= 4 that is under half a
    # step (code spacing >= 1/16 relative), so there a code can only move to its neighbour
    big = np.abs(q) >= 4.0
    assert err <= P.TOL["fp8"], err
    assert not ((step > 1) & big).any(), (gq[(step > 1) & big][:8], q[(step > 1) & big][:8])
    assert float(np.mean(step > 0)) <= 1e-2, float(np.mean(step > 0))
    return q, s


@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_swiglu_e4m3_h_and_fp8_down_projection(block_m):
    """Both expert GEMMs in fp8: L1's epilogue quantizes H to e4m3 with 1x128
    scales, L2 runs on those codes and scales.  H and y on every valid row."""
    counts = [70, 0, 300, 6, 129, 3]
    K, I, N2 = 256, 256, 512
    G, R = len(counts), sum(counts)
    announce("expert MLP fp8 H", counts, "block_m", block_m)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=16, device="cuda", l2="fp8")
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=block_m, N=2 * I)
    H = torch.empty((R, I), dtype=torch.float8_e4m3fn, device="cuda")
    Hs = torch.full((R, I // 128), float("nan"), device="cuda")
    Y = P.sentinel_like((R, N2))
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, inp["A_scale"], inp["W1_scale"],
                                     block_m=block_m, H_scale=Hs)
    mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], block_m=block_m,
                                         b_layout=mg.B_NK)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), counts)
    rows = list(range(R))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    assert bool(torch.isfinite(Hs).all())
    q, s = check_fp8_h(H, Hs, h, rows)
    qa = torch.from_numpy(q).float().to(torch.float8_e4m3fn).contiguous()
    y = og.contiguous(qa, cpu["W2"].transpose(1, 2).contiguous(), counts, rows,
                      A_scale=torch.from_numpy(s).float().contiguous(), B_scale=cpu["W2_scale"])
    P.check_gemm(P.rows_as_float(Y, rows), y, "fp8", bound="chain_e4m3", what=f"mlp fp8 H block_m={block_m} y")


def run_mlp_fp4(counts, K, I, N2, block_m, seed, w1_layout=mg.B_NK):
    """L1 with fp4 gate/up weights (fp8 activations, E8M0 scales) and the e4m3 H
    epilogue, then the fp8 L2 on H.  w1_layout B_NK_PANEL: W1 in 256-row panels."""
    G, R = len(counts), sum(counts)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=seed, device="cuda", l2="fp8",
                             w1_format="e2m1")
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=block_m, N=2 * I)
    H = torch.empty((R, I), dtype=torch.float8_e4m3fn, device="cuda")
    Hs = torch.full((R, I // 128), float("nan"), device="cuda")
    Y = P.sentinel_like((R, N2))
    W1 = inp["W1"] if w1_layout == mg.B_NK else mg.pack_panels(inp["W1"], mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
    mg.grouped_gemm_swiglu_scheduled(inp["A"], W1, H, G, ws, inp["A_scale_e8m0"], inp["W1_scale_e8m0"],
                                     block_m=block_m, H_scale=Hs, b_layout=w1_layout)
    mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], block_m=block_m,
                                         b_layout=mg.B_NK)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), counts)
    return inp, H, Hs, Y


@pytest.mark.parametrize("block_m", [0, 64, 256, mg.BLOCK_M_PER_EXPERT])
def test_swiglu_fp4_weights(block_m):
    """Expert MLP with fp4 gate/up weights: H (e4m3) and y on every valid row."""
    counts = [70, 0, 300, 6, 129, 3]                     # 508 rows: a multiple of 4 (E8M0 scale rows)
    K, I, N2 = 256, 256, 512
    announce("expert MLP fp4 L1", counts, "block_m", block_m)
    inp, H, Hs, Y = run_mlp_fp4(counts, K, I, N2, block_m, seed=26)
    rows = list(range(sum(counts)))
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows_fp4(cpu["A"], cpu["A_scale"], cpu["W1"], cpu["W1_scale"], counts, rows)
    q, s = check_fp8_h(H, Hs, h, rows)
    qa = torch.from_numpy(q).float().to(torch.float8_e4m3fn).contiguous()
    y = og.contiguous(qa, cpu["W2"].transpose(1, 2).contiguous(), counts, rows,
                      A_scale=torch.from_numpy(s).float().contiguous(), B_scale=cpu["W2_scale"])
    P.check_gemm(P.rows_as_float(Y, rows), y, "fp8", bound="chain_e4m3", what=f"mlp fp4 L1 block_m={block_m} y")


@pytest.mark.parametrize("block_m", [0, mg.BLOCK_M_PER_EXPERT])
def test_swiglu_fp4_panels_bit_exact(block_m):
    """fp4 gate/up weights in 256-row panels: H, its scales and y bit for bit
    as with [G, 2I, K/2]."""
    counts = [70, 0, 300, 6, 129, 3]
    announce("expert MLP fp4 L1 panels", counts, "block_m", block_m)
    outs = [run_mlp_fp4(counts, 256, 256, 512, block_m, seed=31, w1_layout=lay)[1:]
            for lay in (mg.B_NK, mg.B_NK_PANEL)]
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_expert_mlp_fp4_full_size():
    """fp4 gate/up weights at the DeepSeek-V3 expert shape on the Zipf histogram
    (the configuration bench.py --mlp --weights e2m1 times); sampled rows."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    announce("expert MLP fp4 L1 full size")
    inp, H, Hs, Y = run_mlp_fp4(counts, K, I, N2, 0, seed=27)
    rows = P.sample_rows_contiguous(counts, 1, 256, extra=24, seed=19)
    got_y = P.rows_as_float(Y, rows)
    cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("W_gate", "W_up")}
    del inp
    h = omlp.swiglu_rows_fp4(cpu["A"], cpu["A_scale"], cpu["W1"], cpu["W1_scale"], counts, rows)
    q, s = check_fp8_h(H, Hs, h, rows)
    offs = acc.segment_offsets(counts, 1)
    ex = [next(e for e in range(len(counts)) if offs[e] <= r < offs[e] + counts[e]) for r in rows]
    y = np.empty((len(rows), N2))
    for e in sorted(set(ex)):
        idx = [i for i, x in enumerate(ex) if x == e]
        w2e = cpu["W2"][e].float().double().numpy() * np.repeat(
            np.repeat(cpu["W2_scale"][e].double().numpy(), 128, 0), 128, 1).T
        y[idx] = (q[idx] * np.repeat(s[idx], 128, axis=1)) @ w2e.T
    P.check_gemm(got_y, y, "fp8", bound="chain_e4m3", what="mlp fp4 L1 full size y")


def test_expert_mlp_fp8_full_size():
    """Both GEMMs fp8 at the DeepSeek-V3 expert shape on the Zipf histogram; sampled rows."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    G, R = len(counts), sum(counts)
    announce("expert MLP fp8 full size")
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=17, device="cuda", l2="fp8")
    for k in ("W_gate", "W_up"):
        inp.pop(k)
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=0, N=2 * I)
    H = torch.empty((R, I), dtype=torch.float8_e4m3fn, device="cuda")
    Hs = torch.empty((R, I // 128), device="cuda")
    Y = torch.empty((R, N2), dtype=torch.bfloat16, device="cuda")
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, inp["A_scale"], inp["W1_scale"], H_scale=Hs)
    mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], b_layout=mg.B_NK)
    torch.cuda.synchronize()
    rows = P.sample_rows_contiguous(counts, 1, 256, extra=32, seed=18)
    got_y = P.rows_as_float(Y, rows)
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    del inp
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    q, s = check_fp8_h(H, Hs, h, rows)
    # L2 on the oracle's own codes for the sampled rows: a compact [rows, I] operand, one expert per row
    offs = acc.segment_offsets(counts, 1)
    ex = [next(e for e in range(G) if offs[e] <= r < offs[e] + counts[e]) for r in rows]
    w2 = cpu["W2"]
    y = np.empty((len(rows), N2))
    for e in sorted(set(ex)):
        idx = [i for i, x in enumerate(ex) if x == e]
        w2e = w2[e].float().double().numpy() * np.repeat(np.repeat(cpu["W2_scale"][e].double().numpy(), 128, 0),
                                                          128, 1).T
        y[idx] = (q[idx] * np.repeat(s[idx], 128, axis=1)) @ w2e.T
    P.check_gemm(got_y, y, "fp8", bound="chain_e4m3", what="mlp fp8 full size y")


def test_swiglu_leaves_other_rows_alone_and_handles_empty():
    counts = [0, 37, 0, 0]
    K, I, N2 = 128, 128, 256
    announce("expert MLP gaps", counts)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="bf16", seed=13, device="cuda")
    R = 64                                                   # rows past the segment stay untouched
    A = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
    A[:37] = inp["A"]
    H = P.sentinel_like((R, I))
    ws = mg.workspace(4, R)
    mg.schedule(inp["counts"], R, ws, block_m=64, N=2 * I)
    mg.grouped_gemm_swiglu_scheduled(A, inp["W1"], H, 4, ws, block_m=64)
    torch.cuda.synchronize()
    assert bool((H[37:].view(torch.int16) == P.SENTINEL_BITS).all())
    cpu = {k: P.cpu(v) for k, v in inp.items()}
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, list(range(37)))
    P.check_gemm(P.rows_as_float(H, range(37)), h, "bf16", what="mlp gaps h")
    ws0 = mg.workspace(4, R)
    mg.schedule(torch.zeros(4, dtype=torch.int32, device="cuda"), R, ws0, block_m=0, N=2 * I)
    H0 = P.sentinel_like((R, I))
    mg.grouped_gemm_swiglu_scheduled(A, inp["W1"], H0, 4, ws0, block_m=0)
    torch.cuda.synchronize()
    assert bool((H0.view(torch.int16) == P.SENTINEL_BITS).all())


def test_expert_mlp_full_size():
    """DeepSeek-V3-shaped experts on the Zipf histogram (64 experts, 32768 rows):
    K = 7168, I = 2048, N2 = 7168; fp8 L1 with fp32 scales, bf16 L2; sampled rows."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    announce("expert MLP full size", K, I, N2)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=14, device="cuda")
    H, Y, ws = run_mlp(counts, inp, 0, N2)
    P.check_stats(mg.stats_read(ws), counts)
    rows = P.sample_rows_contiguous(counts, 1, 256, extra=32, seed=15)
    got_h, got_y = P.rows_as_float(H, rows), P.rows_as_float(Y, rows)
    cpu = {k: P.cpu(v) for k, v in inp.items() if k not in ("W_gate", "W_up")}
    del inp
    h = omlp.swiglu_rows(cpu["A"], cpu["W1"], counts, rows, A_scale=cpu["A_scale"], W1_scale=cpu["W1_scale"])
    y = omlp.down_rows(h, cpu["W2"], counts, rows)
    P.check_gemm(got_h, h, "fp8", what="mlp full size h")
    P.check_gemm(got_y, y, "fp8", bound="chain", what="mlp full size y")


# ----------------------------------------------------------------- K-grouped


def run_k_grouped(t_sizes, Mw, Nw, seed=5, values="normal_unit", dtype="bf16", scales="fp32"):
    """scales "e8m0": power-of-two scales, passed to the library as exponent bytes
    (the oracle takes the same scales as fp32 values)."""
    w = wl.Workload("kg", "k_grouped", dtype, t_sizes, Mw=Mw, Nw=Nw, values=values, seed=seed, scales=scales)
    inp = wl.materialize(w, "cuda")
    dW = torch.full((w.G, Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(w.G, 0)
    e8 = scales == "e8m0"
    mg.grouped_gemm_k_grouped(inp["X"], inp["dY"], dW, inp["counts"], ws,
                              inp.get("X_scale_e8m0" if e8 else "X_scale"), inp.get("dY_scale_e8m0" if e8 else "dY_scale"))
    torch.cuda.synchronize()
    return w, inp, dW, ws


def k_grouped_ref(w, inp, pairs):
    """fp8 with either scale form: the oracle takes the fp32 scales (for E8M0 the
    powers of two the bytes encode)."""
    X, dY = P.cpu(inp["X"]), P.cpu(inp["dY"])
    if w.dtype == "fp8":
        return og.k_grouped_fp8(X, P.cpu(inp["X_scale"]), dY, P.cpu(inp["dY_scale"]), w.counts,
                                [e for e, _ in pairs], [i for _, i in pairs])
    return og.k_grouped(X, dY, w.counts, [e for e, _ in pairs], [i for _, i in pairs])


def check_k_grouped(w, inp, dW, pairs, ref=None):
    """dW rows against the oracle: fp32 output, so only the accumulation separates them
    (rel. Frobenius <= 1e-4 and the fp32 per-element bound; with e4m3 operands plus
    the term for the fp8 MFMA's group sums, S from the oracle on |X| and |dY|)."""
    ref = k_grouped_ref(w, inp, pairs) if ref is None else ref
    abs_sum = None
    if w.dtype == "fp8":
        mag = {k: (v.float().abs().to(torch.float8_e4m3fn) if k in ("X", "dY") else v) for k, v in inp.items()}
        abs_sum = k_grouped_ref(w, mag, pairs)
    got = dW[torch.tensor([e for e, _ in pairs]), torch.tensor([i for _, i in pairs])].cpu().double().numpy()
    return P.check_gemm(got, ref, "fp32", bound="fp32", what=f"k-grouped {w.dtype} G={w.G} Mw={w.Mw} Nw={w.Nw}",
                        abs_sum=abs_sum)


def k_rows_every_block(G, Mw, seed):
    """One dW row from every 16-row block of every 256-row i-tile of every expert."""
    rng = random.Random(seed)
    return [(e, b + rng.randrange(16)) for e in range(G) for b in range(0, Mw, 16)]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_k_grouped_small(dtype):
    t = [100, 0, 37, 200, 1, 129]
    announce("k-grouped small", dtype, t)
    w, inp, dW, ws = run_k_grouped(t, 512, 512, dtype=dtype)
    pairs = [(e, i) for e in range(w.G) for i in range(w.Mw)]
    check_k_grouped(w, inp, dW, pairs)
    assert not dW[1].any()                        # t_e = 0 -> zeros
    st = mg.stats_read(ws)
    assert st.U == sum(t) and st.active == 5 and st.sum_sq == sum(x * x for x in t) and st.error_flags == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_k_grouped_config_full_size(dtype):
    """The Dirichlet weight-gradient workload (16 experts, 65536 rows, dW [16, 2048,
    7168]): one dW row from every 16-row block of every i-tile of every expert,
    whole rows, so every 16 x 16 MFMA block of every tile is compared."""
    w0 = wl.workload(5)
    announce("k-grouped config 5", dtype, w0.counts)
    w, inp, dW, ws = run_k_grouped(w0.counts, w0.Mw, w0.Nw, dtype=dtype)
    pairs = k_rows_every_block(w.G, w.Mw, seed=5)
    check_k_grouped(w, inp, dW, pairs)
    for e, t in enumerate(w.counts):
        if t == 0:
            assert not dW[e].any()
    st = mg.stats_read(ws)
    assert st.U == sum(w.counts) and st.error_flags == 0


def k_grouped_matches_fp32_scales(inp, dW, ws):
    """Every element against the fp32-scale call on the same power-of-two scales.
    The two differ only in where each group's scaled partial sum is rounded (into
    the accumulator inside the MFMA, or on its own and then added), one rounding
    of the accumulator per group either way: at most 512 groups (65536 rows) of
    2^-24 each stay far below 2^-10 of the row's rms, which one wrong 16 x 16
    block or one lost group exceeds."""
    ref = torch.full_like(dW, float("nan"))
    mg.grouped_gemm_k_grouped(inp["X"], inp["dY"], ref, inp["counts"], ws, inp["X_scale"], inp["dY_scale"])
    torch.cuda.synchronize()
    rms = ref.double().pow(2).mean(dim=-1, keepdim=True).sqrt()
    diff = (dW.double() - ref.double()).abs()
    worst = float(torch.where(diff == 0, torch.zeros_like(diff), diff / (2.0 ** -10 * rms)).max())
    print(f"e8m0 call against the fp32-scale call: max |diff| / (2^-10 rms(row)) = {worst:.3e}", flush=True)
    assert bool(torch.isfinite(dW).all()) and worst <= 1.0


def test_k_grouped_e8m0_small():
    """E8M0 scale bytes, applied by the MFMA: ragged segments around the 128-row
    group, every dW row against the oracle, and every element against the
    fp32-scale call."""
    t = [100, 0, 37, 200, 1, 129, 256, 300]
    announce("k-grouped e8m0 small", t)
    w, inp, dW, ws = run_k_grouped(t, 512, 512, dtype="fp8", scales="e8m0", seed=28)
    assert bool((torch.exp2(inp["X_scale_e8m0"].float() - 127) == inp["X_scale"]).all())
    pairs = [(e, i) for e in range(w.G) for i in range(w.Mw)]
    check_k_grouped(w, inp, dW, pairs)
    assert not dW[1].any()
    st = mg.stats_read(ws)
    assert st.U == sum(t) and st.error_flags == 0
    k_grouped_matches_fp32_scales(inp, dW, ws)


def test_k_grouped_e8m0_full_size():
    """The Dirichlet weight-gradient workload with E8M0 scales: one dW row from
    every 16-row block of every i-tile of every expert against the oracle, and
    the whole dW against the fp32-scale call."""
    w0 = wl.workload(5)
    announce("k-grouped e8m0 config 5", w0.counts)
    w, inp, dW, ws = run_k_grouped(w0.counts, w0.Mw, w0.Nw, dtype="fp8", scales="e8m0")
    pairs = k_rows_every_block(w.G, w.Mw, seed=6)
    check_k_grouped(w, inp, dW, pairs)
    for e, t in enumerate(w.counts):
        if t == 0:
            assert not dW[e].any()
    assert mg.stats_read(ws).error_flags == 0
    k_grouped_matches_fp32_scales(inp, dW, ws)


def test_k_grouped_e8m0_integer_exact_and_deterministic():
    """e4m3 codes in {-1, 0, 1} with scale bytes 124..130 (2^-3..2^3) per group
    and column: every partial sum is exact in fp32, so GPU == oracle bit for bit,
    and two runs agree.  Segments straddle the 128-row group."""
    t = [1, 127, 128, 129, 255, 0, 300]
    T, Mw, Nw = sum(t), 256, 512
    announce("k-grouped e8m0 integer exact", t)
    g = torch.Generator().manual_seed(11)
    X = torch.randint(-1, 2, (T, Mw), generator=g).float().to(torch.float8_e4m3fn)
    dY = torch.randint(-1, 2, (T, Nw), generator=g).float().to(torch.float8_e4m3fn)
    S = mg.k_scale_groups(t)
    bx = torch.randint(124, 131, (S, Mw), generator=g).to(torch.uint8)
    by = torch.randint(124, 131, (S, Nw), generator=g).to(torch.uint8)
    outs = []
    ws = mg.workspace(len(t), 0)
    for _ in range(2):
        dW = torch.full((len(t), Mw, Nw), float("nan"), device="cuda")
        mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws,
                                  bx.cuda(), by.cuda())
        torch.cuda.synchronize()
        outs.append(dW.cpu())
    assert torch.equal(outs[0], outs[1])
    pairs = [(e, i) for e in range(len(t)) for i in range(Mw)]
    sx, sy = torch.exp2(bx.float() - 127), torch.exp2(by.float() - 127)
    ref = og.k_grouped_fp8(X, sx, dY, sy, t, [e for e, _ in pairs], [i for _, i in pairs])
    assert np.array_equal(outs[0].double().numpy().reshape(len(t) * Mw, Nw), ref)
    assert mg.stats_read(ws).error_flags == 0


def test_k_grouped_e8m0_too_few_scale_groups_is_flagged():
    """E8M0 scale arrays short of the histogram's groups: the flag is set and the
    missing groups' bytes read as 0 (2^-127), which flushes their products to 0."""
    t = [200, 100]
    announce("k-grouped e8m0 scale groups flag", t)
    Mw = Nw = 256
    g = torch.Generator().manual_seed(13)
    X, sx = wl.quantize_k_groups_e4m3(torch.randn(300, Mw, generator=g), t, pow2=True)
    dY, sy = wl.quantize_k_groups_e4m3(torch.randn(300, Nw, generator=g), t, pow2=True)
    bx, by = wl.e8m0_bytes(sx), wl.e8m0_bytes(sy)
    dW = torch.full((2, Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(2, 0)
    mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws,
                              bx[:2].contiguous().cuda(), by[:2].contiguous().cuda())
    torch.cuda.synchronize()
    assert mg.stats_read(ws).error_flags & mg.FLAG_SCALE_GROUPS
    pairs = [(0, i) for i in range(0, Mw, 5)]
    ref = og.k_grouped_fp8(X, sx, dY, sy, t, [e for e, _ in pairs], [i for _, i in pairs])
    P.check_gemm(dW[0, 0:Mw:5].cpu().double().numpy(), ref, "fp32", bound="fp32", what="k-grouped e8m0 complete")
    assert not dW[1].any()


def test_k_grouped_integer_exact_and_ragged():
    """Inputs in {-1, 0, 1}: every dW entry is an integer of magnitude <= t_e,
    exact in fp32, so GPU == oracle bit for bit.  Segment lengths straddle the
    64-row reduction step (1, 63, 64, 65, 127, 0)."""
    t = [1, 63, 64, 65, 127, 0]
    T, Mw, Nw = sum(t), 256, 512
    announce("k-grouped integer exact", t)
    g = torch.Generator().manual_seed(9)
    X = torch.randint(-1, 2, (T, Mw), generator=g).to(torch.bfloat16)
    dY = torch.randint(-1, 2, (T, Nw), generator=g).to(torch.bfloat16)
    dW = torch.full((len(t), Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(len(t), 0)
    mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws)
    torch.cuda.synchronize()
    pairs = [(e, i) for e in range(len(t)) for i in range(Mw)]
    ref = og.k_grouped(X, dY, t, [e for e, _ in pairs], [i for _, i in pairs])
    got = dW.cpu().double().numpy().reshape(len(t) * Mw, Nw)
    assert np.array_equal(got, ref)


def test_k_grouped_fp8_integer_exact():
    """e4m3 codes in {-1, 0, 1} with power-of-two scales 2^-3..2^3 per group and
    column: every product and every partial sum is a multiple of 2^-6 well
    inside fp32's exact range, so GPU == oracle bit for bit.  Segment lengths
    straddle the 128-row scale group (1, 127, 128, 129, 255, 0, 300): a group
    index off by one anywhere changes the result."""
    t = [1, 127, 128, 129, 255, 0, 300]
    T, Mw, Nw = sum(t), 256, 512
    announce("k-grouped fp8 integer exact", t)
    g = torch.Generator().manual_seed(10)
    X = torch.randint(-1, 2, (T, Mw), generator=g).float().to(torch.float8_e4m3fn)
    dY = torch.randint(-1, 2, (T, Nw), generator=g).float().to(torch.float8_e4m3fn)
    S = mg.k_scale_groups(t)
    sx = torch.exp2(torch.randint(-3, 4, (S, Mw), generator=g).float())
    sy = torch.exp2(torch.randint(-3, 4, (S, Nw), generator=g).float())
    dW = torch.full((len(t), Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(len(t), 0)
    mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws,
                              sx.cuda(), sy.cuda())
    torch.cuda.synchronize()
    pairs = [(e, i) for e in range(len(t)) for i in range(Mw)]
    ref = og.k_grouped_fp8(X, sx, dY, sy, t, [e for e, _ in pairs], [i for _, i in pairs])
    got = dW.cpu().double().numpy().reshape(len(t) * Mw, Nw)
    assert np.array_equal(got, ref)
    assert mg.stats_read(ws).error_flags == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_k_grouped_empty_truncated_and_deterministic(dtype):
    """All experts empty -> dW all zero; counts past T are truncated (flag set);
    two runs give identical bits."""
    announce("k-grouped empty / truncated / deterministic", dtype)
    Mw, Nw = 256, 256
    d = torch.float8_e4m3fn if dtype == "fp8" else torch.bfloat16
    scales = lambda S: (torch.ones(S, Mw, device="cuda"), torch.ones(S, Nw, device="cuda")) \
        if dtype == "fp8" else (None, None)
    X = torch.zeros(0, Mw).to(d).cuda()
    dY = torch.zeros(0, Nw).to(d).cuda()
    dW = torch.full((3, Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(3, 0)
    mg.grouped_gemm_k_grouped(X, dY, dW, torch.zeros(3, dtype=torch.int32, device="cuda"), ws, *scales(1))
    torch.cuda.synchronize()
    assert not dW.any()
    assert mg.stats_read(ws).U == 0
    # counts summing past T: the last segment is cut at T
    t, T = [50, 80, 40], 100
    clamped = [50, 50, 0]                                   # the reading the device takes
    g = torch.Generator().manual_seed(4)
    x, dy = torch.randn(T, Mw, generator=g), torch.randn(T, Nw, generator=g)
    if dtype == "fp8":
        X, sx = wl.quantize_k_groups_e4m3(x, clamped)
        dY, sy = wl.quantize_k_groups_e4m3(dy, clamped)
        sc = (sx.cuda(), sy.cuda())
    else:
        X, dY, sc = x.to(torch.bfloat16), dy.to(torch.bfloat16), (None, None)
    outs = []
    for _ in range(2):
        dW = torch.full((3, Mw, Nw), float("nan"), device="cuda")
        mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws,
                                  *sc)
        torch.cuda.synchronize()
        outs.append(dW.cpu())
    st = mg.stats_read(ws)
    assert st.error_flags & mg.FLAG_ROWS_OVERFLOW and st.U == T
    assert torch.equal(outs[0], outs[1])
    pairs = [(e, i) for e in range(2) for i in range(0, Mw, 7)]
    if dtype == "fp8":
        ref = og.k_grouped_fp8(X, sx, dY, sy, clamped, [e for e, _ in pairs], [i for _, i in pairs])
    else:
        ref = og.k_grouped(X, dY, clamped, [e for e, _ in pairs], [i for _, i in pairs])
    got = outs[0][torch.tensor([e for e, _ in pairs]), torch.tensor([i for _, i in pairs])].double().numpy()
    P.check_gemm(got, ref, "fp32", bound="fp32", what=f"k-grouped truncated {dtype}")
    assert not outs[0][2].any()                             # the segment that starts at T is empty


def test_k_grouped_fp8_too_few_scale_groups_is_flagged():
    """Scale arrays with fewer rows than the histogram's groups: the call runs, the
    missing groups read as zero scales, and MOEGG_FLAG_SCALE_GROUPS is set."""
    t = [200, 100]                                          # 2 + 1 = 3 groups
    announce("k-grouped fp8 scale groups flag", t)
    Mw = Nw = 256
    g = torch.Generator().manual_seed(12)
    X, sx = wl.quantize_k_groups_e4m3(torch.randn(300, Mw, generator=g), t)
    dY, sy = wl.quantize_k_groups_e4m3(torch.randn(300, Nw, generator=g), t)
    dW = torch.full((2, Mw, Nw), float("nan"), device="cuda")
    ws = mg.workspace(2, 0)
    mg.grouped_gemm_k_grouped(X.cuda(), dY.cuda(), dW, torch.tensor(t, dtype=torch.int32, device="cuda"), ws,
                              sx[:2].contiguous().cuda(), sy[:2].contiguous().cuda())
    torch.cuda.synchronize()
    assert mg.stats_read(ws).error_flags & mg.FLAG_SCALE_GROUPS
    assert bool(torch.isfinite(dW).all())
    # expert 0 (groups 0 and 1) is complete; expert 1's group 2 is missing and reads as 0
    pairs = [(0, i) for i in range(0, Mw, 5)]
    ref = og.k_grouped_fp8(X, sx, dY, sy, t, [e for e, _ in pairs], [i for _, i in pairs])
    got = dW[0, 0:Mw:5].cpu().double().numpy()
    P.check_gemm(got, ref, "fp32", bound="fp32", what="k-grouped fp8 complete expert")
    assert not dW[1].any()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_k_grouped_maximum_expert_count(dtype):
    """G = 4096 experts with tiny ragged segments (a third empty): the expert
    order comes from the scheduler's sort; every expert's dW, zeros included."""
    rng = random.Random(43)
    t = [0 if rng.random() < 0.33 else rng.randint(1, 3) for _ in range(4096)]
    announce("k-grouped G=4096", dtype, sum(t))
    w, inp, dW, ws = run_k_grouped(t, 256, 256, seed=43, dtype=dtype)
    rows = [(e, i) for e in range(w.G) for i in range(0, w.Mw, 37)]
    check_k_grouped(w, inp, dW, rows)
    empty = torch.tensor([e for e, x in enumerate(t) if x == 0], device="cuda")
    assert not dW[empty].any()
    st = mg.stats_read(ws)
    assert st.U == sum(t) and st.active == sum(1 for x in t if x) and st.error_flags == 0


# ----------------------------------------------------------------- weights in column panels


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("b_layout", [mg.B_KN_PANEL, mg.B_NK_PANEL])
@pytest.mark.parametrize("block_m", [0, 64, 128, 256, mg.BLOCK_M_PER_EXPERT])
def test_contiguous_panel_layouts(dtype, b_layout, block_m):
    """The same weights repacked in 256-column panels: every valid row against the
    oracle (which reads them as [G, K, N]); rows outside segments untouched."""
    counts = [300, 0, 17, 513, 64, 1]
    announce("contiguous panels", dtype, b_layout, block_m, counts)
    w, inp = small_contig(counts, 512, 768, dtype)
    B = mg.pack_panels(inp["B"], b_layout, mg.PANEL_CONTIGUOUS)
    C = P.sentinel_like((w.rows_total, w.N))
    ws = mg.workspace(w.G, w.rows_total)
    mg.grouped_gemm_contiguous(inp["A"], B, C, inp["counts"], ws, A_scale=inp.get("A_scale"),
                               B_scale=inp.get("B_scale"), block_m=block_m, b_layout=b_layout)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), counts)
    rows = list(range(w.rows_total))
    ref = P.oracle_contiguous_rows(w, {k: P.cpu(v) for k, v in inp.items()}, rows)
    valid = ~np.isnan(ref[:, 0])
    P.check_gemm(P.rows_as_float(C, rows)[valid], ref[valid], dtype, what=f"panels {dtype} {b_layout} {block_m}")
    assert P.untouched_rows_ok(C, counts, 1)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("b_layout", [mg.B_KN_PANEL, mg.B_NK_PANEL])
def test_masked_panel_layouts(dtype, b_layout):
    """128-column panels in the masked layout, with experts of one row tile (weights
    streamed) and of several (64, 65, 130 rows)."""
    counts = [3, 0, 64, 65, 130, 1]
    announce("masked panels", dtype, b_layout, counts)
    w, inp = masked_case(counts, 160, 512, 256, dtype)
    B = mg.pack_panels(inp["B"], b_layout, mg.PANEL_MASKED)
    C = P.sentinel_like((w.G, w.cap, w.N))
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], None, inp.get("A_scale"), inp.get("B_scale"), b_layout)
    torch.cuda.synchronize()
    check_masked(w, inp, C, counts)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_masked_panel_full_size(dtype):
    """The decode workload (32 experts, cap 256, K 2048, N 7168) with weights in
    128-column panels, as the benchmark runs it: every valid row."""
    w0 = wl.workload(4)
    announce("masked panels full size", dtype)
    w = wl.Workload("masked " + dtype, "masked", dtype, w0.counts, K=w0.K, N=w0.N, cap=w0.cap, seed=w0.seed)
    inp = wl.materialize(w, "cuda")
    B = mg.pack_panels(inp["B"], mg.B_KN_PANEL, mg.PANEL_MASKED)
    C = P.sentinel_like((w.G, w.cap, w.N))
    ws = mg.workspace(w.G, w.G * w.cap)
    mg.grouped_gemm_masked(inp["A"], B, C, inp["counts"], ws, inp.get("A_scale"), inp.get("B_scale"),
                           mg.B_KN_PANEL)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), w.counts)
    check_masked(w, inp, C, w.counts)


def test_contiguous_panel_full_size():
    """The Zipf fp8 workload with weights in K-step panels, device-chosen height:
    one row from every 16-row block of every expert segment."""
    w = wl.workload(3)
    announce("contiguous nk panels full size", w.name)
    inp = wl.materialize(w, "cuda")
    B = mg.pack_panels(inp["B"], mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
    C = P.sentinel_like((w.rows_total, w.N))
    ws = mg.workspace(w.G, w.rows_total)
    mg.grouped_gemm_contiguous(inp["A"], B, C, inp["counts"], ws, A_scale=inp["A_scale"], B_scale=inp["B_scale"],
                               b_layout=mg.B_NK_PANEL)
    torch.cuda.synchronize()
    P.check_stats(mg.stats_read(ws), w.counts)
    rows = full_size_rows(w)
    ref = full_size_ref(w, inp, rows)
    del inp
    P.check_gemm(P.rows_as_float(C, rows), ref, "fp8", what="nk panels full size")
    assert P.untouched_rows_ok(C, w.counts, w.seg_align)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_swiglu_panel_layout(dtype):
    """L1 with the SwiGLU epilogue reading W1 in K-step panels, bit for bit the
    [G, 2I, K] result."""
    counts = [70, 0, 300, 6, 129, 3]
    K, I, N2 = 256, 256, 512
    G, R = len(counts), sum(counts)
    announce("swiglu panels", dtype, counts)
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype=dtype, seed=12, device="cuda")
    ws = mg.workspace(G, R)
    mg.schedule(inp["counts"], R, ws, block_m=0, N=2 * I)
    H0, H1 = P.sentinel_like((R, I)), P.sentinel_like((R, I))
    mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H0, G, ws, inp["A_scale"], inp["W1_scale"])
    W1p = mg.pack_panels(inp["W1"].transpose(1, 2).contiguous(), mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
    mg.grouped_gemm_swiglu_scheduled(inp["A"], W1p, H1, G, ws, inp["A_scale"], inp["W1_scale"],
                                     b_layout=mg.B_NK_PANEL)
    torch.cuda.synchronize()
    assert torch.equal(H0.view(torch.int16), H1.view(torch.int16))
