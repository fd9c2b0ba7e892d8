"""Benchmark: the MoE grouped GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input
already resident in HBM:
    device scheduler (counts -> accounting, tile height, tile list)
    + the fp8 contiguous grouped GEMM with per-128 fp32 scale promotion.

Default workload: 64 local experts, 32768 routed rows on a seeded Zipf(1.2)
histogram with some experts empty, K = 7168, N = 4096, e4m3 operands with
fp32 scales per 1x128 activation group and per 128x128 weight block, bf16
output, contiguous layout.

Metric: effective TFLOPS = 2 * U * K * N / step time (valid rows only), and its
fraction of the MI355X dense fp8 MFMA peak.  Physical TFLOPS counts the rows
the MFMAs actually executed (P_exec).

Prints ONE JSON line on stdout.  `--config n` times another problem (1..5) for
reporting; the JSON `config.workload` names it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_grouped_gemm_sizes_amd as mg  # noqa: E402
import workloads as wl  # noqa: E402

PEAK = {"fp8": 5000.0, "bf16": 2500.0}      # dense MFMA TFLOP/s, MI355X
HBM_PEAK = 8000.0                           # GB/s
METRIC = "effective TFLOPS (valid rows) + % of MFMA peak, V3-shaped fp8 grouped GEMM"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_step(w: wl.Workload, inp, block_m_hint: int, b_layout: int, sched_block_m: int = 0, exemplars=None,
               hysteresis: int = 0, scale_km: bool = False):
    """Returns (scheduler, gemm, workspace) closures for one workload.  With an
    exemplar table the scheduler picks the tile height by exemplar matching."""
    dev = "cuda"
    if w.layout == "contiguous":
        C = torch.empty((w.rows_total, w.N), dtype=torch.bfloat16, device=dev)
        ws = mg.workspace(w.G, w.rows_total)

        def sched():
            if exemplars is not None:
                mg.schedule_exemplar(inp["counts"], w.rows_total, ws, exemplars, hysteresis=hysteresis,
                                     seg_align=w.seg_align, N=w.N)
            else:
                mg.schedule(inp["counts"], w.rows_total, ws, seg_align=w.seg_align, block_m=sched_block_m, N=w.N)

        def gemm():
            mg.grouped_gemm_contiguous_scheduled(inp["A"], inp["B"], C, w.G, ws, inp.get("A_scale"),
                                                 inp.get("B_scale"), block_m=block_m_hint, b_layout=b_layout,
                                                 scale_km=scale_km)
        return sched, gemm, ws
    if w.layout == "masked":
        C = torch.empty((w.G, w.cap, w.N), dtype=torch.bfloat16, device=dev)
        ws = mg.workspace(w.G, w.G * w.cap)

        def gemm():
            mg.grouped_gemm_masked(inp["A"], inp["B"], C, inp["counts"], None, inp.get("A_scale"),
                                   inp.get("B_scale"), b_layout=b_layout, scale_km=scale_km)
        return None, gemm, ws
    dW = torch.empty((w.G, w.Mw, w.Nw), dtype=torch.float32, device=dev)
    ws = mg.workspace(w.G, 0)

    e8 = w.scales == "e8m0"

    def gemm():
        mg.grouped_gemm_k_grouped(inp["X"], inp["dY"], dW, inp["counts"], ws,
                                  inp.get("X_scale_e8m0" if e8 else "X_scale"),
                                  inp.get("dY_scale_e8m0" if e8 else "dY_scale"))
    return None, gemm, ws


def algorithmic_bytes(w: wl.Workload) -> int:
    """Bytes the method must move once: active experts' weights, valid rows in and out (plus scales)."""
    active = sum(1 for c in w.counts if c > 0)
    U = sum(w.counts)
    if w.layout == "k_grouped":
        if w.dtype == "fp8":
            groups = mg.k_scale_groups(w.counts)
            ssz = 1 if w.scales == "e8m0" else 4
            return U * (w.Mw + w.Nw) + groups * (w.Mw + w.Nw) * ssz + w.G * w.Mw * w.Nw * 4
        return U * (w.Mw + w.Nw) * 2 + w.G * w.Mw * w.Nw * 4
    esz = 1 if w.dtype == "fp8" else 2
    w_bytes = w.K * w.N // 2 if w.weights == "e2m1" else w.K * w.N * esz
    b = active * w_bytes + U * w.K * esz + U * w.N * 2
    if w.dtype == "fp8":
        ssz = 1 if w.scales == "e8m0" else 4
        b += U * (w.K // 128) * ssz + active * (w.K // 128) * (w.N // 128) * ssz
    return b


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "device.hpp", "tile_order.hpp"):
        with open(os.path.join(ROOT, "moe_grouped_gemm_sizes_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_key(w: wl.Workload, b_layout: int, scale_km: bool = True) -> str:
    """The entry of profiles/traffic.json that holds this workload's counters."""
    layout = {mg.B_KN: "kn", mg.B_NK: "nk", mg.B_KN_PANEL: "kn-panel", mg.B_NK_PANEL: "nk-panel"}[b_layout]
    return f"{w.name}|{layout}" + ("|e8m0" if w.scales == "e8m0" else "") + \
        ("|e2m1" if w.weights == "e2m1" else "") + \
        ("|rows" if w.dtype == "fp8" and w.scales != "e8m0" and not scale_km else "")


def traffic_for(w: wl.Workload, b_layout: int, scale_km: bool = True):
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on this exact kernel source and workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get("entries", {}).get(traffic_key(w, b_layout, scale_km))
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e["hbm_bytes_per_launch"]


def cpu_baseline(w: wl.Workload, inp, target_s: float = 15.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of rows."""
    from oracle import gemm as og
    from tests.parity import sample_rows_contiguous
    og.lib()
    if w.layout != "contiguous":
        return None
    cpu = {k: (v.cpu().contiguous() if v is not None else None) for k, v in inp.items()}
    if w.weights == "e2m1":
        from oracle import fp4

        def run(rows):
            fp4.contiguous_fp8_fp4(cpu["A"], cpu["A_scale"], cpu["B"], cpu["B_scale"], w.counts, rows,
                                   seg_align=w.seg_align)
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    else:
        def run(rows):
            og.contiguous(cpu["A"], cpu["B"], w.counts, rows, seg_align=w.seg_align,
                          A_scale=cpu.get("A_scale"), B_scale=cpu.get("B_scale"))
        threads = og.threads()
    rows = sample_rows_contiguous(w.counts, w.seg_align, 256, extra=4096, seed=99)
    probe = rows[:threads]
    t0 = time.perf_counter()
    run(probe)
    dt = time.perf_counter() - t0
    n = max(threads, min(len(rows), int(target_s / max(dt, 1e-6) * len(probe)) // threads * threads))
    sample = rows[:n]
    t0 = time.perf_counter()
    run(sample)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(sample) * w.K * w.N
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{len(sample)} output rows x {w.N} columns of this workload (fp64 oracle, {dt:.1f} s)"}


def settle(fn, ms: float = 100.0):
    """Call fn() back to back until about `ms` of GPU time has passed: in a fresh process, or after the GPU
    has idled, the first tens of milliseconds of work run below the steady state."""
    t = 0.0
    while t < ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        t += a.elapsed_time(b)


def time_candidates(w: wl.Workload, inp, b_layout: int, scale_km: bool, args):
    """Every candidate tile height of the contiguous GEMM timed on its own (the padding page,
    "Build a routing-shaped benchmark": P, padding fraction, tiles, latency, effective and physical
    throughput per candidate), outside the headline's timed steps, same cache mode."""
    rows = []
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.cold else None
    for bm in (64, 128, 256, mg.BLOCK_M_PER_EXPERT):
        sched, gemm, ws = build_step(w, inp, bm, b_layout, bm, None, 0, scale_km=scale_km)
        settle(lambda: (sched(), gemm()), 20.0)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for i, (a, b) in enumerate(ev):
            if scratch is not None:
                scratch.fill_(i & 255)
            sched()
            a.record()
            gemm()
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
        st = mg.stats_read(ws)
        rep = st.report()
        q = 256 if bm == mg.BLOCK_M_PER_EXPERT else bm
        rows.append({"block_m": "per-expert" if bm == mg.BLOCK_M_PER_EXPERT else bm, "tiles": st.tiles,
                     "P_at_block_m": st.P_at[q], "padding_fraction_at_block_m": round(rep.padding_fraction[q], 6),
                     "P_exec": st.P_exec, "active_experts": st.active,
                     "effective_experts": round(rep.effective_experts, 4), "gemm_ms_median": round(ms, 4),
                     "effective_tflops": round(w.useful_flops() / (ms * 1e-3) / 1e12, 2),
                     "physical_tflops": round(2.0 * st.P_exec * w.K * w.N / (ms * 1e-3) / 1e12, 2)})
        del ws
    return rows


def sample_sclk(step, seconds: float = 0.4):
    """The shader clock under this workload: the current DPM level of the GPU's
    sclk (sysfs pp_dpm_sclk), sampled from a thread while about `seconds` of
    steps run back to back after the timed region."""
    import glob
    import re
    import threading
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))

    def read():
        for pth in paths:
            try:
                with open(pth) as f:
                    for line in f:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                return int(m.group(1))
            except OSError:
                pass
        return None
    if not paths or read() is None:
        return {"mhz_median": None, "source": "pp_dpm_sclk not readable on this host"}
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-4)
    samples, done = [], threading.Event()

    def sampler():
        while not done.is_set():
            v = read()
            if v is not None:
                samples.append(v)
            time.sleep(0.002)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    for _ in range(int(seconds / per) + 1):
        step()
    torch.cuda.synchronize()
    done.set()
    th.join()
    samples.sort()
    return {"mhz_median": samples[len(samples) // 2] if samples else None,
            "mhz_min": samples[0] if samples else None, "mhz_max": samples[-1] if samples else None,
            "samples": len(samples), "source": "pp_dpm_sclk current level while steps run back to back"}


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "cpu_affinity": len(os.sched_getaffinity(0))}


def run_mlp(args):
    """Expert MLP on the Zipf histogram (64 experts, 32768 rows), DeepSeek-V3 expert shape: K 7168, I 2048,
    N2 7168.  One step: scheduler, L1 (fp8 e4m3, fp32 scales) with the fused SwiGLU epilogue writing H, L2 on H
    from the same schedule.  --mlp-h fp8 (default): H e4m3 with 1x128 scales quantized in the epilogue and an
    fp8 L2; bf16: H bf16 and a bf16 L2.  Cold caches between steps."""
    counts = wl.workload(3).counts
    K, I, N2 = 7168, 2048, 7168
    G, R = len(counts), sum(counts)
    fp8_h = args.mlp_h == "fp8"
    w4 = args.weights == "e2m1"               # fp4 gate/up weights, E8M0 scales (L1)
    log(f"expert MLP: G={G}, U={R}, K={K}, I={I}, N2={N2}, H {args.mlp_h}, L1 weights {args.weights}")
    inp = wl.materialize_mlp(counts, K=K, I=I, N2=N2, dtype="fp8", seed=14, device="cuda",
                             l2="fp8" if fp8_h else "bf16", w1_format="e2m1" if w4 else "e4m3")
    a_s, w1_s = (inp["A_scale_e8m0"], inp["W1_scale_e8m0"]) if w4 else (inp["A_scale"], inp["W1_scale"])
    # fp32 scales go over transposed, [K/128, rows]: L1's input and the H scales it writes for L2 (an
    # fp4-weight L1 takes E8M0 activation scales and writes H scales [rows, I/128])
    km_l1 = not w4 and args.a_scale == "km"
    km_l2 = fp8_h and km_l1
    if km_l1:
        a_s = a_s.t().contiguous()
    for k in ("W_gate", "W_up"):
        inp.pop(k)
    torch.cuda.empty_cache()
    ws = mg.workspace(G, R)
    H = torch.empty((R, I), dtype=torch.float8_e4m3fn if fp8_h else torch.bfloat16, device="cuda")
    Hs = (torch.empty((I // 128, R) if km_l2 else (R, I // 128), device="cuda")) if fp8_h else None
    Y = torch.empty((R, N2), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    # both GEMMs run whatever height the scheduler chose on the device (block_m = 0, one launch each)
    def sched():
        mg.schedule(inp["counts"], R, ws, block_m=0, N=2 * I)

    w1_layout = mg.B_NK
    if w4 and not args.mlp_fused:
        # fp4 gate/up weights repacked once into 256-row panels: whole lines per K step
        inp["W1"] = mg.pack_panels(inp["W1"], mg.B_NK_PANEL, mg.PANEL_CONTIGUOUS)
        w1_layout = mg.B_NK_PANEL

    def l1():
        mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, a_s, w1_s, block_m=0, H_scale=Hs,
                                         scale_km=km_l1, b_layout=w1_layout)

    def l2():
        mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], block_m=0,
                                             b_layout=mg.B_NK, scale_km=km_l2)
    if args.mlp_fused:
        return run_mlp_fused(args, inp, counts, K, I, N2, a_s, w1_s, km_l1, ws, H, Hs, Y)
    for _ in range(args.warmup):
        sched(); l1(); l2()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        scratch.fill_(i & 255)
        ev[i][0].record(stream)
        sched()
        ev[i][1].record(stream)
        l1()
        ev[i][2].record(stream)
        l2()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = sum(e[0].elapsed_time(e[3]) for e in ev) / args.steps
    l1_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    l2_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    f1, f2 = 2.0 * R * K * 2 * I, 2.0 * R * I * N2
    st = mg.stats_read(ws)
    out = {
        "metric": "effective TFLOPS (valid rows), expert MLP L1 -> SwiGLU -> L2",
        "value": round((f1 + f2) / (ms * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3" if fp8_h else "fp8_e4m3 (L1) + bf16 (L2)", "data": "synthetic",
        "config": {"workload": "zipf 64 experts expert MLP (L1 fp8%s + SwiGLU, L2 %s)" % (
                       " x fp4" if w4 else "", "fp8" if fp8_h else "bf16"),
                   "experts": G,
                   "routed_rows": R, "K": K, "I": I, "N2": N2, "layout": "contiguous", "seed": 3,
                   "weights": "W1 [G,2I,K] gate/up interleaved, W2 [G,N2,I]",
                   "cache": "cold (512 MiB written between steps)"},
        "block_m": "per-expert" if st.block_m == mg.BLOCK_M_PER_EXPERT else st.block_m,
        "l1_swiglu_ms": round(l1_ms, 4), "l2_ms": round(l2_ms, 4),
        "l1_tflops": round(f1 / (l1_ms * 1e-3) / 1e12, 2), "l2_tflops": round(f2 / (l2_ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(f1 / (l1_ms * 1e-3) / 1e12, 2), "peak": PEAK["fp8"],
                     "unit": "TFLOP/s", "frac": round(f1 / (l1_ms * 1e-3) / 1e12 / PEAK["fp8"], 4),
                     "traffic": None, "kernel": "L1 with the SwiGLU epilogue"},
        "l2_roofline_frac": round(f2 / (l2_ms * 1e-3) / 1e12 / PEAK["fp8" if fp8_h else "bf16"], 4),
        "wall_s_timed": round(wall, 4), "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def calib_copy(args):
    """With --calib-copy-mib n: one plain elementwise kernel over n MiB of fp32 after the timed steps (reads n MiB,
    writes n MiB), so a counter run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) can scale HBM counters by a transfer of
    known size."""
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 18                         # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst


def run_mlp_fused(args, inp, counts, K, I, N2, a_s, w1_s, km, ws, H, Hs, Y):
    """The expert MLP in one launch (moegg_expert_mlp_fused: the scheduler, which also clears the completion
    counters, then one kernel with both GEMMs), and beside it the same work as three launches from the same 256-row schedule, each timed
    cold over the same steps."""
    G, R = len(counts), sum(counts)
    stream = torch.cuda.current_stream()

    def fused():
        mg.expert_mlp_fused(inp["A"], inp["W1"], inp["W2"], H, Y, inp["counts"], ws, a_s, w1_s, inp["W2_scale"],
                            Hs, scale_km=km)

    def chain():
        mg.schedule(inp["counts"], R, ws, block_m=256, N=2 * I)
        mg.grouped_gemm_swiglu_scheduled(inp["A"], inp["W1"], H, G, ws, a_s, w1_s, block_m=256, H_scale=Hs,
                                         scale_km=km)
        mg.grouped_gemm_contiguous_scheduled(H, inp["W2"], Y, G, ws, Hs, inp["W2_scale"], block_m=256,
                                             b_layout=mg.B_NK, scale_km=km)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            scratch.fill_(i & 255)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / args.steps
    t_wall = time.perf_counter()
    ms = timed(fused)
    wall = time.perf_counter() - t_wall
    st = mg.stats_read(ws)
    if st.error_flags:
        raise RuntimeError(f"fused expert MLP: error flags {st.error_flags:#x}")
    chain_ms = timed(chain)
    calib_copy(args)
    f1, f2 = 2.0 * R * K * 2 * I, 2.0 * R * I * N2
    tf = (f1 + f2) / (ms * 1e-3) / 1e12
    out = {
        "metric": "effective TFLOPS (valid rows), expert MLP L1 -> SwiGLU -> L2 in one launch",
        "value": round(tf, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "zipf 64 experts expert MLP (L1 fp8 + SwiGLU, e4m3 H, L2 fp8), one launch",
                   "experts": G, "routed_rows": R, "K": K, "I": I, "N2": N2, "layout": "contiguous", "seed": 3,
                   "weights": "W1 [G,2I,K] gate/up interleaved, W2 [G,N2,I]",
                   "scales": "[K/128, rows]" if km else "[rows, K/128]",
                   "cache": "cold (512 MiB written between steps)"},
        "block_m": 256,
        "three_launch_ms_block_m_256": round(chain_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK["fp8"], "unit": "TFLOP/s",
                     "frac": round(tf / PEAK["fp8"], 4), "traffic": None,
                     "kernel": "fused expert MLP (both GEMMs; scheduler included)"},
        "wall_s_timed": round(wall, 4), "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def run_decode_buckets(args):
    """Low-token buckets (the padding page, "Build a routing-shaped benchmark", asks for them beside the large
    histograms).  Contiguous: the Zipf fp8 shape (64 experts, K 7168, N 4096, fp32 scales [K/128, rows]) at U =
    32 ... 1024 routed rows, every tile height timed on its own and the device's own choice (block_m = 0).
    Masked: the decode shape (32 experts, cap 256, K 2048, N 7168, bf16 and fp8 with fp32 scales, weights in
    128-column panels) at Poisson means 1 ... 128.  Cold caches between calls; one JSON line per bucket; these are memory-bound, so the
    rate is algorithmic bytes per second against HBM."""
    args.cold = True
    for U in (32, 64, 128, 256, 512, 1024):
        counts = wl.hist_zipf(3, experts=64, total=U)
        w = wl.Workload(f"zipf 64 experts fp8 contiguous, {U} rows", "contiguous", "fp8", counts, K=7168, N=4096,
                        values="normal", seed=3)
        inp = wl.materialize(w, "cuda")
        inp["B"] = inp["B"].transpose(1, 2).contiguous()
        a_s = inp["A_scale"]
        inp = dict(inp, A_scale=a_s.t().contiguous())
        sched, gemm, ws = build_step(w, inp, 0, mg.B_NK, 0, None, 0, scale_km=True)
        settle(lambda: (sched(), gemm()))
        cands = time_candidates(w, inp, mg.B_NK, True, args)
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        settle(lambda: (sched(), gemm()), 20.0)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i, (a, b) in enumerate(ev):
            scratch.fill_(i & 255)
            sched()
            a.record()
            gemm()
            b.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        st = mg.stats_read(ws)
        nb = algorithmic_bytes(w)
        best = min(cands, key=lambda c: c["gemm_ms_median"])
        print(json.dumps({"bucket": "contiguous", "U": U, "active_experts": st.active,
                          "effective_experts": round(st.report().effective_experts, 3),
                          "device_choice": "per-expert" if st.block_m == mg.BLOCK_M_PER_EXPERT else st.block_m,
                          "device_choice_ms": round(ms, 4), "fastest": best["block_m"],
                          "fastest_ms": best["gemm_ms_median"], "algorithmic_bytes": nb,
                          "gbs": round(nb / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK, 4),
                          "candidates": {str(c["block_m"]): c["gemm_ms_median"] for c in cands}}), flush=True)
        del inp, ws, scratch
        torch.cuda.empty_cache()
    for dtype, mean in [(d, m) for d in ("bf16", "fp8") for m in (1, 2, 4, 8, 16, 32, 64, 128)]:
        counts = wl.hist_poisson_masked(4, experts=32, cap=256, mean=float(mean))
        w = wl.Workload(f"masked decode 32 experts {dtype}, mean {mean}", "masked", dtype, counts, K=2048, N=7168,
                        cap=256, values="normal", seed=4)
        inp = wl.materialize(w, "cuda")
        inp["B"] = mg.pack_panels(inp["B"], mg.B_KN_PANEL, mg.PANEL_MASKED)
        _, gemm, _ = build_step(w, inp, 0, mg.B_KN_PANEL)
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        settle(gemm)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i, (a, b) in enumerate(ev):
            scratch.fill_(i & 255)
            a.record()
            gemm()
            b.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        nb = algorithmic_bytes(w)
        print(json.dumps({"bucket": "masked", "dtype": dtype, "poisson_mean": mean, "U": sum(counts),
                          "active_experts": sum(1 for c in counts if c > 0), "ms": round(ms, 4),
                          "algorithmic_bytes": nb, "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK, 4)}), flush=True)
        del inp, scratch
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps before the timed ones; in a fresh process the first few tens of steps run "
                         "about 5 %% slower than the steady state")
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the clock sample (about 0.4 s of extra back-to-back steps after the timed ones)")
    ap.add_argument("--no-candidates", action="store_true",
                    help="skip the per-candidate report (each tile height timed on its own after the timed steps)")
    cache = ap.add_mutually_exclusive_group()
    cache.add_argument("--cold", dest="cold", action="store_true", default=None,
                       help="write a 512 MiB scratch buffer between steps (more than L2 + MALL), and time each "
                            "step with its own events; ms_per_step is then the mean of those.  The default for "
                            "workloads 2-5, whose operands (0.8-2.2 GB) are streamed once per layer in a model")
    cache.add_argument("--warm", dest="cold", action="store_false",
                       help="back-to-back steps, operands left in L2 and MALL; the default for workload 1")
    ap.add_argument("--dtype", choices=("as-stated", "fp8"), default="as-stated",
                    help="fp8: run the masked decode (4) or the K-grouped weight-gradient (5) workload on e4m3 "
                         "operands with fp32 scales (per 1x128 activation group and 128x128 weight block; "
                         "K-grouped: per 128-row group of each expert's segment and column)")
    ap.add_argument("--scales", choices=("fp32", "e8m0"), default="fp32",
                    help="fp8 block scales: fp32 (the workload as stated, promoted on the VALU), or powers of two "
                         "as E8M0 bytes, applied by the MFMA (the contiguous and masked workloads, and the K-grouped "
                         "one with --dtype fp8)")
    ap.add_argument("--weights", choices=("e4m3", "e2m1"), default="e4m3",
                    help="fp8 workload weights: e4m3 (as stated), or packed fp4 E2M1 [G,N,K/2] with E8M0 scales "
                         "(implies --scales e8m0; contiguous fp8 workloads only)")
    ap.add_argument("--mlp", action="store_true",
                    help="time the expert MLP (scheduler, L1 fp8 with the fused SwiGLU epilogue, L2 bf16) on the "
                         "Zipf histogram at the DeepSeek-V3 expert shape instead of one grouped GEMM")
    ap.add_argument("--a-scale", choices=("km", "rows"), default="km",
                    help="fp32 activation-scale layout for fp8: [K/128, rows] (default) or [rows, K/128]")
    ap.add_argument("--decode-buckets", action="store_true",
                    help="low-token buckets instead of one workload: the contiguous fp8 shape at 32..1024 routed "
                         "rows (every tile height and the device's choice) and the masked decode shape at Poisson "
                         "means 1..128; one JSON line per bucket")
    ap.add_argument("--mlp-fused", action="store_true",
                    help="with --mlp: the expert MLP in one launch (fp8 H), timed beside the same "
                         "work as three launches from the 256-row schedule")
    ap.add_argument("--mlp-h", choices=("fp8", "bf16"), default="fp8",
                    help="with --mlp: H quantized to e4m3 in L1's epilogue and an fp8 L2 (default), or bf16 H and L2")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB, so that a "
                         "counter run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) can scale HBM counters by "
                         "a transfer of known size")
    ap.add_argument("--block-m", default="auto", choices=("auto", "exemplar", "per-expert", "64", "128", "256"),
                    help="tile height: auto = chosen on the device by the cost rule; exemplar = chosen on the "
                         "device by matching the histogram to the MI355X exemplar table (hysteresis 4096); "
                         "per-expert = 256-row tiles plus a remainder tile per expert sized 64/128/256")
    ap.add_argument("--b-layout", choices=("auto", "kn", "nk", "kn-panel", "nk-panel"), default="auto",
                    help="weight storage: [G,K,N] (kn) or [G,N,K] (nk, the K-contiguous form fp8 MoE weights "
                         "are usually kept in; repacking is one-time, outside the timed steps).  auto: nk for "
                         "the contiguous workloads, kn-panel for the masked one, nk-panel for fp4 weights.  "
                         "kn-panel / nk-panel: the same weights repacked in column panels of the call's tile "
                         "width, so that each K step's weight tile is one contiguous block (one-time repack)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mg.lib()
    if args.mlp_fused and (not args.mlp or args.mlp_h != "fp8" or args.weights != "e4m3"):
        print("--mlp-fused goes with --mlp, fp8 H and e4m3 weights", file=sys.stderr)
        sys.exit(2)
    if args.mlp:
        run_mlp(args)
        return
    if args.decode_buckets:
        run_decode_buckets(args)
        return
    w = wl.workload(args.config)
    if args.dtype == "fp8":
        if w.layout == "contiguous":
            print("--dtype fp8 applies to the masked (4) and K-grouped (5) workloads", file=sys.stderr)
            sys.exit(2)
        if w.dtype != "fp8":
            w.dtype, w.name = "fp8", w.name.replace("bf16", "fp8")
    if args.weights == "e2m1":
        args.scales = "e8m0"
        w.weights = "e2m1"
    if args.scales == "e8m0":
        if w.layout == "masked" and w.dtype == "bf16":
            # the decode workload with fp8 activations (power-of-two 1x128 scales) in place of bf16
            w.dtype, w.name = "fp8", w.name.replace("bf16", "fp8")
        if w.dtype != "fp8" or (w.layout == "k_grouped" and w.weights == "e2m1"):
            print("--scales e8m0 applies to the fp8 workloads (--dtype fp8 for the K-grouped one), --weights e2m1 "
                  "to the contiguous and masked ones", file=sys.stderr)
            sys.exit(2)
        w.scales = "e8m0"
    if args.cold is None:
        args.cold = args.config != 1
    log(f"workload {args.config}: {w.name}, G={w.G}, U={sum(w.counts)}")
    inp = wl.materialize(w, "cuda")
    # auto: K-contiguous [G,N,K] for the contiguous workloads; for the decode workload its [G,K,N] weights
    # repacked once into 128-column panels, which it streams; fp4 weights, drawn [G,N,K/2], repacked once
    # into panels of the call's column tile, so that each K step reads whole lines
    layout = args.b_layout if args.b_layout != "auto" else \
        ("nk-panel" if w.weights == "e2m1" else "kn-panel" if w.layout == "masked" else "nk")
    if w.weights == "e2m1" and layout not in ("nk", "nk-panel"):
        print("fp4 weights are stored [G,N,K/2] (nk) or in its panels (nk-panel)", file=sys.stderr)
        sys.exit(2)
    b_layout = {"kn": mg.B_KN, "nk": mg.B_NK, "kn-panel": mg.B_KN_PANEL, "nk-panel": mg.B_NK_PANEL}[layout]
    oracle_inp = dict(inp)                # the oracle reads the weights as drawn, [G, K, N]
    if b_layout == mg.B_NK and "B" in inp and w.weights != "e2m1":
        inp["B"] = inp["B"].transpose(1, 2).contiguous()       # static weights, stored K-contiguous
    elif b_layout in (mg.B_KN_PANEL, mg.B_NK_PANEL):
        if w.layout == "k_grouped":
            print("panel layouts apply to the contiguous and masked workloads", file=sys.stderr)
            sys.exit(2)
        inp["B"] = mg.pack_panels(inp["B"], b_layout,
                                  mg.PANEL_MASKED if w.layout == "masked" else mg.PANEL_CONTIGUOUS)
    torch.cuda.synchronize()

    # the tile height stays on the device: the timed step is the scheduler, then the GEMM with block_m = 0
    # (one launch that runs whatever height the scheduler chose) unless --block-m fixes a height
    bm_req = {"auto": 0, "exemplar": 0, "per-expert": mg.BLOCK_M_PER_EXPERT}[args.block_m] \
        if not args.block_m.isdigit() else int(args.block_m)
    exemplars = mg.exemplar_table(dtype=w.dtype) if args.block_m == "exemplar" and w.layout == "contiguous" \
        else None
    # the kernels take E8M0 bytes; the oracle (cpu_baseline) keeps the same scales as fp32 (the K-grouped
    # step picks its byte arrays itself)
    inp_gpu = dict(inp, A_scale=inp["A_scale_e8m0"], B_scale=inp["B_scale_e8m0"]) \
        if w.scales == "e8m0" and w.layout != "k_grouped" else inp
    # fp32 activation scales handed over [K/128, rows] (the quantizer upstream writes them so; the
    # transpose here is input preparation, outside the timed region); the oracle keeps [rows, K/128]
    scale_km = w.dtype == "fp8" and w.scales != "e8m0" and args.a_scale == "km" and w.layout != "k_grouped"
    if scale_km:
        a_s = inp["A_scale"]
        inp_gpu = dict(inp, A_scale=a_s.reshape(-1, a_s.shape[-1]).t().contiguous())
    sched, gemm, ws = build_step(w, inp_gpu, bm_req, b_layout, bm_req, exemplars, 4096, scale_km=scale_km)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        if sched is not None:
            sched()
        gemm()
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 2)]
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] if args.cold else None
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.cold else None
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        if args.cold:
            scratch.fill_(i & 255)                   # evict the inputs from L2 and MALL
            step_ev[i].record(stream)
        if sched is not None:
            sched()
        ev[1 + 2 * i].record(stream)
        gemm()
        ev[2 + 2 * i].record(stream)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = ev[0].elapsed_time(ev[-1])
    gemm_ms = [ev[1 + 2 * i].elapsed_time(ev[2 + 2 * i]) for i in range(args.steps)]
    if args.cold:
        ms_step = sum(step_ev[i].elapsed_time(ev[2 + 2 * i]) for i in range(args.steps)) / args.steps
    else:
        ms_step = total_ms / args.steps
    gemm_avg = sum(gemm_ms) / len(gemm_ms)

    st = mg.stats_read(ws) if sched is not None or w.layout != "k_grouped" else None
    U = sum(w.counts)
    flops = w.useful_flops()
    eff = flops / (ms_step * 1e-3) / 1e12
    peak = PEAK[w.dtype]
    out = {
        "metric": METRIC if args.config == 3 else f"effective TFLOPS (valid rows), workload {args.config}",
        "value": round(eff, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_e4m3 x fp4_e2m1" if w.weights == "e2m1" else "fp8_e4m3") if w.dtype == "fp8" else "bf16",
        # operands' storage type; accumulation is fp32 and the output bf16 (fp32 dW for the K-grouped gradient)
        "data": "synthetic",
        "config": {"workload": w.name, "experts": w.G, "routed_rows": U,
                   "K": w.K or None, "N": w.N or None, "layout": w.layout, "seed": w.seed,
                   "weights": {mg.B_KN: "[G,K,N]", mg.B_KN_PANEL: "[G,N/P,K,P] column panels",
                               mg.B_NK_PANEL: "[G,N/P,K/S,P,S] column panels by K step",
                               mg.B_NK: "[G,N,K/2] packed e2m1" if w.weights == "e2m1" else "[G,N,K]"}[b_layout],
                   "scales": ("e8m0 (powers of two, applied by the MFMA)" if w.scales == "e8m0" else
                              "fp32, activation scales [K/128, rows]" if scale_km else "fp32")
                   if w.dtype == "fp8" else None,
                   "cache": "cold (512 MiB written between steps)" if args.cold else "warm",
                   "tile_choice": f"exemplar table (MI355X, {w.dtype})" if exemplars is not None else
                   ("cost rule" if args.block_m == "auto" else "fixed")},
        "pct_mfma_peak": round(100.0 * eff / peak, 2),
    }
    if w.layout == "contiguous":
        phys = 2.0 * st.P_exec * w.K * w.N / (ms_step * 1e-3) / 1e12
        rep = st.report()                       # ratios derived by the library (moegg_stats_report)
        out.update({"physical_tflops": round(phys, 2),
                    "block_m": "per-expert" if st.block_m == mg.BLOCK_M_PER_EXPERT else st.block_m,
                    "U": st.U, "P_exec": st.P_exec, "active_experts": st.active,
                    # rows the MFMAs ran without a valid row: every height skips 16-row blocks past a tile's
                    # valid rows, so the executed rows are P(16) whatever the height
                    "padding_fraction_exec": round(rep.exec_padding_fraction, 6),
                    "padding_fraction_by_q": {q: round(v, 6) for q, v in rep.padding_fraction.items()},
                    "effective_experts": round(rep.effective_experts, 4)})
    # roofline of the dominant kernel (the GEMM), from HIP events on its own stream
    achieved_tflops = flops / (gemm_avg * 1e-3) / 1e12
    bytes_alg = algorithmic_bytes(w)
    # the binding roof: algorithmic bytes at HBM peak against algorithmic flops at MFMA peak
    if bytes_alg / (HBM_PEAK * 1e9) > flops / (peak * 1e12):
        gbs = bytes_alg / (gemm_avg * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK, 4), "traffic": None}
    else:
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": peak,
                           "unit": "TFLOP/s", "frac": round(achieved_tflops / peak, 4), "traffic": None}
    tr = traffic_for(w, b_layout, scale_km)
    if tr is not None:
        out["roofline"]["traffic"] = tr
    out["traffic_key"] = traffic_key(w, b_layout, scale_km)
    out["gemm_kernel_ms"] = round(gemm_avg, 4)
    out["algorithmic_bytes"] = bytes_alg
    out["wall_s_timed"] = round(wall, 4)
    # after the timed steps: the other candidate heights, and the clock under this load
    if w.layout == "contiguous" and exemplars is None and not args.no_candidates:
        out["candidates"] = time_candidates(w, inp_gpu, b_layout, scale_km, args)
    out["sclk"] = None if args.no_sclk else sample_sclk(lambda: (sched() if sched is not None else None, gemm()))
    out["host"] = host_info()
    calib_copy(args)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)...")
        out["cpu_baseline"] = cpu_baseline(w, oracle_inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
