"""Measure the exemplar table of the distribution-aware tile-height selector
(moegg_schedule_exemplar) on this GPU and write it as JSON.

The padding page ("MoE GroupGEMM padding under expert skew") asks for kernel
choice from the routing histogram on the device, matched against exemplars
tuned offline ("Adapt kernels without adding a CPU stall"), and for the
candidates to be benchmarked on the deployed GPU rather than chosen from the
padding formula ("Padding is not the whole cost model").  This tool does the
benchmarking:

  - exemplar histograms: 64 experts, U in {256, 512, ..., 32768} (powers of
    two) routed rows, Zipf exponents 0 (uniform), 0.8, 1.2 and 2.0 over the
    experts, a fifth of the experts empty (the seeded generator of the
    workloads module);
  - for each, the contiguous GEMM (K = 7168, N = 4096; --dtype fp8: e4m3 with
    fp32 block scales, the default; --dtype bf16: bf16 operands; [G, N, K]
    weights, 512 MiB written between calls so the operands come from HBM) at
    every tile configuration: 64, 128 and 256 rows and per-expert heights; the
    median of 8 timed calls;
  - each entry keeps the histogram, its descriptor as the device computes it
    (moegg_selection_read), the times, and the fastest configuration.

With --evaluate, it instead times held-out histograms (sizes and skews
between the table's grid points, other seeds) at every configuration and
reports, for the exemplar choice and for the cost rule of the contiguous call
(block_m = 0), the time of the chosen configuration over the fastest one.

Usage, on the GPU:  python -m moe_grouped_gemm_sizes_amd.tune_exemplars [--dtype bf16] [--out PATH]
                    python -m moe_grouped_gemm_sizes_amd.tune_exemplars --evaluate [--dtype bf16] [--out PATH]
Each dtype has its own table (mg.EXEMPLAR_TABLE_PATHS).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import moe_grouped_gemm_sizes_amd as mg  # noqa: E402
import workloads as wl  # noqa: E402

SIZES = (256, 512, 1024, 2048, 4096, 8192, 16384, 32768)
SKEWS = (0.0, 0.8, 1.2, 2.0)
CONFIGS = (64, 128, 256, mg.BLOCK_M_PER_EXPERT)
EVAL_SIZES = (384, 2500, 6000, 12000, 24000)
EVAL_SKEWS = (0.4, 1.0, 1.6)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="default: the package's table for --dtype")
    ap.add_argument("--dtype", choices=sorted(mg.EXEMPLAR_TABLE_PATHS), default="fp8")
    ap.add_argument("--iters", type=int, default=8)
    ap.add_argument("--settle", type=int, default=100, help="untimed full-workload GEMMs before the first timing")
    ap.add_argument("--evaluate", action="store_true")
    ap.add_argument("--hysteresis", type=int, default=0)
    args = ap.parse_args()
    out_path = args.out or mg.EXEMPLAR_TABLE_PATHS[args.dtype]
    w = wl.workload(3)                        # shapes of the fp8 Zipf workload: 64 experts, K 7168, N 4096
    if args.dtype == "bf16":
        w = wl.Workload("exemplar tuning, bf16", "contiguous", "bf16", w.counts, K=w.K, N=w.N, values="normal",
                        seed=w.seed)
    inp = wl.materialize(w, "cuda", nan_padding=False)
    A, As, Bs = inp["A"], inp.get("A_scale"), inp.get("B_scale")
    B = inp["B"].transpose(1, 2).contiguous()
    del inp
    G, R, N = w.G, w.rows_total, w.N
    C = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    ws = mg.workspace(G, R)
    ws_d = torch.zeros_like(ws)
    probe = torch.zeros((1, mg.EXEMPLAR_FIELDS), dtype=torch.int32, device="cuda")
    probe[0, -1] = 256
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    # the first few tens of GEMMs in a fresh process run below the steady state: settle on the full workload
    # first, so the histograms timed first are not handicapped
    ct = torch.tensor(w.counts, dtype=torch.int32, device="cuda")
    mg.schedule(ct, R, ws, block_m=mg.BLOCK_M_PER_EXPERT, N=N)
    for _ in range(args.settle):
        mg.grouped_gemm_contiguous_scheduled(A, B, C, G, ws, As, Bs, block_m=mg.BLOCK_M_PER_EXPERT, b_layout=mg.B_NK)
    torch.cuda.synchronize()
    entries = []
    table = mg.exemplar_table(dtype=args.dtype) if args.evaluate else None
    grid = [(U, s) for U in (EVAL_SIZES if args.evaluate else SIZES) for s in (EVAL_SKEWS if args.evaluate else SKEWS)]
    for U, s in grid:
        seed = (5000 if args.evaluate else 1000) + U + int(10 * s)
        counts = wl.hist_zipf(seed=seed, experts=G, total=U, s=s)
        ct = torch.tensor(counts, dtype=torch.int32, device="cuda")
        ws_d.zero_()
        mg.schedule_exemplar(ct, R, ws_d, table if args.evaluate else probe, hysteresis=args.hysteresis, N=N)
        d = mg.selection_read(ws_d)
        picked = mg.stats_read(ws_d).block_m
        mg.schedule(ct, R, ws, block_m=0, N=N)
        rule = mg.stats_read(ws).block_m
        times = {}
        for bm in CONFIGS:
            mg.schedule(ct, R, ws, block_m=bm, N=N)

            def gemm():
                mg.grouped_gemm_contiguous_scheduled(A, B, C, G, ws, As, Bs, block_m=bm, b_layout=mg.B_NK)
            gemm()
            gemm()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.iters)]
            for i, (e0, e1) in enumerate(ev):
                scratch.fill_(i & 255)
                e0.record()
                gemm()
                e1.record()
            torch.cuda.synchronize()
            t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
            times[str(bm)] = round(t[len(t) // 2], 4)
        best = int(min(times, key=times.get))
        e = {"name": f"zipf{s}_U{U}", "U": U, "counts": counts, "size_class": d.size_class,
             "lorenz": list(d.lorenz), "block_m": best, "times_ms": times}
        if args.evaluate:
            e.update({"exemplar": d.exemplar, "exemplar_block_m": picked, "rule_block_m": rule,
                      "exemplar_over_best": round(times[str(picked)] / times[str(best)], 4),
                      "rule_over_best": round(times[str(rule)] / times[str(best)], 4)})
        entries.append(e)
        print(f"U={U:6d} s={s:3.1f} size_class={d.size_class} best={best:4d} "
              + (f"exemplar={picked:4d} rule={rule:4d} " if args.evaluate else "") + f"{times}", flush=True)
    if args.evaluate:
        import math
        gx = math.exp(sum(math.log(e["exemplar_over_best"]) for e in entries) / len(entries))
        gr = math.exp(sum(math.log(e["rule_over_best"]) for e in entries) / len(entries))
        print(f"geomean time over the fastest: exemplar {gx:.4f}, cost rule {gr:.4f}", flush=True)
        out = {"device": torch.cuda.get_device_name(0),
               "command": "python -m moe_grouped_gemm_sizes_amd.tune_exemplars --evaluate --dtype " + args.dtype,
               "geomean_exemplar_over_best": round(gx, 4), "geomean_rule_over_best": round(gr, 4),
               "held_out": entries}
        with open(out_path, "w") as f:
            json.dump(out, f, indent=1)
        return
    out = {"device": torch.cuda.get_device_name(0),
           "workload": "64 experts, K 7168, N 4096, %s, [G,N,K] weights, contiguous, cold caches; median of %d "
                       "calls per configuration" % ("fp8 e4m3 with fp32 block scales" if args.dtype == "fp8" else
                                                    "bf16", args.iters),
           "command": "python -m moe_grouped_gemm_sizes_amd.tune_exemplars --dtype " + args.dtype,
           "exemplars": entries}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {len(entries)} exemplars to {out_path}", flush=True)


if __name__ == "__main__":
    main()
