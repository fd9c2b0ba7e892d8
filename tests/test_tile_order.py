"""Work order of the contiguous GEMM (csrc/tile_order.hpp), checked on the host:
tests/tile_order_driver.hip is built with hipcc (host code only, nothing is
launched) and maps every work item of the oracle's tile lists (every height and
per-expert heights, 200 random histograms plus the workloads, several
column-tile counts) to its (row tile, column tile): each pair once, all in
range.  The groups of row tiles the order forms are also checked to stay within
one expert.  The one-launch expert MLP's grid (L1 blocks, then L2 blocks) is
checked over the same lists: each (phase, row tile, column tile) once, every L1
block ahead of every L2 block."""
import os
import random
import subprocess

import pytest

import workloads as wl
from moe_grouped_gemm_sizes_amd import build as B
from oracle import accounting as acc

HERE = os.path.dirname(os.path.abspath(__file__))


def _lists():
    rng = random.Random(5)
    hists = [wl.workload(n).counts for n in (1, 2, 3)] + [[300], [1], [0, 0, 5], [257, 0, 1000, 128, 129, 3000]]
    for _ in range(200):
        G = rng.randrange(1, 70)
        hists.append([rng.choice([0, 1, 128, 129, 256, 257, rng.randrange(0, 3000)]) for _ in range(G)])
    for h in hists:
        for n_ct in (1, 3, 16):
            for bm in (64, 128, 256):
                yield n_ct, 0, acc.tile_list(h, bm)
            yield n_ct, 1, acc.tile_list_per_expert(h)


@pytest.mark.timeout(300)
def test_contiguous_work_order(tmp_path):
    exe = str(tmp_path / "tile_order_driver")
    r = subprocess.run([B.hipcc(), "-O1", "-std=c++17", f"--offload-arch={B.ARCH}",
                        os.path.join(HERE, "tile_order_driver.hip"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = []
    n = 0
    for n_ct, pe, tiles in _lists():
        lines.append(f"{n_ct} {pe} {len(tiles)}")
        lines += [f"{e} {i} {rv}" for e, i, _, rv in tiles]
        n += 1
    path = tmp_path / "lists.txt"
    path.write_text("\n".join(lines) + "\n")
    r = subprocess.run([exe, str(path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == f"{n} cases ok", r.stdout[-2000:]
