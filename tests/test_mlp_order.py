"""Work order of the one-launch expert MLP (csrc/mlp_order.hpp), checked on the
host: tests/mlp_order_driver.hip is built with hipcc (host code only, nothing
is launched) and run.  It checks that every item is handed out once, that each
row tile's down-projection items follow all of its SwiGLU-projection items
with the next group's L1 work between them (what keeps the bounded waits
short), and that the queues' row ranges cover every row tile."""
import os
import subprocess

import pytest

from moe_grouped_gemm_sizes_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(300)
def test_mlp_work_order(tmp_path):
    exe = str(tmp_path / "mlp_order_driver")
    r = subprocess.run([B.hipcc(), "-O1", "-std=c++17", f"--offload-arch={B.ARCH}",
                        os.path.join(HERE, "mlp_order_driver.hip"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:]
