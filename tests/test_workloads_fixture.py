"""The frozen histograms (tests/golden/histograms.json) are the ones the
seeded generators draw, and the workloads use them (CPU only)."""
import json

import workloads as wl


def test_generators_reproduce_the_fixture():
    with open(wl.FIXTURE_PATH) as f:
        fx = json.load(f)
    assert fx["zipf64"]["counts"] == wl.hist_zipf(3)
    assert fx["poisson32"]["counts"] == wl.hist_poisson_masked(4)
    assert fx["dirichlet16"]["counts"] == wl.hist_dirichlet(5)


def test_workloads_take_the_fixture():
    assert wl.workload(3).counts == wl.fixture_counts("zipf64")
    assert wl.workload(4).counts == wl.fixture_counts("poisson32")
    assert wl.workload(5).counts == wl.fixture_counts("dirichlet16")


def test_fixture_shapes():
    z, p, d = (wl.fixture_counts(k) for k in ("zipf64", "poisson32", "dirichlet16"))
    assert len(z) == 64 and sum(z) == 32768 and 0 in z
    assert len(p) == 32 and all(0 <= c <= 256 for c in p) and 0 in p
    assert len(d) == 16 and sum(d) == 65536
