"""Write tests/golden/histograms.json: the per-expert counts of the three
seeded workloads (Zipf routing over 64 experts, Poisson decode counts over 32
experts, Dirichlet weight-gradient split over 16 experts), drawn once by the
generators in workloads/ and frozen.  The fixture is what the benchmark and
the tests use; tests/test_workloads_fixture.py checks that the generators
still reproduce it.

Usage: python tests/golden/make_histograms.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as wl  # noqa: E402


def histograms():
    return {
        "zipf64": {"recipe": "hist_zipf(seed=3, experts=64, total=32768, s=1.2, p_zero=0.2)",
                   "counts": wl.hist_zipf(3)},
        "poisson32": {"recipe": "hist_poisson_masked(seed=4, experts=32, cap=256, mean=24, p_zero=0.2)",
                      "counts": wl.hist_poisson_masked(4)},
        "dirichlet16": {"recipe": "hist_dirichlet(seed=5, experts=16, total=65536, alpha=0.3)",
                        "counts": wl.hist_dirichlet(5)},
    }


if __name__ == "__main__":
    out = {"_note": "Seeded synthetic histograms (no routing traces ship with the pages); "
                    "written by tests/golden/make_histograms.py with numpy's default_rng.",
           **histograms()}
    with open(os.path.join(HERE, "histograms.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
