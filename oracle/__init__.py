"""The oracle: a plain CPU reference for the MoE grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
and the cpu_baseline leg of bench.py may import it.  The HIP library and its
Python binding never import it, and it shares no code with them.

Parts:
- accounting.py: the exact integer padding accounting and tile lists, in
  Python ints and Fractions.
- oracle.c with gemm.py: fp64 per-expert dot products for the contiguous,
  masked and K-grouped layouts (bf16, and e4m3 with fp32 scales).  They read the same bf16 / e4m3 bits the GPU
  receives and decode them with their own decoders.
- fp4.py: fp8 activations times packed E2M1 weights with power-of-two block
  scales (the contiguous layout), with its own E2M1 decoder.
- select.py: the distribution-aware tile-height choice (sorted, normalized
  histogram matched against an exemplar table, with hysteresis).
- choice.py: the integer cost rule that picks the tile height for block_m = 0.
- mlp.py: the expert MLP, L1 projection -> SwiGLU -> L2 projection, in fp64.

Every function states the page and section it follows.  Parity pins live in
tests/test_oracle_*.py and tests/golden/.
"""
from . import accounting  # noqa: F401
from . import gemm  # noqa: F401
from . import fp4  # noqa: F401
from . import select  # noqa: F401
from . import choice  # noqa: F401
from . import mlp  # noqa: F401
