"""Expert MLP of a MoE layer on one GPU: L1 projection -> SwiGLU -> L2
projection, written out in fp64 (test infrastructure only).

The DeepGEMM record's Mega MoE fuses an expert's two GEMMs and the SwiGLU
between them.  For each valid row R of expert e (contiguous layout):

    g[R, c] = sum_k A[R, k] * Wgate_e[k, c]
    u[R, c] = sum_k A[R, k] * Wup_e[k, c]
    h[R, c] = silu(g) * u,   silu(x) = x / (1 + e^-x)
    y[R, n] = sum_c h[R, c] * W2_e[c, n]

The library takes the gate and up weights as one matrix W1 [G, 2I, K] whose
row 32q + w is gate column 16q + w and row 32q + 16 + w is up column 16q + w
(w < 16); `split_gate_up` undoes that order by its definition.  The two L1
sums come from the C oracle (gemm.contiguous, fp64 on the decoded bf16/e4m3
bits and fp32 scales); silu, the product and the L2 sum are plain numpy fp64.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np
import torch

from . import accounting as acc
from . import gemm as og


def silu(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):             # e^-x = inf for very negative x: the limit -0
        return x / (1.0 + np.exp(-x))


def split_gate_up(c: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Columns of an interleaved [.., 2I] result -> (gate [.., I], up [.., I])."""
    n2 = c.shape[-1]
    I = n2 // 2
    cols = np.arange(I)
    gate_idx = 32 * (cols // 16) + cols % 16
    return c[..., gate_idx], c[..., gate_idx + 16]


def swiglu_rows(A: torch.Tensor, W1: torch.Tensor, counts: Sequence[int], rows: Sequence[int],
                A_scale=None, W1_scale=None, seg_align: int = 1) -> np.ndarray:
    """h for the given rows, fp64 [len(rows), I].  A [rows_total, K] and W1
    [G, 2I, K] hold the bits the GPU receives (bf16, or e4m3 with fp32
    1x128 / 128x128 scales over W1's interleaved rows)."""
    B = W1.transpose(1, 2).contiguous()                   # [G, K, 2I]: the oracle's B layout
    c = og.contiguous(A, B, counts, rows, seg_align=seg_align, A_scale=A_scale, B_scale=W1_scale)
    g, u = split_gate_up(c)
    return silu(g) * u


def swiglu_rows_fp4(A: torch.Tensor, A_scale, W1: torch.Tensor, W1_scale, counts: Sequence[int],
                    rows: Sequence[int], seg_align: int = 1) -> np.ndarray:
    """As swiglu_rows for fp8 activations times packed E2M1 gate/up weights
    W1 [G, 2I, K/2] (same row order) with power-of-two scales given as fp32."""
    from . import fp4
    c = fp4.contiguous_fp8_fp4(A, A_scale, W1, W1_scale, counts, rows, seg_align=seg_align)
    g, u = split_gate_up(c)
    return silu(g) * u


def _e4m3_positive() -> np.ndarray:
    """Values of the non-negative finite e4m3 codes 0x00 .. 0x7E, ascending with the code."""
    return np.array([og.dec_e4m3(c) for c in range(0x7F)], dtype=np.float64)


_E4M3_POS = None


def e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value to each |x| <= 448, ties to the even code (the code's
    last mantissa bit 0), sign kept."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = _e4m3_positive()
    v = _E4M3_POS
    a = np.abs(x)
    hi = np.clip(np.searchsorted(v, a), 1, len(v) - 1)
    lo = hi - 1
    dlo, dhi = a - v[lo], v[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.sign(x) * v[pick]


def quantize_groups(h: np.ndarray, group: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """h [rows, I] -> (e4m3 values [rows, I], scales [rows, I / group]): per
    1 x group slice s = amax / 448 (1 if the amax is 0), value = e4m3_rne of
    h / s clamped to +-448."""
    r, n = h.shape
    g = h.reshape(r, n // group, group)
    amax = np.abs(g).max(axis=2)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    q = e4m3_rne(np.clip(g / s[:, :, None], -448.0, 448.0))
    return np.ascontiguousarray(q.reshape(r, n)), np.ascontiguousarray(s)


def down_rows(h: np.ndarray, W2: torch.Tensor, counts: Sequence[int], rows: Sequence[int],
              seg_align: int = 1) -> np.ndarray:
    """y = h @ W2_e for the given rows (h fp64, as swiglu_rows returns it);
    W2 [G, N2, I] bf16 (K-contiguous).  fp64 [len(rows), N2]."""
    offs = acc.segment_offsets(counts, seg_align)
    out = np.empty((len(rows), W2.shape[1]), dtype=np.float64)
    by_e = {}
    for i, r in enumerate(rows):
        e = next(e for e in range(len(counts)) if offs[e] <= r < offs[e] + counts[e])
        by_e.setdefault(e, []).append(i)
    for e, idx in by_e.items():
        w2 = W2[e].double().numpy()                  # [N2, I]
        out[idx] = h[idx] @ w2.T
    return out
