"""fp8 activations times fp4 (E2M1) weights with power-of-two block scales:
the plain per-expert definition in fp64 (test infrastructure only).

The DeepGEMM record lists low-precision weights (FP8 x FP4) next to the
SM100 UE8M0 scale format; this is that product written out.  For each valid
row R of expert e and each column n:

    C[R, n] = sum_k (dec8(A[R, k]) * sa[R, k/128]) * (dec4(W[e, n, k]) * sb[e, k/128, n/128])

with dec8 the oracle's own OCP E4M3FN decoder (gemm.dec_e4m3) and dec4 the
OCP E2M1 decoder below.  Weights are stored [G, N, K/2], two codes per byte,
element 2i in the low nibble.  Both operands are dequantized in fp64 exactly as
the formula reads (each code times its own group's scale), and a library
float64 matmul takes the sum over k; nothing is blocked or reordered.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np
import torch

from . import accounting as acc
from . import gemm as og


def e2m1_value(code: int) -> float:
    """OCP E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0
    is subnormal (0 or 0.5); no infinities or NaN."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def dec_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> float64 [..., K]; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = E2M1[p & 0xF]
    out[..., 1::2] = E2M1[p >> 4]
    return out


def _e4m3_table() -> np.ndarray:
    return np.array([og.dec_e4m3(c) for c in range(256)], dtype=np.float64)


def _dequant_rows(codes: np.ndarray, scales: np.ndarray, dec8: np.ndarray) -> np.ndarray:
    """e4m3 codes [m, K] and their 1x128 scales [m, K/128] -> values [m, K] (fp64)."""
    return dec8[codes] * np.repeat(scales, 128, axis=1)


def _dequant_weight(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's packed E2M1 weights [N, K/2] and block scales [K/128, N/128] -> W [N, K] (fp64)."""
    w = dec_e2m1_packed(packed)                                      # [N, K]
    s = np.repeat(np.repeat(scales, 128, axis=0), 128, axis=1)       # [K, N]: the scale of each (k, n)
    return w * s.T


def contiguous_fp8_fp4(A: torch.Tensor, A_scale: torch.Tensor, W: torch.Tensor, W_scale: torch.Tensor,
                       counts: Sequence[int], rows: Sequence[int], seg_align: int = 1) -> np.ndarray:
    """Rows `rows` of C for the contiguous layout (segment starts as in the tile
    list of the accounting module).  A: e4m3 codes [rows_total, K]; A_scale fp32
    [rows_total, K/128]; W: packed E2M1 [G, N, K/2]; W_scale fp32 [G, K/128, N/128]."""
    dec8 = _e4m3_table()
    a_codes = A.contiguous().view(torch.uint8).numpy()
    sa = A_scale.double().numpy()
    w = W.contiguous().numpy()
    sb = W_scale.double().numpy()
    N = w.shape[1]
    offs = acc.segment_offsets(counts, seg_align)
    out = np.zeros((len(rows), N), dtype=np.float64)
    expert_of = {}
    for e, c in enumerate(counts):
        for r in range(offs[e], offs[e] + c):
            expert_of[r] = e
    by_e = {}
    for i, r in enumerate(rows):
        by_e.setdefault(expert_of[r], []).append(i)
    for e, idx in by_e.items():
        rr = [rows[i] for i in idx]
        a = _dequant_rows(a_codes[rr], sa[rr], dec8)                  # [m, K]
        we = _dequant_weight(w[e], sb[e])                             # [N, K]
        out[idx] = a @ we.T
    return out


def masked_fp8_fp4(A: torch.Tensor, A_scale: torch.Tensor, W: torch.Tensor, W_scale: torch.Tensor,
                   masked_m: Sequence[int], pairs: Sequence[tuple]) -> np.ndarray:
    """Masked layout: C[e, r, n] for each (e, r) in `pairs` (r < masked_m[e]).
    A: e4m3 codes [G, cap, K]; A_scale fp32 [G, cap, K/128]; W packed E2M1
    [G, N, K/2]; W_scale fp32 [G, K/128, N/128].  Same product as
    contiguous_fp8_fp4, with row r of expert e at A[e, r]."""
    dec8 = _e4m3_table()
    a_codes = A.contiguous().view(torch.uint8).numpy()
    sa = A_scale.double().numpy()
    w = W.contiguous().numpy()
    sb = W_scale.double().numpy()
    N = w.shape[1]
    out = np.zeros((len(pairs), N), dtype=np.float64)
    by_e = {}
    for i, (e, r) in enumerate(pairs):
        assert 0 <= r < masked_m[e]
        by_e.setdefault(e, []).append(i)
    for e, idx in by_e.items():
        rr = [pairs[i][1] for i in idx]
        a = _dequant_rows(a_codes[e, rr], sa[e, rr], dec8)
        we = _dequant_weight(w[e], sb[e])
        out[idx] = a @ we.T
    return out
