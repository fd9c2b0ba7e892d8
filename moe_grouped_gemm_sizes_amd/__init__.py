"""MI355X (gfx950) MoE grouped GEMM: a thin Python binding over libmoegg.so.

The binding only marshals arguments.  Every step of the grouped GEMM runs in
the HIP kernels behind the C ABI declared in include/moegg.h:
  - scheduler: counts -> padding accounting + tile list;
  - contiguous, masked and K-grouped GEMMs.
PyTorch supplies device memory and the current stream.  If the library has
not been built, `lib()` raises.  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from fractions import Fraction
from typing import List, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegg.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moegg.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, FP8_E4M3, FP8_E4M3_E8M0, FP8_E4M3_FP4_E2M1, FP8_E4M3_SCALE_KM = 0, 1, 2, 3, 4
B_KN, B_NK = 0, 1
FLAG_NEGATIVE_COUNT, FLAG_ROWS_OVERFLOW, FLAG_COUNT_OVER_CAP, FLAG_BAD_EXEMPLAR = 0x1, 0x2, 0x4, 0x8
Q_VALUES = (8, 16, 32, 64, 128, 256)
BLOCK_M_PER_EXPERT = -1          # per-expert tile heights (include/moegg.h)


class MoeggError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib().moegg_status_string(status).decode()} (status {status})")
        self.status = status


class _Stats(ctypes.Structure):
    _fields_ = [("U", ctypes.c_int64), ("P_exec", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("active", ctypes.c_int64), ("sum_sq", ctypes.c_int64), ("capacity_rows", ctypes.c_int64),
                ("P_at", ctypes.c_int64 * 6), ("block_m", ctypes.c_int32), ("error_flags", ctypes.c_uint32)]


class _Tile(ctypes.Structure):
    _fields_ = [("expert", ctypes.c_int32), ("tile", ctypes.c_int32), ("row_start", ctypes.c_int32),
                ("rows_valid", ctypes.c_int32)]


@dataclass
class Stats:
    """Device-computed padding accounting of one scheduled call."""
    U: int
    P_exec: int
    tiles: int
    active: int
    sum_sq: int
    capacity_rows: int
    P_at: dict
    block_m: int
    error_flags: int

    @property
    def effective_experts(self) -> Fraction:
        return Fraction(0) if self.sum_sq == 0 else Fraction(self.U * self.U, self.sum_sq)

    def padding_fraction(self, q: int) -> Fraction:
        p = self.P_at[q]
        return Fraction(0) if p == 0 else Fraction(p - self.U, p)


_lib = None
_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

EXPORTS = {
    "moegg_version": (ctypes.c_int, []),
    "moegg_status_string": (ctypes.c_char_p, [_I32]),
    "moegg_workspace_bytes": (_SZ, [_I32, _I64]),
    "moegg_schedule": (_I32, [_VP, _I32, _I64, _I32, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_schedule_exemplar": (_I32, [_VP, _I32, _I64, _I32, _I32, _VP, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_selection_read": (_I32, [_VP, _VP, _VP]),
    "moegg_grouped_gemm_contiguous_scheduled": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                                       _I32, _I32, _VP, _SZ, _VP]),
    "moegg_grouped_gemm_contiguous": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                             _I32, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_grouped_gemm_swiglu_scheduled": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                                   _I32, _I32, _VP, _SZ, _VP]),
    "moegg_grouped_gemm_masked": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32,
                                         _VP, _SZ, _VP]),
    "moegg_grouped_gemm_k_grouped": (_I32, [_VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_stats_read": (_I32, [_VP, ctypes.POINTER(_Stats), _VP]),
    "moegg_tile_list_read": (_I32, [_VP, ctypes.POINTER(_Tile), _I64, ctypes.POINTER(_I64), _VP]),
}


def lib():
    """The loaded HIP library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m moe_grouped_gemm_sizes_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        raise MoeggError(status, what)


def _dtype(t: torch.Tensor, scale: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
           scale_km: bool = False) -> int:
    """Operand type code: fp8 with uint8 (E8M0) scales is MOEGG_FP8_E4M3_E8M0,
    and with uint8 weights (packed E2M1 [G, N, K/2]) MOEGG_FP8_E4M3_FP4_E2M1.
    scale_km: fp32 activation scales stored [K/128, rows]
    (MOEGG_FP8_E4M3_SCALE_KM)."""
    if t.dtype == torch.bfloat16:
        code = BF16
    elif t.dtype == torch.float8_e4m3fn:
        if w is not None and w.dtype == torch.uint8:
            code = FP8_E4M3_FP4_E2M1
        else:
            code = FP8_E4M3_E8M0 if scale is not None and scale.dtype == torch.uint8 else FP8_E4M3
    else:
        raise TypeError(f"bf16 or float8_e4m3fn operands expected, got {t.dtype}")
    if scale_km:
        if code != FP8_E4M3:
            raise ValueError("scale_km applies to e4m3 operands with fp32 scales")
        return FP8_E4M3_SCALE_KM
    return code


def workspace_bytes(G: int, max_rows: int) -> int:
    return int(lib().moegg_workspace_bytes(G, max_rows))


def workspace(G: int, max_rows: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(G, max_rows)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.empty(n, dtype=torch.uint8, device=device)


def schedule(m_sizes: torch.Tensor, rows_total: int, ws: torch.Tensor, seg_align: int = 1, block_m: int = 0,
             N: int = 256, stream=None):
    _check(lib().moegg_schedule(_p(m_sizes), m_sizes.numel(), rows_total, seg_align, block_m, N, _p(ws),
                                ws.numel(), _stream(stream)), "moegg_schedule")


EXEMPLAR_FIELDS = 10            # moegg_exemplar_t: size_class, lorenz[8], block_m (int32 each)
EXEMPLAR_TABLE_PATH = os.path.join(_HERE, "exemplars_mi355x.json")


def exemplar_table(device="cuda", path: Optional[str] = None) -> torch.Tensor:
    """The exemplar table as an int32 [n, 10] device tensor (moegg_exemplar_t rows).
    Default: the table measured on MI355X that ships with the package."""
    import json
    with open(path or EXEMPLAR_TABLE_PATH) as f:
        rows = json.load(f)["exemplars"]
    t = torch.tensor([[r["size_class"], *r["lorenz"], r["block_m"]] for r in rows], dtype=torch.int32)
    return t.to(device)


def schedule_exemplar(m_sizes: torch.Tensor, rows_total: int, ws: torch.Tensor, exemplars: torch.Tensor,
                      hysteresis: int = 0, seg_align: int = 1, N: int = 256, stream=None):
    """moegg_schedule with the tile height matched to an exemplar on the device (see moegg.h)."""
    if exemplars.dtype != torch.int32 or exemplars.dim() != 2 or exemplars.shape[1] != EXEMPLAR_FIELDS:
        raise ValueError("exemplars: int32 [n, 10] expected")
    _check(lib().moegg_schedule_exemplar(_p(m_sizes), m_sizes.numel(), rows_total, seg_align, N, _p(exemplars),
                                         exemplars.shape[0], hysteresis, _p(ws), ws.numel(), _stream(stream)),
           "moegg_schedule_exemplar")


class _Selection(ctypes.Structure):
    _fields_ = [("exemplar", ctypes.c_int32), ("size_class", ctypes.c_int32), ("lorenz", ctypes.c_int32 * 8),
                ("distance", ctypes.c_int64)]


@dataclass
class Selection:
    exemplar: int
    size_class: int
    lorenz: Tuple[int, ...]
    distance: int


def selection_read(ws: torch.Tensor, stream=None) -> Selection:
    s = _Selection()
    _check(lib().moegg_selection_read(_p(ws), ctypes.c_void_p(ctypes.addressof(s)), _stream(stream)),
           "moegg_selection_read")
    return Selection(s.exemplar, s.size_class, tuple(s.lorenz), s.distance)


def grouped_gemm_contiguous_scheduled(A, B, C, G: int, ws, A_scale=None, B_scale=None, block_m: int = 0,
                                      b_layout: int = B_KN, stream=None, scale_km: bool = False):
    """The contiguous GEMM from the tile list already in ws (see moegg.h).
    scale_km: A_scale is fp32 [K/128, rows] (MOEGG_FP8_E4M3_SCALE_KM)."""
    K = A.shape[1]
    N = B.shape[2] if b_layout == B_KN else B.shape[1]
    _check(lib().moegg_grouped_gemm_contiguous_scheduled(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), G, A.shape[0], K, N, _dtype(A, A_scale, B, scale_km), b_layout,
        block_m, _p(ws), ws.numel(), _stream(stream)), "moegg_grouped_gemm_contiguous_scheduled")


def grouped_gemm_contiguous(A, B, C, m_sizes, ws, A_scale=None, B_scale=None, seg_align: int = 1,
                            block_m: int = 0, b_layout: int = B_KN, stream=None, scale_km: bool = False):
    """C[rows of expert e] = A[rows of expert e] @ B_e (see moegg.h).
    scale_km: A_scale is fp32 [K/128, rows] (MOEGG_FP8_E4M3_SCALE_KM)."""
    K = A.shape[1]
    N = B.shape[2] if b_layout == B_KN else B.shape[1]
    _check(lib().moegg_grouped_gemm_contiguous(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), _p(m_sizes), m_sizes.numel(), A.shape[0], K, N,
        seg_align, _dtype(A, A_scale, B, scale_km), b_layout, block_m, _p(ws), ws.numel(), _stream(stream)),
        "moegg_grouped_gemm_contiguous")


def interleave_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """Gate and up weights [G, I, K] (K-contiguous) -> W1 [G, 2I, K] in the row
    order moegg_grouped_gemm_swiglu_scheduled takes: 16 gate rows, then the 16
    up rows of the same outputs.  A one-time weight transform."""
    G, I, K = w_gate.shape
    if w_up.shape != w_gate.shape or I % 16:
        raise ValueError("gate and up weights [G, I, K] with I % 16 == 0 expected")
    return torch.stack([w_gate.reshape(G, I // 16, 16, K), w_up.reshape(G, I // 16, 16, K)], dim=2) \
        .reshape(G, 2 * I, K).contiguous()


def grouped_gemm_swiglu_scheduled(A, W1, H, G: int, ws, A_scale=None, W1_scale=None, block_m: int = 0,
                                  H_scale=None, stream=None, scale_km: bool = False):
    """H = silu(A W_gate) * (A W_up) per expert, from the tile list in ws (see moegg.h).
    H bf16 [rows, I]; or, with H_scale (fp32 [rows, I/128]), H float8_e4m3fn codes.
    scale_km: A_scale fp32 [K/128, rows] in, H_scale [I/128, rows] out."""
    K = A.shape[1]
    I = W1.shape[1] // 2
    if (H_scale is None) != (H.dtype == torch.bfloat16):
        raise ValueError("H: bf16 without H_scale, float8_e4m3fn with it")
    _check(lib().moegg_grouped_gemm_swiglu_scheduled(
        _p(A), _p(A_scale), _p(W1), _p(W1_scale), _p(H), _p(H_scale), G, A.shape[0], K, I,
        _dtype(A, A_scale, W1, scale_km),
        B_NK, block_m, _p(ws), ws.numel(), _stream(stream)), "moegg_grouped_gemm_swiglu_scheduled")


def grouped_gemm_masked(A, B, C, masked_m, ws=None, A_scale=None, B_scale=None, b_layout: int = B_KN,
                        stream=None, scale_km: bool = False):
    """C[e, r] = A[e, r] @ B_e for r < masked_m[e] (see moegg.h).
    scale_km: A_scale is fp32 [K/128, G * cap] (MOEGG_FP8_E4M3_SCALE_KM)."""
    G, cap, K = A.shape
    N = B.shape[2] if b_layout == B_KN else B.shape[1]
    _check(lib().moegg_grouped_gemm_masked(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), _p(masked_m), G, cap, K, N, _dtype(A, A_scale, B, scale_km), b_layout,
        _p(ws), 0 if ws is None else ws.numel(), _stream(stream)), "moegg_grouped_gemm_masked")


def grouped_gemm_k_grouped(X, dY, dW, t_sizes, ws, stream=None):
    """dW[e] = X_e^T @ dY_e over expert e's rows (see moegg.h)."""
    T, Mw = X.shape
    Nw = dY.shape[1]
    _check(lib().moegg_grouped_gemm_k_grouped(
        _p(X), _p(dY), _p(dW), _p(t_sizes), t_sizes.numel(), T, Mw, Nw, _p(ws), ws.numel(), _stream(stream)),
        "moegg_grouped_gemm_k_grouped")


def stats_read(ws: torch.Tensor, stream=None) -> Stats:
    s = _Stats()
    _check(lib().moegg_stats_read(_p(ws), ctypes.byref(s), _stream(stream)), "moegg_stats_read")
    return Stats(s.U, s.P_exec, s.tiles, s.active, s.sum_sq, s.capacity_rows,
                 {q: int(s.P_at[i]) for i, q in enumerate(Q_VALUES)}, s.block_m, s.error_flags)


def tile_list_read(ws: torch.Tensor, cap_tiles: int, stream=None) -> List[Tuple[int, int, int, int]]:
    buf = (_Tile * max(1, cap_tiles))()
    n = _I64(0)
    _check(lib().moegg_tile_list_read(_p(ws), buf, cap_tiles, ctypes.byref(n), _stream(stream)),
           "moegg_tile_list_read")
    return [(buf[i].expert, buf[i].tile, buf[i].row_start, buf[i].rows_valid) for i in range(min(n.value, cap_tiles))]
