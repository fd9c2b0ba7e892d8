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
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegg.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moegg.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, FP8_E4M3, FP8_E4M3_E8M0, FP8_E4M3_FP4_E2M1, FP8_E4M3_SCALE_KM = 0, 1, 2, 3, 4
B_KN, B_NK, B_KN_PANEL, B_NK_PANEL = 0, 1, 2, 3
PANEL_CONTIGUOUS, PANEL_MASKED = 256, 128     # panel width P of the contiguous / SwiGLU and the masked calls
FLAG_NEGATIVE_COUNT, FLAG_ROWS_OVERFLOW, FLAG_COUNT_OVER_CAP, FLAG_BAD_EXEMPLAR = 0x1, 0x2, 0x4, 0x8
FLAG_SCALE_GROUPS = 0x10
FLAG_SYNC_TIMEOUT = 0x20
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


class _Report(ctypes.Structure):
    _fields_ = [("effective_experts", ctypes.c_double), ("padding_fraction", ctypes.c_double * 6),
                ("useful_share", ctypes.c_double * 6), ("exec_padding_fraction", ctypes.c_double),
                ("physical_over_effective", ctypes.c_double)]


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

    def report(self) -> "Report":
        """The derived ratios, computed by the library (moegg_stats_report)."""
        st = _Stats(self.U, self.P_exec, self.tiles, self.active, self.sum_sq, self.capacity_rows,
                    (ctypes.c_int64 * 6)(*[self.P_at[q] for q in Q_VALUES]), self.block_m, self.error_flags)
        r = _Report()
        _check(lib().moegg_stats_report(ctypes.byref(st), ctypes.byref(r)), "moegg_stats_report")
        return Report(r.effective_experts, {q: r.padding_fraction[i] for i, q in enumerate(Q_VALUES)},
                      {q: r.useful_share[i] for i, q in enumerate(Q_VALUES)}, r.exec_padding_fraction,
                      r.physical_over_effective)

    @property
    def effective_experts(self) -> float:
        return self.report().effective_experts

    def padding_fraction(self, q: int) -> float:
        return self.report().padding_fraction[q]


@dataclass
class Report:
    """Ratios derived from Stats by the library: effective experts U^2 / sum m^2,
    padding fraction (P(q) - U) / P(q), useful share U / P(q), the executed rows'
    padding fraction and physical / effective work."""
    effective_experts: float
    padding_fraction: dict
    useful_share: dict
    exec_padding_fraction: float
    physical_over_effective: float


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
    "moegg_grouped_gemm_contiguous_noalloc": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                                     _I32, _I32, _I32, _VP]),
    "moegg_grouped_gemm_swiglu_scheduled": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                                   _I32, _I32, _VP, _SZ, _VP]),
    "moegg_expert_mlp_fused": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32,
                                      _I32, _I32, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_grouped_gemm_masked": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32,
                                         _VP, _SZ, _VP]),
    "moegg_grouped_gemm_k_grouped": (_I32, [_VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _VP, _SZ, _VP]),
    "moegg_grouped_gemm_k_grouped_fp8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I64,
                                                _VP, _SZ, _VP]),
    "moegg_grouped_gemm_k_grouped_e8m0": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I64,
                                                 _VP, _SZ, _VP]),
    "moegg_stats_read": (_I32, [_VP, ctypes.POINTER(_Stats), _VP]),
    "moegg_stats_report": (_I32, [ctypes.POINTER(_Stats), ctypes.POINTER(_Report)]),
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


_E4M3 = torch.float8_e4m3fn


def _need(t: Optional[torch.Tensor], name: str, shape: Sequence[Optional[int]], dtypes):
    """ValueError unless `t` is a tensor of this shape (None matches any extent) and one of `dtypes`.
    The library sees only pointers, so every extent it will index is checked here."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: tensor expected")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.dim() != len(shape) or any(x is not None and d != x for d, x in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if x is None else str(x) for x in shape) + "]"
        raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")


def _none(t, name: str, why: str):
    if t is not None:
        raise ValueError(f"{name}: must be None {why}")


def _one_device(*ts):
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(str(d) for d in devs)}")


def _ws(ws, G: int, max_rows: int):
    _need(ws, "ws", [None], (torch.uint8,))
    # the library checks the byte count too; this names the problem
    need = workspace_bytes(G, max_rows)
    if ws.numel() < need:
        raise ValueError(f"ws: {ws.numel()} bytes, need {need} (workspace_bytes({G}, {max_rows}))")


def _counts(t, name: str, G: Optional[int] = None):
    _need(t, name, [G], (torch.int32,))
    if t.numel() < 1:
        raise ValueError(f"{name}: at least one expert expected")


def pack_panels(B: torch.Tensor, b_layout: int, P: int) -> torch.Tensor:
    """Weights [G, K, N] -> the paneled layout the kernels stream (include/moegg.h):
    B_KN_PANEL [G, N/P, K, P]; B_NK_PANEL [G, N/P, K/S, P, S] with S = 128 bytes of
    K.  Packed E2M1 weights (uint8) come as they are stored, [G, N, K/2], and go to
    B_NK_PANEL [G, N/P, K/128, P, 64].  P: PANEL_CONTIGUOUS for the contiguous and
    SwiGLU calls, PANEL_MASKED for the masked call.  A one-time weight transform."""
    if B.dtype == torch.uint8:
        if b_layout != B_NK_PANEL:
            raise ValueError("packed E2M1 weights have the B_NK_PANEL panel layout only")
        G, N, KB = B.shape
        if N % P or KB % 64:
            raise ValueError(f"[G, N, K/2] = {list(B.shape)}: N % {P} and K/2 % 64 must be 0")
        return B.reshape(G, N // P, P, KB // 64, 64).permute(0, 1, 3, 2, 4).contiguous()
    G, K, N = B.shape
    if N % P:
        raise ValueError(f"N = {N} is not a multiple of the panel width {P}")
    if b_layout == B_KN_PANEL:
        return B.reshape(G, K, N // P, P).permute(0, 2, 1, 3).contiguous()
    if b_layout == B_NK_PANEL:
        S = 128 // B.element_size()
        if K % S:
            raise ValueError(f"K = {K} is not a multiple of {S}")
        return B.reshape(G, K // S, S, N // P, P).permute(0, 3, 1, 4, 2).contiguous()
    raise ValueError(f"b_layout {b_layout} is not a panel layout")


def _weight_n(B, K: int, G: int, b_layout: int, P: int, dtypes) -> int:
    """N of weights B in layout b_layout, after checking B's shape against K and G."""
    if b_layout == B_KN:
        _need(B, "B", [G, K, None], dtypes)
        return B.shape[2]
    if b_layout == B_NK:
        _need(B, "B", [G, None, K], dtypes)
        return B.shape[1]
    if b_layout == B_KN_PANEL:
        _need(B, "B", [G, None, K, P], dtypes)
        return B.shape[1] * P
    if b_layout == B_NK_PANEL:
        S = 128 // B.element_size()
        _need(B, "B", [G, None, K // S, P, S], dtypes)
        if K % S:
            raise ValueError(f"K = {K}: the panel layout needs K % {S} == 0")
        return B.shape[1] * P
    raise ValueError(f"b_layout: {b_layout}")


def _operands(rows: int, K: int, A, A_scale, B, B_scale, G: int, b_layout: int, scale_km: bool,
              a_scale_rows_shape=None, P: int = PANEL_CONTIGUOUS) -> Tuple[int, int]:
    """Operand type code and N, after checking B, A_scale and B_scale against A's
    dtype, `rows` rows of K and G experts.  a_scale_rows_shape: the shape of a
    row-major fp32 activation-scale array ([rows, K/128] unless given).
    Formats (include/moegg.h): bf16 x bf16, no scales; e4m3 x e4m3 with fp32
    scales ([rows, K/128], or [K/128, rows] with scale_km) or E8M0 bytes
    ([K/128, rows]); e4m3 x packed E2M1 [G, N, K/2] (uint8) or its panels with E8M0
    bytes."""
    if b_layout not in (B_KN, B_NK, B_KN_PANEL, B_NK_PANEL):
        raise ValueError(f"b_layout: {b_layout}")
    if A.dtype == torch.bfloat16:
        _none(A_scale, "A_scale", "for bf16 operands")
        _none(B_scale, "B_scale", "for bf16 operands")
        if scale_km:
            raise ValueError("scale_km applies to e4m3 operands with fp32 scales")
        return BF16, _weight_n(B, K, G, b_layout, P, (torch.bfloat16,))
    if A.dtype != _E4M3:
        raise ValueError(f"A: bf16 or float8_e4m3fn expected, got {A.dtype}")
    if K % 128:
        raise ValueError(f"K = {K}: e4m3 operands need K % 128 == 0")
    if A_scale is None or B_scale is None:
        raise ValueError("e4m3 operands need A_scale and B_scale")
    if not isinstance(B, torch.Tensor):
        raise ValueError("B: tensor expected")
    if B.dtype == torch.uint8:                              # packed E2M1 weights [G, N, K/2] or its panels
        if b_layout == B_NK:
            N = B.shape[1]
            _need(B, "B", [G, N, K // 2], (torch.uint8,))
        elif b_layout == B_NK_PANEL:
            _need(B, "B", [G, None, K // 128, P, 64], (torch.uint8,))
            N = B.shape[1] * P
        else:
            raise ValueError("packed E2M1 weights are [G, N, K/2] (B_NK) or its panels (B_NK_PANEL)")
        _need(A_scale, "A_scale", [K // 128, rows], (torch.uint8,))
        _need(B_scale, "B_scale", [G, K // 128, N // 128], (torch.uint8,))
        if scale_km:
            raise ValueError("scale_km applies to e4m3 operands with fp32 scales")
        return FP8_E4M3_FP4_E2M1, N
    N = _weight_n(B, K, G, b_layout, P, (_E4M3,))
    if N % 128:
        raise ValueError(f"N = {N}: e4m3 operands need N % 128 == 0")
    if A_scale.dtype == torch.uint8:                        # E8M0 exponent bytes
        if scale_km:
            raise ValueError("scale_km applies to e4m3 operands with fp32 scales")
        _need(A_scale, "A_scale", [K // 128, rows], (torch.uint8,))
        _need(B_scale, "B_scale", [G, K // 128, N // 128], (torch.uint8,))
        return FP8_E4M3_E8M0, N
    if scale_km:
        _need(A_scale, "A_scale", [K // 128, rows], (torch.float32,))
    else:
        _need(A_scale, "A_scale", a_scale_rows_shape or [rows, K // 128], (torch.float32,))
    _need(B_scale, "B_scale", [G, K // 128, N // 128], (torch.float32,))
    return (FP8_E4M3_SCALE_KM if scale_km else FP8_E4M3), N


def workspace_bytes(G: int, max_rows: int) -> int:
    return int(lib().moegg_workspace_bytes(G, max_rows))


def workspace(G: int, max_rows: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(G, max_rows)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.empty(n, dtype=torch.uint8, device=device)


def schedule(m_sizes: torch.Tensor, rows_total: int, ws: torch.Tensor, seg_align: int = 1, block_m: int = 0,
             N: int = 256, stream=None):
    _counts(m_sizes, "m_sizes")
    _ws(ws, m_sizes.numel(), rows_total)
    _one_device(m_sizes, ws)
    _check(lib().moegg_schedule(_p(m_sizes), m_sizes.numel(), rows_total, seg_align, block_m, N, _p(ws),
                                ws.numel(), _stream(stream)), "moegg_schedule")


EXEMPLAR_FIELDS = 10            # moegg_exemplar_t: size_class, lorenz[8], block_m (int32 each)
EXEMPLAR_TABLE_PATH = os.path.join(_HERE, "exemplars_mi355x.json")           # fp8 e4m3, fp32 block scales
EXEMPLAR_TABLE_PATHS = {"fp8": EXEMPLAR_TABLE_PATH, "bf16": os.path.join(_HERE, "exemplars_mi355x_bf16.json")}


def exemplar_table(device="cuda", path: Optional[str] = None, dtype: str = "fp8") -> torch.Tensor:
    """The exemplar table as an int32 [n, 10] device tensor (moegg_exemplar_t rows).
    Default: the table measured on MI355X for the operand type that ships with the
    package (dtype "fp8": e4m3 with fp32 block scales; "bf16")."""
    import json
    if path is None and dtype not in EXEMPLAR_TABLE_PATHS:
        raise ValueError(f"dtype: one of {sorted(EXEMPLAR_TABLE_PATHS)} expected, got {dtype!r}")
    with open(path or EXEMPLAR_TABLE_PATHS[dtype]) as f:
        rows = json.load(f)["exemplars"]
    t = torch.tensor([[r["size_class"], *r["lorenz"], r["block_m"]] for r in rows], dtype=torch.int32)
    return t.to(device)


def schedule_exemplar(m_sizes: torch.Tensor, rows_total: int, ws: torch.Tensor, exemplars: torch.Tensor,
                      hysteresis: int = 0, seg_align: int = 1, N: int = 256, stream=None):
    """moegg_schedule with the tile height matched to an exemplar on the device (see moegg.h)."""
    if exemplars.dtype != torch.int32 or exemplars.dim() != 2 or exemplars.shape[1] != EXEMPLAR_FIELDS:
        raise ValueError("exemplars: int32 [n, 10] expected")
    _counts(m_sizes, "m_sizes")
    _ws(ws, m_sizes.numel(), rows_total)
    _one_device(m_sizes, ws, exemplars)
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
    _need(A, "A", [None, None], (torch.bfloat16, _E4M3))
    rows, K = A.shape
    code, N = _operands(rows, K, A, A_scale, B, B_scale, G, b_layout, scale_km)
    _need(C, "C", [rows, N], (torch.bfloat16,))
    _ws(ws, G, rows)
    _one_device(A, A_scale, B, B_scale, C, ws)
    _check(lib().moegg_grouped_gemm_contiguous_scheduled(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), G, rows, K, N, code, b_layout,
        block_m, _p(ws), ws.numel(), _stream(stream)), "moegg_grouped_gemm_contiguous_scheduled")


def grouped_gemm_contiguous(A, B, C, m_sizes, ws, A_scale=None, B_scale=None, seg_align: int = 1,
                            block_m: int = 0, b_layout: int = B_KN, stream=None, scale_km: bool = False):
    """C[rows of expert e] = A[rows of expert e] @ B_e (see moegg.h).
    scale_km: A_scale is fp32 [K/128, rows] (MOEGG_FP8_E4M3_SCALE_KM)."""
    _counts(m_sizes, "m_sizes")
    G = m_sizes.numel()
    _need(A, "A", [None, None], (torch.bfloat16, _E4M3))
    rows, K = A.shape
    code, N = _operands(rows, K, A, A_scale, B, B_scale, G, b_layout, scale_km)
    _need(C, "C", [rows, N], (torch.bfloat16,))
    _ws(ws, G, rows)
    _one_device(A, A_scale, B, B_scale, C, m_sizes, ws)
    _check(lib().moegg_grouped_gemm_contiguous(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), _p(m_sizes), G, rows, K, N,
        seg_align, code, b_layout, block_m, _p(ws), ws.numel(), _stream(stream)),
        "moegg_grouped_gemm_contiguous")


NOALLOC_SCRATCH_BYTES = 1 << 20          # MOEGG_NOALLOC_SCRATCH_BYTES


def grouped_gemm_contiguous_noalloc(A, B, C, m_sizes, A_scale=None, B_scale=None, seg_align: int = 1,
                                    block_m: int = 0, b_layout: int = B_KN, stream=None, scale_km: bool = False):
    """grouped_gemm_contiguous without a workspace: the library's fixed per-GPU
    scratch array holds the schedule (see moegg.h); nothing is allocated."""
    _counts(m_sizes, "m_sizes")
    G = m_sizes.numel()
    _need(A, "A", [None, None], (torch.bfloat16, _E4M3))
    rows, K = A.shape
    code, N = _operands(rows, K, A, A_scale, B, B_scale, G, b_layout, scale_km)
    _need(C, "C", [rows, N], (torch.bfloat16,))
    _one_device(A, A_scale, B, B_scale, C, m_sizes)
    _check(lib().moegg_grouped_gemm_contiguous_noalloc(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), _p(m_sizes), G, rows, K, N,
        seg_align, code, b_layout, block_m, _stream(stream)), "moegg_grouped_gemm_contiguous_noalloc")


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
                                  H_scale=None, stream=None, scale_km: bool = False, b_layout: int = B_NK):
    """H = silu(A W_gate) * (A W_up) per expert, from the tile list in ws (see moegg.h).
    H bf16 [rows, I]; or, with H_scale (fp32 [rows, I/128]), H float8_e4m3fn codes.
    scale_km: A_scale fp32 [K/128, rows] in, H_scale [I/128, rows] out."""
    _need(A, "A", [None, None], (torch.bfloat16, _E4M3))
    rows, K = A.shape
    if b_layout not in (B_NK, B_NK_PANEL):
        raise ValueError("W1: [G, 2I, K] (B_NK) or its panels (B_NK_PANEL)")
    code, N = _operands(rows, K, A, A_scale, W1, W1_scale, G, b_layout, scale_km)
    if N % 256:
        raise ValueError(f"W1: {N} interleaved gate/up rows, a multiple of 256 expected")
    I = N // 2
    if H_scale is None:
        _need(H, "H", [rows, I], (torch.bfloat16,))
    else:
        _need(H, "H", [rows, I], (_E4M3,))
        _need(H_scale, "H_scale", [I // 128, rows] if scale_km else [rows, I // 128], (torch.float32,))
    _ws(ws, G, rows)
    _one_device(A, A_scale, W1, W1_scale, H, H_scale, ws)
    _check(lib().moegg_grouped_gemm_swiglu_scheduled(
        _p(A), _p(A_scale), _p(W1), _p(W1_scale), _p(H), _p(H_scale), G, rows, K, I, code,
        b_layout, block_m, _p(ws), ws.numel(), _stream(stream)), "moegg_grouped_gemm_swiglu_scheduled")


def expert_mlp_fused(A, W1, W2, H, Y, m_sizes, ws, A_scale, W1_scale, W2_scale, H_scale, seg_align: int = 1,
                     b_layout: int = B_NK, scale_km: bool = False, stream=None):
    """Y = SwiGLU(A W1) W2 per expert in one launch (see moegg.h): e4m3 A [rows, K], W1
    [G, 2I, K] (gate/up interleaved), W2 [G, N2, I], fp32 scales; H e4m3 [rows, I] with H_scale the
    caller's intermediate, written and read back by the kernel; Y bf16 [rows, N2].  b_layout B_NK or
    B_NK_PANEL (P = PANEL_CONTIGUOUS) for both weights; scale_km: A_scale [K/128, rows] in and
    H_scale [I/128, rows]."""
    _need(A, "A", [None, None], (_E4M3,))
    rows, K = A.shape
    if b_layout not in (B_NK, B_NK_PANEL):
        raise ValueError("W1, W2: [G, N, K] (B_NK) or its panels (B_NK_PANEL)")
    _counts(m_sizes, "m_sizes")
    G = m_sizes.numel()
    code, N = _operands(rows, K, A, A_scale, W1, W1_scale, G, b_layout, scale_km)
    if N % 256:
        raise ValueError(f"W1: {N} interleaved gate/up rows, a multiple of 256 expected")
    I = N // 2
    _need(H, "H", [rows, I], (_E4M3,))
    _need(H_scale, "H_scale", [I // 128, rows] if scale_km else [rows, I // 128], (torch.float32,))
    code2, N2 = _operands(rows, I, H, H_scale, W2, W2_scale, G, b_layout, scale_km)
    if code2 != code or N2 % 256:
        raise ValueError(f"W2: e4m3 [G, N2, I] with N2 % 256 == 0 expected, got N2 = {N2}")
    _need(Y, "Y", [rows, N2], (torch.bfloat16,))
    _ws(ws, G, rows)
    _one_device(A, A_scale, W1, W1_scale, W2, W2_scale, H, H_scale, Y, m_sizes, ws)
    _check(lib().moegg_expert_mlp_fused(
        _p(A), _p(A_scale), _p(W1), _p(W1_scale), _p(W2), _p(W2_scale), _p(H), _p(H_scale), _p(Y),
        _p(m_sizes), G, rows, K, I, N2, seg_align, code, b_layout, _p(ws), ws.numel(), _stream(stream)),
        "moegg_expert_mlp_fused")


def grouped_gemm_masked(A, B, C, masked_m, ws=None, A_scale=None, B_scale=None, b_layout: int = B_KN,
                        stream=None, scale_km: bool = False):
    """C[e, r] = A[e, r] @ B_e for r < masked_m[e] (see moegg.h).
    scale_km: A_scale is fp32 [K/128, G * cap] (MOEGG_FP8_E4M3_SCALE_KM)."""
    _need(A, "A", [None, None, None], (torch.bfloat16, _E4M3))
    G, cap, K = A.shape
    _counts(masked_m, "masked_m", G)
    code, N = _operands(G * cap, K, A, A_scale, B, B_scale, G, b_layout, scale_km,
                        a_scale_rows_shape=[G, cap, K // 128], P=PANEL_MASKED)
    _need(C, "C", [G, cap, N], (torch.bfloat16,))
    if ws is not None:
        _ws(ws, G, G * cap)
    _one_device(A, A_scale, B, B_scale, C, masked_m, ws)
    _check(lib().moegg_grouped_gemm_masked(
        _p(A), _p(A_scale), _p(B), _p(B_scale), _p(C), _p(masked_m), G, cap, K, N, code, b_layout,
        _p(ws), 0 if ws is None else ws.numel(), _stream(stream)), "moegg_grouped_gemm_masked")


def k_scale_groups(t_sizes: Sequence[int]) -> int:
    """Rows the K-grouped fp8 scale arrays need: sum over experts of ceil(t_e / 128)."""
    return sum((max(int(t), 0) + 127) // 128 for t in t_sizes)


def grouped_gemm_k_grouped(X, dY, dW, t_sizes, ws, X_scale=None, dY_scale=None, stream=None):
    """dW[e] = X_e^T @ dY_e over expert e's rows (see moegg.h).  bf16 X and dY;
    or e4m3 X and dY with scales X_scale [S, Mw], dY_scale [S, Nw], one row per
    128-row group of each expert's segment (k_scale_groups gives S): fp32, or
    uint8 E8M0 exponent bytes (2^(b - 127))."""
    _counts(t_sizes, "t_sizes")
    G = t_sizes.numel()
    _need(X, "X", [None, None], (torch.bfloat16, _E4M3))
    T, Mw = X.shape
    _need(dY, "dY", [T, None], (X.dtype,))
    Nw = dY.shape[1]
    _need(dW, "dW", [G, Mw, Nw], (torch.float32,))
    _ws(ws, G, 0)
    if X.dtype == torch.bfloat16:
        _none(X_scale, "X_scale", "for bf16 operands")
        _none(dY_scale, "dY_scale", "for bf16 operands")
        _one_device(X, dY, dW, t_sizes, ws)
        _check(lib().moegg_grouped_gemm_k_grouped(
            _p(X), _p(dY), _p(dW), _p(t_sizes), G, T, Mw, Nw, _p(ws), ws.numel(), _stream(stream)),
            "moegg_grouped_gemm_k_grouped")
        return
    _need(X_scale, "X_scale", [None, Mw], (torch.float32, torch.uint8))
    S = X_scale.shape[0]
    _need(dY_scale, "dY_scale", [S, Nw], (X_scale.dtype,))
    _one_device(X, X_scale, dY, dY_scale, dW, t_sizes, ws)
    if X_scale.dtype == torch.uint8:
        _check(lib().moegg_grouped_gemm_k_grouped_e8m0(
            _p(X), _p(X_scale), _p(dY), _p(dY_scale), _p(dW), _p(t_sizes), G, T, Mw, Nw, S, _p(ws), ws.numel(),
            _stream(stream)), "moegg_grouped_gemm_k_grouped_e8m0")
        return
    _check(lib().moegg_grouped_gemm_k_grouped_fp8(
        _p(X), _p(X_scale), _p(dY), _p(dY_scale), _p(dW), _p(t_sizes), G, T, Mw, Nw, S, _p(ws), ws.numel(),
        _stream(stream)), "moegg_grouped_gemm_k_grouped_fp8")


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
