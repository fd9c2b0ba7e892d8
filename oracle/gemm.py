"""ctypes front end of the fp64 C oracle (test infrastructure only).

The C source, oracle.c, sits beside this file.  `build()` compiles it with
gcc into liboracle.so.  The wrappers take CPU torch tensors holding the same
bf16 / e4m3 bit patterns the GPU receives, and return float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP8 = 0, 1
B_KN, B_NK = 0, 1


def build() -> str:
    """Compile oracle.c (plain C, OpenMP, fp64, no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.oracle_dec_bf16.restype = ctypes.c_double
        L.oracle_dec_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_dec_e4m3.restype = ctypes.c_double
        L.oracle_dec_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_contiguous.restype = i32
        L.oracle_contiguous.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, vp, i64, vp]
        L.oracle_masked.restype = i32
        L.oracle_masked.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i64, vp]
        L.oracle_k_grouped.restype = i32
        L.oracle_k_grouped.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp, i64, vp]
        L.oracle_k_grouped_fp8.restype = i32
        L.oracle_k_grouped_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i64, vp, vp, i64, vp]
        L.oracle_threads.restype = i32
        _lib = L
    return _lib


def threads() -> int:
    return lib().oracle_threads()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8
    raise TypeError(f"oracle takes bf16 or float8_e4m3fn operands, not {t.dtype}")


def contiguous(A, B, counts: Sequence[int], rows: Sequence[int], seg_align: int = 1,
               A_scale=None, B_scale=None, b_layout: int = B_KN) -> np.ndarray:
    """Rows `rows` of C for the M-grouped contiguous layout (NaN rows = no expert)."""
    A, B = A.contiguous(), B.contiguous()
    K = A.shape[1]
    N = B.shape[2] if b_layout == B_KN else B.shape[1]
    m = torch.tensor(list(counts), dtype=torch.int32)
    r = torch.tensor(list(rows), dtype=torch.int64)
    out = np.empty((len(rows), N), dtype=np.float64)
    rc = lib().oracle_contiguous(_dtype_code(A), b_layout, _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale),
                                 _ptr(m), len(counts), A.shape[0], K, N, seg_align, _ptr(r), len(rows),
                                 ctypes.c_void_p(out.ctypes.data))
    if rc != 0:
        raise ValueError("oracle_contiguous rejected its arguments")
    return out


def masked(A, B, masked_m: Sequence[int], experts: Sequence[int], rs: Sequence[int],
           A_scale=None, B_scale=None, b_layout: int = B_KN) -> np.ndarray:
    """Rows C[e, r, :] of the masked layout for each (e, r) request."""
    A, B = A.contiguous(), B.contiguous()
    G, cap, K = A.shape
    N = B.shape[2] if b_layout == B_KN else B.shape[1]
    m = torch.tensor(list(masked_m), dtype=torch.int32)
    e = torch.tensor(list(experts), dtype=torch.int32)
    r = torch.tensor(list(rs), dtype=torch.int32)
    out = np.empty((len(e), N), dtype=np.float64)
    rc = lib().oracle_masked(_dtype_code(A), b_layout, _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale),
                             _ptr(m), G, cap, K, N, _ptr(e), _ptr(r), len(e),
                             ctypes.c_void_p(out.ctypes.data))
    if rc != 0:
        raise ValueError("oracle_masked rejected its arguments")
    return out


def k_grouped(X, dY, t_sizes: Sequence[int], experts: Sequence[int], is_: Sequence[int]) -> np.ndarray:
    """Rows dW[e, i, :] of the K-grouped weight gradient for each (e, i) request."""
    X, dY = X.contiguous(), dY.contiguous()
    assert X.dtype == torch.bfloat16 and dY.dtype == torch.bfloat16
    T, Mw = X.shape
    Nw = dY.shape[1]
    t = torch.tensor(list(t_sizes), dtype=torch.int32)
    e = torch.tensor(list(experts), dtype=torch.int32)
    i = torch.tensor(list(is_), dtype=torch.int32)
    out = np.empty((len(e), Nw), dtype=np.float64)
    rc = lib().oracle_k_grouped(_ptr(X), _ptr(dY), _ptr(t), len(t_sizes), T, Mw, Nw, _ptr(e), _ptr(i),
                                len(e), ctypes.c_void_p(out.ctypes.data))
    if rc != 0:
        raise ValueError("oracle_k_grouped rejected its arguments")
    return out


def k_grouped_fp8(X, X_scale, dY, dY_scale, t_sizes: Sequence[int], experts: Sequence[int],
                  is_: Sequence[int]) -> np.ndarray:
    """Rows dW[e, i, :] of the K-grouped weight gradient on e4m3 operands with
    fp32 scales per 128-row group of each expert's segment (see oracle.c):
    X e4m3 [T, Mw], X_scale fp32 [n_groups, Mw], dY e4m3 [T, Nw], dY_scale fp32
    [n_groups, Nw]."""
    X, dY = X.contiguous(), dY.contiguous()
    assert X.dtype == torch.float8_e4m3fn and dY.dtype == torch.float8_e4m3fn
    Xs, dYs = X_scale.float().contiguous(), dY_scale.float().contiguous()
    T, Mw = X.shape
    Nw = dY.shape[1]
    assert Xs.shape[0] == dYs.shape[0] and Xs.shape[1] == Mw and dYs.shape[1] == Nw
    t = torch.tensor(list(t_sizes), dtype=torch.int32)
    e = torch.tensor(list(experts), dtype=torch.int32)
    i = torch.tensor(list(is_), dtype=torch.int32)
    out = np.empty((len(e), Nw), dtype=np.float64)
    rc = lib().oracle_k_grouped_fp8(_ptr(X), _ptr(Xs), _ptr(dY), _ptr(dYs), _ptr(t), len(t_sizes), T, Mw, Nw,
                                    Xs.shape[0], _ptr(e), _ptr(i), len(e), ctypes.c_void_p(out.ctypes.data))
    if rc != 0:
        raise ValueError("oracle_k_grouped_fp8 rejected its arguments")
    return out


def dec_bf16(bits: int) -> float:
    return lib().oracle_dec_bf16(bits)


def dec_e4m3(code: int) -> float:
    return lib().oracle_dec_e4m3(code)


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F over the given (valid) entries, in fp64.

    With ||ref|| = 0 the error is 0 if got is exactly 0 everywhere, else inf.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    den = float(np.sqrt(np.sum(ref ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
