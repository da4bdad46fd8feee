"""ctypes loader of ``mx_fast.c`` -- TEST INFRASTRUCTURE ONLY (oracle).

The oracle's MXFP8 rule (reading R7 of ``moe_oracle.py``) for bf16 rows,
in plain C with OpenMP over rows, for tensors too large for the numpy
implementation (the full-size weight matrices).  Pinned bit for bit against
``moe_oracle.mx_quantize_blocks`` in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mx_fast.c")
LIB = os.path.join(_HERE, "libmx_fast.so")
_lib = None
_lock = threading.Lock()


def build() -> str:
    """Compile libmx_fast.so next to the source (gcc, OpenMP)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if (not os.path.exists(LIB) or
                    os.path.getmtime(LIB) < os.path.getmtime(SRC)):
                build()
            lib = ctypes.CDLL(LIB)
            lib.mx_fast_rows_bf16.argtypes = [
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.mx_fast_rows_bf16.restype = None
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def quantize_rows(bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 bit patterns [R, C] (C % 32 == 0) -> (codes u8 [R, C], scales u8
    [R, C/32]): moe_oracle.mxfp8_quantize_rows for bf16 input."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    R, C = b.shape
    if C % 32:
        raise ValueError("cols must be a multiple of 32")
    codes = np.empty((R, C), dtype=np.uint8)
    scales = np.empty((R, C // 32), dtype=np.uint8)
    _load().mx_fast_rows_bf16(_ptr(b), R, C, _ptr(codes), _ptr(scales), None)
    return codes, scales


def dequantized_rows(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [R, C] -> float64 decode(code) * 2^s, i.e.
    moe_oracle._mx_rows (the value an MXFP8 GEMM consumes)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    R, C = b.shape
    if C % 32:
        raise ValueError("cols must be a multiple of 32")
    out = np.empty((R, C), dtype=np.float64)
    _load().mx_fast_rows_bf16(_ptr(b), R, C, None, None, _ptr(out))
    return out
