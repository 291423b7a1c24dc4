"""CPU oracle for the FP8-blk dense linear -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package. The HIP library never does, and the
two share no source: the oracle is plain C (``fp8blk_oracle.c`` for the FP8-blk
dense linear, ``fp4_expert_oracle.c`` for the native expert arm) built with
gcc, called here through ctypes with numpy arrays.

Functions and the passages they follow are documented in the C files:
  e4m3 / e8m0 / bf16 decode (O1, O2), bf16 exactness (O3), load check (O4),
  dequant slab (O5), double-precision GEMV (O6), documented-order f32 GEMV (O7);
  e2m1 decode (O8), FP4 element value (O9), FP4 load check (O10), FP4 bf16
  slab (O11), act_quant (O12), native expert GEMV in double (O13).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "fp8blk_oracle.c"), os.path.join(HERE, "fp4_expert_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")

OK, ARG, SCALE_FF, NAN_CODE, INEXACT, BAD_SCALE = 0, 1, 2, 3, 4, 7
MXFP4, NVFP4 = 0, 1
FP4_BLOCK = {MXFP4: 32, NVFP4: 16}

GCC_CMD = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-pthread", "-Wall", "-Wextra", "-o", LIB, *SRCS, "-lm"]


def build() -> str:
    """Compile the oracle with gcc (no contraction of a*b+c, no fast-math)."""
    subprocess.run(GCC_CMD, check=True)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or any(os.path.getmtime(LIB) < os.path.getmtime(f) for f in SRCS):
            build()
        L = ctypes.CDLL(LIB)
        u8p, u16p = ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint16)
        f32p, f64p = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)
        i64, i64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)
        L.orc_e4m3.argtypes = [ctypes.c_uint8, f64p]
        L.orc_e8m0.argtypes = [ctypes.c_uint8, f64p]
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_bf16.restype = ctypes.c_double
        L.orc_is_bf16_exact.argtypes = [ctypes.c_double]
        L.orc_load_check.argtypes = [u8p, u8p, i64, i64, f32p, i64p]
        L.orc_dequant_bf16.argtypes = [u8p, u8p, i64, i64, u16p, i64p]
        L.orc_gemv_f64.argtypes = [u8p, u8p, i64, i64, u16p, i64, f64p, f64p, ctypes.c_int]
        L.orc_gemv_f64.restype = None
        L.orc_gemv_f32_order.argtypes = [ctypes.c_int, u8p, u8p, u16p, i64, i64, u16p, i64,
                                         ctypes.c_int, f32p, ctypes.c_int]
        L.orc_e2m1.argtypes = [ctypes.c_int]
        L.orc_e2m1.restype = ctypes.c_double
        L.orc_fp4_element.argtypes = [ctypes.c_int, u8p, u8p, i64, i64, i64, f64p]
        L.orc_fp4_load_check.argtypes = [ctypes.c_int, u8p, u8p, i64, i64, i64p]
        L.orc_fp4_dequant_bf16.argtypes = [ctypes.c_int, u8p, u8p, i64, i64, u16p, i64p]
        L.orc_act_quant.argtypes = [u16p, i64, i64, u8p, u8p]
        L.orc_fp4_gemv_f64.argtypes = [ctypes.c_int, u8p, u8p, ctypes.c_double, i64, i64, u8p, u8p, i64,
                                       f64p, f64p, ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray | None, ct):
    if a is None:
        return ctypes.POINTER(ct)()
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ct))


def e4m3(code: int) -> float | None:
    """O1: value of one e4m3 byte, None for NaN."""
    v = ctypes.c_double()
    return v.value if lib().orc_e4m3(code, ctypes.byref(v)) else None


def e8m0(code: int) -> float | None:
    """O2: value of one e8m0 byte, None for the refused 0xFF."""
    v = ctypes.c_double()
    return v.value if lib().orc_e8m0(code, ctypes.byref(v)) else None


def bf16(bits: int) -> float:
    return lib().orc_bf16(bits)


def is_bf16_exact(v: float) -> bool:
    """O3."""
    return bool(lib().orc_is_bf16_exact(v))


def load_check(codes: np.ndarray, scales: np.ndarray):
    """O4: (status, first_bad, f32 grid). first_bad is -1 on success."""
    rows, cols = codes.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    grid = np.zeros(scales.shape, dtype=np.float32)
    fb = ctypes.c_int64(-1)
    st = lib().orc_load_check(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                              _p(grid, ctypes.c_float), ctypes.byref(fb))
    return st, fb.value, grid


def dequant_bf16(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """O5: uint16 bf16 slab [rows, cols]; raises on an inexact element."""
    rows, cols = codes.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.zeros((rows, cols), dtype=np.uint16)
    fb = ctypes.c_int64(-1)
    st = lib().orc_dequant_bf16(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                                _p(out, ctypes.c_uint16), ctypes.byref(fb))
    if st != OK:
        raise ValueError(f"dequant refused: status {st} at element {fb.value}")
    return out


def gemv_f64(codes: np.ndarray, scales: np.ndarray, x: np.ndarray, nthreads: int | None = None):
    """O6: (y, yabs) as float64 [M, rows]."""
    rows, cols = codes.shape
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    M = x.shape[0]
    assert x.shape[1] == cols
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.zeros((M, rows), dtype=np.float64)
    ya = np.zeros((M, rows), dtype=np.float64)
    lib().orc_gemv_f64(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                       _p(x, ctypes.c_uint16), M, _p(y, ctypes.c_double), _p(ya, ctypes.c_double),
                       nthreads or os.cpu_count() or 1)
    return y, ya


def gemv_f32_order(x: np.ndarray, *, codes: np.ndarray | None = None,
                   scales: np.ndarray | None = None, w_bf16: np.ndarray | None = None,
                   variant: int = 0, nthreads: int | None = None) -> np.ndarray:
    """O7: float32 [M, rows] in the documented order. Give codes+scales for the
    in-register decode (B) or w_bf16 for the bf16 slab (A)."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    M = x.shape[0]
    if w_bf16 is not None:
        wsrc = 0
        w_bf16 = np.ascontiguousarray(w_bf16, dtype=np.uint16)
        rows, cols = w_bf16.shape
    else:
        wsrc = 1
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        rows, cols = codes.shape
    assert x.shape[1] == cols
    y = np.zeros((M, rows), dtype=np.float32)
    st = lib().orc_gemv_f32_order(wsrc, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8),
                                  _p(w_bf16, ctypes.c_uint16), rows, cols, _p(x, ctypes.c_uint16),
                                  M, variant, _p(y, ctypes.c_float), nthreads or os.cpu_count() or 1)
    if st != OK:
        raise ValueError(f"gemv_f32_order: status {st}")
    return y


# --- native expert arm (fp4_expert_oracle.c) --------------------------------

def e2m1(code: int) -> float:
    """O8: value of one e2m1 code (low 4 bits)."""
    return lib().orc_e2m1(code)


def _fp4_args(fmt: int, codes: np.ndarray, scales: np.ndarray):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    assert scales.shape == (rows, cols // FP4_BLOCK[fmt]), (scales.shape, rows, cols)
    return codes, scales, rows, cols


def fp4_element(fmt: int, codes: np.ndarray, scales: np.ndarray, r: int, c: int) -> float | None:
    """O9: exact value of element (r, c); None for a refused scale."""
    codes, scales, rows, cols = _fp4_args(fmt, codes, scales)
    v = ctypes.c_double()
    ok = lib().orc_fp4_element(fmt, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), cols, r, c,
                               ctypes.byref(v))
    return v.value if ok else None


def fp4_load_check(fmt: int, codes: np.ndarray, scales: np.ndarray):
    """O10: (status, first_bad); first_bad is -1 on success."""
    codes, scales, rows, cols = _fp4_args(fmt, codes, scales)
    fb = ctypes.c_int64(-1)
    st = lib().orc_fp4_load_check(fmt, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                                  ctypes.byref(fb))
    return st, fb.value


def fp4_dequant_bf16(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """O11: uint16 bf16 slab [rows, cols]; raises on a refused or inexact element."""
    codes, scales, rows, cols = _fp4_args(fmt, codes, scales)
    out = np.zeros((rows, cols), dtype=np.uint16)
    fb = ctypes.c_int64(-1)
    st = lib().orc_fp4_dequant_bf16(fmt, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                                    _p(out, ctypes.c_uint16), ctypes.byref(fb))
    if st != OK:
        raise ValueError(f"fp4 dequant refused: status {st} at element {fb.value}")
    return out


def act_quant(x: np.ndarray):
    """O12: (codes uint8 [M, cols], e8m0 scale codes uint8 [M, ceil(cols/128)])."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    M, cols = x.shape
    codes = np.zeros((M, cols), dtype=np.uint8)
    scales = np.zeros((M, (cols + 127) // 128), dtype=np.uint8)
    st = lib().orc_act_quant(_p(x, ctypes.c_uint16), M, cols, _p(codes, ctypes.c_uint8),
                             _p(scales, ctypes.c_uint8))
    if st != OK:
        raise ValueError(f"act_quant: status {st}")
    return codes, scales


def fp4_gemv_f64(fmt: int, codes: np.ndarray, scales: np.ndarray, xq: np.ndarray, xs: np.ndarray,
                 global_scale: float = 1.0, nthreads: int | None = None):
    """O13: (y, yabs) as float64 [M, rows]."""
    codes, scales, rows, cols = _fp4_args(fmt, codes, scales)
    xq = np.ascontiguousarray(np.atleast_2d(xq), dtype=np.uint8)
    xs = np.ascontiguousarray(np.atleast_2d(xs), dtype=np.uint8)
    M = xq.shape[0]
    assert xq.shape == (M, cols) and xs.shape == (M, (cols + 127) // 128)
    y = np.zeros((M, rows), dtype=np.float64)
    ya = np.zeros((M, rows), dtype=np.float64)
    st = lib().orc_fp4_gemv_f64(fmt, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), float(global_scale),
                                rows, cols, _p(xq, ctypes.c_uint8), _p(xs, ctypes.c_uint8), M,
                                _p(y, ctypes.c_double), _p(ya, ctypes.c_double), nthreads or os.cpu_count() or 1)
    if st != OK:
        raise ValueError(f"fp4_gemv_f64: status {st}")
    return y, ya
