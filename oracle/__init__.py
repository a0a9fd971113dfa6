"""CPU oracle for the FP8 block-scaled GEMM (numpy front end of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package; the library path never does.  It shares no code with the HIP
implementation.  What each function computes, and the passages it follows, is stated in
``oracle.c``'s header:  D = bf16_rne( sum_kb sa*sb * exact fp64 block dot product ).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain C11 + OpenMP) into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_bits.restype = ctypes.c_uint16
        lib.oracle_bf16_bits.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_code.restype = ctypes.c_uint8
        lib.oracle_e4m3_code.argtypes = [ctypes.c_double]
        lib.oracle_quantize_1x128.restype = ctypes.c_int
        lib.oracle_quantize_1x128.argtypes = [P, I64, I64, P, P, ctypes.c_int]
        lib.oracle_swiglu_quantize_1x128.argtypes = [P, I64, I64, P, P, P, ctypes.c_int]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_grouped_masked_fp4.restype = ctypes.c_int
        lib.oracle_grouped_masked_fp4.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64,
                                                  P, P, P, ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_gemm_nt.restype = ctypes.c_int
        lib.oracle_gemm_nt.argtypes = [P, P, P, P, I64, I64, I64, P, P, ctypes.c_int]
        lib.oracle_grouped_contiguous.restype = ctypes.c_int
        lib.oracle_grouped_contiguous.argtypes = [P, P, P, P, P, I64, I64, I64, ctypes.c_int32,
                                                  P, P, P, ctypes.c_int]
        lib.oracle_grouped_masked.restype = ctypes.c_int
        lib.oracle_grouped_masked.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64,
                                              P, P, P, ctypes.c_int]
        lib.oracle_elements.restype = ctypes.c_int
        lib.oracle_elements.argtypes = [P, P, P, P, I64, P, P, P, I64, P, P, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def num_threads(nthreads: int = 0) -> int:
    return _load().oracle_num_threads(nthreads)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def bf16_bits(x: float) -> int:
    return _load().oracle_bf16_bits(float(x))


def e4m3_code(x: float) -> int:
    return _load().oracle_e4m3_code(float(x))


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gemm_nt(A, sa, B, sb, with_acc: bool = False, nthreads: int = 0):
    """Dense: A uint8 [M,K], sa f32 [M,ceil(K/128)], B uint8 [N,K], sb f32 [ceil(N/128),ceil(K/128)].
    Returns D as bf16 bits (uint16 [M,N]) and, if asked, the fp64 values before rounding."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    M, K = A.shape
    N = B.shape[0]
    nkb = -(-K // 128)
    assert B.shape == (N, K) and sa.shape == (M, nkb) and sb.shape == (-(-N // 128), nkb)
    D = np.empty((M, N), dtype=np.uint16)
    acc = np.empty((M, N), dtype=np.float64) if with_acc else None
    rc = _load().oracle_gemm_nt(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), M, N, K, _ptr(D),
                                _ptr(acc), nthreads)
    if rc:
        raise MemoryError("oracle_gemm_nt")
    return (D, acc) if with_acc else D


def grouped_contiguous(A, sa, B, sb, m_indices, with_acc: bool = False, nthreads: int = 0):
    """Contiguous MoE layout.  Returns (D bits [M,N], valid uint8 [M]) (+ fp64 values)."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    m_indices = _c(m_indices, np.int32)
    M, K = A.shape
    G, N, K2 = B.shape
    assert K2 == K and m_indices.shape == (M,)
    D = np.empty((M, N), dtype=np.uint16)
    valid = np.empty((M,), dtype=np.uint8)
    acc = np.empty((M, N), dtype=np.float64) if with_acc else None
    rc = _load().oracle_grouped_contiguous(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(m_indices),
                                           M, N, K, G, _ptr(D), _ptr(valid), _ptr(acc), nthreads)
    if rc:
        raise MemoryError("oracle_grouped_contiguous")
    return (D, valid, acc) if with_acc else (D, valid)


def grouped_masked(A, sa, B, sb, masked_m, with_acc: bool = False, nthreads: int = 0):
    """Masked MoE layout: A [G,M_max,K].  Returns (D bits [G,M_max,N], valid [G,M_max])."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    masked_m = _c(masked_m, np.int32)
    G, M_max, K = A.shape
    G2, N, K2 = B.shape
    assert G2 == G and K2 == K and masked_m.shape == (G,)
    D = np.empty((G, M_max, N), dtype=np.uint16)
    valid = np.empty((G, M_max), dtype=np.uint8)
    acc = np.empty((G, M_max, N), dtype=np.float64) if with_acc else None
    rc = _load().oracle_grouped_masked(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(masked_m), G,
                                       M_max, N, K, _ptr(D), _ptr(valid), _ptr(acc), nthreads)
    if rc:
        raise MemoryError("oracle_grouped_masked")
    return (D, valid, acc) if with_acc else (D, valid)


def elements(A, sa, B, sb, a_rows, b_rows, sb_rows, with_acc: bool = False, nthreads: int = 0):
    """Selected outputs of a (possibly grouped) problem.  A/sa are viewed as [rows, K] and
    [rows, ceil(K/128)], B/sb flattened over groups ([G*N, K], [G*ceil(N/128), ceil(K/128)]).
    Sample i uses A row a_rows[i], B row b_rows[i] and sb row sb_rows[i]."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    K = A.shape[-1]
    a_rows = _c(np.asarray(a_rows, dtype=np.int64), np.int64)
    b_rows = _c(np.asarray(b_rows, dtype=np.int64), np.int64)
    sb_rows = _c(np.asarray(sb_rows, dtype=np.int64), np.int64)
    n = a_rows.shape[0]
    assert b_rows.shape == (n,) and sb_rows.shape == (n,)
    assert a_rows.size == 0 or (a_rows.min() >= 0 and a_rows.max() < A.size // K)
    assert b_rows.size == 0 or (b_rows.min() >= 0 and b_rows.max() < B.size // K)
    assert sb_rows.size == 0 or (sb_rows.min() >= 0 and sb_rows.max() < sb.size // (-(-K // 128)))
    out = np.empty((n,), dtype=np.uint16)
    acc = np.empty((n,), dtype=np.float64) if with_acc else None
    rc = _load().oracle_elements(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), K, _ptr(a_rows),
                                 _ptr(b_rows), _ptr(sb_rows), n, _ptr(out), _ptr(acc), nthreads)
    if rc:
        raise MemoryError("oracle_elements")
    return (out, acc) if with_acc else out


def quantize_1x128(X_bits, nthreads: int = 0):
    """Activation quantiser: X bf16 bit patterns (uint16 [M,K]) -> (codes uint8 [M,K],
    sa float32 [M, ceil(K/128)]), one scale per 1x128 block (definition in ``oracle.c``)."""
    X = _c(X_bits, np.uint16)
    M, K = X.shape
    codes = np.empty((M, K), dtype=np.uint8)
    sa = np.empty((M, -(-K // 128)), dtype=np.float32)
    _load().oracle_quantize_1x128(_ptr(X), M, K, _ptr(codes), _ptr(sa), nthreads)
    return codes, sa


def swiglu_quantize_1x128(X_bits, nthreads: int = 0):
    """SwiGLU + requantisation: X bf16 bit patterns (uint16 [M, 2I], gate | up) -> (codes uint8
    [M, I], sa float32 [M, ceil(I/128)], h float64 [M, I]) with h = silu(gate) * up (definition
    in ``oracle.c``)."""
    X = _c(X_bits, np.uint16)
    M, I2 = X.shape
    assert I2 % 2 == 0
    I = I2 // 2
    codes = np.empty((M, I), dtype=np.uint8)
    sa = np.empty((M, -(-I // 128)), dtype=np.float32)
    h = np.empty((M, I), dtype=np.float64)
    _load().oracle_swiglu_quantize_1x128(_ptr(X), M, I, _ptr(codes), _ptr(sa), _ptr(h), nthreads)
    return codes, sa, h


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e8m0_value(s: int) -> float:
    return _load().oracle_e8m0_value(int(s))


def grouped_masked_fp4(A, sa, B, sb, masked_m, with_acc: bool = False, nthreads: int = 0):
    """Masked layout with an E2M1 right operand: A uint8 [G,M_max,K] (E4M3), sa float32
    [G,M_max,K/128], B uint8 [G,N,K/2] (two E2M1 codes per byte, even element low), sb uint8
    [G,N,K/32] (E8M0), masked_m int32 [G] -> (D bf16 bits [G,M_max,N], valid [G,M_max])."""
    A, sa, B = _c(A, np.uint8), _c(sa, np.float32), _c(B, np.uint8)
    sb, mm = _c(sb, np.uint8), _c(masked_m, np.int32)
    G, M_max, K = A.shape
    N = B.shape[1]
    assert B.shape == (G, N, K // 2) and sb.shape == (G, N, K // 32) and K % 32 == 0
    assert sa.shape == (G, M_max, -(-K // 128)) and mm.shape == (G,)
    D = np.empty((G, M_max, N), dtype=np.uint16)
    valid = np.empty((G, M_max), dtype=np.uint8)
    acc = np.empty((G, M_max, N), dtype=np.float64) if with_acc else None
    rc = _load().oracle_grouped_masked_fp4(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(mm), G, M_max, N, K,
                                           _ptr(D), _ptr(valid), _ptr(acc), nthreads)
    if rc:
        raise MemoryError("oracle_grouped_masked_fp4")
    return (D, valid, acc) if with_acc else (D, valid)
