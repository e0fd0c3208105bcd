"""CPU oracle for the non-TN operand GEMM and for attention's P*V product (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
import this package; the product package never does. It shares no code with the HIP
path: the arithmetic lives in ``oracle.c`` (built with gcc into ``liboracle.so``), the
host-side rules below are written out from the pages' text.

Contents and the passage each follows:
  * ``gemm``            -- C = A*B by definition (decode, logical map, fp64 sum, one
                           rounding). Non-TN operands: Triton PR 5223, "Feature
                           description"; int4 weights: BitBLAS PR 268, dequantize example.
  * ``dequant_u4``      -- (q - zero) * s rounded once to binary16.
  * ``decode(.., "f8")`` -- 8-bit E4M3 operands (OCP convention: bias 7, no infinity,
                           one NaN pattern per sign), exact in fp64.
  * ``attention``       -- softmax(scale * Q K^T) V by definition (fp64 scores, exp of the
                           shifted scores, fp64 sums, one division, one rounding): the
                           flash-attention second dot named in Triton PR 5223, "Introduction".
  * ``splitk_factor``   -- BitBLAS PR 268, "SplitK Infer" code block, with ceil grid.
  * ``perm_fwd/perm_inv`` -- rocm-libraries PR 2487, "Add support for permuting perpDim",
                           forward and inverse mapping formulas.

Every function here is pinned by ``tests/test_oracle_pins.py`` against values that do
not come from this package (exact rationals, closed forms, numpy/torch conversions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"f16": 0, "bf16": 1, "f32": 2, "f8": 3}   # f8: E4M3 (OCP), decode only


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, strict IEEE: no -ffast-math, no FMA
    contraction) into liboracle.so next to it. Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        lib.oracle_decode.argtypes = [vp, i64, ctypes.c_int, dp]
        lib.oracle_encode.argtypes = [dp, i64, ctypes.c_int, vp]
        lib.oracle_logical.argtypes = [dp, i64, i64, ctypes.c_int, dp]
        lib.oracle_dequant_u4.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, dp]
        lib.oracle_gemm_f64.argtypes = [dp, dp, i64, i64, i64, i64, i64, dp]
        lib.oracle_threads.argtypes = []
        lib.oracle_attention_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_double,
                                             i64, i64, dp]
        for f in (lib.oracle_decode, lib.oracle_encode, lib.oracle_logical,
                  lib.oracle_dequant_u4, lib.oracle_gemm_f64, lib.oracle_threads,
                  lib.oracle_attention_f64):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """OpenMP threads the oracle's product loop uses."""
    return _L().oracle_threads()


def decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Stored bit patterns (uint16 for f16/bf16, uint32 for f32, uint8 for the fp8 E4M3
    format) -> exact fp64 values."""
    want = np.uint32 if fmt == "f32" else (np.uint8 if fmt == "f8" else np.uint16)
    b = np.ascontiguousarray(bits).view(want) if bits.dtype != want else np.ascontiguousarray(bits)
    out = np.empty(b.size, dtype=np.float64)
    if _L().oracle_decode(b.ctypes.data, b.size, FMT[fmt], _dp(out)):
        raise ValueError(fmt)
    return out.reshape(b.shape)


def encode(x: np.ndarray, fmt: str) -> np.ndarray:
    """fp64 values -> bit patterns of ``fmt`` after one round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32 if fmt == "f32" else np.uint16)
    if _L().oracle_encode(_dp(x), x.size, FMT[fmt], out.ctypes.data):
        raise ValueError(fmt)
    return out


def logical(stored: np.ndarray, rows: int, cols: int, layout: str) -> np.ndarray:
    """rows x cols logical matrix from a flat stored array ("row" or "col" major)."""
    s = np.ascontiguousarray(stored, dtype=np.float64).reshape(-1)
    assert s.size == rows * cols
    out = np.empty((rows, cols), dtype=np.float64)
    _L().oracle_logical(_dp(s), rows, cols, 1 if layout == "col" else 0, _dp(out))
    return out


def dequant_u4(packed: np.ndarray, scales_bits: np.ndarray, K: int, N: int,
               group: int = 128, zero: int = 8) -> np.ndarray:
    """Logical K x N fp64 weights from nibbles packed along K (byte n*K/2 + k/2, low
    nibble = even k) and binary16 scales laid out [K/group][N]."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    s = np.ascontiguousarray(scales_bits).view(np.uint16).reshape(-1)
    assert p.size == N * K // 2 and s.size == (K // group) * N
    out = np.empty((K, N), dtype=np.float64)
    if _L().oracle_dequant_u4(p.ctypes.data, s.ctypes.data, K, N, group, zero, _dp(out)):
        raise ValueError("bad dequant shape")
    return out


def gemm_f64(a: np.ndarray, b: np.ndarray, rows: tuple[int, int] | None = None) -> np.ndarray:
    """Plain fp64 product of logical a (M x K) and b (K x N); optionally rows [r0, r1)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    M, K = a.shape
    K2, N = b.shape
    assert K == K2
    r0, r1 = rows if rows is not None else (0, M)
    c = np.empty((r1 - r0, N), dtype=np.float64)
    if _L().oracle_gemm_f64(_dp(a), _dp(b), M, N, K, r0, r1, _dp(c)):
        raise ValueError("bad row range")
    return c


def operand_a(A_bits: np.ndarray, M: int, K: int, layout: str, fmt: str) -> np.ndarray:
    """Logical fp64 A (M x K) from its stored bits."""
    return logical(decode(A_bits.reshape(-1), fmt), M, K, layout)


def operand_b(B_bits, K: int, N: int, layout: str, fmt: str, scales_bits=None,
              group: int = 128, zero: int = 8) -> np.ndarray:
    """Logical fp64 B (K x N) from its stored bits, or from packed int4 codes."""
    if fmt == "u4":
        return dequant_u4(B_bits, scales_bits, K, N, group, zero)
    return logical(decode(B_bits.reshape(-1), fmt), K, N, layout)


def gemm(A_bits, B_bits, M: int, N: int, K: int, layout_a: str, layout_b: str,
         fmt_ab: str, fmt_c: str, scales_bits=None, group: int = 128, zero: int = 8,
         rows: tuple[int, int] | None = None):
    """C = A*B by definition. Returns (c64, c_bits): the exact-as-fp64 sums and the
    sums rounded once to ``fmt_c`` (bit patterns). ``fmt_ab`` is the A format; B uses the
    same format unless ``scales_bits`` is given (B is then int4 codes, "u4")."""
    a = operand_a(A_bits, M, K, layout_a, fmt_ab)
    b = operand_b(B_bits, K, N, layout_b, "u4" if scales_bits is not None else fmt_ab,
                  scales_bits, group, zero)
    c64 = gemm_f64(a, b, rows)
    return c64, encode(c64, fmt_c)


def attention_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  rows: tuple[int, int] | None = None) -> np.ndarray:
    """softmax(scale * q k^T) v per slice for fp64 q [BH, Sq, D], k and v [BH, Sk, D].
    Returns [BH, Sq, D], or the flattened rows [r0, r1) of (slice, query) as [r1 - r0, D]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    BH, Sq, D = q.shape
    assert k.shape[0] == BH and k.shape[2] == D and v.shape == k.shape
    Sk = k.shape[1]
    r0, r1 = rows if rows is not None else (0, BH * Sq)
    o = np.empty((r1 - r0, D), dtype=np.float64)
    if _L().oracle_attention_f64(_dp(q), _dp(k), _dp(v), BH, Sq, Sk, D, float(scale), r0, r1, _dp(o)):
        raise ValueError("bad attention arguments")
    return o.reshape(BH, Sq, D) if rows is None else o


def attention(q_bits, k_bits, v_bits, BH: int, Sq: int, Sk: int, D: int, fmt: str,
              fmt_o: str, scale: float, rows: tuple[int, int] | None = None):
    """Attention forward by definition from stored bits ([BH][S][D], head dim contiguous).
    Returns (o64, o_bits): fp64 outputs and their single rounding to ``fmt_o``."""
    q = decode(np.asarray(q_bits).reshape(-1), fmt).reshape(BH, Sq, D)
    k = decode(np.asarray(k_bits).reshape(-1), fmt).reshape(BH, Sk, D)
    v = decode(np.asarray(v_bits).reshape(-1), fmt).reshape(BH, Sk, D)
    o64 = attention_f64(q, k, v, scale, rows)
    return o64, encode(o64, fmt_o)


def splitk_factor(M: int, N: int, K: int, block_m: int, block_n: int, block_k: int,
                  num_cus: int, threshold: float = 5e-2, cap: int = 16) -> int:
    """Split-K factor by the waste-ratio search of BitBLAS PR 268 ("SplitK Infer").

    Start at 1; the grid is tiles * factor; the waste is grid mod num_cus and the ratio
    waste / grid. Stop once the ratio is at most the threshold; otherwise double the
    factor, unless the doubled factor times block_k reaches K. Readings: tile counts use
    ceiling division (the page's floor gives an empty grid when a block exceeds M), and
    the factor never exceeds ``cap``.
    """
    tiles = (-(-M // block_m)) * (-(-N // block_n))
    f = 1
    while True:
        grid = tiles * f
        waste = grid - (grid // num_cus) * num_cus
        if waste / grid <= threshold:
            break
        nxt = f * 2
        if nxt * block_k >= K or nxt > cap:
            break
        f = nxt
    return f


def perm_fwd(I: int, B: int, S: int) -> int:
    """Forward map of rocm-libraries PR 2487: with S' = B / S, I' = S*(I mod S') + I div S'."""
    Sp = B // S
    return S * (I % Sp) + I // Sp


def perm_inv(Ip: int, B: int, S: int) -> int:
    """Inverse map of the same page: with S' = B / S, I = S'*(I' mod S) + I' div S."""
    Sp = B // S
    return Sp * (Ip % S) + Ip // S
