"""CPU oracle for the block-wise int4 weight-only matmul (ONNX MatMulNBits).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
library never calls it, and it imports nothing from the product package.

This module is a thin ctypes loader over ``mnb_oracle.c`` (plain C, fp64,
naive loops) plus the per-element acceptance rule.  All arithmetic of the
method lives in the C file; see its header for the passages each function
follows.  Every function here is pinned by ``tests/test_oracle.py``.

Acceptance rule (the method's stated tolerance):
an output y is accepted against the fp64 oracle value Y when
``|y - Y| <= 1e-3 * sum_k |a_k * w_nk| + 1e-5``; NaN against NaN and equal
infinities count as agreement (the NaN convention of ferrox-cuda gpu.rs, test
helper assert_close_relative).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mnb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmnb_oracle.so")
_lib = None

REL_TOL = 1e-3
ABS_TOL = 1e-5


def build(force: bool = True) -> str:
    """Compile the C oracle: -O2, no fast-math, OpenMP over output elements."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # rebuilt when missing or older than its source, so a test never runs a
    # stale oracle
    if not os.path.exists(_LIB_PATH) or (os.path.exists(_SRC) and
                                         os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [p, i64, p]
    lib.oracle_decode_f32.argtypes = [p, i64, p]
    lib.oracle_code.argtypes = [p, i64, i64, i64, i64]
    lib.oracle_code.restype = ctypes.c_int
    lib.oracle_zero_point.argtypes = [p, i64, i64, i64]
    lib.oracle_zero_point.restype = ctypes.c_int
    lib.oracle_unpack_codes.argtypes = [p, i64, i64, i64, p]
    lib.oracle_unpack_zero_points.argtypes = [p, i64, i64, p]
    lib.oracle_dequant.argtypes = [p, p, p, i64, i64, i64, p]
    lib.oracle_matmul.argtypes = [p, p, i64, i64, i64, p, p, ctypes.c_int]
    lib.oracle_matmul_nbits_at.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p, p, ctypes.c_int]
    lib.oracle_matmul_nbits.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p, ctypes.c_int]
    lib.oracle_swiglu.argtypes = [p, p, i64, p]
    lib.oracle_pack_codes.argtypes = [p, i64, i64, i64, p]
    lib.oracle_pack_zero_points.argtypes = [p, i64, i64, p]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_dequant_gidx.argtypes = [p, p, p, p, i64, i64, i64, p]
    lib.oracle_round_f16.argtypes = [ctypes.c_double]
    lib.oracle_round_f16.restype = ctypes.c_uint16
    lib.oracle_round_f16_array.argtypes = [p, i64, p]
    lib.oracle_bias_f16.argtypes = [ctypes.c_float, ctypes.c_uint16, ctypes.c_int]
    lib.oracle_bias_f16.restype = ctypes.c_uint16
    lib.oracle_bias_f16_array.argtypes = [p, p, i64, ctypes.c_int, p]
    lib.oracle_acc4_quantize.argtypes = [p, i64, i64, p, p]
    lib.oracle_acc4_matmul.argtypes = [p, i64, i64, p, p, p, i64, i64, p, p, p, p, p]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def k_blocks(K: int, g: int) -> int:
    return (K + g - 1) // g


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# ---- decoding -------------------------------------------------------------

def decode(x: np.ndarray) -> np.ndarray:
    """fp16 (decoded from the IEEE-754 binary16 definition) or fp32 -> fp64."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    if x.dtype == np.float16 or x.dtype == np.uint16:
        _load().oracle_decode_f16(_ptr(x.view(np.uint16)), x.size, _ptr(out))
    elif x.dtype == np.float32:
        _load().oracle_decode_f32(_ptr(x), x.size, _ptr(out))
    else:
        raise TypeError("decode: fp16 or fp32 expected, got %s" % x.dtype)
    return out


def code(packed: np.ndarray, n: int, k: int, K: int, g: int) -> int:
    return int(_load().oracle_code(_ptr(np.ascontiguousarray(packed, np.uint8)), n, k, K, g))


def zero_point(zp: Optional[np.ndarray], n: int, b: int, kb: int) -> int:
    zp = None if zp is None else np.ascontiguousarray(zp, np.uint8)
    return int(_load().oracle_zero_point(_ptr(zp), n, b, kb))


def unpack_codes(packed: np.ndarray, N: int, K: int, g: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    assert packed.size == N * k_blocks(K, g) * (g // 2)
    out = np.empty((N, K), dtype=np.uint8)
    _load().oracle_unpack_codes(_ptr(packed), N, K, g, _ptr(out))
    return out


def unpack_zero_points(zp: Optional[np.ndarray], N: int, K: int, g: int) -> np.ndarray:
    kb = k_blocks(K, g)
    if zp is not None:
        zp = np.ascontiguousarray(zp, np.uint8)
        assert zp.size == N * ((kb + 1) // 2)
    out = np.empty((N, kb), dtype=np.uint8)
    _load().oracle_unpack_zero_points(_ptr(zp), N, kb, _ptr(out))
    return out


def dequant(packed: np.ndarray, scales: np.ndarray, zp: Optional[np.ndarray],
            N: int, K: int, g: int) -> np.ndarray:
    """fp64 dense W[N,K] = (code - zp) * scale."""
    kb = k_blocks(K, g)
    packed = np.ascontiguousarray(packed, np.uint8)
    s64 = decode(scales).reshape(-1)
    assert s64.size == N * kb and packed.size == N * kb * (g // 2)
    if zp is not None:
        zp = np.ascontiguousarray(zp, np.uint8)
        assert zp.size == N * ((kb + 1) // 2)
    w = np.empty((N, K), dtype=np.float64)
    _load().oracle_dequant(_ptr(packed), _ptr(s64), _ptr(zp), N, K, g, _ptr(w))
    return w


def dequant_gidx(packed: np.ndarray, scales: np.ndarray, zp: Optional[np.ndarray],
                 g_idx: np.ndarray, N: int, K: int, g: int) -> np.ndarray:
    """fp64 dense W[N,K] = (code - zp[g_idx[k]]) * scale[g_idx[k]] (act order)."""
    kb = k_blocks(K, g)
    packed = np.ascontiguousarray(packed, np.uint8)
    s64 = decode(scales).reshape(-1)
    assert s64.size == N * kb and packed.size == N * kb * (g // 2)
    if zp is not None:
        zp = np.ascontiguousarray(zp, np.uint8)
        assert zp.size == N * ((kb + 1) // 2)
    gi = np.ascontiguousarray(g_idx, np.int32)
    assert gi.size == K
    w = np.empty((N, K), dtype=np.float64)
    _load().oracle_dequant_gidx(_ptr(packed), _ptr(s64), _ptr(zp), _ptr(gi), N, K, g, _ptr(w))
    return w


def matmul(A64: np.ndarray, W64: np.ndarray, threads: int = 0):
    """Y = A . W^T and the magnitude sum Bnd, naive fp64 loops."""
    A64 = np.ascontiguousarray(A64, np.float64)
    W64 = np.ascontiguousarray(W64, np.float64)
    M, K = A64.shape
    N, K2 = W64.shape
    assert K == K2
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul(_ptr(A64), _ptr(W64), M, N, K, _ptr(Y), _ptr(B), threads)
    return Y, B


def matmul_lib(A64: np.ndarray, W64: np.ndarray):
    """Y = A . W^T and Bnd = |A| . |W|^T with a library matrix product
    (numpy's fp64 matmul) as the step: the same sums as ``matmul`` in another
    order, each within K * 2^-53 * Bnd of the exact value, for products too
    large for the naive loops (a full prefill output)."""
    A64 = np.ascontiguousarray(A64, np.float64)
    W64 = np.ascontiguousarray(W64, np.float64)
    assert A64.shape[1] == W64.shape[1]
    Y = A64 @ W64.T
    B = np.abs(A64) @ np.abs(W64).T
    return Y, B


def acc4_matmul_lib(A, packed, scales, zp, N: int, K: int, g: int, bias=None) -> tuple:
    """acc4_matmul for every output with a library matrix product as the
    step: the oracle's int8 rows q and scales s, the oracle's dequantized
    weights w = (c - z) * scale in fp64, then s[m] * (q . w^T) + b in fp64.
    The block sums of acc4_matmul are exact integers; here the same value is
    summed in another order, within K * 2^-53 * Bnd of it.  Returns (Y, Bnd, q, s)."""
    A = np.ascontiguousarray(A, np.float32).reshape(-1, K)
    q, sc = acc4_quantize(A)
    W64 = dequant(packed, scales, zp, N, K, g)
    inner, mag = matmul_lib(q.astype(np.float64), W64)
    s64 = sc.astype(np.float64)[:, None]
    b = np.zeros(N) if bias is None else np.asarray(bias, np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        Y = np.where(s64 != 0, s64 * inner, 0.0) + b[None, :]
        Bnd = np.where(s64 != 0, np.abs(s64) * mag, 0.0) + np.abs(b)[None, :]
    return Y, Bnd, q, sc


def matmul_nbits(A: np.ndarray, packed, scales, zp, N: int, K: int, g: int, threads: int = 0):
    """The whole method (dequantize on the fly) for every output: (Y, Bnd) [M,N]."""
    A64 = decode(np.ascontiguousarray(A)).reshape(-1, K)
    M = A64.shape[0]
    s64 = decode(scales).reshape(-1)
    packed = np.ascontiguousarray(packed, np.uint8)
    zp = None if zp is None else np.ascontiguousarray(zp, np.uint8)
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul_nbits(_ptr(A64), _ptr(packed), _ptr(s64), _ptr(zp),
                                M, N, K, g, _ptr(Y), _ptr(B), threads)
    return Y, B


def matmul_nbits_at(A: np.ndarray, packed, scales, zp, N: int, K: int, g: int,
                    ms: np.ndarray, ns: np.ndarray, threads: int = 0):
    """The whole method at chosen outputs (ms[i], ns[i]): (Y, Bnd) [count]."""
    A64 = decode(np.ascontiguousarray(A)).reshape(-1, K)
    s64 = decode(scales).reshape(-1)
    packed = np.ascontiguousarray(packed, np.uint8)
    zp = None if zp is None else np.ascontiguousarray(zp, np.uint8)
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    assert ms.shape == ns.shape
    assert (ms >= 0).all() and (ms < A64.shape[0]).all() and (ns >= 0).all() and (ns < N).all()
    Y = np.empty(ms.shape, dtype=np.float64)
    B = np.empty(ms.shape, dtype=np.float64)
    _load().oracle_matmul_nbits_at(_ptr(A64), _ptr(packed), _ptr(s64), _ptr(zp), N, K, g,
                                   _ptr(ms), _ptr(ns), ms.size, _ptr(Y), _ptr(B), threads)
    return Y, B


def swiglu(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    G = np.ascontiguousarray(G, np.float64)
    U = np.ascontiguousarray(U, np.float64)
    assert G.shape == U.shape
    S = np.empty(G.shape, dtype=np.float64)
    _load().oracle_swiglu(_ptr(G), _ptr(U), G.size, _ptr(S))
    return S


def pack_codes(codes: np.ndarray, g: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    N, K = codes.shape
    out = np.empty(N * k_blocks(K, g) * (g // 2), dtype=np.uint8)
    _load().oracle_pack_codes(_ptr(codes), N, K, g, _ptr(out))
    return out.reshape(N, k_blocks(K, g), g // 2)


def pack_zero_points(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, np.uint8)
    N, kb = z.shape
    out = np.empty(N * ((kb + 1) // 2), dtype=np.uint8)
    _load().oracle_pack_zero_points(_ptr(z), N, kb, _ptr(out))
    return out.reshape(N, (kb + 1) // 2)


# ---- output rounding and the bias epilogue ---------------------------------

def round_f16(x) -> np.ndarray:
    """binary16 nearest to each value (ties to even), as float16."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_f16_array(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


def bias_epilogue_f16(acc, bias, after_round: bool) -> np.ndarray:
    """fp16 outputs of the bias epilogue from fp32 accumulators and fp16
    biases (same shape): fp16(acc + b) or, after_round, fp16(fp16(acc) + b)."""
    acc = np.ascontiguousarray(acc, np.float32)
    b = np.ascontiguousarray(bias, np.float16).view(np.uint16)
    assert acc.shape == b.shape
    out = np.empty(acc.shape, dtype=np.uint16)
    _load().oracle_bias_f16_array(_ptr(acc), _ptr(b), acc.size, int(bool(after_round)), _ptr(out))
    return out.view(np.float16)


def bias_bound(Y: np.ndarray, Bnd: np.ndarray, bias64: np.ndarray) -> np.ndarray:
    """Tolerance of a biased fp16 output against Y + b (fp64), a reading: the
    matmul's own rule for the accumulator, then one binary32 addition and one
    binary16 rounding of the sum (together at most 2^-10 of its magnitude,
    plus half the binary16 subnormal spacing, 2^-25, for sums below the
    binary16 normal range)."""
    e = REL_TOL * np.asarray(Bnd, np.float64) + ABS_TOL
    return e + 2.0 ** -10 * (np.abs(np.asarray(Y, np.float64) + bias64) + e) + 2.0 ** -25


# ---- int8 activations (accuracy_level 4) -----------------------------------

def acc4_quantize(A) -> tuple:
    """Rows of fp32 A [M,K] to int8 with one binary32 scale each:
    (q int8 [M,K], scale float32 [M])."""
    A = np.ascontiguousarray(A, np.float32)
    M, K = A.shape
    q = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    _load().oracle_acc4_quantize(_ptr(A), M, K, _ptr(q), _ptr(sc))
    return q, sc


def acc4_matmul(A, packed, scales, zp, N: int, K: int, g: int, bias=None) -> tuple:
    """The accuracy_level=4 product of fp32 A [M,K]: (Y, Bnd) [M,N] in fp64
    from the int8 rows, plus those rows and their scales (q [M,K], scale [M])."""
    A = np.ascontiguousarray(A, np.float32).reshape(-1, K)
    M = A.shape[0]
    kb = k_blocks(K, g)
    s64 = decode(scales).reshape(-1)
    packed = np.ascontiguousarray(packed, np.uint8)
    assert s64.size == N * kb and packed.size == N * kb * (g // 2)
    zp = None if zp is None else np.ascontiguousarray(zp, np.uint8)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    assert b is None or b.size == N
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    q = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    _load().oracle_acc4_matmul(_ptr(A), M, K, _ptr(packed), _ptr(s64), _ptr(zp), N, g, _ptr(b),
                               _ptr(Y), _ptr(B), _ptr(q), _ptr(sc))
    return Y, B, q, sc


def acc4_bound(Bnd, K: int, g: int) -> np.ndarray:
    """Tolerance of a binary32 evaluation of the int8-activation product, a
    reading (the stated tolerance is for fp16 arithmetic).  Every product and
    every sum of products within a block is an integer below 2^24, exact in
    binary32; the errors are the roundings of running values, each at most
    2^-24 of a partial total, itself at most Bnd.  The evaluation with the
    most of them keeps one accumulator in units of the current block's scale:
    one rounding per 16-k partial sum added to it, two per block for the
    change of units (the ratio of scales and the product), then the last
    block's scale, the activation scale and the bias: k_blocks*(g/16 + 2) + 4
    roundings, which also covers one rounding per block term (the pages' two
    binary32 orders).  Plus one smallest subnormal per rounding for results
    below the normal range."""
    kb = k_blocks(K, g)
    n = kb * (g // 16 + 2) + 4
    return n * 2.0 ** -24 * np.asarray(Bnd, np.float64) + n * 2.0 ** -149


# ---- acceptance ------------------------------------------------------------

def within_bound(y, Y: np.ndarray, Bnd, rel: float = REL_TOL,
                 abs_: float = ABS_TOL, tol=None) -> np.ndarray:
    """Per-element verdict |y - Y| <= rel*Bnd + abs_ (or <= tol, a per-element
    tolerance given instead of Bnd), NaN==NaN, equal infs."""
    y = np.asarray(y, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    if tol is None:
        tol = rel * np.asarray(Bnd, dtype=np.float64) + abs_
    tol = np.asarray(tol, dtype=np.float64)
    both_nan = np.isnan(y) & np.isnan(Y)
    same_inf = np.isinf(y) & np.isinf(Y) & (np.sign(y) == np.sign(Y))
    with np.errstate(invalid="ignore"):
        # the distance test applies to finite expected values only: an
        # infinite Y (whose bound is infinite too) is matched only by the
        # same infinity, a NaN only by a NaN
        ok = np.isfinite(Y) & (np.abs(y - Y) <= tol)
    return ok | both_nan | same_inf


def swiglu_bound(G: np.ndarray, BG: np.ndarray, U: np.ndarray, BU: np.ndarray) -> np.ndarray:
    """Tolerance of a fused silu(gate)*up output, propagated to first order
    from the matmul bound of each projection (a reading: the stated tolerance
    covers only the matmul).  Eg, Eu bound the projections including an
    optional fp16 rounding of each; 1.1 bounds |silu'|; 2^-11 covers the final
    fp16 rounding of S."""
    eps16 = 2.0 ** -11
    Eg = REL_TOL * BG + ABS_TOL + eps16 * np.abs(G)
    Eu = REL_TOL * BU + ABS_TOL + eps16 * np.abs(U)
    S = swiglu(G, U)
    silu = swiglu(G, np.ones_like(G))
    return 1.1 * Eg * (np.abs(U) + Eu) + np.abs(silu) * Eu + eps16 * np.abs(S) + ABS_TOL
