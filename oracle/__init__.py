"""ORACLE — test infrastructure, not part of the product.

Python access (ctypes + numpy) to the plain-C oracle in ``oracle.c``.  Only
the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  It never imports the GPU package and the GPU
package never imports it.

Functions (parity status in ``oracle.c``):
  gemm_i32(x, w)                 O1  integer product, exact
  gemm_i32_threads(x, w, t)      O1  the same C function on t host threads, each
                                     over its own block of weight rows (same result)
  ternarize_absmean(W)           O2  absmean ternarization -> (wq, sw)
  quant_act(x_bf16_bits)         O3  per-token absmax int8 quantization
  epilogue(acc, sa, sw)          O4  fp32 scale epilogue
  pack(w) / unpack(p, N, K)      a2  2-bit packing per the T32x128 layout
  packed_bytes(N, K)
  quant_act_a4(x_bf16_bits)      O5  per-token absmax int4 quantization
  pack_act4(q) / unpack_act4(b, M, K), act4_bytes(M, K)
                                     int4 activation layout "A4I"
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_gemm_i32.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_gemm_i32.restype = ctypes.c_int
    lib.oracle_ternarize_absmean.argtypes = [P, I64, I64, P, P]
    lib.oracle_ternarize_absmean.restype = None
    lib.oracle_quant_act.argtypes = [P, I64, I64, P, P]
    lib.oracle_quant_act.restype = None
    lib.oracle_epilogue.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.oracle_epilogue.restype = None
    lib.oracle_packed_bytes.argtypes = [I64, I64]
    lib.oracle_packed_bytes.restype = I64
    lib.oracle_pack.argtypes = [P, I64, I64, P]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [P, I64, I64, P]
    lib.oracle_unpack.restype = ctypes.c_int
    lib.oracle_quant_act_a4.argtypes = [P, I64, I64, P, P]
    lib.oracle_quant_act_a4.restype = None
    lib.oracle_act4_bytes.argtypes = [I64, I64]
    lib.oracle_act4_bytes.restype = I64
    lib.oracle_pack_act4.argtypes = [P, I64, I64, P]
    lib.oracle_pack_act4.restype = ctypes.c_int
    lib.oracle_unpack_act4.argtypes = [P, I64, I64, P]
    lib.oracle_unpack_act4.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def gemm_i32(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x int8 [M, K] (or [K]); w int8 [N, K] -> int32 [M, N] (or [N])."""
    squeeze = x.ndim == 1
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.int8)
    w2 = np.ascontiguousarray(w, dtype=np.int8)
    M, K = x2.shape
    N, K2 = w2.shape
    if K != K2:
        raise ValueError("K mismatch")
    y = np.empty((M, N), dtype=np.int32)
    if _load().oracle_gemm_i32(_ptr(x2), _ptr(w2), M, N, K, _ptr(y)) != 0:
        raise OverflowError("int32 overflow in oracle product")
    return y[0] if squeeze else y


def gemm_i32_threads(x: np.ndarray, w: np.ndarray, threads: int) -> np.ndarray:
    """gemm_i32 with the output columns (rows of w) split into `threads`
    contiguous blocks, each computed by the same C function on its own host
    thread (ctypes releases the GIL during the call).  Every output element is
    the same int64 sum as in gemm_i32, so the result is identical."""
    from concurrent.futures import ThreadPoolExecutor

    squeeze = x.ndim == 1
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.int8)
    w2 = np.ascontiguousarray(w, dtype=np.int8)
    M, K = x2.shape
    N, K2 = w2.shape
    if K != K2:
        raise ValueError("K mismatch")
    threads = max(1, min(int(threads), N))
    bounds = [N * i // threads for i in range(threads + 1)]
    y = np.empty((M, N), dtype=np.int32)

    def block(i):
        n0, n1 = bounds[i], bounds[i + 1]
        if n1 > n0:
            y[:, n0:n1] = gemm_i32(x2, w2[n0:n1])

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(block, range(threads)))
    return y[0] if squeeze else y


def ternarize_absmean(W: np.ndarray):
    W2 = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W2.shape
    wq = np.empty((N, K), dtype=np.int8)
    sw = np.zeros(1, dtype=np.float32)
    _load().oracle_ternarize_absmean(_ptr(W2), N, K, _ptr(wq), _ptr(sw))
    return wq, np.float32(sw[0])


def quant_act(xb: np.ndarray):
    """xb: uint16 bf16 bit patterns [M, K] -> (xq int8 [M, K], sa fp32 [M])."""
    x2 = np.ascontiguousarray(np.atleast_2d(xb), dtype=np.uint16)
    M, K = x2.shape
    xq = np.empty((M, K), dtype=np.int8)
    sa = np.empty(M, dtype=np.float32)
    _load().oracle_quant_act(_ptr(x2), M, K, _ptr(xq), _ptr(sa))
    return xq, sa


def epilogue(acc: np.ndarray, sa: np.ndarray, sw) -> np.ndarray:
    a2 = np.ascontiguousarray(np.atleast_2d(acc), dtype=np.int32)
    M, N = a2.shape
    s2 = np.ascontiguousarray(np.atleast_1d(sa), dtype=np.float32)
    if s2.shape[0] != M:
        raise ValueError("sa must have one entry per row")
    y = np.empty((M, N), dtype=np.float32)
    _load().oracle_epilogue(_ptr(a2), _ptr(s2), ctypes.c_float(float(sw)), M, N, _ptr(y))
    return y[0] if np.ndim(acc) == 1 else y


def packed_bytes(N: int, K: int) -> int:
    return int(_load().oracle_packed_bytes(N, K))


def pack(w: np.ndarray) -> np.ndarray:
    w2 = np.ascontiguousarray(w, dtype=np.int8)
    N, K = w2.shape
    out = np.empty(packed_bytes(N, K), dtype=np.uint8)
    if _load().oracle_pack(_ptr(w2), N, K, _ptr(out)) != 0:
        raise ValueError("weight outside {-1, 0, 1}")
    return out


def unpack(p: np.ndarray, N: int, K: int) -> np.ndarray:
    p2 = np.ascontiguousarray(p, dtype=np.uint8)
    if p2.size < packed_bytes(N, K):
        raise ValueError("packed buffer too small")
    w = np.empty((N, K), dtype=np.int8)
    if _load().oracle_unpack(_ptr(p2), N, K, _ptr(w)) != 0:
        raise ValueError("code 11 found in packed matrix")
    return w


def quant_act_a4(xb: np.ndarray):
    """xb: uint16 bf16 bit patterns [M, K] -> (q int8 [M, K] in -7..7, sa fp32 [M])."""
    x2 = np.ascontiguousarray(np.atleast_2d(xb), dtype=np.uint16)
    M, K = x2.shape
    q = np.empty((M, K), dtype=np.int8)
    sa = np.empty(M, dtype=np.float32)
    _load().oracle_quant_act_a4(_ptr(x2), M, K, _ptr(q), _ptr(sa))
    return q, sa


def act4_bytes(M: int, K: int) -> int:
    return int(_load().oracle_act4_bytes(M, K))


def pack_act4(q: np.ndarray) -> np.ndarray:
    """q int8 [M, K] (values -8..7) -> uint8 [act4_bytes(M, K)] in the A4I layout."""
    q2 = np.ascontiguousarray(np.atleast_2d(q), dtype=np.int8)
    M, K = q2.shape
    out = np.empty(act4_bytes(M, K), dtype=np.uint8)
    if _load().oracle_pack_act4(_ptr(q2), M, K, _ptr(out)) != 0:
        raise ValueError("activation outside -8..7")
    return out


def unpack_act4(b: np.ndarray, M: int, K: int) -> np.ndarray:
    b2 = np.ascontiguousarray(b, dtype=np.uint8)
    if b2.size < act4_bytes(M, K):
        raise ValueError("buffer too small")
    q = np.empty((M, K), dtype=np.int8)
    _load().oracle_unpack_act4(_ptr(b2), M, K, _ptr(q))
    return q
