"""ctypes loader for ``oracle/liboracle.so`` (the plain C oracle).

Oracle (test infrastructure).  ``build()`` compiles ``liboracle.c`` with gcc
(no GPU code, no shared source with the GPU library).  The wrappers take and
return numpy arrays; every definition is the one stated in ``liboracle.c``
and in the matching Python module.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "liboracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=True):
    """Compile liboracle.so (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        for name, args in {
            "oracle_dyadic_quantize": [P, I64, I64, P, P],
            "oracle_dyadic_dequant": [P, P, I64, I64, P],
            "oracle_lut16_indices": [P, P, P, I64, I64, P],
            "oracle_signmag8_indices": [P, P, I64, I64, P],
            "oracle_lut16_fit": [P, I64, I64, ctypes.c_int, P, P],
            "oracle_signmag8_fit": [P, I64, I64, ctypes.c_int, P],
            "oracle_dyadic_matmul": [P, P, P, I64, I64, I64, P],
        }.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc):
    if rc != 0:
        raise ValueError("liboracle rejected the shape")


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    lib().oracle_set_num_threads(int(n))


def dyadic_quantize(w_bits):
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    idx = np.empty((n, k), np.uint8)
    s = np.empty((n, k // 64), np.uint16)
    _check(lib().oracle_dyadic_quantize(_p(w), n, k, _p(idx), _p(s)))
    return idx, s


def dyadic_dequant(idx, s_bits):
    idx = _c(idx, np.uint8)
    s = _c(s_bits, np.uint16)
    n, k = idx.shape
    out = np.empty((n, k), np.uint16)
    _check(lib().oracle_dyadic_dequant(_p(idx), _p(s), n, k, _p(out)))
    return out


def dyadic_matmul(packed, s_bits, x_bits):
    """y [m, n] (fp64) = x [m, k] @ w_hat [n, k]^T for dyadic (packed, scales)."""
    p = _c(packed, np.uint8)
    s = _c(s_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    n, k = p.shape[0], 2 * p.shape[1]
    m = x.shape[0]
    y = np.empty((m, n), np.float64)
    _check(lib().oracle_dyadic_matmul(_p(p), _p(s), _p(x), n, k, m, _p(y)))
    return y


def lut16_indices(w_bits, s_bits, lut_bits):
    w = _c(w_bits, np.uint16)
    s = _c(s_bits, np.uint16)
    L = _c(lut_bits, np.uint16)
    n, k = w.shape
    idx = np.empty((n, k), np.uint8)
    _check(lib().oracle_lut16_indices(_p(w), _p(s), _p(L), n, k, _p(idx)))
    return idx


def signmag8_indices(w_bits, cb_bits):
    w = _c(w_bits, np.uint16)
    cb = _c(cb_bits, np.uint16)
    n, k = w.shape
    nib = np.empty((n, k), np.uint8)
    _check(lib().oracle_signmag8_indices(_p(w), _p(cb), n, k, _p(nib)))
    return nib


def lut16_fit(w_bits, iters=25):
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    s = np.empty((n, k // 64), np.uint16)
    L = np.empty((n, k // 64, 16), np.uint16)
    _check(lib().oracle_lut16_fit(_p(w), n, k, iters, _p(s), _p(L)))
    return s, L


def signmag8_fit(w_bits, iters=25):
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    cb = np.empty((n, k // 32, 8), np.uint16)
    _check(lib().oracle_signmag8_fit(_p(w), n, k, iters, _p(cb)))
    return cb
