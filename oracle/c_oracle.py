"""ctypes wrapper of the plain C fp64 oracle (oracle/c/externd_oracle.c).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this module.  The C library implements T_tau (§2.2, with the
fixed-point mean reading), the greedy sequential decomposition (§2.3) and
the plain batched block ALS (§2.4) of
"ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with Accuracy
Approaching Any Quantization Level" in plain loops; it shares no code with
the GPU library or with the numpy oracle.  build() in __graft_entry__.py
compiles it with the system C compiler (build_c below).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "externd_oracle.c")
LIB = os.path.join(HERE, "c", "liboracle_c.so")

__all__ = ["build_c", "splitmix64_mix", "start_vector", "threshold", "ternarize", "decompose_seq",
           "decompose_block"]


def build_c():
    """Compile the C oracle into oracle/c/liboracle_c.so (gcc, -O2, strict fp)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is missing: run build() in __graft_entry__.py")
        lib = ctypes.CDLL(LIB)
        i64, u64, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
        p = ctypes.c_void_p
        lib.orc_splitmix64_mix.restype = u64
        lib.orc_splitmix64_mix.argtypes = [u64]
        lib.orc_start_vector.restype = None
        lib.orc_start_vector.argtypes = [u64, i64, i64, p]
        lib.orc_threshold.restype = ctypes.c_double
        lib.orc_threshold.argtypes = [p, i64, f32, p]
        lib.orc_ternarize.restype = i64
        lib.orc_ternarize.argtypes = [p, i64, f32, p]
        lib.orc_decompose_seq.restype = ctypes.c_int
        lib.orc_decompose_seq.argtypes = [p, i64, i64, i64, f32, ctypes.c_int, u64, p, p, p, p, p]
        lib.orc_decompose_block.restype = ctypes.c_int
        lib.orc_decompose_block.argtypes = [p, i64, i64, i64, ctypes.c_int, f32, ctypes.c_int, u64, p, p, p, p,
                                            p, p]
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def splitmix64_mix(x):
    return int(_load().orc_splitmix64_mix(x & ((1 << 64) - 1)))


def start_vector(seed, i, m):
    u = np.zeros(m, dtype=np.float64)
    _load().orc_start_vector(seed, i, m, _ptr(u))
    return u


def threshold(x, tau):
    """(thr, max|x|) of T_tau on the 1-D vector x."""
    xv = np.ascontiguousarray(x, dtype=np.float64)
    big = ctypes.c_double(0.0)
    thr = _load().orc_threshold(_ptr(xv), xv.size, float(tau), ctypes.byref(big))
    return thr, big.value


def ternarize(x, tau):
    xv = np.ascontiguousarray(x, dtype=np.float64)
    if xv.ndim != 1 or xv.size == 0:
        raise ValueError("ternarize takes a non-empty 1-D vector")
    t = np.zeros(xv.size, dtype=np.int8)
    _load().orc_ternarize(_ptr(xv), xv.size, float(tau), _ptr(t))
    return t


def decompose_seq(A, k, tau, iters=15, seed=0):
    """Returns (B m x k, C k x n, D, trace, E); B and C int8, D and trace fp64."""
    A32 = np.ascontiguousarray(A, dtype=np.float32)
    m, n = A32.shape
    Bt = np.zeros((k, m), dtype=np.int8)
    C = np.zeros((k, n), dtype=np.int8)
    D = np.zeros(k, dtype=np.float64)
    trace = np.zeros(k, dtype=np.float64)
    E = ctypes.c_double(0.0)
    rc = _load().orc_decompose_seq(_ptr(A32), m, n, k, float(tau), iters, seed, _ptr(Bt), _ptr(C), _ptr(D),
                                   _ptr(trace), ctypes.byref(E))
    if rc != 0:
        raise MemoryError("C oracle: out of memory")
    return Bt.T.copy(), C, D, trace, E.value


def decompose_block(A, k, b, tau, iters=15, seed=0):
    """Block ALS with exactly width b (the last block takes the rest).
    Returns (B m x k, C k x n, D, trace per block, E, ridge retries)."""
    A32 = np.ascontiguousarray(A, dtype=np.float32)
    m, n = A32.shape
    Bt = np.zeros((k, m), dtype=np.int8)
    C = np.zeros((k, n), dtype=np.int8)
    D = np.zeros(k, dtype=np.float64)
    trace = np.zeros((k + b - 1) // b, dtype=np.float64)
    E = ctypes.c_double(0.0)
    retries = ctypes.c_int64(0)
    rc = _load().orc_decompose_block(_ptr(A32), m, n, k, b, float(tau), iters, seed, _ptr(Bt), _ptr(C), _ptr(D),
                                     _ptr(trace), ctypes.byref(E), ctypes.byref(retries))
    if rc == -1:
        raise MemoryError("C oracle: out of memory")
    if rc != 0:
        raise ArithmeticError("C oracle: a ridge-regularised Gram is not positive definite")
    return Bt.T.copy(), C, D, trace, E.value, retries.value
