"""ctypes marshalling for oracle.c (test infrastructure only; see the package docstring).

Every function takes numpy arrays, checks shapes, and hands raw pointers to the C code.
Weights may be float16, float32 or float64; the C side widens them exactly to double.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import subprocess

import numpy as np

F32, F16, F64 = 0, 1, 2
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
OMP_LIB_PATH = os.path.join(_HERE, "liboracle_omp.so")
_lib = None
_FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C11, no fast-math, no FP
    contraction, single-threaded: the OpenMP pragmas are ignored), and the same source with
    -fopenmp into liboracle_omp.so (the CPU baseline's all-core timing; same arithmetic)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *_FLAGS, "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB_PATH)
    if force or not os.path.exists(OMP_LIB_PATH):
        tmp = OMP_LIB_PATH + ".tmp"
        subprocess.run(["gcc", *_FLAGS, "-fopenmp", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, OMP_LIB_PATH)
    return _LIB_PATH


def _configure(lib):
    P, I32, I64, D = C.c_void_p, C.c_int32, C.c_int64, C.c_double
    lib.oracle_half_to_double.argtypes = [C.c_uint16]
    lib.oracle_half_to_double.restype = D
    lib.oracle_predict.argtypes = [I32, I32, I32, I32, P, P, P, I32, P, P, P]
    lib.oracle_threshold.argtypes = [I32, I32, P, D, P]
    lib.oracle_compact.argtypes = [I32, I32, P, P, P, P]
    lib.oracle_forward.argtypes = [I32, I32, I32, I32, P, P, P, P, I32, P, P, P, I32, P, P]
    lib.oracle_dense.argtypes = [I32, I32, I32, I32, P, P, P, P, I32, P, P, P]
    lib.oracle_dense_f16act.argtypes = [I32, I32, I32, I32, P, P, P, P, I32, P, P, P]
    lib.oracle_round_half_array.argtypes = [I64, P, P]
    lib.oracle_preact.argtypes = [I32, I32, I32, P, P, I32, P, P]
    lib.oracle_profile_counts.argtypes = [I32, I32, I32, P, P, I32, P, P]
    lib.oracle_permutation.argtypes = [P, I32, I32, P]
    lib.oracle_pack_rows.argtypes = [P, P, P, I32, I64]
    for name in ("predict", "threshold", "compact", "forward", "dense", "dense_f16act",
                 "round_half_array", "preact", "profile_counts", "permutation", "pack_rows"):
        getattr(lib, "oracle_" + name).restype = C.c_int
    if hasattr(lib, "oracle_threads"):
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = C.c_int
    return lib


def threads() -> int:
    """Threads the active oracle library runs its loops on (1 unless the OpenMP build is
    routed in with set_library)."""
    lib = load()
    return int(lib.oracle_threads()) if hasattr(lib, "oracle_threads") else 1


def open_library(path: str):
    """Open an oracle shared library at `path` (the tests use this for planted-mistake copies)."""
    return _configure(C.CDLL(path))


def set_library(lib):
    """Route every wrapper call to `lib`; returns the previous library (may be None)."""
    global _lib
    prev, _lib = _lib, lib
    return prev


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = open_library(_LIB_PATH)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported weight dtype {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle_{what} rejected its arguments (rc={rc})")


def half_to_double(bits: np.ndarray) -> np.ndarray:
    """Decode uint16 binary16 bit patterns with the oracle's own decoder."""
    lib = load()
    return np.array([lib.oracle_half_to_double(int(b)) for b in np.asarray(bits, np.uint16).ravel()])


def predict(X, P1, P2, c=None, return_q=False):
    """Scores S[B, n] = P2 @ (P1 @ x) + c per token, fp64."""
    X = _c(X, np.float32)
    P1, P2 = _c(P1), _c(P2)
    c = _c(c, np.float32)
    B, d = X.shape
    r, d2 = P1.shape
    n, r2 = P2.shape
    assert d2 == d and r2 == r and P1.dtype == P2.dtype
    assert c is None or c.shape == (n,)
    S = np.empty((B, n), np.float64)
    Q = np.empty((B, r), np.float64)
    _check(load().oracle_predict(d, n, r, B, _ptr(X), _ptr(P1), _ptr(P2), _dtype_code(P1),
                                 _ptr(c), _ptr(S), _ptr(Q)), "predict")
    return (S, Q) if return_q else S


def threshold(S, tau=0.0):
    """Mask M[B, n] (uint8) = S > tau, strictly; NaN is inactive. S is widened to float64."""
    S = np.ascontiguousarray(np.asarray(S, np.float64))
    if S.ndim == 1:
        S = S[None, :]
    B, n = S.shape
    M = np.empty((B, n), np.uint8)
    _check(load().oracle_threshold(B, n, _ptr(S), float(tau), _ptr(M)), "threshold")
    return M


def compact(M):
    """(idx int32[count], count, tokmask uint64[count]) from a mask M[B, n]."""
    M = np.ascontiguousarray(np.asarray(M, np.uint8))
    if M.ndim == 1:
        M = M[None, :]
    B, n = M.shape
    idx = np.empty(n, np.int32)
    tok = np.empty(n, np.uint64)
    cnt = np.zeros(1, np.int32)
    _check(load().oracle_compact(B, n, _ptr(M), _ptr(idx), _ptr(cnt), _ptr(tok)), "compact")
    k = int(cnt[0])
    return idx[:k].copy(), k, tok[:k].copy()


def forward(X, Wa, Wo, idx, tokmask=None, *, Wu=None, b_a=None, b_o=None):
    """Y[B, d] (fp64) over the active list idx (with per-token bits tokmask when given)."""
    X = _c(X, np.float32)
    Wa, Wo, Wu = _c(Wa), _c(Wo), _c(Wu)
    b_a, b_o = _c(b_a, np.float32), _c(b_o, np.float32)
    idx = _c(np.asarray(idx, np.int32))
    B, d = X.shape
    n, d2 = Wa.shape
    assert d2 == d and Wo.shape == (n, d) and Wo.dtype == Wa.dtype
    assert Wu is None or (Wu.shape == (n, d) and Wu.dtype == Wa.dtype)
    count = int(idx.shape[0])
    if tokmask is not None:
        tokmask = _c(np.asarray(tokmask, np.uint64))
        assert tokmask.shape == (count,)
    Y = np.empty((B, d), np.float64)
    _check(load().oracle_forward(d, n, B, 1 if Wu is not None else 0, _ptr(X), _ptr(Wa),
                                 _ptr(Wu), _ptr(Wo), _dtype_code(Wa), _ptr(b_a), _ptr(b_o),
                                 _ptr(idx), count, _ptr(tokmask), _ptr(Y)), "forward")
    return Y


def dense(X, Wa, Wo, *, Wu=None, b_a=None, b_o=None):
    """Y[B, d] (fp64): the FFN over every neuron, no mask."""
    X = _c(X, np.float32)
    Wa, Wo, Wu = _c(Wa), _c(Wo), _c(Wu)
    b_a, b_o = _c(b_a, np.float32), _c(b_o, np.float32)
    B, d = X.shape
    n = Wa.shape[0]
    Y = np.empty((B, d), np.float64)
    _check(load().oracle_dense(d, n, B, 1 if Wu is not None else 0, _ptr(X), _ptr(Wa), _ptr(Wu),
                               _ptr(Wo), _dtype_code(Wa), _ptr(b_a), _ptr(b_o), _ptr(Y)), "dense")
    return Y


def dense_f16act(X, Wa, Wo, *, Wu=None, b_a=None, b_o=None):
    """Y[B, d] (fp64): dense with fp16 activations, x rounded to binary16 (nearest, ties
    to even) before the up products and h before the down product."""
    X = _c(X, np.float32)
    Wa, Wo, Wu = _c(Wa), _c(Wo), _c(Wu)
    b_a, b_o = _c(b_a, np.float32), _c(b_o, np.float32)
    B, d = X.shape
    n = Wa.shape[0]
    Y = np.empty((B, d), np.float64)
    _check(load().oracle_dense_f16act(d, n, B, 1 if Wu is not None else 0, _ptr(X), _ptr(Wa),
                                      _ptr(Wu), _ptr(Wo), _dtype_code(Wa), _ptr(b_a), _ptr(b_o),
                                      _ptr(Y)), "dense_f16act")
    return Y


def round_half(v):
    """Each value (fp64) rounded to the nearest binary16 value, ties to even (overflow to
    infinity from 65520 on), returned as fp64."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty_like(v)
    _check(load().oracle_round_half_array(v.size, _ptr(v), _ptr(out)), "round_half")
    return out


def preact(X, Wa, b_a=None):
    """A[B, n] (fp64) = Wa @ x + b_a: the ReLU input (the gate, for the gated form)."""
    X = _c(X, np.float32)
    Wa = _c(Wa)
    b_a = _c(b_a, np.float32)
    B, d = X.shape
    n = Wa.shape[0]
    A = np.empty((B, n), np.float64)
    _check(load().oracle_preact(d, n, B, _ptr(X), _ptr(Wa), _dtype_code(Wa), _ptr(b_a), _ptr(A)),
           "preact")
    return A


def profile_counts(Xprof, Wa, b_a=None):
    """counts[n] int64: number of profiling tokens whose pre-activation is > 0."""
    X = _c(Xprof, np.float32)
    Wa = _c(Wa)
    b_a = _c(b_a, np.float32)
    N, d = X.shape
    n = Wa.shape[0]
    counts = np.empty(n, np.int64)
    _check(load().oracle_profile_counts(d, n, N, _ptr(X), _ptr(Wa), _dtype_code(Wa), _ptr(b_a),
                                        _ptr(counts)), "profile_counts")
    return counts


def n_hot_for(n: int, hot_frac: float) -> int:
    """Number of hot neurons for a hot fraction: ceil(hot_frac * n), evaluated in double."""
    return int(math.ceil(float(hot_frac) * n))


def permutation(counts, n_hot):
    """perm[new] = old: n_hot hottest first (count desc, index asc), then the rest ascending."""
    counts = _c(np.asarray(counts, np.int64))
    n = counts.shape[0]
    perm = np.empty(n, np.int32)
    _check(load().oracle_permutation(_ptr(counts), n, int(n_hot), _ptr(perm)), "permutation")
    return perm


def pack_rows(src, perm):
    """dst[i] = src[perm[i]] row by row (byte copy); src is any array with rows on axis 0."""
    src = np.ascontiguousarray(src)
    perm = _c(np.asarray(perm, np.int32))
    rows = src.shape[0]
    assert perm.shape == (rows,)
    dst = np.empty_like(src)
    row_bytes = src.nbytes // rows
    _check(load().oracle_pack_rows(_ptr(src), _ptr(perm), _ptr(dst), rows, row_bytes), "pack_rows")
    return dst
