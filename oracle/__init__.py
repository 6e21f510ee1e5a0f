"""CPU oracle for batched LU with partial pivoting, getrs and gesv, and for
batched Cholesky (potrf, potrs, posv).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports it,
and it imports nothing from the product package.

The arithmetic lives in ``lu_oracle.c`` and ``chol_oracle.c`` (plain C,
working precision, explicit fma, built with ``-ffp-contract=off``); this
module builds and loads them and adds numpy helpers for unpacking factors and
for residual checks.  Which passage of the BatchLAS pages each step follows
is stated in the C files.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "lu_oracle.c"), os.path.join(_HERE, "chol_oracle.c"),
         os.path.join(_HERE, "lu_rect_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DTYPES = {"s": (0, np.float32), "d": (1, np.float64), "c": (2, np.complex64), "z": (3, np.complex128)}
_CODE_OF = {np.dtype(v[1]): v[0] for v in DTYPES.values()}


def build(force: bool = False) -> str:
    """Compile the oracle's C sources into liboracle.so with gcc (no fused
    contraction)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(s) for s in _SRCS)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread"] + _SRCS + ["-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            vp, ip, dp, i32, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
            lib.oracle_getrf_batch.argtypes = [i32, i32, vp, i32, i64, ip, i64, ip, dp, i32, i32]
            lib.oracle_getrf_batch.restype = i32
            lib.oracle_getrs_batch.argtypes = [i32, i32, i32, vp, i32, i64, ip, i64, vp, i32, i64, i32, i32]
            lib.oracle_getrs_batch.restype = i32
            lib.oracle_getrs_trans_batch.argtypes = [i32, i32, i32, i32, vp, i32, i64, ip, i64, vp, i32, i64,
                                                     i32, i32]
            lib.oracle_getrs_trans_batch.restype = i32
            lib.oracle_getri_batch.argtypes = [i32, i32, vp, i32, i64, ip, i64, vp, i32, i64, i32, i32]
            lib.oracle_getri_batch.restype = i32
            lib.oracle_gesv_batch.argtypes = [i32, i32, i32, vp, i32, i64, ip, i64, vp, i32, i64, ip, dp, i32, i32]
            lib.oracle_gesv_batch.restype = i32
            lib.oracle_chol_batch.argtypes = [i32, i32, i32, i32, i32, vp, i32, i64, ip, vp, i32, i64, i32, i32]
            lib.oracle_chol_batch.restype = i32
            lib.oracle_getrf_rect_batch.argtypes = [i32, i32, i32, vp, i32, i64, ip, i64, ip, dp, i32, i32]
            lib.oracle_getrf_rect_batch.restype = i32
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _code(a: np.ndarray) -> int:
    try:
        return _CODE_OF[a.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {a.dtype}") from None


def _check_flat(a, need, name):
    if not (isinstance(a, np.ndarray) and a.ndim == 1 and a.flags.c_contiguous):
        raise ValueError(f"{name} must be a 1-D contiguous numpy array")
    if a.size < need:
        raise ValueError(f"{name} too small: {a.size} < {need}")


def getrf(A, n, lda, strideA, batch, strideP=None, want_margins=False, nthreads=0):
    """Factor ``batch`` matrices stored in the flat column-major buffer ``A``
    (element (i, j) of matrix b at ``b*strideA + i + j*lda``) in place.

    Returns ``(ipiv, info, margins, threads_used)``; ipiv is int32
    (batch, strideP) 1-based, info int32 (batch,), margins float64
    (batch, n) or None."""
    strideP = n if strideP is None else strideP
    if batch > 0 and n > 0:
        _check_flat(A, (batch - 1) * strideA + (n - 1) * lda + n, "A")
    ipiv = np.zeros((max(batch, 0), max(strideP, 1)), np.int32)
    info = np.zeros(max(batch, 0), np.int32)
    margins = np.zeros((max(batch, 0), max(n, 1)), np.float64) if want_margins else None
    used = _load().oracle_getrf_batch(_code(A), n, _ptr(A), lda, strideA, _ptr(ipiv), ipiv.shape[1],
                                      _ptr(info), _ptr(margins), batch, nthreads)
    return ipiv[:, :max(n, 0)] if strideP == n else ipiv, info, margins, used


def getrs(LU, n, lda, strideA, ipiv, B, nrhs, ldb, strideB, batch, nthreads=0, trans="N"):
    """Solve op(A) X = B in place of ``B`` from the oracle's (or any) LU + ipiv;
    op is A for trans 'N', A^T for 'T', A^H for 'C' (A^T for real types)."""
    ipiv = np.ascontiguousarray(ipiv, dtype=np.int32).reshape(batch, -1)
    code = {"N": 0, "T": 1, "C": 2}[trans.upper()]
    if batch > 0 and n > 0 and nrhs > 0:
        _check_flat(B, (batch - 1) * strideB + (nrhs - 1) * ldb + n, "B")
        if LU.dtype != B.dtype:
            raise TypeError("LU and B dtypes differ")
    if code == 0:
        return _load().oracle_getrs_batch(_code(B), n, nrhs, _ptr(LU), lda, strideA, _ptr(ipiv), ipiv.shape[1],
                                          _ptr(B), ldb, strideB, batch, nthreads)
    return _load().oracle_getrs_trans_batch(_code(B), code, n, nrhs, _ptr(LU), lda, strideA, _ptr(ipiv),
                                            ipiv.shape[1], _ptr(B), ldb, strideB, batch, nthreads)


def getri(LU, n, lda, strideA, ipiv, C, ldc, strideC, batch, nthreads=0):
    """C = A^{-1} (out of place) from the oracle's (or any) LU + ipiv."""
    ipiv = np.ascontiguousarray(ipiv, dtype=np.int32).reshape(batch, -1)
    if batch > 0 and n > 0:
        _check_flat(C, (batch - 1) * strideC + (n - 1) * ldc + n, "C")
        if LU.dtype != C.dtype:
            raise TypeError("LU and C dtypes differ")
    return _load().oracle_getri_batch(_code(C), n, _ptr(LU), lda, strideA, _ptr(ipiv), ipiv.shape[1],
                                      _ptr(C), ldc, strideC, batch, nthreads)


def gesv(A, n, lda, strideA, B, nrhs, ldb, strideB, batch, want_margins=False, nthreads=0):
    """getrf then getrs for every matrix whose info is 0 (B left as is otherwise)."""
    if batch > 0 and n > 0:
        _check_flat(A, (batch - 1) * strideA + (n - 1) * lda + n, "A")
        if nrhs > 0:
            _check_flat(B, (batch - 1) * strideB + (nrhs - 1) * ldb + n, "B")
    ipiv = np.zeros((max(batch, 0), max(n, 1)), np.int32)
    info = np.zeros(max(batch, 0), np.int32)
    margins = np.zeros((max(batch, 0), max(n, 1)), np.float64) if want_margins else None
    used = _load().oracle_gesv_batch(_code(A), n, nrhs, _ptr(A), lda, strideA, _ptr(ipiv), n, _ptr(B), ldb,
                                     strideB, _ptr(info), _ptr(margins), batch, nthreads)
    return ipiv[:, :max(n, 0)], info, margins, used


def getrf_rect(A, m, n, lda, strideA, batch, strideP=None, want_margins=False, nthreads=0):
    """LU with partial pivoting of ``batch`` m x n matrices in place (min(m, n)
    steps).  Returns ``(ipiv (batch, strideP), info, margins, threads_used)``;
    ipiv holds min(m, n) 1-based entries per matrix."""
    k = min(m, n)
    strideP = max(k, 1) if strideP is None else strideP
    if batch > 0 and m > 0 and n > 0:
        _check_flat(A, (batch - 1) * strideA + (n - 1) * lda + m, "A")
    ipiv = np.zeros((max(batch, 0), max(strideP, 1)), np.int32)
    info = np.zeros(max(batch, 0), np.int32)
    margins = np.zeros((max(batch, 0), max(k, 1)), np.float64) if want_margins else None
    used = _load().oracle_getrf_rect_batch(_code(A), m, n, _ptr(A), lda, strideA, _ptr(ipiv), ipiv.shape[1],
                                           _ptr(info), _ptr(margins), batch, nthreads)
    return ipiv[:, :k], info, margins, used


def _uplo(uplo):
    u = uplo.upper()
    if u not in ("L", "U"):
        raise ValueError("uplo must be 'L' or 'U'")
    return 1 if u == "U" else 0


def potrf(A, n, lda, strideA, batch, uplo="L", nthreads=0):
    """Cholesky factor of ``batch`` Hermitian positive definite matrices in
    place: 'L' overwrites the lower triangle with L (A = L L^H), 'U' the
    upper with U (A = U^H U); the other triangle is neither read nor written.
    Returns ``(info, threads_used)``; info[b] = j + 1 for the first column
    whose diagonal value is not positive (the factorisation stops there)."""
    if batch > 0 and n > 0:
        _check_flat(A, (batch - 1) * strideA + (n - 1) * lda + n, "A")
    info = np.zeros(max(batch, 0), np.int32)
    used = _load().oracle_chol_batch(0, _code(A), _uplo(uplo), n, 0, _ptr(A), lda, strideA, _ptr(info),
                                     None, 1, 0, batch, nthreads)
    return info, used


def potrs(F, n, lda, strideA, B, nrhs, ldb, strideB, batch, uplo="L", nthreads=0):
    """Solve A X = B in place of ``B`` from the Cholesky factor in ``F``."""
    if batch > 0 and n > 0 and nrhs > 0:
        _check_flat(B, (batch - 1) * strideB + (nrhs - 1) * ldb + n, "B")
        if F.dtype != B.dtype:
            raise TypeError("factor and B dtypes differ")
    return _load().oracle_chol_batch(1, _code(B), _uplo(uplo), n, nrhs, _ptr(F), lda, strideA, None,
                                     _ptr(B), ldb, strideB, batch, nthreads)


def posv(A, n, lda, strideA, B, nrhs, ldb, strideB, batch, uplo="L", nthreads=0):
    """potrf, then potrs for every matrix whose info is 0 (B left as is
    otherwise).  Returns ``(info, threads_used)``."""
    if batch > 0 and n > 0:
        _check_flat(A, (batch - 1) * strideA + (n - 1) * lda + n, "A")
        if nrhs > 0:
            _check_flat(B, (batch - 1) * strideB + (nrhs - 1) * ldb + n, "B")
    info = np.zeros(max(batch, 0), np.int32)
    used = _load().oracle_chol_batch(2, _code(A), _uplo(uplo), n, nrhs, _ptr(A), lda, strideA, _ptr(info),
                                     _ptr(B), ldb, strideB, batch, nthreads)
    return info, used


# ---------------------------------------------------------------------------
# views and checks (numpy, double or extended precision)
# ---------------------------------------------------------------------------

def matrix(flat, b, rows, cols, ld, stride):
    """Copy of matrix ``b`` (rows x cols) out of a flat column-major buffer."""
    base = b * stride
    return np.array(np.lib.stride_tricks.as_strided(flat[base:], shape=(rows, cols),
                                                    strides=(flat.itemsize, ld * flat.itemsize)))


def unpack(LU):
    """Unit-lower L and upper U of a square packed factor."""
    n = LU.shape[0]
    L = np.tril(LU, -1) + np.eye(n, dtype=LU.dtype)
    U = np.triu(LU)
    return L, U


def perm_from_ipiv(ipiv, n):
    """Row order after applying the transpositions ipiv[0..n) (1-based) in turn:
    (P A)[i] = A[perm[i]]."""
    perm = np.arange(n)
    for k in range(n):
        p = int(ipiv[k]) - 1
        perm[k], perm[p] = perm[p], perm[k]
    return perm


_EPS = {np.dtype(np.float32): 2.0 ** -23, np.dtype(np.complex64): 2.0 ** -23,
        np.dtype(np.float64): 2.0 ** -52, np.dtype(np.complex128): 2.0 ** -52}


def eps_of(dtype) -> float:
    """Machine epsilon of the working precision (2^-23 single, 2^-52 double)."""
    return _EPS[np.dtype(dtype)]


def _wide(x):
    x = np.asarray(x)
    if x.dtype in (np.float64, np.complex128):
        return x.astype(np.clongdouble if np.iscomplexobj(x) else np.longdouble)
    return x.astype(np.complex128 if np.iscomplexobj(x) else np.float64)


def factor_residual(A, LU, ipiv):
    """||P A - L U||_F / (n eps ||A||_F) in wider precision than the data."""
    n = A.shape[0]
    if n == 0:
        return 0.0
    L, U = unpack(_wide(LU))
    PA = _wide(A)[perm_from_ipiv(ipiv, n)]
    num = np.sqrt(np.sum(np.abs(PA - L @ U) ** 2))
    den = n * eps_of(A.dtype) * np.sqrt(np.sum(np.abs(_wide(A)) ** 2))
    return float(num / den) if den > 0 else float(num)


def solve_residual(A, X, B):
    """max_j ||A x_j - b_j||_inf / (n eps ||A||_inf ||x_j||_inf)."""
    n = A.shape[0]
    if n == 0 or X.shape[1] == 0:
        return 0.0
    Aw, Xw, Bw = _wide(A), _wide(X), _wide(B)
    R = Aw @ Xw - Bw
    anorm = np.max(np.sum(np.abs(Aw), axis=1))
    worst = 0.0
    for j in range(X.shape[1]):
        den = n * eps_of(A.dtype) * anorm * np.max(np.abs(Xw[:, j]))
        num = np.max(np.abs(R[:, j]))
        worst = max(worst, float(num / den) if den > 0 else float(num))
    return worst


def hermitian_from(A, uplo="L"):
    """The full Hermitian matrix whose named triangle is that of ``A`` (the
    diagonal's imaginary part is dropped, as potrf never reads it)."""
    n = A.shape[0]
    T = np.tril(A) if uplo.upper() == "L" else np.triu(A).conj().T
    H = T + np.tril(T, -1).conj().T
    H[np.diag_indices(n)] = H.diagonal().real
    return H


def chol_factor(F, uplo="L"):
    """The lower factor L (A = L L^H) held in the named triangle of ``F``."""
    return np.tril(F) if uplo.upper() == "L" else np.triu(F).conj().T


def chol_residual(A, F, uplo="L"):
    """||A - L L^H||_F / (n eps ||A||_F) in wider precision, A taken as the
    Hermitian matrix of its named triangle."""
    n = A.shape[0]
    if n == 0:
        return 0.0
    H = _wide(hermitian_from(A, uplo))
    L = _wide(chol_factor(F, uplo))
    num = np.sqrt(np.sum(np.abs(H - L @ L.conj().T) ** 2))
    den = n * eps_of(A.dtype) * np.sqrt(np.sum(np.abs(H) ** 2))
    return float(num / den) if den > 0 else float(num)


def rect_residual(A, LU, ipiv):
    """||P A - L U||_F / (max(m, n) eps ||A||_F) for an m x n factorisation
    (L m x k unit lower trapezoidal, U k x n upper trapezoidal, k = min(m, n))."""
    m, n = A.shape
    k = min(m, n)
    if k == 0:
        return 0.0
    W = _wide(LU)
    L = np.tril(W[:, :k], -1) + np.eye(m, k, dtype=W.dtype)
    U = np.triu(W[:k, :])
    perm = np.arange(m)
    for j in range(k):
        p = int(ipiv[j]) - 1
        perm[j], perm[p] = perm[p], perm[j]
    PA = _wide(A)[perm]
    num = np.sqrt(np.sum(np.abs(PA - L @ U) ** 2))
    den = max(m, n) * eps_of(A.dtype) * np.sqrt(np.sum(np.abs(_wide(A)) ** 2))
    return float(num / den) if den > 0 else float(num)
