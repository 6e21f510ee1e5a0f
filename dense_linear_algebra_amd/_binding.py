"""ctypes binding of libbatchlu.so: the C ABI under the same names.

Argument marshalling only.  Every step of the computation runs in the HIP
library; a missing library is an error, never a fallback.  Pointer arguments
accept a torch tensor (its data_ptr is passed), a plain int (a device
address) or None (NULL).  ``stream`` accepts a torch.cuda.Stream, an int
handle or None (torch's current stream when torch is initialised on a GPU,
else the null stream).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbatchlu.so")

R32, R64, C64, C128 = 0, 1, 2, 3
TIER_AUTO, TIER_TINY, TIER_CTA, TIER_BLOCKED, TIER_CTA_LDS = 0, 1, 2, 3, 4
TIER_NAMES = {TIER_TINY: "tiny", TIER_CTA: "cta", TIER_BLOCKED: "blocked", TIER_CTA_LDS: "cta_lds"}
OK, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_LAUNCH = 0, -100, -101, -102

_lib = None


class BatchLUError(RuntimeError):
    def __init__(self, func, status):
        self.status = status
        super().__init__(f"{func} returned {status}: {status_string(status)}")


def load():
    """Load libbatchlu.so (built by ``python -m dense_linear_algebra_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dense_linear_algebra_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, ch = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_char
    lib.batchlu_getrf.argtypes = [i32, i32, vp, i32, i64, vp, i64, vp, i32, vp]
    lib.batchlu_getrs.argtypes = [i32, ch, i32, i32, vp, i32, i64, vp, i64, vp, i32, i64, i32, vp]
    lib.batchlu_gesv.argtypes = [i32, i32, i32, vp, i32, i64, vp, i64, vp, i32, i64, vp, i32, vp]
    lib.batchlu_getri.argtypes = [i32, i32, vp, i32, i64, vp, i64, vp, i32, i64, i32, vp]
    lib.batchlu_potrf.argtypes = [i32, ch, i32, vp, i32, i64, vp, i32, vp]
    lib.batchlu_getrf_rect.argtypes = [i32, i32, i32, vp, i32, i64, vp, i64, vp, i32, vp]
    lib.batchlu_getrf_vbatched.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.batchlu_getrs_vbatched.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
    lib.batchlu_gesv_vbatched.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
    lib.batchlu_potrs.argtypes = [i32, ch, i32, i32, vp, i32, i64, vp, i32, i64, i32, vp]
    lib.batchlu_posv.argtypes = [i32, ch, i32, i32, vp, i32, i64, vp, i32, i64, vp, i32, vp]
    lib.batchlu_check_reciprocal.argtypes = [ctypes.c_uint, ctypes.c_uint, vp, vp, vp]
    lib.batchlu_check_reciprocal.restype = i32
    lib.batchlu_select_tier.argtypes = [i32, i32, i32, i32, i32]
    lib.batchlu_set_tier.argtypes = [i32]
    lib.batchlu_status_string.argtypes = [i32]
    lib.batchlu_status_string.restype = ctypes.c_char_p
    lib.batchlu_version.argtypes = []
    lib.batchlu_version.restype = ctypes.c_char_p
    for f in ("batchlu_getrf", "batchlu_getrs", "batchlu_gesv", "batchlu_getri", "batchlu_potrf", "batchlu_potrs",
              "batchlu_posv", "batchlu_getrf_rect", "batchlu_getrf_vbatched", "batchlu_getrs_vbatched",
              "batchlu_gesv_vbatched", "batchlu_select_tier", "batchlu_set_tier"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        try:
            import torch
            if torch.cuda.is_available() and torch.cuda.is_initialized():
                return torch.cuda.current_stream().cuda_stream
        except Exception:
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def dtype_code(dtype) -> int:
    """Library code of a torch or numpy dtype."""
    name = str(dtype).replace("torch.", "")
    codes = {"float32": R32, "float64": R64, "complex64": C64, "complex128": C128}
    if name not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[name]


def _check(func, status, raise_on_error):
    if raise_on_error and status != OK:
        raise BatchLUError(func, status)
    return status


def batchlu_getrf(t, n, A, lda, strideA, ipiv, strideP, info, batch, stream=None, raise_on_error=True):
    st = load().batchlu_getrf(t, n, _ptr(A), lda, strideA, _ptr(ipiv), strideP, _ptr(info), batch, _stream(stream))
    return _check("batchlu_getrf", st, raise_on_error)


def batchlu_getrs(t, trans, n, nrhs, A, lda, strideA, ipiv, strideP, B, ldb, strideB, batch, stream=None,
                  raise_on_error=True):
    tr = trans.encode() if isinstance(trans, str) else bytes([trans])
    st = load().batchlu_getrs(t, tr, n, nrhs, _ptr(A), lda, strideA, _ptr(ipiv), strideP, _ptr(B), ldb, strideB,
                              batch, _stream(stream))
    return _check("batchlu_getrs", st, raise_on_error)


def batchlu_getri(t, n, A, lda, strideA, ipiv, strideP, C, ldc, strideC, batch, stream=None,
                  raise_on_error=True):
    st = load().batchlu_getri(t, n, _ptr(A), lda, strideA, _ptr(ipiv), strideP, _ptr(C), ldc, strideC, batch,
                              _stream(stream))
    return _check("batchlu_getri", st, raise_on_error)


def batchlu_gesv(t, n, nrhs, A, lda, strideA, ipiv, strideP, B, ldb, strideB, info, batch, stream=None,
                 raise_on_error=True):
    st = load().batchlu_gesv(t, n, nrhs, _ptr(A), lda, strideA, _ptr(ipiv), strideP, _ptr(B), ldb, strideB,
                             _ptr(info), batch, _stream(stream))
    return _check("batchlu_gesv", st, raise_on_error)


def batchlu_getrf_rect(t, m, n, A, lda, strideA, ipiv, strideP, info, batch, stream=None, raise_on_error=True):
    st = load().batchlu_getrf_rect(t, m, n, _ptr(A), lda, strideA, _ptr(ipiv), strideP, _ptr(info), batch,
                                   _stream(stream))
    return _check("batchlu_getrf_rect", st, raise_on_error)


def batchlu_getrf_vbatched(t, m, n, A, lda, ipiv, info, max_m, max_n, batch, stream=None, raise_on_error=True):
    """m, n, lda, info: device int32 arrays; A, ipiv: device arrays of device
    pointers (int64 tensors holding the addresses)."""
    st = load().batchlu_getrf_vbatched(t, _ptr(m), _ptr(n), _ptr(A), _ptr(lda), _ptr(ipiv), _ptr(info), max_m,
                                       max_n, batch, _stream(stream))
    return _check("batchlu_getrf_vbatched", st, raise_on_error)


def batchlu_getrs_vbatched(t, n, nrhs, A, lda, ipiv, B, ldb, max_n, batch, stream=None, raise_on_error=True):
    st = load().batchlu_getrs_vbatched(t, _ptr(n), _ptr(nrhs), _ptr(A), _ptr(lda), _ptr(ipiv), _ptr(B), _ptr(ldb),
                                       max_n, batch, _stream(stream))
    return _check("batchlu_getrs_vbatched", st, raise_on_error)


def batchlu_gesv_vbatched(t, n, nrhs, A, lda, ipiv, B, ldb, info, max_n, batch, stream=None, raise_on_error=True):
    st = load().batchlu_gesv_vbatched(t, _ptr(n), _ptr(nrhs), _ptr(A), _ptr(lda), _ptr(ipiv), _ptr(B), _ptr(ldb),
                                      _ptr(info), max_n, batch, _stream(stream))
    return _check("batchlu_gesv_vbatched", st, raise_on_error)


def _uplo(uplo):
    return uplo.encode() if isinstance(uplo, str) else bytes([uplo])


def batchlu_potrf(t, uplo, n, A, lda, strideA, info, batch, stream=None, raise_on_error=True):
    st = load().batchlu_potrf(t, _uplo(uplo), n, _ptr(A), lda, strideA, _ptr(info), batch, _stream(stream))
    return _check("batchlu_potrf", st, raise_on_error)


def batchlu_potrs(t, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, stream=None, raise_on_error=True):
    st = load().batchlu_potrs(t, _uplo(uplo), n, nrhs, _ptr(A), lda, strideA, _ptr(B), ldb, strideB, batch,
                              _stream(stream))
    return _check("batchlu_potrs", st, raise_on_error)


def batchlu_posv(t, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, info, batch, stream=None,
                 raise_on_error=True):
    st = load().batchlu_posv(t, _uplo(uplo), n, nrhs, _ptr(A), lda, strideA, _ptr(B), ldb, strideB, _ptr(info),
                             batch, _stream(stream))
    return _check("batchlu_posv", st, raise_on_error)


def batchlu_check_reciprocal(lo_bits, hi_bits, mismatches, first_bad, stream=None, raise_on_error=True):
    st = load().batchlu_check_reciprocal(lo_bits, hi_bits, _ptr(mismatches), _ptr(first_bad), _stream(stream))
    return _check("batchlu_check_reciprocal", st, raise_on_error)


def batchlu_select_tier(t, op, n, nrhs, batch):
    return load().batchlu_select_tier(t, op, n, nrhs, batch)


def batchlu_set_tier(tier):
    return load().batchlu_set_tier(tier)


def status_string(status):
    return load().batchlu_status_string(status).decode()


def version():
    return load().batchlu_version().decode()
