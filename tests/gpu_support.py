"""Helpers for GPU parity tests: move flat host buffers to the device, call
the C ABI through the binding, bring results back, and compare them with the
CPU oracle run on the same bytes."""
from __future__ import annotations

import numpy as np

import oracle

try:
    import torch
except Exception:      # pragma: no cover - torch is part of the image
    torch = None

TORCH_DT = {np.dtype(np.float32): "float32", np.dtype(np.float64): "float64",
            np.dtype(np.complex64): "complex64", np.dtype(np.complex128): "complex128"}


def gpu_available() -> bool:
    return torch is not None and torch.cuda.is_available()


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns, so that -0 and +0 differ.  Every NaN is first mapped
    to one canonical NaN: the position of a NaN is part of the result, its
    sign and payload are not (x86 and gfx950 produce different default NaNs)."""
    a = np.array(a, copy=True, order="C")
    real = a.view(np.float32 if a.dtype in (np.float32, np.complex64) else np.float64)
    real[np.isnan(real)] = np.nan
    return a.view({4: np.uint32, 8: np.uint64, 16: np.uint64}[a.dtype.itemsize])


def gesv_gpu(lib, A, B, n, nrhs, batch, lda=None, sA=None, ldb=None, sB=None, sP=None, op="gesv"):
    """Run gesv (or getrf / getrf then getrs) on copies of the flat host
    buffers; returns (A_out, B_out, ipiv (batch, sP), info)."""
    lda = n if lda is None else lda
    ldb = n if ldb is None else ldb
    sA = lda * n if sA is None else sA
    sB = ldb * nrhs if sB is None else sB
    sP = n if sP is None else sP
    t = lib.dtype_code(A.dtype)
    dA = to_dev(A)
    dB = to_dev(B) if B is not None and B.size else to_dev(np.zeros(1, A.dtype))
    dP = torch.full((max(batch, 1) * max(sP, 1),), -7, dtype=torch.int32, device="cuda")
    dI = torch.full((max(batch, 1),), -7, dtype=torch.int32, device="cuda")
    if op == "gesv":
        lib.batchlu_gesv(t, n, nrhs, dA, lda, sA, dP, sP, dB, ldb, sB, dI, batch)
    elif op == "getrf":
        lib.batchlu_getrf(t, n, dA, lda, sA, dP, sP, dI, batch)
    elif op == "getrf+getrs":
        lib.batchlu_getrf(t, n, dA, lda, sA, dP, sP, dI, batch)
        lib.batchlu_getrs(t, "N", n, nrhs, dA, lda, sA, dP, sP, dB, ldb, sB, batch)
    else:
        raise ValueError(op)
    torch.cuda.synchronize()
    return to_host(dA), to_host(dB), to_host(dP).reshape(max(batch, 1), max(sP, 1)), to_host(dI)


def oracle_run(A, B, n, nrhs, batch, lda=None, sA=None, ldb=None, sB=None, op="gesv"):
    lda = n if lda is None else lda
    ldb = n if ldb is None else ldb
    sA = lda * n if sA is None else sA
    sB = ldb * nrhs if sB is None else sB
    a = A.copy()
    b = B.copy() if B is not None else None
    if op == "gesv":
        ipiv, info, margins, _ = oracle.gesv(a, n, lda, sA, b, nrhs, ldb, sB, batch, want_margins=True)
    else:
        ipiv, info, margins, _ = oracle.getrf(a, n, lda, sA, batch, want_margins=True)
        if op == "getrf+getrs":
            oracle.getrs(a, n, lda, sA, ipiv, b, nrhs, ldb, sB, batch)
    return a, b, ipiv, info, margins


def matrices_equal_bits(X, Y, n, cols, ld, stride, batch):
    """Element-wise bit equality of the n x cols blocks of two flat buffers;
    returns the list of matrix indices that differ."""
    bad = []
    for b in range(batch):
        x = oracle.matrix(X, b, n, cols, ld, stride)
        y = oracle.matrix(Y, b, n, cols, ld, stride)
        if not np.array_equal(bits(x), bits(y)):
            bad.append(b)
    return bad
