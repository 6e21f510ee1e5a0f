"""Pins for the Cholesky part of the CPU oracle (potrf, potrs, posv).

Each test checks the oracle against something other than the oracle itself:
hand-worked cases whose last bits depend on each reading (tests/golden/
chol_hand_worked.json), closed forms whose factor and solution are exact
integers (the symmetric Pascal matrix, complex integer factors), and LAPACK
through numpy as a secondary check within the residual bound.  The
triangle that uplo does not name is filled with NaN and must come back
untouched, which also shows that it is never read."""
import json
import math
import os

import numpy as np
import pytest

import lu_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chol_hand_worked.json")
DT = {"float32": np.float32, "float64": np.float64, "complex64": np.complex64, "complex128": np.complex128}


def _num(v):
    if isinstance(v, list):
        return complex(_num(v[0]), _num(v[1]))
    if isinstance(v, str):
        if v.startswith("f32:0x"):
            return float(np.array([int(v[4:], 16)], np.uint32).view(np.float32)[0])
        if v.startswith("f64:0x"):
            return float(np.array([int(v[4:], 16)], np.uint64).view(np.float64)[0])
        if "*2^" in v:
            m, e = v.split("*2^")
            return math.ldexp(float(m), int(e))
        return float(v)
    return float(v)


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view({4: np.uint32, 8: np.uint64, 16: np.uint64}[a.dtype.itemsize])


def _same(got, want):
    """Bit equality of two scalars of one dtype, any NaN matching any NaN."""
    g = np.array([got]).view(np.float32 if got.dtype in (np.float32, np.complex64) else np.float64)
    w = np.array([want], got.dtype).view(g.dtype)
    return all((np.isnan(a) and np.isnan(b)) or _bits(np.array([a]))[0] == _bits(np.array([b]))[0]
               for a, b in zip(g, w))


def _poisoned(M, uplo):
    """Column-major flat copy of M whose other triangle is NaN."""
    n = M.shape[0]
    P = M.copy()
    mask = np.triu(np.ones((n, n), bool), 1) if uplo == "L" else np.tril(np.ones((n, n), bool), -1)
    P[mask] = np.nan
    return np.ascontiguousarray(P.T).reshape(-1).copy(), mask


def _cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        for dt in c["dtypes"]:
            yield pytest.param(c, DT[dt], id=f"{c['name']}-{dt}")


@pytest.mark.parametrize("case,dtype", list(_cases()))
def test_hand_worked_case(case, dtype):
    M = np.array([[_num(x) for x in r] for r in case["A"]], dtype=dtype)
    n = M.shape[0]
    uplo = case["uplo"]
    flat, mask = _poisoned(M, uplo)
    before = flat.copy()
    info, _ = oracle.potrf(flat, n, n, n * n, 1, uplo=uplo)
    assert int(info[0]) == case["info"]
    F = oracle.matrix(flat, 0, n, n, n, n * n)
    for i, j, v in case["entries"]:
        assert _same(F[i, j], np.array(_num(v), dtype)), f"entry ({i},{j}) = {F[i, j]!r}, expected {v}"
    # the other triangle is neither read nor written
    after = flat.reshape(n, n).T
    assert np.array_equal(_bits(after[mask]), _bits(before.reshape(n, n).T[mask]))
    if "B" in case:
        B = np.array([[_num(x) for x in r] for r in case["B"]], dtype=dtype)
        nrhs = B.shape[1]
        fb = np.ascontiguousarray(B.T).reshape(-1).copy()
        oracle.potrs(flat, n, n, n * n, fb, nrhs, n, n * nrhs, 1, uplo=uplo)
        X = fb.reshape(nrhs, n).T
        want = np.array([[_num(x) for x in r] for r in case["X"]], dtype=dtype)
        for i in range(n):
            for c in range(nrhs):
                assert _same(X[i, c], want[i, c]), f"X[{i},{c}] = {X[i, c]!r}, expected {case['X'][i][c]}"


def _pascal(n):
    return np.array([[math.comb(i + j, i) for j in range(n)] for i in range(n)], dtype=np.float64)


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("dtype,n", [(np.float32, 10), (np.float64, 20), (np.complex64, 10), (np.complex128, 20)])
def test_pascal_closed_form(dtype, n, uplo):
    """The symmetric Pascal matrix is L L^T with L the lower Pascal matrix of
    binomial coefficients and a unit diagonal: every step of potrf and potrs
    is exact in integers here, so a dropped or misplaced term anywhere shows
    as a wrong integer.  B = A x for x in {-1, 0, 1} comes back as x."""
    P = _pascal(n).astype(dtype)
    Lp = np.array([[math.comb(i, j) if j <= i else 0 for j in range(n)] for i in range(n)], dtype=dtype)
    flat, mask = _poisoned(P, uplo)
    info, _ = oracle.potrf(flat, n, n, n * n, 1, uplo=uplo)
    assert info[0] == 0
    F = oracle.matrix(flat, 0, n, n, n, n * n)
    got = np.tril(F) if uplo == "L" else np.triu(F).T
    assert np.array_equal(got, Lp)
    rng = np.random.default_rng(n)
    x = rng.integers(-1, 2, size=(n, 3)).astype(dtype)
    b = (_pascal(n) @ x.real.astype(np.float64)).astype(dtype)
    fb = np.ascontiguousarray(b.T).reshape(-1).copy()
    oracle.potrs(flat, n, n, n * n, fb, 3, n, n * 3, 1, uplo=uplo)
    assert np.array_equal(fb.reshape(3, n).T, x)


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("dtype", [np.complex64, np.complex128])
def test_complex_integer_closed_form(dtype, uplo):
    """A = L L^H for a complex integer L with diagonal 1 and 2 (so every
    reciprocal is exact): potrf must return L exactly (this fixes where the
    conjugate goes: L L^T or conj(L) L^T give other matrices), and potrs must
    return the complex integer X with B = A X."""
    L = np.array([[1, 0, 0, 0, 0],
                  [1 + 2j, 2, 0, 0, 0],
                  [3 - 1j, 2 + 1j, 1, 0, 0],
                  [-2 + 0j, 1 - 3j, -1 + 1j, 2, 0],
                  [1j, -1 - 1j, 2 + 2j, 3 - 2j, 1]], dtype=np.complex128)
    A = L @ L.conj().T
    n = 5
    flat, mask = _poisoned(A.astype(dtype), uplo)
    info, _ = oracle.potrf(flat, n, n, n * n, 1, uplo=uplo)
    assert info[0] == 0
    F = oracle.matrix(flat, 0, n, n, n, n * n)
    got = np.tril(F) if uplo == "L" else np.triu(F).conj().T
    assert np.array_equal(got, L.astype(dtype))
    X = np.array([[1 + 1j, 0], [-2j, 3], [2, 1 - 1j], [0, -1], [1 - 2j, 2j]], dtype=np.complex128)
    B = (A @ X).astype(dtype)
    fb = np.ascontiguousarray(B.T).reshape(-1).copy()
    oracle.potrs(flat, n, n, n * n, fb, 2, n, n * 2, 1, uplo=uplo)
    assert np.array_equal(fb.reshape(2, n).T, X.astype(dtype))


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [1, 7, 33, 70])
def test_matches_lapack_within_bound(dtype, n, uplo):
    """Secondary: the factor agrees with LAPACK's (numpy.linalg.cholesky) to
    a few units of rounding, the reconstruction and the solve residual are
    within the bound 20, and the diagonal is real and positive."""
    batch, nrhs = 3, 4
    A, B = lu_inputs.spd_problem(500 + n, dtype, n, nrhs, batch)
    F = A.copy()
    info, _ = oracle.potrf(F, n, n, n * n, batch, uplo=uplo)
    assert not info.any()
    X = B.copy()
    oracle.potrs(F, n, n, n * n, X, nrhs, n, n * nrhs, batch, uplo=uplo)
    eps = oracle.eps_of(dtype)
    for b in range(batch):
        Am = oracle.matrix(A, b, n, n, n, n * n)
        Fm = oracle.matrix(F, b, n, n, n, n * n)
        L = oracle.chol_factor(Fm, uplo)
        assert np.all(L.diagonal().real > 0) and np.all(L.diagonal().imag == 0)
        assert oracle.chol_residual(Am, Fm, uplo) <= 20
        ref = np.linalg.cholesky(Am.astype(np.complex128 if np.iscomplexobj(Am) else np.float64))
        assert np.max(np.abs(L - ref)) <= 64 * n * eps * np.max(np.abs(ref))
        res = oracle.solve_residual(oracle.hermitian_from(Am, uplo), oracle.matrix(X, b, n, nrhs, n, n * nrhs),
                                    oracle.matrix(B, b, n, nrhs, n, n * nrhs))
        assert res <= 20


def test_posv_leaves_b_when_not_positive_definite():
    """posv = potrf, then potrs only where info == 0 (B untouched elsewhere)."""
    n, nrhs = 4, 2
    A, B = lu_inputs.spd_problem(9, np.float64, n, nrhs, 3)
    A[n * n + 2 + 2 * n] = -50.0         # matrix 1: a22 very negative
    A0, B0 = A.copy(), B.copy()
    info, _ = oracle.posv(A, n, n, n * n, B, nrhs, n, n * nrhs, 3)
    assert list(info) == [0, 3, 0]
    assert np.array_equal(B[n * nrhs: 2 * n * nrhs], B0[n * nrhs: 2 * n * nrhs])
    F = A0.copy()
    oracle.potrf(F, n, n, n * n, 3)
    X = B0.copy()
    oracle.potrs(F, n, n, n * n, X, nrhs, n, n * nrhs, 3)
    for b in (0, 2):
        assert np.array_equal(B[b * n * nrhs: (b + 1) * n * nrhs], X[b * n * nrhs: (b + 1) * n * nrhs])


def test_zero_order_and_zero_batch():
    A = np.zeros(0, np.float32)
    info, _ = oracle.potrf(A, 0, 1, 0, 2)
    assert list(info) == [0, 0]
    info, _ = oracle.potrf(A, 3, 3, 9, 0)
    assert info.size == 0
