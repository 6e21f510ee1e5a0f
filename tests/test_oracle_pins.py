"""Pins for the CPU oracle: hand-worked cases, closed forms, exact brute force
and invariants.  Each test checks the oracle against something other than the
oracle itself (a hand derivation, a closed form, an exact enumeration, or an
independent library), chosen so that a dropped term, a wrong sign or index, a
transposed operand or a reversed tie-break fails at least one of them."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import lu_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
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


def _mat(rows, dtype):
    return np.array([[_num(x) for x in r] for r in rows], dtype=dtype)


def _flat_colmajor(M):
    return np.ascontiguousarray(M.T).reshape(-1).copy()


def _factor_one(M):
    n = M.shape[0]
    flat = _flat_colmajor(M)
    ipiv, info, margins, _ = oracle.getrf(flat, n, n, n * n, 1, want_margins=True)
    return oracle.matrix(flat, 0, n, n, n, n * n), ipiv[0], int(info[0]), margins[0]


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view({4: np.uint32, 8: np.uint64, 16: np.uint64}[a.dtype.itemsize])


def _cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        for dt in c["dtypes"]:
            yield pytest.param(c, DT[dt], id=f"{c['name']}-{dt}")


@pytest.mark.parametrize("case,dtype", list(_cases()))
def test_hand_worked(case, dtype):
    A = _mat(case["A"], dtype)
    LU, ipiv, info, _ = _factor_one(A)
    assert list(ipiv) == case["ipiv"]
    assert info == case["info"]
    if case["LU"] is not None:
        want = _mat(case["LU"], dtype)
        # bit for bit: -0 differs from +0, and a last-bit difference fails
        assert np.array_equal(_bits(LU), _bits(want)), f"LU {LU!r} != {want!r}"
    if "B" in case:
        n = A.shape[0]
        B = _mat(case["B"], dtype)
        flatA = _flat_colmajor(A)
        flatB = _flat_colmajor(B)
        ipiv2, info2, _, _ = oracle.gesv(flatA, n, n, n * n, flatB, B.shape[1], n, n * B.shape[1], 1)
        X = oracle.matrix(flatB, 0, n, B.shape[1], n, n * B.shape[1])
        assert np.array_equal(_bits(X), _bits(_mat(case["X"], dtype))), f"X {X!r}"


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype,n", [(np.float32, 8), (np.float32, 32), (np.float64, 50), (np.complex64, 20)])
def test_wilkinson_growth_matrix(dtype, n):
    """1 on the diagonal, -1 below, 1 in the last column: every pivot step is a
    tie resolved to the diagonal, L is the -1 pattern and the last column of U
    doubles at each row (2^i), exactly."""
    W = np.tril(-np.ones((n, n)), -1) + np.eye(n)
    W[:, -1] = 1
    LU, ipiv, info, margins = _factor_one(W.astype(dtype))
    assert list(ipiv) == list(range(1, n + 1))
    assert info == 0
    L, U = oracle.unpack(LU)
    np.testing.assert_array_equal(L, (np.tril(-np.ones((n, n)), -1) + np.eye(n)).astype(dtype))
    expect_u = np.eye(n)
    expect_u[:, -1] = 2.0 ** np.arange(n)
    np.testing.assert_array_equal(U, expect_u.astype(dtype))
    assert np.all(margins[:-1] == 1.0)


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [1, 5, 17, 40])
def test_permutation_matrix(dtype, n):
    """A = a permutation matrix: L = U = I and the recorded transpositions
    rebuild exactly the rows of A."""
    rng = np.random.default_rng(1000 + n)
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype)
    P[np.arange(n), perm] = 1
    LU, ipiv, info, _ = _factor_one(P)
    assert info == 0
    np.testing.assert_array_equal(LU, np.eye(n, dtype=dtype))
    order = oracle.perm_from_ipiv(ipiv, n)
    np.testing.assert_array_equal(P[order], np.eye(n, dtype=dtype))


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64])
def test_upper_triangular_is_its_own_factor(dtype):
    rng = np.random.default_rng(7)
    n = 24
    U = np.triu(rng.uniform(-1, 1, (n, n))).astype(dtype)
    if np.iscomplexobj(U):
        U = U + 1j * np.triu(rng.uniform(-1, 1, (n, n))).astype(dtype)
    np.fill_diagonal(U, 2.0)
    LU, ipiv, info, _ = _factor_one(U)
    assert list(ipiv) == list(range(1, n + 1)) and info == 0
    np.testing.assert_array_equal(LU, U)


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
def test_column_diagonally_dominant_never_swaps(dtype):
    """Classical result: a column diagonally dominant matrix needs no row
    interchange under partial pivoting."""
    rng = np.random.default_rng(11)
    n = 33
    A = rng.uniform(-1, 1, (n, n))
    np.fill_diagonal(A, 0)
    A[np.diag_indices(n)] = np.abs(A).sum(axis=0) * 1.5 + 1
    LU, ipiv, info, _ = _factor_one(A.astype(dtype))
    assert list(ipiv) == list(range(1, n + 1)) and info == 0


def test_integer_solve_is_exact():
    """A unimodular integer matrix with an integer solution: the solve is exact
    in double (all intermediate values small integers / dyadics)."""
    A = np.array([[2, 1, 0, 0], [4, 3, 1, 0], [0, 2, 2, 1], [0, 0, 4, 3]], np.float64)
    x = np.array([[1, -2], [3, 0], [-1, 5], [2, 1]], np.float64)
    b = A @ x
    flatA, flatB = _flat_colmajor(A), _flat_colmajor(b)
    _, info, _, _ = oracle.gesv(flatA, 4, 4, 16, flatB, 2, 4, 8, 1)
    assert info[0] == 0
    np.testing.assert_allclose(oracle.matrix(flatB, 0, 4, 2, 4, 8), x, rtol=0, atol=1e-14)


# --------------------------------------------------- exact brute force (n <= 4)

def _exact(v):
    if isinstance(v, (complex, np.complexfloating)):
        return (Fraction(float(v.real)), Fraction(float(v.imag)))
    return (Fraction(float(v)), Fraction(0))


def _cmul(a, b):
    return (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])


def _cdiv(a, b):
    d = b[0] * b[0] + b[1] * b[1]
    return ((a[0] * b[0] + a[1] * b[1]) / d, (a[1] * b[0] - a[0] * b[1]) / d)


def _csub(a, b):
    return (a[0] - b[0], a[1] - b[1])


def _metric(z, is_complex):
    return abs(z[0]) + abs(z[1]) if is_complex else abs(z[0])


def _exact_gepp_orders(M, is_complex):
    """Every row order r (P A = A[r]) under which elimination WITHOUT pivoting,
    in exact rational arithmetic, picks at each step an entry of largest pivot
    metric in its column of the Schur complement.  Returns a list of
    (order, L, U, strict) where strict says every step's maximum was unique."""
    n = M.shape[0]
    out = []
    for order in itertools.permutations(range(n)):
        S = [[_exact(M[i, k]) for k in range(n)] for i in order]
        L = [[(Fraction(int(i == k)), Fraction(0)) for k in range(n)] for i in range(n)]
        ok, strict = True, True
        for j in range(n):
            mj = _metric(S[j][j], is_complex)
            others = [_metric(S[i][j], is_complex) for i in range(j + 1, n)]
            if any(o > mj for o in others) or mj == 0:
                ok = False
                break
            if any(o == mj for o in others):
                strict = False
            for i in range(j + 1, n):
                l = _cdiv(S[i][j], S[j][j])
                L[i][j] = l
                for k in range(j, n):
                    S[i][k] = _csub(S[i][k], _cmul(l, S[j][k]))
        if ok:
            out.append((order, L, S, strict))
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_brute_force_pivot_order(dtype, n):
    """For random inputs the exact partial-pivoting row order is unique; the
    oracle must find it, and its factors must lie within rounding of the exact
    L and U."""
    is_complex = np.dtype(dtype).kind == "c"
    A_all, _ = lu_inputs.random_problem(4242 + n, dtype, n, 0, 30)
    eps = oracle.eps_of(dtype)
    checked = 0
    for b in range(30):
        M = A_all[b * n * n:(b + 1) * n * n].reshape(n, n).T.copy()
        cands = _exact_gepp_orders(M, is_complex)
        LU, ipiv, info, margins = _factor_one(M)
        if len(cands) != 1 or not cands[0][3]:
            continue
        order, Lx, Ux, _ = cands[0]
        if np.max(margins[:-1], initial=0.0) > 1 - 1e3 * eps:
            continue   # rounding could legitimately flip this near-tie
        checked += 1
        assert tuple(oracle.perm_from_ipiv(ipiv, n)) == order
        L, U = oracle.unpack(LU)
        lx = np.array([[complex(float(z[0]), float(z[1])) for z in r] for r in Lx])
        ux = np.array([[complex(float(Ux[i][k][0]), float(Ux[i][k][1])) if k >= i else 0
                        for k in range(n)] for i in range(n)])
        scale = np.max(np.abs(M)) * 8
        assert np.max(np.abs(L - lx)) <= 64 * n * eps * 8
        assert np.max(np.abs(U - ux)) <= 64 * n * eps * scale
    assert checked >= 20


def test_brute_force_sees_ties_in_small_integers():
    """Small-integer matrices produce exact ties; the oracle must pick the
    lowest-position candidate, i.e. the lexicographically first exact order
    among those the enumeration accepts."""
    rng = np.random.default_rng(99)
    seen_tie = 0
    for _ in range(200):
        M = rng.integers(-2, 3, (4, 4)).astype(np.float64)
        cands = _exact_gepp_orders(M, False)
        if not cands:
            continue   # singular: no order with non-zero pivots
        LU, ipiv, info, _ = _factor_one(M)
        if info != 0:
            continue
        order = tuple(oracle.perm_from_ipiv(ipiv, 4))
        assert order in [c[0] for c in cands]
        if len(cands) > 1:
            seen_tie += 1
            # the oracle's choice at each step is the lowest current position:
            # replay the transpositions against the candidates' first rows
            assert order == _lowest_position_order(M, cands)
    assert seen_tie > 10


def _lowest_position_order(M, cands):
    """Walk the steps: among accepted orders consistent with the choices so
    far, the next pivot is the candidate row currently at the lowest position
    (positions move by the transpositions of the earlier steps)."""
    n = M.shape[0]
    current = list(range(n))       # current[pos] = original row
    chosen = []
    for j in range(n):
        allowed = {c[0][j] for c in cands if list(c[0][:j]) == chosen}
        pos = min(p for p in range(j, n) if current[p] in allowed)
        current[j], current[pos] = current[pos], current[j]
        chosen.append(current[j])
    return tuple(chosen)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [1, 7, 32, 65])
def test_invariants_random(dtype, n):
    A_all, _ = lu_inputs.random_problem(77 + n, dtype, n, 0, 6)
    flat = A_all.copy()
    ipiv, info, margins, _ = oracle.getrf(flat, n, n, n * n, 6, want_margins=True)
    is_complex = np.dtype(dtype).kind == "c"
    for b in range(6):
        A = oracle.matrix(A_all, b, n, n, n, n * n)
        LU = oracle.matrix(flat, b, n, n, n, n * n)
        assert info[b] == 0
        assert np.all((ipiv[b] >= np.arange(1, n + 1)) & (ipiv[b] <= n))
        assert np.all((margins[b] >= 0) & (margins[b] <= 1))
        assert oracle.factor_residual(A, LU, ipiv[b]) <= 20
        L, U = oracle.unpack(LU)
        if is_complex:
            # cabs1 pivoting: cabs1(l * u_jj) <= cabs1(u_jj) up to rounding
            cab = lambda z: np.abs(z.real) + np.abs(z.imag)
            lu_j = L * np.diag(U)[None, :]
            assert np.all(cab(np.tril(lu_j, -1)) <= cab(np.diag(U))[None, :] * (1 + 8 * oracle.eps_of(dtype)))
        else:
            assert np.max(np.abs(L)) <= 1.0


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
def test_info_and_singular_structure(dtype):
    """Rank-deficient input: info names the first zero pivot, ipiv stays in
    range and the factorisation still satisfies P A = L U."""
    n = 6
    rng = np.random.default_rng(5)
    A = rng.uniform(-1, 1, (n, n)).astype(dtype)
    A[:, 2] = 0                    # stays exactly zero through steps 0 and 1
    LU, ipiv, info, _ = _factor_one(A)
    U = np.triu(LU)
    zero = [j for j in range(n) if U[j, j] == 0]
    assert info == 3 and zero[0] == 2
    assert ipiv[2] == 3            # tie of zeros: the lowest position
    assert oracle.factor_residual(A, LU, ipiv) <= 20


# -------------------------------------------- independent library cross-check

@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [5, 24, 64])
def test_against_lapack_getrf(dtype, n):
    """LAPACK getrf (scipy) as a secondary check, in the pages' own manner:
    pivots compared up to the first step whose margin is close to 1, and only
    where LAPACK passes its own residual check."""
    scipy_linalg = pytest.importorskip("scipy.linalg")
    A_all, _ = lu_inputs.random_problem(3030 + n, dtype, n, 0, 8)
    eps = oracle.eps_of(dtype)
    flat = A_all.copy()
    ipiv, info, margins, _ = oracle.getrf(flat, n, n, n * n, 8, want_margins=True)
    compared = 0
    for b in range(8):
        A = oracle.matrix(A_all, b, n, n, n, n * n)
        lu_ref, piv_ref = scipy_linalg.lu_factor(A, check_finite=False)
        if oracle.factor_residual(A, lu_ref, piv_ref + 1) > 20:
            continue
        near = np.nonzero(margins[b] > 1 - 64 * n * eps)[0]
        stop = int(near[0]) if near.size else n
        assert list(ipiv[b][:stop]) == list(piv_ref[:stop] + 1)
        compared += stop
        if stop == n:
            LU = oracle.matrix(flat, b, n, n, n, n * n)
            tol = 64 * n * eps * max(1.0, float(np.max(np.abs(lu_ref))))
            assert np.max(np.abs(LU - lu_ref)) <= tol
    assert compared >= 4 * n


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n,nrhs", [(4, 1), (32, 8), (64, 3)])
def test_solve_against_lapack(dtype, n, nrhs):
    A_all, B_all = lu_inputs.random_problem(555 + n, dtype, n, nrhs, 4)
    fa, fb = A_all.copy(), B_all.copy()
    ipiv, info, _, _ = oracle.gesv(fa, n, n, n * n, fb, nrhs, n, n * nrhs, 4)
    for b in range(4):
        A = oracle.matrix(A_all, b, n, n, n, n * n)
        B = oracle.matrix(B_all, b, n, nrhs, n, n * nrhs)
        X = oracle.matrix(fb, b, n, nrhs, n, n * nrhs)
        assert info[b] == 0
        assert oracle.solve_residual(A, X, B) <= 20
        Xref = np.linalg.solve(A.astype(np.complex128 if np.iscomplexobj(A) else np.float64),
                               B.astype(np.complex128 if np.iscomplexobj(B) else np.float64))
        cond = np.linalg.cond(A.astype(np.complex128))
        err = np.max(np.abs(X - Xref)) / np.max(np.abs(Xref))
        assert err <= 64 * n * oracle.eps_of(dtype) * cond


def test_integer_transposed_solve_is_exact():
    """A^T x = b and A^H x = b with a unimodular integer matrix whose
    factorisation swaps rows: exact in double, so undoing the interchanges in
    the wrong order, or taking L^T / U^T from the wrong triangle, fails."""
    A = np.array([[2, 1, 0, 0], [4, 3, 1, 0], [0, 2, 2, 1], [0, 0, 4, 3]], np.float64)
    x = np.array([[1, -2], [3, 0], [-1, 5], [2, 1]], np.float64)
    flatA = _flat_colmajor(A)
    ipiv, info, _, _ = oracle.getrf(flatA, 4, 4, 16, 1)
    assert info[0] == 0 and list(ipiv[0]) != [1, 2, 3, 4]
    for trans in ("T", "C"):
        flatB = _flat_colmajor(A.T @ x)
        oracle.getrs(flatA, 4, 4, 16, ipiv, flatB, 2, 4, 8, 1, trans=trans)
        np.testing.assert_allclose(oracle.matrix(flatB, 0, 4, 2, 4, 8), x, rtol=0, atol=1e-14)
    Ac = A + 1j * np.array([[0, 1, 0, 0], [1, 0, 0, 0], [0, 0, 1, 0], [0, 1, 0, 2]])
    xc = x + 1j * x[::-1]
    flatA = _flat_colmajor(Ac.astype(np.complex128))
    ipiv, info, _, _ = oracle.getrf(flatA, 4, 4, 16, 1)
    assert info[0] == 0
    for trans, op in (("T", Ac.T), ("C", Ac.conj().T)):
        flatB = _flat_colmajor(op @ xc)
        oracle.getrs(flatA, 4, 4, 16, ipiv, flatB, 2, 4, 8, 1, trans=trans)
        np.testing.assert_allclose(oracle.matrix(flatB, 0, 4, 2, 4, 8), xc, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n,nrhs", [(5, 1), (40, 3)])
@pytest.mark.parametrize("trans", ["T", "C"])
def test_transposed_solve_against_lapack(dtype, n, nrhs, trans):
    A_all, B_all = lu_inputs.random_problem(808 + n, dtype, n, nrhs, 3)
    fa, fb = A_all.copy(), B_all.copy()
    ipiv, info, _, _ = oracle.getrf(fa, n, n, n * n, 3)
    oracle.getrs(fa, n, n, n * n, ipiv, fb, nrhs, n, n * nrhs, 3, trans=trans)
    wide = np.complex128 if np.iscomplexobj(A_all) else np.float64
    for b in range(3):
        A = oracle.matrix(A_all, b, n, n, n, n * n).astype(wide)
        op = A.T if trans == "T" else A.conj().T
        B = oracle.matrix(B_all, b, n, nrhs, n, n * nrhs).astype(wide)
        X = oracle.matrix(fb, b, n, nrhs, n, n * nrhs)
        assert info[b] == 0
        Xref = np.linalg.solve(op, B)
        err = np.max(np.abs(X - Xref)) / np.max(np.abs(Xref))
        assert err <= 64 * n * oracle.eps_of(dtype) * np.linalg.cond(op)


def test_integer_inverse_is_exact():
    """A unimodular integer matrix (det -1) whose factorisation swaps rows and
    whose pivots are powers of two (4, 1, 2, 1/8): every intermediate value
    is dyadic, so getri reproduces the integer inverse exactly in double and
    a wrong interchange order or a transposed operand fails."""
    A = np.array([[-2, 1, -4, -1], [2, 1, -3, 3], [1, 1, -2, -1], [4, 0, 3, -1]], np.float64)
    Ainv = np.round(np.linalg.inv(A))
    np.testing.assert_array_equal(A @ Ainv, np.eye(4))   # the inverse is integral
    flatA = _flat_colmajor(A)
    ipiv, info, _, _ = oracle.getrf(flatA, 4, 4, 16, 1)
    assert info[0] == 0 and list(ipiv[0]) != [1, 2, 3, 4]
    C = np.full(6 * 4 + 3, 9.0)
    oracle.getri(flatA, 4, 4, 16, ipiv, C, 6, 27, 1)
    np.testing.assert_array_equal(oracle.matrix(C, 0, 4, 4, 6, 27), Ainv)
    assert np.all(C[[4, 5, 10, 11, 16, 17, 22, 23, 24, 25, 26]] == 9.0)   # pads untouched


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [1, 6, 37])
def test_inverse_against_lapack(dtype, n):
    A_all, _ = lu_inputs.random_problem(4242 + n, dtype, n, 0, 3)
    fa = A_all.copy()
    ipiv, info, _, _ = oracle.getrf(fa, n, n, n * n, 3)
    C = np.zeros(3 * n * n, dtype)
    oracle.getri(fa, n, n, n * n, ipiv, C, n, n * n, 3)
    wide = np.complex128 if np.iscomplexobj(A_all) else np.float64
    for b in range(3):
        A = oracle.matrix(A_all, b, n, n, n, n * n).astype(wide)
        ref = np.linalg.inv(A)
        X = oracle.matrix(C, b, n, n, n, n * n)
        err = np.max(np.abs(X - ref)) / np.max(np.abs(ref))
        assert err <= 64 * n * oracle.eps_of(dtype) * np.linalg.cond(A)


def test_gesv_leaves_b_for_singular_matrix():
    A = np.array([[1, 2], [2, 4]], np.float32)
    B = np.array([[3.0], [7.0]], np.float32)
    fa, fb = _flat_colmajor(A), _flat_colmajor(B)
    ipiv, info, _, _ = oracle.gesv(fa, 2, 2, 4, fb, 1, 2, 2, 1)
    assert info[0] == 2
    np.testing.assert_array_equal(fb, [3.0, 7.0])


def test_padded_layout_and_strides_are_respected():
    """ld > n and a batch stride larger than ld*n: the pad is never touched."""
    n, lda, sA, batch = 5, 8, 50, 3
    A_all, _ = lu_inputs.random_problem(8, np.float64, n, 0, batch)
    dense = A_all.copy()
    ip1, info1, _, _ = oracle.getrf(dense, n, n, n * n, batch)
    padded = lu_inputs.relayout(A_all, n, n, batch, n, n * n, lda, sA, poison=1e300)
    ip2, info2, _, _ = oracle.getrf(padded, n, lda, sA, batch)
    np.testing.assert_array_equal(ip1, ip2)
    back = lu_inputs.relayout(padded, n, n, batch, lda, sA, n, n * n)
    np.testing.assert_array_equal(back, dense)
    mask = np.ones(padded.size, bool)
    for b in range(batch):
        for j in range(n):
            mask[b * sA + j * lda: b * sA + j * lda + n] = False
    assert np.all(padded[mask] == 1e300)
