"""Pins for the rectangular (m x n) LU oracle.

Each test checks the oracle against something other than itself: hand-worked
cases (tests/golden/rect_hand_worked.json) that reach beyond the square part
in both directions (a pivot from a row below n, an update of a column beyond
m), the independently written square oracle on m = n, an exact brute force
over every row order for tiny shapes, and LAPACK's getrf (scipy) as a
secondary, margin-gated check.  A mutation check at the end plants the
plausible rectangular mistakes in a private copy and sees a named pin fail."""
import ctypes
import itertools
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import lu_inputs
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "rect_hand_worked.json")
SRC = os.path.join(os.path.dirname(HERE), "oracle", "lu_rect_oracle.c")
DT = {"float32": np.float32, "float64": np.float64, "complex64": np.complex64, "complex128": np.complex128}


def _flat(M):
    return np.ascontiguousarray(M.T).reshape(-1).copy()


def _fixtures():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def _run_case(getrf, case, dtype):
    M = np.array(case["A"], dtype=dtype)
    m, n = M.shape
    f = _flat(M)
    ipiv, info = getrf(f, m, n)
    return list(ipiv), int(info), f.reshape(n, m).T


def _oracle_getrf(f, m, n):
    ipiv, info, _, _ = oracle.getrf_rect(f, m, n, m, m * n, 1)
    return ipiv[0], info[0]


@pytest.mark.parametrize("name,dtype", [(c["name"], d) for c in _fixtures().values() for d in c["dtypes"]])
def test_hand_worked(name, dtype):
    case = _fixtures()[name]
    ipiv, info, LU = _run_case(_oracle_getrf, case, DT[dtype])
    assert ipiv == case["ipiv"] and info == case["info"]
    if case["LU"] is not None:
        assert np.array_equal(LU, np.array(case["LU"], dtype=DT[dtype]))


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("n", [1, 5, 17, 40])
def test_square_agrees_with_the_square_oracle(dtype, n):
    """Two independently written implementations of the same steps."""
    A, _ = lu_inputs.random_problem(77 + n, dtype, n, 0, 4)
    a1, a2 = A.copy(), A.copy()
    p1, i1, _, _ = oracle.getrf_rect(a1, n, n, n, n * n, 4)
    p2, i2, _, _ = oracle.getrf(a2, n, n, n * n, 4)
    assert np.array_equal(p1, p2) and np.array_equal(i1, i2)
    assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8))


def _exact(v):
    v = complex(v)
    return (Fraction(v.real), Fraction(v.imag))


def _exact_orders(M, is_complex):
    """Row orders under which elimination without pivoting, in exact
    arithmetic, meets a largest-metric pivot at each of the min(m, n) steps;
    (order, strict) pairs, strict when every maximum was unique."""
    m, n = M.shape
    k = min(m, n)
    met = (lambda z: abs(z[0]) + abs(z[1])) if is_complex else (lambda z: abs(z[0]))
    out = []
    seen = set()
    for order in itertools.permutations(range(m)):
        key = order[:k]
        if key in seen:
            continue
        seen.add(key)
        S = [[_exact(M[i, c]) for c in range(n)] for i in order]
        ok, strict = True, True
        for j in range(k):
            mj = met(S[j][j])
            others = [met(S[i][j]) for i in range(j + 1, m)]
            if mj == 0 or any(o > mj for o in others):
                ok = False
                break
            strict = strict and not any(o == mj for o in others)
            d = S[j][j]
            den = d[0] * d[0] + d[1] * d[1]
            for i in range(j + 1, m):
                a = S[i][j]
                l = ((a[0] * d[0] + a[1] * d[1]) / den, (a[1] * d[0] - a[0] * d[1]) / den)
                for c in range(j, n):
                    u = S[j][c]
                    S[i][c] = (S[i][c][0] - (l[0] * u[0] - l[1] * u[1]), S[i][c][1] - (l[0] * u[1] + l[1] * u[0]))
        if ok:
            out.append((key, strict))
    return out


@pytest.mark.parametrize("dtype", [np.float64, np.complex128])
@pytest.mark.parametrize("m,n", [(3, 2), (4, 2), (2, 4), (4, 3), (3, 1), (1, 3)])
def test_brute_force_pivot_order(dtype, m, n):
    """The exact partial-pivoting choice of the first min(m, n) rows is unique
    for random inputs; the oracle must make it."""
    is_complex = np.dtype(dtype).kind == "c"
    rng = np.random.default_rng(m * 10 + n)
    checked = 0
    for _ in range(25):
        M = rng.uniform(-1, 1, (m, n))
        if is_complex:
            M = M + 1j * rng.uniform(-1, 1, (m, n))
        M = M.astype(dtype)
        cands = _exact_orders(M, is_complex)
        f = _flat(M)
        ipiv, info, margins, _ = oracle.getrf_rect(f, m, n, m, m * n, 1, want_margins=True)
        if len(cands) != 1 or not cands[0][1] or np.max(margins[0]) > 1 - 1e-9:
            continue
        perm = list(range(m))
        for j in range(min(m, n)):
            p = int(ipiv[0][j]) - 1
            perm[j], perm[p] = perm[p], perm[j]
        assert tuple(perm[:min(m, n)]) == cands[0][0]
        checked += 1
    assert checked >= 15


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
@pytest.mark.parametrize("m,n", [(50, 20), (20, 50), (64, 63), (100, 3), (3, 100), (129, 257)])
def test_matches_lapack_and_residual(dtype, m, n):
    """Secondary: LAPACK's getrf (scipy) picks the same rows wherever the
    oracle's margins leave room for rounding, |L| <= 1 (cabs1 bound sqrt(2)
    for complex) and P A = L U within the bound 20."""
    scipy_linalg = pytest.importorskip("scipy.linalg")
    batch = 3
    rng = np.random.default_rng(m + 1000 * n)
    eps = oracle.eps_of(dtype)
    for b in range(batch):
        M = rng.uniform(-1, 1, (m, n))
        if np.dtype(dtype).kind == "c":
            M = M + 1j * rng.uniform(-1, 1, (m, n))
        M = M.astype(dtype)
        f = _flat(M)
        ipiv, info, margins, _ = oracle.getrf_rect(f, m, n, m, m * n, 1, want_margins=True)
        LU = f.reshape(n, m).T
        assert info[0] == 0
        assert oracle.rect_residual(M, LU, ipiv[0]) <= 20
        k = min(m, n)
        L = np.tril(LU[:, :k], -1)
        bound = np.sqrt(2) + 1e-6 if np.dtype(dtype).kind == "c" else 1.0
        assert np.max(np.abs(L), initial=0) <= bound
        if np.dtype(dtype).kind != "c" and np.max(margins[0]) < 1 - 1e4 * k * eps:
            _, piv = scipy_linalg.lu_factor(M.astype(np.float64))
            assert np.array_equal(piv[:k] + 1, ipiv[0])


# --------------------------------------------------------------- mutation check

MUTATIONS = [
    ("pivot search stops at row n", [("for (int i = j + 1; i < m; ++i) {                                      \\\n"
                                      "            T v = FABS(A[RT_IDX(i, j)]);",
                                      "for (int i = j + 1; i < n && i < m; ++i) {                             \\\n"
                                      "            T v = FABS(A[RT_IDX(i, j)]);", 1)],
     ["tall_3x2_pivot_from_a_row_below_n"]),
    ("update stops at column m", [("        for (int k = j + 1; k < n; ++k) {                       /* R4 */       \\\n"
                                   "            const T u = A[RT_IDX(j, k)];",
                                   "        for (int k = j + 1; k < n && k < m; ++k) {              /* R4 */       \\\n"
                                   "            const T u = A[RT_IDX(j, k)];", 1)],
     ["wide_2x3_update_reaches_the_extra_column"]),
    ("row swap stops at column m", [("            for (int k = 0; k < n; ++k) {                                      \\\n"
                                     "                T t = A[RT_IDX(j, k)];",
                                     "            for (int k = 0; k < n && k < m; ++k) {                             \\\n"
                                     "                T t = A[RT_IDX(j, k)];", 1)],
     ["tall_3x2_pivot_from_a_row_below_n", "wide_2x3_update_reaches_the_extra_column"]),
    ("real multiplier by division", [("A[RT_IDX(i, j)] = A[RT_IDX(i, j)] * r;", "A[RT_IDX(i, j)] = A[RT_IDX(i, j)] / piv;", 1)],
     ["@square_oracle"]),
    ("ties go to the last row", [("    return x > best;", "    return x >= best;", 1)],
     ["tall_4x2_zero_column_then_later_pivot"]),
]


def _build(tmp_path, edits):
    text = open(SRC).read()
    for old, new, count in edits:
        assert text.count(old) == count, f"mutation text {old!r} occurs {text.count(old)} times"
        text = text.replace(old, new)
    (tmp_path / "m.c").write_text(text)
    lib = tmp_path / "libm.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
                           str(tmp_path / "m.c"), "-o", str(lib), "-lm"])
    L = ctypes.CDLL(str(lib))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    L.oracle_getrf_rect_batch.argtypes = [i32, i32, i32, vp, i32, i64, vp, i64, vp, vp, i32, i32]
    return L


def _lib_getrf(L):
    codes = {np.dtype(np.float32): 0, np.dtype(np.float64): 1, np.dtype(np.complex64): 2,
             np.dtype(np.complex128): 3}

    def run(f, m, n):
        ipiv = np.zeros(max(min(m, n), 1), np.int32)
        info = np.zeros(1, np.int32)
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        L.oracle_getrf_rect_batch(codes[f.dtype], m, n, p(f), m, m * n, p(ipiv), ipiv.size, p(info), None, 1, 1)
        return ipiv[:min(m, n)], info[0]
    return run


def _caught(L, name):
    if name == "@square_oracle":
        n = 9
        A, _ = lu_inputs.random_problem(5, np.float32, n, 0, 2)
        a1, a2 = A.copy(), A.copy()
        run = _lib_getrf(L)
        for b in range(2):
            run(a1[b * n * n:(b + 1) * n * n], n, n)
        oracle.getrf(a2, n, n, n * n, 2)
        return not np.array_equal(a1.view(np.uint8), a2.view(np.uint8))
    case = _fixtures()[name]
    for d in case["dtypes"]:
        ipiv, info, LU = _run_case(_lib_getrf(L), case, DT[d])
        if ipiv != case["ipiv"] or info != case["info"]:
            return True
        if case["LU"] is not None and not np.array_equal(LU, np.array(case["LU"], dtype=DT[d])):
            return True
    return False


@pytest.mark.parametrize("name,edits,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, edits, catchers):
    L = _build(tmp_path, edits)
    assert any(_caught(L, c) for c in catchers), f"mutation '{name}' passes {catchers}"


def test_unmutated_copy_passes(tmp_path):
    L = _build(tmp_path, [])
    for name in list(_fixtures()) + ["@square_oracle"]:
        assert not _caught(L, name), name
