"""Mutation check of the Cholesky oracle's pins (CPU only).

Each mutation plants one plausible mistake in a private copy of the oracle's
Cholesky source -- a division where the pages' potf2 multiplies by one
reciprocal, a reciprocal where their trsm divides, a multiply then subtract
instead of one fused multiply-add, complex fmas in the other order, the
conjugate on the wrong operand, the diagonal sum in descending k, no stop at
the first non-positive diagonal -- builds it with gcc into a temporary
directory and runs the hand-worked fixtures and the closed forms on it.  At
least one check named for the mutation must then disagree.  A mutation whose
text no longer occurs in the source fails loudly, so the check cannot pass
vacuously after the oracle is edited.

The oracle itself is never modified and nothing here runs on a GPU.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest

from test_oracle_chol_pins import DT, _num, _same

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "chol_oracle.c")
GOLDEN = os.path.join(HERE, "golden", "chol_hand_worked.json")

# (name, [(old text, new text, expected occurrences)], fixtures that must catch it)
MUTATIONS = [
    ("potf2 divides instead of multiplying by one reciprocal",
     [("*PFX##_at(A, lda, up, i, j) = s * r;", "*PFX##_at(A, lda, up, i, j) = s / ljj;", 1)],
     ["real_2x2_potrf_reciprocal_then_multiply_float32", "real_2x2_potrf_reciprocal_then_multiply_float64",
      "real_2x2_potrf_reciprocal_then_multiply_upper_float32"]),
    ("potrs multiplies by a reciprocal instead of dividing",
     [("b[k] = b[k] / *PFX##_at(A, lda, up, k, k);", "b[k] = b[k] * ((T)1 / *PFX##_at(A, lda, up, k, k));", 2)],
     ["real_1x1_potrs_divides_float32", "real_1x1_potrs_divides_float64"]),
    ("diagonal: multiply, then subtract",
     [("d = FMA(-l, l, d);", "d = d - l * l;", 1)],
     ["real_2x2_potrf_diagonal_fused_float32", "real_2x2_potrf_diagonal_fused_float64"]),
    ("diagonal summed in descending k",
     [("        for (int k = 0; k < j; ++k) {                                          \\\n"
       "            T l = *PFX##_at(A, lda, up, j, k);",
       "        for (int k = j - 1; k >= 0; --k) {                                     \\\n"
       "            T l = *PFX##_at(A, lda, up, j, k);", 1)],
     ["real_3x3_potrf_diagonal_ascending_k_float32", "real_3x3_potrf_diagonal_ascending_k_float64"]),
    ("complex diagonal: imaginary term first",
     [("            d = FMA(-l[0], l[0], d);                                           \\\n"
       "            d = FMA(-l[1], l[1], d);",
       "            d = FMA(-l[1], l[1], d);                                           \\\n"
       "            d = FMA(-l[0], l[0], d);", 1)],
     ["complex_2x2_potrf_diagonal_fma_order_complex64", "complex_2x2_potrf_diagonal_fma_order_complex128"]),
    ("complex update: real-part fmas in the other order",
     [("    T re = FMA(-x[0], y[0], z[0]);                                             \\\n"
       "    re = FMA(-x[1], y[1], re);                                                 \\\n"
       "    T im = FMA(x[0], y[1], z[1]);",
       "    T re = FMA(-x[1], y[1], z[0]);                                             \\\n"
       "    re = FMA(-x[0], y[0], re);                                                 \\\n"
       "    T im = FMA(x[0], y[1], z[1]);", 1)],
     ["complex_3x3_potrf_update_fma_order_complex64", "complex_3x3_potrf_update_fma_order_complex128"]),
    ("complex update: imaginary-part fmas in the other order",
     [("    T im = FMA(x[0], y[1], z[1]);                                              \\\n"
       "    im = FMA(-x[1], y[0], im);",
       "    T im = FMA(-x[1], y[0], z[1]);                                             \\\n"
       "    im = FMA(x[0], y[1], im);", 1)],
     ["complex_3x3_potrf_update_fma_order_complex64", "complex_3x3_potrf_update_fma_order_upper_complex128"]),
    ("complex update conjugates the other operand",
     [("PFX##_fms_conj(s, x, y);", "PFX##_fms_conj(s, y, x);", 1)],
     ["@complex_integer_closed_form", "complex_3x3_potrf_update_fma_order_complex64"]),
    ("complex back solve without the conjugate",
     [("PFX##_fms_cx(&b[2 * i], l, &b[2 * k]);", "PFX##_fms(&b[2 * i], l, &b[2 * k]);", 1)],
     ["@complex_integer_closed_form", "complex_2x2_potrs_fma_order_complex64"]),
    ("complex forward solve: fmas in the other order",
     [("    T re = FMA(-x[0], y[0], z[0]);                                             \\\n"
       "    re = FMA(x[1], y[1], re);",
       "    T re = FMA(x[1], y[1], z[0]);                                              \\\n"
       "    re = FMA(-x[0], y[0], re);", 1)],
     ["complex_2x2_potrs_fma_order_complex64", "complex_2x2_potrs_fma_order_complex128"]),
    ("complex back solve: fmas in the other order",
     [("    T im = FMA(-x[0], y[1], z[1]);                                             \\\n"
       "    im = FMA(x[1], y[0], im);",
       "    T im = FMA(x[1], y[0], z[1]);                                              \\\n"
       "    im = FMA(-x[0], y[1], im);", 1)],
     ["complex_2x2_potrs_fma_order_complex64", "complex_2x2_potrs_fma_order_complex128"]),
    ("no stop at the first non-positive diagonal",
     [("            *info = j + 1;                                                     \\\n"
       "            return;",
       "            if (!*info) *info = j + 1;                                         \\\n"
       "            continue;", 2)],
     ["real_3x3_potrf_stops_at_first_failure"]),
    ("a zero diagonal counts as positive",
     [("if (!(d > (T)0)) {", "if (d < (T)0 || d != d) {", 2)],
     ["real_2x2_potrf_zero_pivot_is_not_positive"]),
    ("the imaginary part of the diagonal is read",
     [("T d = djj[0];", "T d = djj[0] + djj[1];", 1)],
     ["complex_1x1_potrf_imaginary_diagonal_ignored"]),
    ("update adds instead of subtracting",
     [("s = FMA(-*PFX##_at(A, lda, up, i, k),", "s = FMA(*PFX##_at(A, lda, up, i, k),", 1)],
     ["@pascal_closed_form"]),
]


def _fixtures():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def _build(tmp_path, edits):
    with open(SRC) as f:
        text = f.read()
    for old, new, count in edits:
        found = text.count(old)
        assert found == count, f"mutation text {old!r} occurs {found} times in the oracle, expected {count}"
        text = text.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
                           str(src), "-o", str(lib), "-lm"])
    L = ctypes.CDLL(str(lib))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    L.oracle_chol_batch.argtypes = [i32, i32, i32, i32, i32, vp, i32, i64, vp, vp, i32, i64, i32, i32]
    return L


_CODE = {np.float32: 0, np.float64: 1, np.complex64: 2, np.complex128: 3}


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _run(L, op, M, uplo, B=None):
    """Run the library on one matrix (and B); return (info, factor, X)."""
    dtype = M.dtype.type
    n = M.shape[0]
    flat = np.ascontiguousarray(M.T).reshape(-1).copy()
    info = np.zeros(1, np.int32)
    up = 1 if uplo == "U" else 0
    if B is None:
        L.oracle_chol_batch(0, _CODE[dtype], up, n, 0, _p(flat), n, n * n, _p(info), None, 1, 0, 1, 1)
        return int(info[0]), flat.reshape(n, n).T, None
    nr = B.shape[1]
    fb = np.ascontiguousarray(B.T).reshape(-1).copy()
    L.oracle_chol_batch(2, _CODE[dtype], up, n, nr, _p(flat), n, n * n, _p(info), _p(fb), n, n * nr, 1, 1)
    return int(info[0]), flat.reshape(n, n).T, fb.reshape(nr, n).T


def _case_disagrees(L, case, dtype):
    M = np.array([[_num(x) for x in r] for r in case["A"]], dtype=dtype)
    B = np.array([[_num(x) for x in r] for r in case["B"]], dtype=dtype) if "B" in case else None
    info, F, X = _run(L, 0 if B is None else 2, M, case["uplo"], B)
    if info != case["info"]:
        return True
    for i, j, v in case["entries"]:
        if not _same(F[i, j], np.array(_num(v), dtype)):
            return True
    if B is not None:
        want = np.array([[_num(x) for x in r] for r in case["X"]], dtype=dtype)
        return any(not _same(X[i, c], want[i, c]) for i in range(X.shape[0]) for c in range(X.shape[1]))
    return False


def _pascal_disagrees(L):
    n = 10
    P = np.array([[math.comb(i + j, i) for j in range(n)] for i in range(n)], dtype=np.float64)
    Lp = np.array([[math.comb(i, j) if j <= i else 0 for j in range(n)] for i in range(n)], dtype=np.float64)
    info, F, _ = _run(L, 0, P, "L")
    return info != 0 or not np.array_equal(np.tril(F), Lp)


def _complex_closed_disagrees(L):
    Lc = np.array([[1, 0, 0], [1 + 2j, 2, 0], [3 - 1j, 2 + 1j, 1]], dtype=np.complex128)
    A = Lc @ Lc.conj().T
    X = np.array([[1 + 1j], [-2j], [2]], dtype=np.complex128)
    info, F, Xg = _run(L, 2, A, "L", A @ X)
    return info != 0 or not np.array_equal(np.tril(F), Lc) or not np.array_equal(Xg, X)


def _disagrees(L, name):
    if name == "@pascal_closed_form":
        return [name] if _pascal_disagrees(L) else []
    if name == "@complex_integer_closed_form":
        return [name] if _complex_closed_disagrees(L) else []
    case = _fixtures()[name]
    return [f"{name}-{dt}" for dt in case["dtypes"] if _case_disagrees(L, case, DT[dt])]


@pytest.mark.parametrize("name,edits,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, edits, catchers):
    L = _build(tmp_path, edits)
    caught = [c for n in catchers for c in _disagrees(L, n)]
    assert caught, f"mutation '{name}' passes every check meant to catch it: {catchers}"


def test_unmutated_copy_passes_every_check(tmp_path):
    """The harness itself: the oracle's source built the same way agrees with
    every fixture and closed form, so a caught mutation is the mutation's
    doing."""
    L = _build(tmp_path, [])
    for name in list(_fixtures()) + ["@pascal_closed_form", "@complex_integer_closed_form"]:
        assert not _disagrees(L, name), name
