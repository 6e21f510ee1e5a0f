"""Mutation check of the oracle's pins (CPU only).

Each mutation plants one plausible mistake in a private copy of the oracle's
C source -- a divide where the pages' reading multiplies by one reciprocal,
the two fused multiply-adds of a complex update in the other order, the
other product fused in a complex multiply, the small-pivot division branch
dropped, a pivot metric or tie rule changed -- builds it with gcc into a
temporary directory, and runs the hand-worked fixtures on it.  At least one
fixture named for the mutation must then disagree (ipiv, info, or a bit of LU
or X).  A mutation whose text no longer occurs in the source fails loudly, so
the check cannot pass vacuously after the oracle is edited.

The oracle itself is never modified and nothing here runs on a GPU.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

import oracle

from test_oracle_pins import DT, _bits, _flat_colmajor, _mat

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "lu_oracle.c")
GOLDEN = os.path.join(HERE, "golden", "hand_worked.json")

# (name, [(old text, new text, expected number of occurrences)], fixtures that must catch it)
MUTATIONS = [
    ("real multiplier by division instead of one reciprocal",
     [("A[i + (size_t)j * lda] *= r;", "A[i + (size_t)j * lda] /= piv;", 1)],
     ["real_2x2_reciprocal_then_multiply", "real_2x2_reciprocal_then_multiply_double"]),
    ("complex multiplier by Smith division instead of one reciprocal",
     [("PFX##_mul(a, r, a);", "PFX##_div(a[0], a[1], piv[0], piv[1], a);", 1)],
     ["complex_2x2_update_fma_order", "complex_2x2_multiplier_fused_product",
      "complex_2x2_multiplier_fused_product_double"]),
    ("complex update: real-part fmas in the other order",
     [("T re = FMA(-x[0], y[0], z[0]);", "T re = FMA(x[1], y[1], z[0]);", 1),
      ("re = FMA(x[1], y[1], re);", "re = FMA(-x[0], y[0], re);", 1)],
     ["complex_2x2_update_fma_order", "complex_2x2_update_fma_order_double"]),
    ("complex update: imaginary-part fmas in the other order",
     [("T im = FMA(-x[0], y[1], z[1]);", "T im = FMA(-x[1], y[0], z[1]);", 1),
      ("im = FMA(-x[1], y[0], im);", "im = FMA(-x[0], y[1], im);", 1)],
     ["complex_2x2_update_fma_order", "complex_2x2_update_fma_order_double",
      "complex_2x2_multiplier_fused_product"]),
    ("complex multiplier fuses the other product",
     [("T t = a[1] * r[1];", "T t = a[0] * r[0];", 1),
      ("T re = FMA(a[0], r[0], -t);", "T re = FMA(-a[1], r[1], t);", 1),
      ("T t2 = a[1] * r[0];", "T t2 = a[0] * r[1];", 1),
      ("T im = FMA(a[0], r[1], t2);", "T im = FMA(a[1], r[0], t2);", 1)],
     ["complex_2x2_multiplier_fused_product", "complex_2x2_multiplier_fused_product_double"]),
    ("complex pivot below the smallest normal still takes the reciprocal",
     [("if (pm >= SFMIN) {", "if (1) {", 1)],
     ["complex_2x2_subnormal_pivot_divides", "complex_2x2_subnormal_pivot_divides_other_branch",
      "complex128_subnormal_pivot_divides"]),
    ("real pivot below the smallest normal still takes the reciprocal",
     [("if (FABS(piv) >= SFMIN) {", "if (1) {", 1)],
     ["float32_subnormal_pivot_divides", "float64_subnormal_pivot_divides"]),
    ("complex pivot metric from the real part only",
     [("return FABS(z[0]) + FABS(z[1]);", "return FABS(z[0]);", 1)],
     ["complex_3x3_first_nan_in_imaginary_part_wins", "complex_2x2_cabs1_tie"]),
    ("a later NaN displaces an earlier one",
     [("if (isnan(best)) return 0;", "if (isnan(best) && !isnan(x)) return 0;", 1)],
     ["real_3x3_first_nan_wins", "complex_3x3_first_nan_in_imaginary_part_wins"]),
    ("ties go to the last row",
     [("return x > best;", "return x >= best;", 1)],
     ["real_2x2_tie_lowest_row", "complex_2x2_cabs1_tie", "real_3x3_tie_then_singular"]),
    ("a zero pivot still scales and updates",
     [("if (FABS(piv) == (T)0) {", "if (0) {", 1)],
     ["real_2x2_zero_column", "real_2x2_singular_last_step"]),
    ("back substitution multiplies by the reciprocal of u_kk",
     [("b[k] = b[k] / A[k + (size_t)k * lda];", "b[k] = b[k] * ((T)1 / A[k + (size_t)k * lda]);", 2)],
     ["real_1x1_solve_divides"]),
    ("rank-1 update adds instead of subtracting",
     [("FMA(-A[i + (size_t)j * lda], u, A[i + (size_t)k * lda]);",
       "FMA(A[i + (size_t)j * lda], u, A[i + (size_t)k * lda]);", 1)],
     ["real_2x2_basic", "real_3x3_solve"]),
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
    L.oracle_getrf_batch.argtypes = [i32, i32, vp, i32, i64, vp, i64, vp, vp, i32, i32]
    L.oracle_gesv_batch.argtypes = [i32, i32, i32, vp, i32, i64, vp, i64, vp, i32, i64, vp, vp, i32, i32]
    return L


def _disagrees(L, case, dtype):
    """True when the library's result for the fixture differs from it."""
    code = {np.float32: 0, np.float64: 1, np.complex64: 2, np.complex128: 3}[dtype]
    A = _mat(case["A"], dtype)
    n = A.shape[0]
    flat = _flat_colmajor(A)
    ipiv = np.zeros(n, np.int32)
    info = np.zeros(1, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    if "B" in case:
        B = _mat(case["B"], dtype)
        nr = B.shape[1]
        flatB = _flat_colmajor(B)
        L.oracle_gesv_batch(code, n, nr, p(flat), n, n * n, p(ipiv), n, p(flatB), n, n * nr, p(info), None, 1, 1)
        X = oracle.matrix(flatB, 0, n, nr, n, n * nr)
        if not np.array_equal(_bits(X), _bits(_mat(case["X"], dtype))):
            return True
    else:
        L.oracle_getrf_batch(code, n, p(flat), n, n * n, p(ipiv), n, p(info), None, 1, 1)
    if list(ipiv) != case["ipiv"] or int(info[0]) != case["info"]:
        return True
    if case["LU"] is not None:
        LU = oracle.matrix(flat, 0, n, n, n, n * n)
        return not np.array_equal(_bits(LU), _bits(_mat(case["LU"], dtype)))
    return False


@pytest.mark.parametrize("name,edits,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, edits, catchers):
    fx = _fixtures()
    L = _build(tmp_path, edits)
    caught = []
    for cname in catchers:
        case = fx[cname]
        for dt in case["dtypes"]:
            if _disagrees(L, case, DT[dt]):
                caught.append(f"{cname}-{dt}")
    assert caught, f"mutation '{name}' passes every fixture meant to catch it: {catchers}"


def test_unmutated_copy_passes_every_fixture(tmp_path):
    """The harness itself: the oracle's source built the same way agrees with
    every fixture, so a caught mutation is the mutation's doing."""
    L = _build(tmp_path, [])
    for cname, case in _fixtures().items():
        for dt in case["dtypes"]:
            assert not _disagrees(L, case, DT[dt]), f"{cname}-{dt}"


ZERO_PIVOT_UPDATES = [
    ("continue;", ";", 2),
    ("if (FABS(piv) >= SFMIN) {", "if (FABS(piv) == (T)0) {} else if (FABS(piv) >= SFMIN) {", 1),
    ("if (pm >= SFMIN) {", "if (pm == (T)0) {} else if (pm >= SFMIN) {", 1),
]


def _canon_bits(a):
    a = np.array(a, copy=True)
    real = a.view(np.float32 if a.dtype in (np.float32, np.complex64) else np.float64)
    real[np.isnan(real)] = np.nan
    return _bits(a)


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
def test_zero_pivot_inputs_discriminate(tmp_path, dtype):
    """The zero-pivot inputs that the GPU tests use are sensitive to the rule
    that a zero pivot's step changes nothing: an oracle that still runs the
    rank-1 update of such a step (with the unscaled zero multipliers) gives
    different bits (0 * inf, +0 replacing -0) or a different pivot order."""
    import lu_inputs
    n, batch = 70, 3
    A, _ = lu_inputs.zero_pivot_problem(11, dtype, n, 1, batch)
    L = _build(tmp_path, ZERO_PIVOT_UPDATES)
    code = {np.float32: 0, np.float64: 1, np.complex64: 2, np.complex128: 3}[dtype]
    mA = A.copy()
    ipiv = np.zeros(batch * n, np.int32)
    info = np.zeros(batch, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    L.oracle_getrf_batch(code, n, p(mA), n, n * n, p(ipiv), n, p(info), None, batch, 1)
    oA = A.copy()
    oP, oI, _, _ = oracle.getrf(oA, n, n, n * n, batch)
    assert np.array_equal(info, oI) and np.all(oI > 0)
    for b in range(batch):
        same = (np.array_equal(ipiv[b * n:(b + 1) * n], oP[b]) and
                np.array_equal(_canon_bits(mA[b * n * n:(b + 1) * n * n]), _canon_bits(oA[b * n * n:(b + 1) * n * n])))
        assert not same, f"matrix {b}: the zero-pivot rule changes nothing on this input"
