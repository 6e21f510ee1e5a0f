"""GPU parity of getrs with op(A) = A^T ('T') and A^H ('C') against the
oracle's transposed solve, through the C ABI.

The factors come from the library's getrf; the oracle solves with those same
factors, so the comparison isolates the solve.  Bar: X bit-identical (the
kernel accumulates each element in the oracle's order: ascending k against
U^T with true division by u_kk, descending k against L^T), plus the solve
residual of op(A) X = B for well-conditioned inputs.  Edge cases: n = 1,
block and wavefront boundaries, n = 1024 (the one-launch solve's largest
order), the block-row-by-block-row solve above it up to n = 4096 (also for
'N'), ragged right-hand-side tiles, padded leading dimensions and batch
strides (pads untouched), and n > 4096, which must be refused."""
import numpy as np
import pytest

import lu_inputs
import oracle
from gpu_support import bits, gesv_gpu, gpu_available, matrices_equal_bits, to_dev, to_host

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    import dense_linear_algebra_amd as lib
else:
    lib = None


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _op(A, trans):
    return A.T if trans == "T" else A.conj().T


def _getrs_gpu(LU, ipiv, B, n, nrhs, batch, trans, lda, sA, ldb, sB, sP):
    t = lib.dtype_code(LU.dtype)
    dA, dB = to_dev(LU), to_dev(B)
    dP = torch.from_numpy(np.ascontiguousarray(ipiv, dtype=np.int32).reshape(-1).copy()).cuda()
    lib.batchlu_getrs(t, trans, n, nrhs, dA, lda, sA, dP, sP, dB, ldb, sB, batch)
    torch.cuda.synchronize()
    return to_host(dB)


CASES = ([(np.float32, n, r) for n, r in ((1, 1), (5, 2), (31, 4), (33, 5), (64, 1), (100, 7), (257, 3))]
         + [(np.float64, n, r) for n, r in ((32, 3), (65, 1), (130, 6))]
         + [(np.complex64, n, r) for n, r in ((24, 2), (96, 3), (200, 5))]
         + [(np.complex128, n, r) for n, r in ((17, 1), (63, 3))])


@pytest.mark.parametrize("trans", ["T", "C"])
@pytest.mark.parametrize("dtype,n,nrhs", CASES, ids=lambda v: getattr(v, "__name__", str(v)))
def test_getrs_trans_matches_oracle_bitwise(dtype, n, nrhs, trans):
    batch = 4
    A, B = lu_inputs.random_problem(9100 + n, dtype, n, nrhs, batch)
    print(f"case getrs trans={trans} dtype={np.dtype(dtype).name} n={n} nrhs={nrhs}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    assert np.all(gI == 0)
    gB = _getrs_gpu(gA, gP[:, :n], B, n, nrhs, batch, trans, n, n * n, n, n * nrhs, n)
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch, trans=trans)
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []
    for b in range(batch):
        Am = oracle.matrix(A, b, n, n, n, n * n)
        X = oracle.matrix(gB, b, n, nrhs, n, n * nrhs)
        assert oracle.solve_residual(_op(Am, trans), X, oracle.matrix(B, b, n, nrhs, n, n * nrhs)) <= 20


# orders to 256 with many right-hand sides at batches of 512 or more take
# wider column tiles (16 for the real types above 8 right-hand sides, 8 for
# complex double above 4); every case ends in a partly filled tile
WIDE = [(np.float32, 100, 19), (np.float64, 256, 17), (np.float64, 33, 40), (np.complex128, 64, 11),
        (np.complex128, 200, 9)]


@pytest.mark.parametrize("trans", ["N", "T", "C"])
@pytest.mark.parametrize("dtype,n,nrhs", WIDE, ids=lambda v: getattr(v, "__name__", str(v)))
def test_wide_tiles_match_oracle_bitwise(dtype, n, nrhs, trans):
    batch = 512
    A, B = lu_inputs.random_problem(9400 + n + nrhs, dtype, n, nrhs, batch)
    print(f"case getrs wide trans={trans} dtype={np.dtype(dtype).name} n={n} nrhs={nrhs}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    assert not gI.any()
    gB = _getrs_gpu(gA, gP[:, :n], B, n, nrhs, batch, trans, n, n * n, n, n * nrhs, n)
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch, trans=trans)
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []


@pytest.mark.parametrize("dtype,trans", [(np.float32, "T"), (np.float64, "T"), (np.complex64, "C"),
                                         (np.complex128, "C")])
def test_getrs_trans_largest_order(dtype, trans):
    """n = 1024, the largest order one work-group solves: sixteen wavefronts,
    32 diagonal blocks.  The factors are the oracle's, so only the solve runs
    on the GPU.  Compared bitwise on every element."""
    n, nrhs, batch = 1024, 3, 2
    A, B = lu_inputs.random_problem(9200, dtype, n, nrhs, batch)
    print(f"case getrs trans={trans} dtype={np.dtype(dtype).name} n={n} nrhs={nrhs}", flush=True)
    LU = A.copy()
    ipiv, info, _, _ = oracle.getrf(LU, n, n, n * n, batch)
    assert np.all(info == 0)
    gB = _getrs_gpu(LU, ipiv, B, n, nrhs, batch, trans, n, n * n, n, n * nrhs, n)
    oB = B.copy()
    oracle.getrs(LU, n, n, n * n, ipiv, oB, nrhs, n, n * nrhs, batch, trans=trans)
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []


@pytest.mark.parametrize("dtype", [np.float32, np.complex128])
def test_getrs_trans_padded_layout(dtype):
    """lda > n, ldb > n, batch strides with gaps, ipiv stride > n: the result
    matches the dense solve and no pad element changes."""
    n, nrhs, batch = 45, 5, 3
    lda, sA, ldb, sB, sP = 50, 50 * 45 + 7, 48, 48 * 5 + 3, 49
    A, B = lu_inputs.random_problem(9300, dtype, n, nrhs, batch)
    print(f"case getrs trans=C padded dtype={np.dtype(dtype).name} n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    LUp = lu_inputs.relayout(gA, n, n, batch, n, n * n, lda, sA, poison=7.5)
    Bp = lu_inputs.relayout(B, n, nrhs, batch, n, n * nrhs, ldb, sB, poison=-3.25)
    Pp = np.full((batch, sP), 99999, np.int32)
    Pp[:, :n] = gP[:, :n]
    gB = _getrs_gpu(LUp, Pp, Bp, n, nrhs, batch, "C", lda, sA, ldb, sB, sP)
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch, trans="C")
    dense = lu_inputs.relayout(gB, n, nrhs, batch, ldb, sB, n, n * nrhs)
    assert matrices_equal_bits(dense, oB, n, nrhs, n, n * nrhs, batch) == []
    pad = np.ones(Bp.shape, bool)
    for b in range(batch):
        for c in range(nrhs):
            pad[b * sB + c * ldb: b * sB + c * ldb + n] = False
    np.testing.assert_array_equal(bits(gB[pad]), bits(Bp[pad]))


BLOCKED = [(np.float32, 1025, "T"), (np.float32, 1100, "N"), (np.float64, 1057, "T"), (np.complex64, 1030, "C"),
           (np.complex64, 1030, "T"), (np.complex128, 1090, "C"), (np.float64, 2048, "N"), (np.float32, 4096, "T"),
           (np.complex64, 4096, "C"), (np.float64, 4096, "C"), (np.complex128, 4096, "T")]


@pytest.mark.parametrize("dtype,n,trans", BLOCKED, ids=lambda v: getattr(v, "__name__", str(v)))
def test_getrs_blocked_orders_match_oracle_bitwise(dtype, n, trans):
    """Above n = 1024 the solve runs block row by block row: a 32-row
    triangular solve, then a GEMM update (transposed and, for 'C',
    conjugated reads of the factor for op(A) = A^T, A^H).  Synthetic packed
    factors and interchanges; X bitwise against the oracle's solve."""
    nrhs, batch = 3, 1 if n > 2048 else 2
    LU, ipiv = lu_inputs.packed_factors(9500 + n, dtype, n, batch)
    _, B = lu_inputs.random_problem(9600 + n, dtype, n, nrhs, batch)
    print(f"case blocked getrs trans={trans} dtype={np.dtype(dtype).name} n={n} nrhs={nrhs}", flush=True)
    gB = _getrs_gpu(LU, ipiv, B, n, nrhs, batch, trans, n, n * n, n, n * nrhs, n)
    oB = B.copy()
    oracle.getrs(LU, n, n, n * n, ipiv, oB, nrhs, n, n * nrhs, batch, trans=trans)
    assert np.isfinite(oB).all()
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []


def test_getrs_trans_blocked_from_gpu_factors():
    """n = 1100 float factored on the GPU (blocked tier), solved with A^T
    above the one-launch order: bitwise against the oracle's solve with the
    same factors, and a small residual of A^T X = B."""
    dtype, n, nrhs, batch = np.float32, 1100, 4, 1
    A, B = lu_inputs.random_problem(9700, dtype, n, nrhs, batch)
    print(f"case blocked getrs trans=T from GPU factors n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    assert np.all(gI == 0)
    gB = _getrs_gpu(gA, gP[:, :n], B, n, nrhs, batch, "T", n, n * n, n, n * nrhs, n)
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch, trans="T")
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []
    Am = oracle.matrix(A, 0, n, n, n, n * n)
    assert oracle.solve_residual(Am.T, oracle.matrix(gB, 0, n, nrhs, n, n * nrhs),
                                 oracle.matrix(B, 0, n, nrhs, n, n * nrhs)) <= 20


def test_getrs_trans_above_limit_is_refused():
    n = 4097
    dA = torch.zeros(n * n, dtype=torch.float32, device="cuda")
    dB = torch.zeros(n, dtype=torch.float32, device="cuda")
    dP = torch.ones(n, dtype=torch.int32, device="cuda")
    st = lib.batchlu_getrs(lib.dtype_code(np.dtype(np.float32)), "T", n, 1, dA, n, n * n, dP, n, dB, n, n, 1,
                           raise_on_error=False)
    assert st == -100
