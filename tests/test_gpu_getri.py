"""GPU parity of getri (C = A^{-1} from the factors, out of place) against
the oracle's getri on the same factors, through the C ABI.

Bar: C bit-identical (the kernel runs the NoTrans solve on the identity in
the oracle's order), plus the residual of A C = I.  Edge cases: n = 1,
block and wavefront boundaries, ragged column tiles, n = 1024 (factors from
the oracle, so only the inverse runs on the GPU), orders above 1024 (the
identity, then the block-row-by-block-row solve), padded ldc and strides
with the pads untouched."""
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


def _getri_gpu(LU, ipiv, C0, n, batch, lda, sA, ldc, sC, sP):
    t = lib.dtype_code(LU.dtype)
    dA, dC = to_dev(LU), to_dev(C0)
    dP = torch.from_numpy(np.ascontiguousarray(ipiv, dtype=np.int32).reshape(-1).copy()).cuda()
    lib.batchlu_getri(t, n, dA, lda, sA, dP, sP, dC, ldc, sC, batch)
    torch.cuda.synchronize()
    return to_host(dC)


CASES = ([(np.float32, n) for n in (1, 5, 32, 33, 64, 100, 257)]
         + [(np.float64, n) for n in (31, 65, 130)]
         + [(np.complex64, n) for n in (24, 96)]
         + [(np.complex128, n) for n in (17, 63)])


@pytest.mark.parametrize("dtype,n", [(np.float32, 70), (np.complex128, 40)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_getri_batch_multiple_of_eight(dtype, n):
    """A batch that is a multiple of eight maps the column tiles of one
    matrix's inverse to one XCD: C bit-identical to the oracle's."""
    batch = 16
    A, _ = lu_inputs.random_problem(9450 + n, dtype, n, 0, batch)
    print(f"case getri batch 16 {np.dtype(dtype).name} n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    assert not gI.any()
    gC = _getri_gpu(gA, gP[:, :n], np.zeros(batch * n * n, dtype), n, batch, n, n * n, n, n * n, n)
    oC = np.zeros(batch * n * n, dtype)
    oracle.getri(gA, n, n, n * n, gP[:, :n], oC, n, n * n, batch)
    assert matrices_equal_bits(gC, oC, n, n, n, n * n, batch) == []


@pytest.mark.parametrize("dtype,n", CASES, ids=lambda v: getattr(v, "__name__", str(v)))
def test_getri_matches_oracle_bitwise(dtype, n):
    batch = 3
    A, _ = lu_inputs.random_problem(9400 + n, dtype, n, 0, batch)
    print(f"case getri dtype={np.dtype(dtype).name} n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    assert np.all(gI == 0)
    gC = _getri_gpu(gA, gP[:, :n], np.zeros(batch * n * n, dtype), n, batch, n, n * n, n, n * n, n)
    oC = np.zeros(batch * n * n, dtype)
    oracle.getri(gA, n, n, n * n, gP[:, :n], oC, n, n * n, batch)
    assert matrices_equal_bits(gC, oC, n, n, n, n * n, batch) == []
    eye = np.eye(n, dtype=dtype)
    for b in range(batch):
        Am = oracle.matrix(A, b, n, n, n, n * n)
        assert oracle.solve_residual(Am, oracle.matrix(gC, b, n, n, n, n * n), eye) <= 20


@pytest.mark.parametrize("dtype", [np.float32, np.complex128])
def test_getri_largest_order(dtype):
    n, batch = 1024, 1
    A, _ = lu_inputs.random_problem(9500, dtype, n, 0, batch)
    print(f"case getri dtype={np.dtype(dtype).name} n={n}", flush=True)
    LU = A.copy()
    ipiv, info, _, _ = oracle.getrf(LU, n, n, n * n, batch)
    assert np.all(info == 0)
    gC = _getri_gpu(LU, ipiv, np.zeros(n * n, dtype), n, batch, n, n * n, n, n * n, n)
    oC = np.zeros(n * n, dtype)
    oracle.getri(LU, n, n, n * n, ipiv, oC, n, n * n, batch)
    assert matrices_equal_bits(gC, oC, n, n, n, n * n, batch) == []


@pytest.mark.parametrize("dtype", [np.float64, np.complex64])
def test_getri_padded_layout(dtype):
    n, batch = 41, 3
    lda, sA, ldc, sC, sP = 44, 44 * 41 + 5, 47, 47 * 41 + 9, 43
    A, _ = lu_inputs.random_problem(9600, dtype, n, 0, batch)
    print(f"case getri padded dtype={np.dtype(dtype).name} n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    LUp = lu_inputs.relayout(gA, n, n, batch, n, n * n, lda, sA, poison=3.5)
    C0 = np.full(batch * sC, -6.75, dtype)
    Pp = np.full((batch, sP), 77777, np.int32)
    Pp[:, :n] = gP[:, :n]
    gC = _getri_gpu(LUp, Pp, C0, n, batch, lda, sA, ldc, sC, sP)
    oC = np.zeros(batch * n * n, dtype)
    oracle.getri(gA, n, n, n * n, gP[:, :n], oC, n, n * n, batch)
    dense = lu_inputs.relayout(gC, n, n, batch, ldc, sC, n, n * n)
    assert matrices_equal_bits(dense, oC, n, n, n, n * n, batch) == []
    pad = np.ones(C0.shape, bool)
    for b in range(batch):
        for c in range(n):
            pad[b * sC + c * ldc: b * sC + c * ldc + n] = False
    np.testing.assert_array_equal(bits(gC[pad]), bits(C0[pad]))


@pytest.mark.parametrize("dtype,n", [(np.float64, 1100), (np.complex64, 1057), (np.float32, 1500)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_getri_blocked_orders(dtype, n):
    """Above n = 1024: C set to the identity, then solved in place block row
    by block row.  Synthetic packed factors; C bitwise against the oracle's
    getri (padded ldc, pads untouched)."""
    batch, ldc = 1, n + 3
    LU, ipiv = lu_inputs.packed_factors(9800 + n, dtype, n, batch)
    print(f"case blocked getri dtype={np.dtype(dtype).name} n={n}", flush=True)
    C0 = np.full(ldc * n, -5.5, dtype)
    gC = _getri_gpu(LU, ipiv, C0, n, batch, n, n * n, ldc, ldc * n, n)
    oC = np.zeros(n * n, dtype)
    oracle.getri(LU, n, n, n * n, ipiv, oC, n, n * n, batch)
    dense = lu_inputs.relayout(gC, n, n, batch, ldc, ldc * n, n, n * n)
    assert matrices_equal_bits(dense, oC, n, n, n, n * n, batch) == []
    pad = np.ones(ldc * n, bool)
    for c in range(n):
        pad[c * ldc: c * ldc + n] = False
    assert (gC[pad] == dtype(-5.5)).all()
