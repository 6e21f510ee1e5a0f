"""GPU parity of the LDS-staged work-group tier (BATCHLU_TIER_CTA_LDS):
getrf and the fused gesv against the CPU oracle, through the C ABI.

Bar: ipiv and info identical, L and U bit-identical, and X bit-identical
too (this tier's back substitution divides by u_kk, in the oracle's
descending order; the forward solve runs as extra columns of the rank-1
updates, the same fused multiply-adds in the same order)."""
import numpy as np
import pytest

import lu_inputs
from gpu_support import bits, gesv_gpu, gpu_available, matrices_equal_bits, oracle_run

pytestmark = pytest.mark.gpu

if gpu_available():
    import dense_linear_algebra_amd as lib
else:
    lib = None


@pytest.fixture(autouse=True)
def _lds_tier():
    if not gpu_available():
        pytest.skip("no GPU")
    lib.batchlu_set_tier(lib.TIER_CTA_LDS)
    yield
    lib.batchlu_set_tier(lib.TIER_AUTO)


CASES = ([(np.float32, n) for n in (1, 2, 5, 31, 32, 33, 64, 65, 100, 128)]
         + [(np.float64, n) for n in (3, 40, 64, 97, 128)]
         + [(np.complex64, n) for n in (7, 33, 64, 80, 128)]
         + [(np.complex128, n) for n in (1, 17, 48, 64)])


@pytest.mark.parametrize("dtype,n", CASES, ids=lambda v: getattr(v, "__name__", str(v)))
@pytest.mark.parametrize("nrhs", [0, 1, 5, 16, 20])
def test_lds_tier_matches_oracle(dtype, n, nrhs):
    batch = 9
    A, B = lu_inputs.random_problem(600 + n + nrhs, dtype, n, max(nrhs, 1), batch)
    if nrhs == 0:
        gA, _, gP, gI = gesv_gpu(lib, A, B, n, 1, batch, op="getrf")
        oA, _, oP, oI, _ = oracle_run(A, B, n, 1, batch, op="getrf")
    else:
        gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
        oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
        assert np.array_equal(bits(gB), bits(oB)), "X differs from the oracle"
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []


def _one(M, dtype):
    return np.ascontiguousarray(np.asarray(M, dtype=dtype).T).reshape(-1).copy()


@pytest.mark.parametrize("dtype,n", [(np.float32, 64), (np.float64, 90), (np.complex64, 70), (np.complex128, 50)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_lds_tier_special_matrices(dtype, n):
    """Wilkinson growth (every step a tie), a zero column (info, the zero
    step changes nothing), +inf and -0 in that pivot's row, a singular last
    step, a NaN; B untouched where info > 0."""
    nrhs = 3
    rng = np.random.default_rng(21)
    W = np.tril(-np.ones((n, n)), -1) + np.eye(n)
    W[:, -1] = 1
    Z = rng.uniform(-1, 1, (n, n))
    for j in range(20):
        Z[j, j] = 64
    Z[:, 20] = 0
    Z[20, 30:] = np.inf
    Z[:, 25] = -0.0
    Z[20, 25] = 1
    S = rng.uniform(-1, 1, (n, n))
    S[-1, :] = 0
    N = rng.uniform(-1, 1, (n, n))
    N[30, 10] = np.nan
    mats = [W, Z, S, N, rng.uniform(-1, 1, (n, n))]
    batch = len(mats)
    A = np.concatenate([_one(M, dtype) for M in mats])
    B = rng.uniform(-1, 1, batch * n * nrhs).astype(dtype)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert np.array_equal(bits(gB), bits(oB))
    assert oI[1] == 21 and oI[2] == n


def test_lds_tier_padded_layout_keeps_poison():
    dtype, n, nrhs, batch = np.complex64, 45, 4, 6
    lda, sA, ldb, sB, sP = n + 3, (n + 3) * n + 9, n + 1, (n + 1) * nrhs + 5, n + 2
    A0, B0 = lu_inputs.random_problem(77, dtype, n, nrhs, batch)
    A = lu_inputs.relayout(A0, n, n, batch, n, n * n, lda, sA, poison=-99.0)
    B = lu_inputs.relayout(B0, n, nrhs, batch, n, n * nrhs, ldb, sB, poison=-55.0)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch, lda=lda, sA=sA, ldb=ldb, sB=sB, sP=sP)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch, lda=lda, sA=sA, ldb=ldb, sB=sB)
    np.testing.assert_array_equal(gI, oI)
    assert np.array_equal(bits(gA), bits(oA)) and np.array_equal(bits(gB), bits(oB))
    assert (gP[:, n:] == -7).all()


def test_lds_tier_full_size_complex_workload():
    """The complex n = 64 workload (nrhs 16, batch 8192) on this tier: LU and
    X bit-identical on matrices spread over the batch."""
    import oracle
    w = lu_inputs.WORKLOADS["cgesv_n64_r16_b8192"]
    A, B = lu_inputs.dense_problem(w)
    n, r = w.n, w.nrhs
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, r, w.batch)
    assert not gI.any()
    for b in np.linspace(0, w.batch - 1, 5).astype(int):
        sa, sb = slice(b * n * n, (b + 1) * n * n), slice(b * n * r, (b + 1) * n * r)
        oA, oB = A[sa].copy(), B[sb].copy()
        oP, oI, _, _ = oracle.gesv(oA, n, n, n * n, oB, r, n, n * r, 1)
        assert np.array_equal(gP[b, :n], oP[0])
        assert np.array_equal(bits(gA[sa]), bits(oA)) and np.array_equal(bits(gB[sb]), bits(oB))
