"""GPU parity of the blocked tier's tallest panels, through the C ABI.

Panels whose rows do not fit the registers of one work-group (complex double
above 512 rows, double and complex float above 2048) are factored in memory,
one column step at a time; float keeps four rows per thread up to 4096.

Bar: ipiv and info identical to the oracle, L and U bit-identical, X
bit-identical (the blocked solve keeps the plain order of operations).  At
n = 4096, where the oracle would take minutes, the first 64 columns of L,
sampled columns of U's first 64 rows and the first 64 pivots are compared
bit for bit with the oracle's LU of the leading n x 64 block (those depend on
nothing else), and the whole factorisation is checked by its invariants."""
import numpy as np
import pytest

import lu_inputs
from gpu_support import bits, gesv_gpu, gpu_available, matrices_equal_bits, oracle_run, to_dev, to_host

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    import dense_linear_algebra_amd as lib
else:
    lib = None


@pytest.fixture(autouse=True)
def _blocked_tier():
    if not gpu_available():
        pytest.skip("no GPU")
    lib.batchlu_set_tier(lib.TIER_BLOCKED)
    yield
    lib.batchlu_set_tier(lib.TIER_AUTO)


# (type, n, batch): complex double 600 / 1100 and double 2100 / complex float
# 2070 start with panels factored in memory; float 2500 runs four rows per
# thread in registers
CASES = [(np.complex128, 600, 3), (np.complex128, 1100, 1), (np.float64, 2100, 1),
         (np.complex64, 2070, 1), (np.float32, 2500, 1)]


@pytest.mark.parametrize("dtype,n,batch", CASES, ids=lambda v: getattr(v, "__name__", str(v)))
def test_tall_panels_match_oracle(dtype, n, batch):
    nrhs = 2
    A, B = lu_inputs.random_problem(9100 + n, dtype, n, nrhs, batch)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert np.array_equal(bits(gB), bits(oB)), "X differs from the oracle"


def _one(M, dtype):
    return np.ascontiguousarray(np.asarray(M, dtype=dtype).T).reshape(-1).copy()


def test_tall_panel_special_matrices():
    """Complex double n = 600 (the first three panels in memory): Wilkinson
    growth (every step a tie), a zero column inside the second panel, a
    singular last step and a NaN in the third panel; B untouched where
    info > 0."""
    dtype, n, nrhs = np.complex128, 600, 2
    rng = np.random.default_rng(5)
    W = np.tril(-np.ones((n, n)), -1) + np.eye(n)
    W[:, -1] = 1
    Z = rng.uniform(-1, 1, (n, n))
    Z[:, 45] = 0
    S = rng.uniform(-1, 1, (n, n))
    S[-1, :] = 0
    N = rng.uniform(-1, 1, (n, n)) + 1j * rng.uniform(-1, 1, (n, n))
    N[70, 70] = np.nan
    mats = [W, Z, S, N, rng.uniform(-1, 1, (n, n)) - 1j * rng.uniform(-1, 1, (n, n))]
    batch = len(mats)
    A = np.concatenate([_one(M, dtype) for M in mats])
    B = lu_inputs.random_problem(31, dtype, n, nrhs, batch)[1]
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert np.array_equal(bits(gB), bits(oB))
    assert oI[1] == 46 and oI[2] == n
    for b in range(batch):
        if oI[b] > 0:
            np.testing.assert_array_equal(bits(gB[b * n * nrhs:(b + 1) * n * nrhs]),
                                          bits(B[b * n * nrhs:(b + 1) * n * nrhs]))


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128],
                         ids=lambda v: v.__name__)
def test_largest_order(dtype):
    import oracle
    n, K = 4096, 64
    A, _ = lu_inputs.random_problem(4242, dtype, n, 1, 1)
    dA = to_dev(A)
    dP = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    dI = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    lib.batchlu_getrf(lib.dtype_code(np.dtype(dtype)), n, dA, n, n * n, dP, n, dI, 1)
    torch.cuda.synchronize()
    gA, gP, gI = to_host(dA), to_host(dP), to_host(dI)
    del dA
    assert gI[0] == 0
    assert ((gP >= np.arange(1, n + 1)) & (gP <= n)).all(), "ipiv[j] must lie in [j + 1, n]"

    # the leading n x K block: pivots, L's columns and U's rows 0..K-1 depend
    # on it alone (and on the later interchanges, applied to L as recorded)
    lead = A[: n * K].copy()
    oP, oI, _, _ = oracle.getrf_rect(lead, n, K, n, n * K, 1)
    assert oI[0] == 0
    np.testing.assert_array_equal(gP[:K], oP[0])
    Lo = oracle.matrix(lead, 0, n, K, n, n * K)
    for j in range(K, n):
        p = int(gP[j]) - 1
        if p != j:
            Lo[[j, p]] = Lo[[p, j]]
    assert np.array_equal(bits(oracle.matrix(gA, 0, n, K, n, n * n)), bits(Lo))
    for c in (K, K + 1, 1000, 2047, 3333, n - 1):
        buf = np.concatenate([A[: n * K], A[c * n:(c + 1) * n]])
        oracle.getrf_rect(buf, n, K + 1, n, n * (K + 1), 1)
        assert np.array_equal(bits(gA[c * n: c * n + K]), bits(buf[K * n: K * n + K])), f"U[:{K}, {c}]"

    # the whole factorisation: |l| bounded by partial pivoting (the pivot's
    # metric |re| + |im| is the column's largest, so |l| <= sqrt 2 for complex
    # types), and P A = L U to a small multiple of n eps ||A||
    wide = np.complex128 if np.iscomplexobj(A) else np.float64
    M = gA.reshape(n, n).T.astype(wide)
    L = np.tril(M, -1)
    bound = (np.sqrt(2.0) if np.iscomplexobj(A) else 1.0) * (1 + 4 * oracle.eps_of(dtype))
    assert np.abs(L).max() <= bound
    L += np.eye(n, dtype=wide)
    U = np.triu(M)
    del M
    A0 = A.reshape(n, n).T.astype(wide)
    R = A0[oracle.perm_from_ipiv(gP, n)] - L @ U
    ratio = np.linalg.norm(R) / (n * oracle.eps_of(dtype) * np.linalg.norm(A0))
    assert ratio < 30, ratio
