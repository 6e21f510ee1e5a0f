"""GPU parity of the blocked tier (panel 32, fused right interchange + TRSM,
MFMA trailing update for real types, deferred left interchange) and of the
blocked getrs, against the CPU oracle through the C ABI.

Bar: ipiv and info identical and L, U bit-identical (the blocked update
chains one fused multiply-add per k in ascending order, as the unblocked
oracle does; an MFMA 16x16x4 accumulates exactly that way, which the
f32/f64 cases here check at scale); getrs X bit-identical to the oracle's
getrs on the same factors (same order, true division by u_kk)."""
import numpy as np
import pytest

import lu_inputs
import oracle
from gpu_support import bits, gesv_gpu, gpu_available, matrices_equal_bits, oracle_run

pytestmark = pytest.mark.gpu

if gpu_available():
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


CASES = ([(np.float32, n) for n in (1, 7, 32, 33, 64, 65, 100, 161, 256, 257, 290, 384, 520, 700)]
         + [(np.float64, n) for n in (31, 64, 96, 130, 256, 300)]
         + [(np.complex64, n) for n in (40, 64, 100, 130, 200, 300)]
         + [(np.complex128, n) for n in (33, 70, 100, 161, 257)])


@pytest.mark.parametrize("dtype,n", CASES, ids=lambda v: getattr(v, "__name__", str(v)))
def test_blocked_getrf_matches_oracle(dtype, n):
    batch = 5
    A, _ = lu_inputs.random_problem(6000 + n, dtype, n, 0, batch)
    print(f"case blocked getrf dtype={np.dtype(dtype).name} n={n}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    oA, _, oP, oI, _ = oracle_run(A, None, n, 0, batch, op="getrf")
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []


@pytest.mark.parametrize("dtype,n,nrhs", [(np.float32, 100, 3), (np.float32, 256, 33), (np.float64, 130, 5),
                                          (np.complex64, 70, 2), (np.complex128, 40, 3)])
def test_blocked_getrs_matches_oracle_bitwise(dtype, n, nrhs):
    batch = 4
    A, B = lu_inputs.random_problem(7000 + n, dtype, n, nrhs, batch)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch, op="getrf+getrs")
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch)
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []
    for b in range(batch):
        Am = oracle.matrix(A, b, n, n, n, n * n)
        assert oracle.solve_residual(Am, oracle.matrix(gB, b, n, nrhs, n, n * nrhs),
                                     oracle.matrix(B, b, n, nrhs, n, n * nrhs)) <= 20


def test_blocked_getrs_beyond_one_launch_solve():
    """n > 1024: getrs runs as the blocked sequence of 32-row triangular
    solves and GEMM updates (ascending k forward, descending k backward)."""
    n, nrhs, batch = 1100, 3, 2
    A, B = lu_inputs.random_problem(7300, np.float32, n, nrhs, batch)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch, op="getrf+getrs")
    oA, _, oP, oI, _ = oracle_run(A, None, n, 0, batch, op="getrf")
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    oB = B.copy()
    oracle.getrs(gA, n, n, n * n, gP[:, :n], oB, nrhs, n, n * nrhs, batch)
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_blocked_gesv_matches_oracle(dtype):
    n, nrhs, batch = 97, 4, 6
    A, B = lu_inputs.random_problem(7100, dtype, n, nrhs, batch)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []


def _one(M, dtype):
    return np.ascontiguousarray(np.asarray(M, dtype=dtype).T).reshape(-1).copy()


@pytest.mark.parametrize("n", [90, 300])
@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64])
def test_blocked_special_matrices(dtype, n):
    """Wilkinson growth across several panels (every step a tie), a zero
    column inside the second panel (info from a later panel), a singular last
    step and a NaN; B untouched where info > 0.  n = 90 runs the one-work-group
    kernel for real types, n = 300 the multi-launch sequence."""
    nrhs = 2
    rng = np.random.default_rng(3)
    W = np.tril(-np.ones((n, n)), -1) + np.eye(n)
    W[:, -1] = 1
    Z = rng.uniform(-1, 1, (n, n))
    Z[:, 45] = 0
    S = rng.uniform(-1, 1, (n, n))
    S[-1, :] = 0
    N = rng.uniform(-1, 1, (n, n))
    N[70, 50] = np.nan
    mats = [W, Z, S, N, rng.uniform(-1, 1, (n, n))]
    batch = len(mats)
    A = np.concatenate([_one(M, dtype) for M in mats])
    B = rng.uniform(-1, 1, batch * n * nrhs).astype(dtype)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert oI[1] == 46 and oI[2] == n
    for b in range(batch):
        if oI[b] > 0:
            np.testing.assert_array_equal(bits(gB[b * n * nrhs:(b + 1) * n * nrhs]),
                                          bits(B[b * n * nrhs:(b + 1) * n * nrhs]))


@pytest.mark.parametrize("dtype,n,nrhs", [(np.float32, 75, 3), (np.float64, 66, 1), (np.complex64, 41, 2)])
def test_blocked_padded_layout_keeps_poison(dtype, n, nrhs):
    batch = 3
    lda, ldb, sP = n + 5, n + 1, n + 3
    sA, sB = lda * n + 11, ldb * nrhs + 3
    A, B = lu_inputs.random_problem(7200 + n, dtype, n, nrhs, batch)
    poison = 1.0e30
    Ap = lu_inputs.relayout(A, n, n, batch, n, n * n, lda, sA, poison)
    Bp = lu_inputs.relayout(B, n, nrhs, batch, n, n * nrhs, ldb, sB, poison)
    gA, gB, gP, gI = gesv_gpu(lib, Ap, Bp, n, nrhs, batch, lda=lda, sA=sA, ldb=ldb, sB=sB, sP=sP)
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert np.all(gP[:, n:] == -7)
    back = lu_inputs.relayout(gA, n, n, batch, lda, sA, n, n * n)
    assert matrices_equal_bits(back, oA, n, n, n, n * n, batch) == []
    Xd = lu_inputs.relayout(gB, n, nrhs, batch, ldb, sB, n, n * nrhs)
    assert matrices_equal_bits(Xd, oB, n, nrhs, n, n * nrhs, batch) == []
    for buf, ld, st, cols in ((gA, lda, sA, n), (gB, ldb, sB, nrhs)):
        mask = np.ones(buf.size, bool)
        for b in range(batch):
            for j in range(cols):
                mask[b * st + j * ld: b * st + j * ld + n] = False
        assert np.all(buf[mask] == poison)


@pytest.mark.parametrize("name", ["dgesv_n256_b1024", "sgetrf_sgetrs_n1024_r32_b64"])
def test_blocked_full_size_workloads(name):
    """The blocked-tier workloads at their full batch under automatic tier
    selection, every matrix compared: ipiv, info and LU bit-identical, X
    bit-identical to the oracle's solve."""
    lib.batchlu_set_tier(lib.TIER_AUTO)
    w = lu_inputs.WORKLOADS[name]
    A, B = lu_inputs.dense_problem(w)
    print(f"case full {name}", flush=True)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, w.n, w.nrhs, w.batch, op="gesv" if w.op == "gesv" else "getrf+getrs")
    oA, oB, oP, oI, _ = oracle_run(A, B, w.n, w.nrhs, w.batch, op="gesv" if w.op == "gesv" else "getrf+getrs")
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :w.n], oP)
    assert matrices_equal_bits(gA, oA, w.n, w.n, w.n, w.n * w.n, w.batch) == []
    assert matrices_equal_bits(gB, oB, w.n, w.nrhs, w.n, w.n * w.nrhs, w.batch) == []
    # the two accuracy bounds of the target on a sample of the batch:
    # ||PA - LU||_F / (n eps ||A||_F) <= 20 and the solve residual <= 20
    sample = sorted({0, w.batch // 3, w.batch // 2, w.batch - 1})
    for b in sample:
        Am = oracle.matrix(A, b, w.n, w.n, w.n, w.n * w.n)
        fr = oracle.factor_residual(Am, oracle.matrix(gA, b, w.n, w.n, w.n, w.n * w.n), gP[b, :w.n])
        assert fr <= 20, f"matrix {b}: factor residual {fr}"
        sr = oracle.solve_residual(Am, oracle.matrix(gB, b, w.n, w.nrhs, w.n, w.n * w.nrhs),
                                   oracle.matrix(B, b, w.n, w.nrhs, w.n, w.n * w.nrhs))
        assert sr <= 20, f"matrix {b}: solve residual {sr}"


@pytest.mark.parametrize("n,batch", [(256, 1100), (96, 1024), (200, 700)])
def test_fused_double_three_and_four_per_compute_unit(n, batch):
    """The double one-work-group kernel budgeted for four work-groups per
    compute unit (batch >= 1024: 64-column U12 stage, pivot row read from LDS
    in the panel update) and for three (batch 513 - 1023: 112-column stage):
    ipiv, info and LU bit-identical to the oracle on matrices spread over
    the batch."""
    dtype = np.float64
    A, _ = lu_inputs.random_problem(4400 + n, dtype, n, 1, batch)
    print(f"case fused f64 3/CU n={n} batch={batch}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    for b in np.linspace(0, batch - 1, 4).astype(int):
        sl = slice(b * n * n, (b + 1) * n * n)
        oA = A[sl].copy()
        oP, oI, _, _ = oracle.getrf(oA, n, n, n * n, 1)
        assert gI[b] == oI[0]
        np.testing.assert_array_equal(gP[b, :n], oP[0])
        assert np.array_equal(bits(gA[sl]), bits(oA))


@pytest.mark.parametrize("dtype,n,batch", [(np.float32, 1600, 12), (np.float64, 1540, 12)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_lookahead_from_1536_rows(dtype, n, batch):
    """From n = 1536 the next panel runs on the look-ahead stream up to two
    64-row strips per compute unit over the batch (here 25 x 12 and 24 x 12):
    LU, ipiv and info bit-identical to the oracle."""
    A, _ = lu_inputs.random_problem(7700 + n, dtype, n, 1, batch)
    print(f"case look-ahead {np.dtype(dtype).name} n={n} batch={batch}", flush=True)
    gA, _, gP, gI = gesv_gpu(lib, A, None, n, 0, batch, op="getrf")
    oA, _, oP, oI, _ = oracle_run(A, None, n, 0, batch, op="getrf")
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []


@pytest.mark.parametrize("dtype,n", [(np.float32, 300), (np.float64, 290), (np.complex64, 130), (np.complex128, 100)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_batch_multiple_of_eight(dtype, n):
    """A batch that is a multiple of eight maps the trailing-update strips
    (and the solve's right-hand-side tiles) of one matrix to one XCD: LU,
    ipiv, info and X bit-identical to the oracle."""
    batch, nrhs = 16, 12
    A, B = lu_inputs.random_problem(7900 + n, dtype, n, nrhs, batch)
    print(f"case batch 16 {np.dtype(dtype).name} n={n}", flush=True)
    gA, gB, gP, gI = gesv_gpu(lib, A, B, n, nrhs, batch, op="getrf+getrs")
    oA, oB, oP, oI, _ = oracle_run(A, B, n, nrhs, batch, op="getrf+getrs")
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :n], oP)
    assert matrices_equal_bits(gA, oA, n, n, n, n * n, batch) == []
    assert matrices_equal_bits(gB, oB, n, nrhs, n, n * nrhs, batch) == []
