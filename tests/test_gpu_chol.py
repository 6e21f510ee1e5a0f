"""GPU parity of batched Cholesky (potrf, potrs, posv) against the CPU oracle,
through the C ABI, on both triangles and every tier.

Bar: info identical; the named triangle of the factor bit-identical to the
oracle's (every tier accumulates each entry over k in ascending order by
fused multiply-adds -- the register kernel one step at a time, the blocked
tier through MFMA chains, which accumulate like fused multiply-adds in k
order -- and scales by one rounded reciprocal of the diagonal); X
bit-identical to the oracle's solve (same order, true division); the other
triangle and every padding element untouched.  Where a matrix is not
positive definite, only columns 0 .. j-1 and a_jj are defined, and only
they are compared; B keeps its bytes."""
import numpy as np
import pytest

import lu_inputs
import oracle
from gpu_support import bits, gpu_available, to_dev, to_host

pytestmark = pytest.mark.gpu

if gpu_available():
    import dense_linear_algebra_amd as lib
    import torch
else:
    lib = None


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    yield
    lib.batchlu_set_tier(lib.TIER_AUTO)


def _poison_other(A, n, batch, uplo):
    """A copy whose triangle that uplo does not name holds NaN."""
    P = A.copy().reshape(batch, n, n)            # [b, col, row] (column-major)
    cols, rows = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    mask = rows < cols if uplo == "L" else rows > cols
    P[:, mask] = np.nan
    return P.reshape(-1), mask


def _defined_mask(n, info, uplo):
    """Stored positions of the defined part of the factor: the named
    triangle, or for info = j + 1 > 0 its columns 0 .. j-1 and a_jj."""
    cols, rows = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")   # [col, row]
    i, k = (rows, cols) if uplo == "L" else (cols, rows)                  # factor element (i, k)
    tri = i >= k
    if info == 0:
        return tri
    j = info - 1
    return tri & ((k < j) | ((k == j) & (i == j)))


def _check_factor(gA, oA, n, batch, info, uplo, mask_other, A_in):
    g = gA.reshape(batch, n, n)
    o = oA.reshape(batch, n, n)
    a0 = A_in.reshape(batch, n, n)
    for b in range(batch):
        d = _defined_mask(n, int(info[b]), uplo)
        assert np.array_equal(bits(g[b][d]), bits(o[b][d])), f"matrix {b}: factor differs from the oracle"
        assert np.array_equal(bits(g[b][mask_other]), bits(a0[b][mask_other])), f"matrix {b}: other triangle"


def _potrf_gpu(A, n, batch, uplo):
    t = lib.dtype_code(A.dtype)
    dA = to_dev(A)
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    lib.batchlu_potrf(t, uplo, n, dA, n, n * n, dI, batch)
    torch.cuda.synchronize()
    return to_host(dA), to_host(dI)


def _posv_gpu(A, B, n, nrhs, batch, uplo):
    t = lib.dtype_code(A.dtype)
    dA, dB = to_dev(A), to_dev(B)
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    lib.batchlu_posv(t, uplo, n, nrhs, dA, n, n * n, dB, n, n * nrhs, dI, batch)
    torch.cuda.synchronize()
    return to_host(dA), to_host(dB), to_host(dI)


TIERS = {"register": 2, "blocked": 3}
REG_CASES = [(np.float32, n) for n in (1, 5, 8, 16, 17, 31, 32, 33, 48, 64)] + \
            [(np.float64, n) for n in (3, 16, 32, 40, 64)] + \
            [(np.complex64, n) for n in (2, 16, 30, 64)] + \
            [(np.complex128, n) for n in (1, 9, 16, 32)]
BLK_CASES = [(np.float32, n) for n in (1, 31, 32, 33, 65, 100, 200, 257, 520, 1024)] + \
            [(np.float64, n) for n in (40, 64, 97, 256, 300)] + \
            [(np.complex64, n) for n in (33, 96, 130, 257)] + \
            [(np.complex128, n) for n in (20, 70, 161, 512)]


def _cases():
    for dt, n in REG_CASES:
        yield "register", dt, n
    for dt, n in BLK_CASES:
        yield "blocked", dt, n


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("tier,dtype,n", list(_cases()), ids=lambda v: getattr(v, "__name__", str(v)))
def test_potrf_matches_oracle(tier, dtype, n, uplo):
    lib.batchlu_set_tier(TIERS[tier])
    batch = 37 if n <= 64 else (5 if n <= 300 else 2)
    A, _ = lu_inputs.spd_problem(1000 + n, dtype, n, 1, batch)
    A, mask = _poison_other(A, n, batch, uplo)
    gA, gI = _potrf_gpu(A, n, batch, uplo)
    oA = A.copy()
    oI, _ = oracle.potrf(oA, n, n, n * n, batch, uplo=uplo)
    np.testing.assert_array_equal(gI, oI)
    assert not oI.any()
    _check_factor(gA, oA, n, batch, oI, uplo, mask, A)


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("tier,dtype,n,nrhs", [
    ("register", np.float32, 32, 8), ("register", np.float32, 16, 1), ("register", np.float64, 50, 16),
    ("register", np.complex64, 64, 3), ("register", np.complex128, 20, 8), ("register", np.float32, 24, 20),
    ("blocked", np.float32, 100, 3), ("blocked", np.float64, 256, 1), ("blocked", np.complex64, 70, 5),
    ("blocked", np.complex128, 97, 2), ("blocked", np.float32, 1024, 32)],
    ids=lambda v: getattr(v, "__name__", str(v)))
def test_posv_matches_oracle(tier, dtype, n, nrhs, uplo):
    """posv: fused in the register kernel (nrhs <= 16) or potrf then the
    one-launch solve; X bit-identical to the oracle's."""
    lib.batchlu_set_tier(TIERS[tier])
    batch = 33 if n <= 64 else 3
    A, B = lu_inputs.spd_problem(2000 + n + nrhs, dtype, n, nrhs, batch)
    A, mask = _poison_other(A, n, batch, uplo)
    gA, gB, gI = _posv_gpu(A, B, n, nrhs, batch, uplo)
    oA, oB = A.copy(), B.copy()
    oI, _ = oracle.posv(oA, n, n, n * n, oB, nrhs, n, n * nrhs, batch, uplo=uplo)
    np.testing.assert_array_equal(gI, oI)
    _check_factor(gA, oA, n, batch, oI, uplo, mask, A)
    assert np.array_equal(bits(gB), bits(oB)), "X differs from the oracle"


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("dtype,n", [(np.float32, 200), (np.float64, 300), (np.complex64, 130), (np.complex128, 100)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_blocked_posv_batch_multiple_of_eight(dtype, n, uplo):
    """A batch that is a multiple of eight maps the trailing-update strips and
    the solve's right-hand-side tiles of one matrix to one XCD: the factor and
    X bit-identical to the oracle's."""
    lib.batchlu_set_tier(TIERS["blocked"])
    batch, nrhs = 16, 12
    A, B = lu_inputs.spd_problem(2500 + n, dtype, n, nrhs, batch)
    A, mask = _poison_other(A, n, batch, uplo)
    gA, gB, gI = _posv_gpu(A, B, n, nrhs, batch, uplo)
    oA, oB = A.copy(), B.copy()
    oI, _ = oracle.posv(oA, n, n, n * n, oB, nrhs, n, n * nrhs, batch, uplo=uplo)
    np.testing.assert_array_equal(gI, oI)
    _check_factor(gA, oA, n, batch, oI, uplo, mask, A)
    assert np.array_equal(bits(gB), bits(oB)), "X differs from the oracle"


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("dtype,n,nrhs", [(np.float32, 40, 4), (np.float64, 300, 3), (np.complex64, 129, 1),
                                          (np.complex128, 64, 5), (np.float32, 1000, 2)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_potrs_matches_oracle(dtype, n, nrhs, uplo):
    """potrs on the oracle's factor (so the solve alone is compared)."""
    batch = 3
    A, B = lu_inputs.spd_problem(3000 + n, dtype, n, nrhs, batch)
    F = A.copy()
    oracle.potrf(F, n, n, n * n, batch, uplo=uplo)
    oB = B.copy()
    oracle.potrs(F, n, n, n * n, oB, nrhs, n, n * nrhs, batch, uplo=uplo)
    dF, dB = to_dev(F), to_dev(B)
    lib.batchlu_potrs(lib.dtype_code(np.dtype(dtype)), uplo, n, nrhs, dF, n, n * n, dB, n, n * nrhs, batch)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(dB)), bits(oB))


def _not_pd_batch(dtype, n, batch, seed):
    """SPD matrices, some made indefinite at a chosen column: a_jj lowered so
    that column j's diagonal value is negative, zero-ish, or NaN."""
    A, B = lu_inputs.spd_problem(seed, dtype, n, 2, batch)
    M = A.reshape(batch, n, n)
    cols = [0, n // 2, n - 1, min(n - 1, 33), min(n - 1, 40)]
    M[1, cols[0], cols[0]] = -1.0
    M[2, cols[1], cols[1]] = -100.0 * n
    M[3, cols[2], cols[2]] = 0.0
    M[4, cols[3], cols[3]] = np.nan
    M[5, cols[4], cols[4]] = -3.0 * n
    return M.reshape(-1).copy(), B


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("tier,dtype,n", [("register", np.float32, 32), ("register", np.float64, 64),
                                          ("register", np.complex64, 45), ("register", np.complex128, 32),
                                          ("blocked", np.float32, 130), ("blocked", np.float64, 70),
                                          ("blocked", np.complex64, 100), ("blocked", np.complex128, 66)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_not_positive_definite(tier, dtype, n, uplo):
    """info names the first failing column; the defined part of the factor
    is bit-identical; posv keeps B where info > 0; later panels and updates
    skip a failed matrix."""
    lib.batchlu_set_tier(TIERS[tier])
    batch, nrhs = 7, 2
    A, B = _not_pd_batch(dtype, n, batch, 4000 + n)
    A, mask = _poison_other(A, n, batch, uplo)
    gA, gB, gI = _posv_gpu(A, B, n, nrhs, batch, uplo)
    oA, oB = A.copy(), B.copy()
    oI, _ = oracle.posv(oA, n, n, n * n, oB, nrhs, n, n * nrhs, batch, uplo=uplo)
    np.testing.assert_array_equal(gI, oI)
    assert (oI[1:6] > 0).all() and oI[0] == 0 and oI[6] == 0
    _check_factor(gA, oA, n, batch, oI, uplo, mask, A)
    for b in range(batch):
        s = slice(b * n * nrhs, (b + 1) * n * nrhs)
        want = B[s] if oI[b] > 0 else oB[s]
        assert np.array_equal(bits(gB[s]), bits(want)), f"matrix {b}"


@pytest.mark.parametrize("tier,dtype,n", [("register", np.float32, 20), ("blocked", np.float64, 90),
                                          ("register", np.complex64, 33), ("blocked", np.complex128, 40)],
                         ids=lambda v: getattr(v, "__name__", str(v)))
def test_padded_layout_keeps_poison(tier, dtype, n):
    """lda > n and strides beyond lda*n: padding is never written."""
    lib.batchlu_set_tier(TIERS[tier])
    batch, nrhs = 5, 3
    lda, sA, ldb, sB = n + 3, (n + 3) * n + 11, n + 2, (n + 2) * nrhs + 5
    A0, B0 = lu_inputs.spd_problem(5000 + n, dtype, n, nrhs, batch)
    A = lu_inputs.relayout(A0, n, n, batch, n, n * n, lda, sA, poison=-77.0)
    B = lu_inputs.relayout(B0, n, nrhs, batch, n, n * nrhs, ldb, sB, poison=-55.0)
    t = lib.dtype_code(np.dtype(dtype))
    dA, dB = to_dev(A), to_dev(B)
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    lib.batchlu_posv(t, "L", n, nrhs, dA, lda, sA, dB, ldb, sB, dI, batch)
    torch.cuda.synchronize()
    gA, gB = to_host(dA), to_host(dB)
    oA, oB = A.copy(), B.copy()
    oI, _ = oracle.posv(oA, n, lda, sA, oB, nrhs, ldb, sB, batch)
    np.testing.assert_array_equal(to_host(dI), oI)
    # the whole buffers: triangle and X identical, upper part and padding unchanged
    assert np.array_equal(bits(gA), bits(oA))
    assert np.array_equal(bits(gB), bits(oB))


def test_argument_errors_and_zero_work():
    t = lib.R32
    dA = torch.zeros(16, dtype=torch.float32, device="cuda")
    dI = torch.zeros(2, dtype=torch.int32, device="cuda")
    assert lib.batchlu_potrf(t, "X", 4, dA, 4, 16, dI, 1, raise_on_error=False) == -2
    assert lib.batchlu_potrf(t, "L", -1, dA, 4, 16, dI, 1, raise_on_error=False) == -3
    assert lib.batchlu_potrf(t, "L", 4, dA, 3, 16, dI, 1, raise_on_error=False) == -5
    assert lib.batchlu_potrf(t, "L", 4, dA, 4, 15, dI, 2, raise_on_error=False) == -6
    assert lib.batchlu_potrf(t, "L", 0, dA, 1, 0, dI, 2, raise_on_error=False) == 0
    assert lib.batchlu_potrf(t, "L", 2048, dA, 2048, 0, dI, 1, raise_on_error=False) == -101
    assert lib.batchlu_posv(t, "U", 4, 2, dA, 4, 16, dA, 3, 8, dI, 1, raise_on_error=False) == -9
    assert lib.batchlu_potrs(t, "L", 4, 0, dA, 4, 16, dA, 4, 0, 1, raise_on_error=False) == 0


@pytest.mark.parametrize("name", ["sposv_n32_r8_b32768", "dposv_n256_b1024"])
def test_full_size_workloads(name):
    """The benchmarked Cholesky shapes at full batch: info, factor and X
    bit-identical on a sample of matrices spread over the batch, and the
    reconstruction and solve residuals within 20."""
    w = lu_inputs.CHOL_WORKLOADS[name]
    A, B = lu_inputs.chol_problem(w)
    n, nrhs, batch = w.n, w.nrhs, w.batch
    gA, gB, gI = _posv_gpu(A, B, n, nrhs, batch, "L")
    assert not gI.any()
    for b in np.linspace(0, batch - 1, 6).astype(int):
        sa = slice(b * n * n, (b + 1) * n * n)
        sb = slice(b * n * nrhs, (b + 1) * n * nrhs)
        oA, oB = A[sa].copy(), B[sb].copy()
        oI, _ = oracle.posv(oA, n, n, n * n, oB, nrhs, n, n * nrhs, 1)
        assert oI[0] == 0
        tri = np.tril(np.ones((n, n), bool)).T.reshape(-1)    # lower triangle, column-major
        assert np.array_equal(bits(gA[sa][tri]), bits(oA[tri])), f"matrix {b}"
        assert np.array_equal(bits(gB[sb]), bits(oB)), f"matrix {b}"
        Am = oracle.matrix(A, b, n, n, n, n * n)
        assert oracle.chol_residual(Am, oracle.matrix(gA, b, n, n, n, n * n)) <= 20
        assert oracle.solve_residual(oracle.hermitian_from(Am), oracle.matrix(gB, b, n, nrhs, n, n * nrhs),
                                     oracle.matrix(B, b, n, nrhs, n, n * nrhs)) <= 20
