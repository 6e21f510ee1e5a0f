"""GPU parity of LU on m x n matrices and on variable-size batches
(batchlu_getrf_rect, batchlu_getrf_vbatched, batchlu_getrs_vbatched,
batchlu_gesv_vbatched) against the CPU oracle, through the C ABI.

Bar: info and ipiv identical, L and U bit-identical to the rectangular
oracle (the kernel keeps the unblocked operation order per element); X
bit-identical to the oracle's getrs on the same factors; padding and
matrices refused as invalid left untouched."""
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


def _rect_gpu(A, m, n, batch, lda=None, sA=None, sP=None):
    lda = m if lda is None else lda
    sA = lda * n if sA is None else sA
    k = min(m, n)
    sP = k if sP is None else sP
    dA = to_dev(A)
    dP = torch.full((batch * max(sP, 1),), -7, dtype=torch.int32, device="cuda")
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    lib.batchlu_getrf_rect(lib.dtype_code(A.dtype), m, n, dA, lda, sA, dP, sP, dI, batch)
    torch.cuda.synchronize()
    return to_host(dA), to_host(dP).reshape(batch, max(sP, 1)), to_host(dI)


SHAPES = ([(np.float32, m, n) for m, n in [(50, 20), (20, 50), (1, 7), (7, 1), (33, 31), (31, 33), (100, 257),
                                           (257, 100), (1024, 300), (300, 1024), (700, 64), (64, 700)]]
          + [(np.float64, m, n) for m, n in [(40, 10), (10, 40), (512, 100), (100, 512), (129, 65)]]
          + [(np.complex64, m, n) for m, n in [(64, 16), (16, 64), (512, 40), (70, 300)]]
          + [(np.complex128, m, n) for m, n in [(48, 20), (20, 48), (256, 33), (33, 256), (100, 1000)]])


@pytest.mark.parametrize("dtype,m,n", SHAPES, ids=lambda v: getattr(v, "__name__", str(v)))
def test_getrf_rect_matches_oracle(dtype, m, n):
    batch = 4 if m * n <= 100000 else 2
    rng = np.random.Generator(np.random.PCG64(m * 7919 + n))
    A = lu_inputs.draw(rng, dtype, batch * m * n)
    gA, gP, gI = _rect_gpu(A, m, n, batch)
    oA = A.copy()
    oP, oI, _, _ = oracle.getrf_rect(oA, m, n, m, m * n, batch)
    np.testing.assert_array_equal(gI, oI)
    np.testing.assert_array_equal(gP[:, :min(m, n)], oP)
    assert np.array_equal(bits(gA), bits(oA))


@pytest.mark.parametrize("dtype,m,n", [(np.float32, 90, 40), (np.float32, 40, 90), (np.float64, 70, 130),
                                       (np.complex64, 130, 70)], ids=lambda v: getattr(v, "__name__", str(v)))
def test_getrf_rect_special_values(dtype, m, n):
    """A zero column (info from a later panel, zero pivot left out of the
    solve and the update), an infinity and a -0 in that pivot's row, a NaN,
    ties; padded lda and batch stride keep their poison."""
    batch = 4
    lda, sA, sP = m + 5, (m + 5) * n + 7, min(m, n) + 3
    rng = np.random.Generator(np.random.PCG64(9 * m + n))
    mats = []
    for b in range(batch):
        M = lu_inputs.draw(rng, dtype, m * n).reshape(n, m).T.copy()
        if b == 0:
            M[:, 35] = 0
            M[34, 37:] = np.inf
            M[:, 38] = -0.0
        elif b == 1:
            M[20, 10] = np.nan
        elif b == 2:
            M[:, :] = np.round(M.real * 2)      # small integers: exact ties
        mats.append(np.ascontiguousarray(M.T).reshape(-1))
    A0 = np.concatenate(mats).astype(dtype)
    A = lu_inputs.relayout(A0, m, n, batch, m, m * n, lda, sA, poison=-99.0)
    gA, gP, gI = _rect_gpu(A, m, n, batch, lda=lda, sA=sA, sP=sP)
    oA = A.copy()
    oP, oI, _, _ = oracle.getrf_rect(oA, m, n, lda, sA, batch, strideP=sP)
    np.testing.assert_array_equal(gI, oI)
    assert oI[0] == 36
    np.testing.assert_array_equal(gP[:, :min(m, n)], oP)
    assert np.array_equal(bits(gA), bits(oA))


def _pack(mats, pad_rows, pad_after, dtype):
    """One device buffer holding every matrix column-major with its own lda
    (rows + pad) and a gap after it; returns (buffer, offsets, ldas)."""
    chunks, offs, ldas, off = [], [], [], 0
    for M, pr, pa in zip(mats, pad_rows, pad_after):
        m, n = M.shape
        ld = m + pr
        block = np.full(max(ld * n, 1) + pa, -33.0, dtype=dtype)
        for j in range(n):
            block[j * ld: j * ld + m] = M[:, j]
        offs.append(off)
        ldas.append(max(ld, 1))
        chunks.append(block)
        off += block.size
    return np.concatenate(chunks), offs, ldas


def _ptrs(base, offs, es):
    return torch.tensor([base.data_ptr() + o * es for o in offs], dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
def test_getrf_vbatched_matches_oracle(dtype):
    """40 matrices of random shapes (1..max) in one launch, each with its own
    lda; one entry with lda < m is refused (info -1, bytes untouched)."""
    rng = np.random.default_rng(5 + np.dtype(dtype).itemsize)
    maxm = {np.float32: 300, np.float64: 300, np.complex64: 200, np.complex128: 120}[dtype]
    batch = 40
    ms = rng.integers(1, maxm + 1, batch)
    ns = rng.integers(1, maxm + 1, batch)
    ms[3], ns[3] = 1, 1
    ms[4], ns[4] = maxm, 17
    ms[5], ns[5] = 9, maxm
    mats = [lu_inputs.draw(rng, dtype, int(m) * int(n)).reshape(int(n), int(m)).T.copy() for m, n in zip(ms, ns)]
    mats[7][:, min(2, int(ns[7]) - 1)] = 0
    pads = list(rng.integers(0, 4, batch))
    buf, offs, ldas = _pack(mats, pads, [5] * batch, dtype)
    ldas[11] = max(int(ms[11]) - 1, 0) if ms[11] > 1 else ldas[11]
    bad = 11 if ms[11] > 1 else None
    es = np.dtype(dtype).itemsize
    dbuf = to_dev(buf)
    kmax = int(np.max(np.minimum(ms, ns)))
    dpiv = torch.full((batch * kmax,), -7, dtype=torch.int32, device="cuda")
    ipiv_ptrs = torch.tensor([dpiv.data_ptr() + 4 * b * kmax for b in range(batch)], dtype=torch.int64,
                             device="cuda")
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    dm = torch.tensor(ms, dtype=torch.int32, device="cuda")
    dn = torch.tensor(ns, dtype=torch.int32, device="cuda")
    dl = torch.tensor(ldas, dtype=torch.int32, device="cuda")
    lib.batchlu_getrf_vbatched(lib.dtype_code(np.dtype(dtype)), dm, dn, _ptrs(dbuf, offs, es), dl, ipiv_ptrs, dI,
                               int(ms.max()), int(ns.max()), batch)
    torch.cuda.synchronize()
    g = to_host(dbuf)
    gP = to_host(dpiv).reshape(batch, kmax)
    gI = to_host(dI)
    o = buf.copy()
    for b in range(batch):
        m, n, ld = int(ms[b]), int(ns[b]), ldas[b]
        seg = slice(offs[b], offs[b] + ld * n)
        if b == bad:
            assert gI[b] == -1
            assert np.array_equal(bits(g[seg]), bits(buf[seg]))
            continue
        a = o[seg].copy()
        oP, oI, _, _ = oracle.getrf_rect(a, m, n, ld, ld * n, 1)
        o[seg] = a
        assert gI[b] == oI[0], f"matrix {b} ({m} x {n})"
        assert np.array_equal(gP[b, :min(m, n)], oP[0]), f"matrix {b} ({m} x {n})"
    assert np.array_equal(bits(g), bits(o))   # factors, and every pad and gap untouched


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.complex64, np.complex128])
def test_gesv_vbatched_matches_oracle(dtype):
    """Square matrices of random orders 1..max with random nrhs (one has 0);
    X bit-identical to the oracle's gesv; a singular matrix keeps its B."""
    rng = np.random.default_rng(11 + np.dtype(dtype).itemsize)
    maxn = {np.float32: 256, np.float64: 200, np.complex64: 160, np.complex128: 100}[dtype]
    batch = 30
    ns = rng.integers(1, maxn + 1, batch)
    ns[0] = maxn
    rs = rng.integers(1, 7, batch)
    rs[2] = 0
    As = [lu_inputs.draw(rng, dtype, int(n) * int(n)).reshape(int(n), int(n)).T.copy() for n in ns]
    Bs = [lu_inputs.draw(rng, dtype, int(n) * int(r)).reshape(int(r), int(n)).T.copy() for n, r in zip(ns, rs)]
    sing = 4
    As[sing][:, min(3, int(ns[sing]) - 1)] = 0
    abuf, aoffs, aldas = _pack(As, list(rng.integers(0, 3, batch)), [3] * batch, dtype)
    bbuf, boffs, bldas = _pack(Bs, list(rng.integers(0, 3, batch)), [3] * batch, dtype)
    es = np.dtype(dtype).itemsize
    dA, dB = to_dev(abuf), to_dev(bbuf)
    dpiv = torch.zeros(batch * maxn, dtype=torch.int32, device="cuda")
    pptr = torch.tensor([dpiv.data_ptr() + 4 * b * maxn for b in range(batch)], dtype=torch.int64, device="cuda")
    dI = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    dn = torch.tensor(ns, dtype=torch.int32, device="cuda")
    dr = torch.tensor(rs, dtype=torch.int32, device="cuda")
    dla = torch.tensor(aldas, dtype=torch.int32, device="cuda")
    dlb = torch.tensor(bldas, dtype=torch.int32, device="cuda")
    lib.batchlu_gesv_vbatched(lib.dtype_code(np.dtype(dtype)), dn, dr, _ptrs(dA, aoffs, es), dla, pptr,
                              _ptrs(dB, boffs, es), dlb, dI, maxn, batch)
    torch.cuda.synchronize()
    gA, gB, gI = to_host(dA), to_host(dB), to_host(dI)
    oA, oB = abuf.copy(), bbuf.copy()
    for b in range(batch):
        n, r = int(ns[b]), int(rs[b])
        sa = slice(aoffs[b], aoffs[b] + aldas[b] * n)
        sb = slice(boffs[b], boffs[b] + bldas[b] * max(r, 1))
        a, bb = oA[sa].copy(), oB[sb].copy()
        _, oI, _, _ = oracle.gesv(a, n, aldas[b], aldas[b] * n, bb, r, bldas[b], bldas[b] * max(r, 1), 1)
        oA[sa], oB[sb] = a, bb
        assert gI[b] == oI[0], f"matrix {b}"
    assert gI[sing] > 0
    assert np.array_equal(bits(gA), bits(oA))
    assert np.array_equal(bits(gB), bits(oB))


def test_argument_errors():
    t = lib.R32
    d = torch.zeros(64, dtype=torch.float32, device="cuda")
    di = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert lib.batchlu_getrf_rect(t, -1, 3, d, 1, 3, di, 1, di, 1, raise_on_error=False) == -2
    assert lib.batchlu_getrf_rect(t, 4, 3, d, 3, 12, di, 3, di, 1, raise_on_error=False) == -5
    assert lib.batchlu_getrf_rect(t, 4, 3, d, 4, 11, di, 3, di, 2, raise_on_error=False) == -6
    assert lib.batchlu_getrf_rect(t, 4, 3, d, 4, 12, di, 2, di, 2, raise_on_error=False) == -8
    assert lib.batchlu_getrf_rect(t, 0, 3, d, 1, 3, di, 0, di, 2, raise_on_error=False) == 0
    assert lib.batchlu_getrf_rect(t, 2000, 3, d, 2000, 6000, di, 3, di, 1, raise_on_error=False) == -101
    assert lib.batchlu_getrf_vbatched(t, di, di, d, di, d, di, 5000, 4, 1, raise_on_error=False) == -101
    assert lib.batchlu_getrf_vbatched(t, None, di, d, di, d, di, 5, 4, 1, raise_on_error=False) == -2
    assert lib.batchlu_gesv_vbatched(t, di, di, d, di, d, d, di, None, 4, 1, raise_on_error=False) == -9
