"""Seeded synthetic inputs for batched LU / solve.

This module only draws numbers and lays them out in memory; it holds none of
the factorisation's arithmetic, so both the CPU oracle side and the GPU side
may use it without sharing any step of the method.

Layout: every matrix is column-major; element (i, j) of matrix b sits at
``b*stride + i + j*ld`` of a flat 1-D buffer.  The workloads follow the five
shapes the BatchLAS pages time (LU page and Blackwell page): small float
systems in the register tier, a complex n = 64 system in the work-group tier,
a double n = 256 and a float n = 1024 system in the blocked tier.  Entries are
iid uniform[-1, 1] (complex: real and imaginary parts drawn as separate
blocks), except the n = 1024 workload, which draws N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: type
    n: int
    nrhs: int
    batch: int
    dist: str           # "uniform" (iid U[-1, 1]) or "normal" (iid N(0, 1))
    op: str             # "gesv", or "getrf+getrs"
    index: int          # 1-based position, sets the seed

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


WORKLOADS = {
    "sgesv_n16_b1024": Workload("sgesv_n16_b1024", np.float32, 16, 1, 1024, "uniform", "gesv", 1),
    "sgesv_n32_r8_b32768": Workload("sgesv_n32_r8_b32768", np.float32, 32, 8, 32768, "uniform", "gesv", 2),
    "cgesv_n64_r16_b8192": Workload("cgesv_n64_r16_b8192", np.complex64, 64, 16, 8192, "uniform", "gesv", 3),
    "dgesv_n256_b1024": Workload("dgesv_n256_b1024", np.float64, 256, 1, 1024, "uniform", "gesv", 4),
    "sgetrf_sgetrs_n1024_r32_b64": Workload("sgetrf_sgetrs_n1024_r32_b64", np.float32, 1024, 32, 64, "normal",
                                            "getrf+getrs", 5),
}


def draw(rng: np.random.Generator, dtype, size: int, dist: str = "uniform") -> np.ndarray:
    """``size`` iid entries of ``dtype``; complex draws the real block first."""
    dt = np.dtype(dtype)
    if dt.kind == "c":
        real = np.float32 if dt == np.complex64 else np.float64
        re = draw(rng, real, size, dist)
        im = draw(rng, real, size, dist)
        out = np.empty(size, dt)
        out.real, out.imag = re, im
        return out
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size).astype(dt)
    if dist == "normal":
        if dt == np.float32:
            return rng.standard_normal(size, dtype=np.float32)
        return rng.standard_normal(size).astype(dt)
    raise ValueError(dist)


def dense_problem(w: Workload, batch: int | None = None):
    """(A, B) as flat buffers with ld = n and strides n*n and n*nrhs.

    ``batch`` below the workload's batch takes the leading matrices of the
    same draw (A for all matrices is drawn before B)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    A = draw(rng, w.dtype, w.batch * w.n * w.n, w.dist)
    B = draw(rng, w.dtype, w.batch * w.n * w.nrhs, w.dist)
    if batch is not None and batch < w.batch:
        A = A[: batch * w.n * w.n].copy()
        B = B[: batch * w.n * w.nrhs].copy()
    return A, B


def random_problem(seed: int, dtype, n: int, nrhs: int, batch: int, dist: str = "uniform"):
    """Same recipe as the named workloads, any shape."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = draw(rng, dtype, batch * n * n, dist)
    B = draw(rng, dtype, batch * n * nrhs, dist)
    return A, B


def relayout(flat: np.ndarray, rows: int, cols: int, batch: int, ld_in: int, stride_in: int,
             ld_out: int, stride_out: int, poison=None) -> np.ndarray:
    """Copy a batch of rows x cols column-major matrices into a new buffer with
    another leading dimension / batch stride; the gaps hold ``poison``."""
    if ld_out < rows or (cols > 0 and stride_out < ld_out * (cols - 1) + rows):
        raise ValueError("output layout too small")
    total = stride_out * batch if batch > 0 else 0
    out = np.empty(max(total, 1), flat.dtype)
    out[:] = poison if poison is not None else 0
    for b in range(batch):
        for j in range(cols):
            src = b * stride_in + j * ld_in
            dst = b * stride_out + j * ld_out
            out[dst: dst + rows] = flat[src: src + rows]
    return out[:total] if total > 0 else out[:0]


def zero_pivot_problem(seed: int, dtype, n: int, nrhs: int, batch: int):
    """Matrices with exactly-zero pivots whose pivot rows carry an infinity
    and signed zeros into the trailing columns.

    Matrix b: iid uniform[-1, 1] entries (complex: both parts), a leading
    diagonal of 64 (so that no rows move before the first zero pivot), one or
    two columns that are entirely +-0 (so that their pivot is exactly zero
    whatever happens before), +inf in the trailing part of the first zero
    pivot's row, and a column of -0 below a 1 in that row.  Used to check
    that a step with a zero pivot changes nothing beyond its own column (no
    0 * inf, no +0 replacing a -0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    mats = []
    for b in range(batch):
        M = draw(rng, dtype, n * n).reshape(n, n)   # row-major view of the draw
        z = [5 + (b % 3)] + ([37 + (b % 5)] if n > 48 else [])
        for j in range(z[0]):
            M[j, j] = 64
        for zc in z:
            col = np.zeros(n, dtype)
            col[1::2] = -0.0
            M[:, zc] = col
        zr = z[0]
        if n > 40:
            cinf, cneg = n - 3, n - 7
            M[zr, cinf] = np.inf
            M[:, cneg] = -0.0
            M[zr, cneg] = 1
        mats.append(np.ascontiguousarray(M.T).reshape(-1))    # column-major
    A = np.concatenate(mats) if mats else np.zeros(0, dtype)
    B = draw(rng, dtype, batch * n * nrhs)
    return A, B


def spd_problem(seed: int, dtype, n: int, nrhs: int, batch: int):
    """Hermitian (real: symmetric) positive definite matrices and right-hand
    sides, both triangles stored.

    Matrix b is (G G^H) / n + I with G iid uniform[-1, 1] (complex: both
    parts), formed in double precision, made exactly Hermitian as (M + M^H)/2
    and then rounded to ``dtype`` (rounding commutes with conjugation, so the
    stored matrix is exactly Hermitian; its diagonal is real).  Its spectrum
    lies in [1, about 1 + 4n/3], so every matrix is well conditioned.  B is
    iid uniform[-1, 1]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = np.dtype(dtype)
    wide = np.complex128 if dt.kind == "c" else np.float64
    G = draw(rng, wide, batch * n * n).reshape(batch, n, n)
    M = np.matmul(G, np.conj(np.swapaxes(G, 1, 2))) / max(n, 1) + np.eye(n)
    M = (M + np.conj(np.swapaxes(M, 1, 2))) / 2
    if dt.kind == "c":
        idx = np.arange(n)
        M[:, idx, idx] = M[:, idx, idx].real
    A = np.ascontiguousarray(np.swapaxes(M, 1, 2)).reshape(-1).astype(dt)   # column-major
    B = draw(rng, dt, batch * n * nrhs)
    return A, B


# Cholesky shapes timed beside the LU workloads: the register-tier LU shape
# (n = 32, eight right-hand sides), the work-group shape (complex n = 64,
# sixteen right-hand sides) and the blocked double shape (n = 256, one
# right-hand side), on Hermitian positive definite inputs (spd_problem).
CHOL_WORKLOADS = {
    "sposv_n32_r8_b32768": Workload("sposv_n32_r8_b32768", np.float32, 32, 8, 32768, "spd", "posv", 6),
    "cposv_n64_r16_b8192": Workload("cposv_n64_r16_b8192", np.complex64, 64, 16, 8192, "spd", "posv", 7),
    "dposv_n256_b1024": Workload("dposv_n256_b1024", np.float64, 256, 1, 1024, "spd", "posv", 8),
}


def chol_problem(w: Workload, batch: int | None = None):
    """(A, B) of a Cholesky workload, flat, ld = n (both triangles stored)."""
    b = w.batch if batch is None else min(batch, w.batch)
    return spd_problem(w.seed, w.dtype, w.n, w.nrhs, b)


# LU shapes outside the square fixed-size batch: tall m x n panels, and a
# batch whose square systems differ in order.
RECT_WORKLOADS = {
    "sgetrf_m512_n128_b2048": Workload("sgetrf_m512_n128_b2048", np.float32, 128, 0, 2048, "uniform",
                                       "getrf_rect", 9),
}
RECT_ROWS = {"sgetrf_m512_n128_b2048": 512}


@dataclass(frozen=True)
class VWorkload:
    """A batch of square systems of orders drawn uniformly from
    [nmin, nmax] (the draw comes first from the seed), nrhs each."""
    name: str
    dtype: type
    nmin: int
    nmax: int
    nrhs: int
    batch: int
    op: str
    index: int

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


VBATCH_WORKLOADS = {
    "sgesv_vbatched_n16_256_r1_b4096": VWorkload("sgesv_vbatched_n16_256_r1_b4096", np.float32, 16, 256, 1, 4096,
                                                 "gesv_vbatched", 10),
}


def vbatch_problem(w: VWorkload):
    """(orders, A, B, a_offsets, b_offsets): matrix b is orders[b] square at
    A[a_offsets[b]:] with lda = its order, its right-hand sides at
    B[b_offsets[b]:] with ldb = its order; entries iid uniform[-1, 1]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    orders = rng.integers(w.nmin, w.nmax + 1, w.batch).astype(np.int32)
    na = orders.astype(np.int64) ** 2
    nb = orders.astype(np.int64) * w.nrhs
    a_off = np.concatenate([[0], np.cumsum(na)[:-1]])
    b_off = np.concatenate([[0], np.cumsum(nb)[:-1]])
    A = draw(rng, w.dtype, int(na.sum()))
    B = draw(rng, w.dtype, int(nb.sum()))
    return orders, A, B, a_off, b_off


def dominant_spd_problem(seed: int, dtype, n: int, nrhs: int, batch: int):
    """Cheap Hermitian positive definite matrices for timing sweeps:
    (M + M^H)/2 + n I with M iid uniform[-1, 1] (complex: both parts), made
    exactly Hermitian in double and rounded; every off-diagonal row sum is
    below n, so the matrix is positive definite (Gershgorin).  B iid
    uniform[-1, 1]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = np.dtype(dtype)
    wide = np.complex128 if dt.kind == "c" else np.float64
    M = draw(rng, wide, batch * n * n).reshape(batch, n, n)
    M = (M + np.conj(np.swapaxes(M, 1, 2))) / 2
    idx = np.arange(n)
    M[:, idx, idx] = M[:, idx, idx].real + n
    A = np.ascontiguousarray(np.swapaxes(M, 1, 2)).reshape(-1).astype(dt)
    B = draw(rng, dt, batch * n * nrhs)
    return A, B


def packed_factors(seed: int, dtype, n: int, batch: int):
    """Stand-in LU factors for solve-only tests at orders where factoring on
    the host would take long: packed unit-lower L and upper U (column-major,
    stride n*n) with off-diagonal entries uniform in [-1, 1] / n and U's
    diagonal 1 + uniform[0, 1) (so every solve stays well scaled), and a
    1-based interchange list with entry k drawn from k+1 .. n."""
    rng = np.random.Generator(np.random.PCG64(seed))
    LU = draw(rng, dtype, batch * n * n) / np.dtype(dtype).type(n)
    d = 1.0 + rng.random((batch, n))
    v = LU.reshape(batch, n, n)        # [b, column, row]
    for b in range(batch):
        v[b][np.arange(n), np.arange(n)] = d[b]
    ipiv = np.empty((batch, n), np.int32)
    for k in range(n):
        ipiv[:, k] = rng.integers(k, n, size=batch) + 1
    return LU, ipiv
