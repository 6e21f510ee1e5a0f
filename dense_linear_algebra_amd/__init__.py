"""Batched LU with partial pivoting (getrf), LU solve (getrs), gesv and getri,
and batched Cholesky (potrf, potrs, posv) on AMD Instinct MI355X (gfx950):
hand-written HIP kernels behind a C ABI (include/batchlu.h), with a thin
ctypes binding of the same names."""
from ._binding import (C64, C128, R32, R64, TIER_AUTO, TIER_BLOCKED, TIER_CTA, TIER_CTA_LDS, TIER_NAMES,
                       TIER_TINY, BatchLUError, batchlu_check_reciprocal, batchlu_gesv, batchlu_gesv_vbatched,
                       batchlu_getrf, batchlu_getrf_rect, batchlu_getrf_vbatched, batchlu_getri, batchlu_getrs,
                       batchlu_getrs_vbatched, batchlu_posv, batchlu_potrf, batchlu_potrs, batchlu_select_tier,
                       batchlu_set_tier, dtype_code, load, status_string, version)

__all__ = ["R32", "R64", "C64", "C128", "TIER_AUTO", "TIER_TINY", "TIER_CTA", "TIER_BLOCKED", "TIER_CTA_LDS",
           "TIER_NAMES",
           "BatchLUError", "batchlu_check_reciprocal", "batchlu_getrf", "batchlu_getrs", "batchlu_getri",
           "batchlu_gesv", "batchlu_getrf_rect", "batchlu_getrf_vbatched", "batchlu_getrs_vbatched",
           "batchlu_gesv_vbatched", "batchlu_potrf", "batchlu_potrs", "batchlu_posv", "batchlu_select_tier",
           "batchlu_set_tier", "dtype_code", "load", "status_string", "version"]
