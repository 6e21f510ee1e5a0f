"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol the header declares, rejects bad arguments with the documented
-k codes before touching the device, treats empty problems as no-ops, and
the selector picks the documented tier for each shape."""
import ctypes
import os
import re

import pytest

import dense_linear_algebra_amd as lib
from dense_linear_algebra_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "batchlu.h")
FAKE = 0x1000   # never dereferenced: every call below fails validation first or has no work


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(batchlu_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(_binding.LIB_PATH)
    names = _declared()
    assert {"batchlu_getrf", "batchlu_getrs", "batchlu_gesv", "batchlu_getri"} <= set(names)
    for name in names:
        assert hasattr(so, name), f"{name} declared in batchlu.h but not exported"


def test_version_and_status_strings():
    assert "batchlu" in lib.version()
    assert lib.status_string(0) == "ok"
    assert lib.status_string(-101).startswith("shape")
    assert lib.status_string(-3) == "invalid argument"


@pytest.mark.parametrize("args,expect", [
    ((9, 4, FAKE, 4, 16, FAKE, 4, FAKE, 1), -1),      # bad dtype
    ((0, -1, FAKE, 4, 16, FAKE, 4, FAKE, 1), -2),     # n < 0
    ((0, 4, FAKE, 3, 16, FAKE, 4, FAKE, 1), -4),      # lda < n
    ((0, 4, FAKE, 4, 15, FAKE, 4, FAKE, 2), -5),      # strideA < lda*n
    ((0, 4, FAKE, 4, 16, FAKE, 3, FAKE, 2), -7),      # strideP < n
    ((0, 4, FAKE, 4, 16, FAKE, 4, FAKE, -1), -9),     # batch < 0
    ((0, 4, None, 4, 16, FAKE, 4, FAKE, 1), -3),      # A null
    ((0, 4, FAKE, 4, 16, None, 4, FAKE, 1), -6),      # ipiv null
    ((0, 4, FAKE, 4, 16, FAKE, 4, None, 1), -8),      # info null
    ((0, 0, None, 1, 0, None, 0, None, 5), 0),        # n == 0: no work
    ((0, 4, None, 4, 16, None, 4, None, 0), 0),       # batch == 0: no work
])
def test_getrf_argument_checks(args, expect):
    assert lib.batchlu_getrf(*args, stream=0, raise_on_error=False) == expect


@pytest.mark.parametrize("args,expect", [
    ((0, "N", 4, 1, FAKE, 4, 16, FAKE, 4, FAKE, 3, 4, 1), -11),   # ldb < n
    ((0, "X", 4, 1, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4, 1), -2),    # bad trans
    ((0, "N", 4, -1, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4, 1), -4),   # nrhs < 0
    ((0, "N", 4, 2, FAKE, 4, 16, FAKE, 4, FAKE, 4, 7, 2), -12),   # strideB < ldb*nrhs
    ((0, "T", 5000, 1, FAKE, 5000, 25000000, FAKE, 5000, FAKE, 5000, 5000, 1), -100),  # 'T' above n = 4096
    ((3, "C", 4097, 2, FAKE, 4097, 16785409, FAKE, 4097, FAKE, 4097, 8194, 1), -100),  # 'C' above n = 4096
    ((0, "T", 0, 1, None, 1, 0, None, 0, None, 1, 1, 3), 0),      # 'T' with n == 0: no work
    ((0, "N", 4, 0, None, 4, 16, None, 4, None, 4, 0, 3), 0),     # nrhs == 0
])
def test_getrs_argument_checks(args, expect):
    assert lib.batchlu_getrs(*args, stream=0, raise_on_error=False) == expect


@pytest.mark.parametrize("args,expect", [
    ((0, -1, FAKE, 4, 16, FAKE, 4, FAKE, 4, 16, 1), -2),          # n < 0
    ((0, 4, FAKE, 3, 16, FAKE, 4, FAKE, 4, 16, 1), -4),           # lda < n
    ((0, 4, FAKE, 4, 16, FAKE, 4, FAKE, 3, 16, 1), -9),           # ldc < n
    ((0, 4, FAKE, 4, 16, FAKE, 4, FAKE, 4, 15, 2), -10),          # strideC < ldc*n
    ((0, 4, FAKE, 4, 16, None, 4, FAKE + 4096, 4, 16, 1), -6),    # ipiv null
    ((0, 4, FAKE, 4, 16, FAKE, 4, FAKE + 60, 4, 16, 1), -8),      # C overlaps A's last element
    ((0, 4, FAKE, 4, 16, FAKE, 4, FAKE, 4, 16, -1), -11),         # batch < 0
    ((0, 4100, FAKE, 4100, 16810000, FAKE, 4100, 1 << 40, 4100, 16810000, 1), -100),  # n > 4096
    ((0, 0, None, 1, 0, None, 0, None, 1, 0, 5), 0),              # n == 0: no work
])
def test_getri_argument_checks(args, expect):
    assert lib.batchlu_getri(*args, stream=0, raise_on_error=False) == expect


@pytest.mark.parametrize("args,expect", [
    ((1, 4, 1, FAKE, 4, 16, FAKE, 4, FAKE, 2, 4, FAKE, 1), -10),  # ldb < n
    ((1, 4, -2, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4, FAKE, 1), -3),  # nrhs < 0
    ((1, 4, 1, FAKE, 4, 16, FAKE, 4, None, 4, 4, FAKE, 1), -9),   # B null with nrhs > 0
    ((1, 4, 1, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4, None, 1), -12),  # info null
    ((1, 4, 1, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4, FAKE, -3), -13), # batch < 0
    ((1, 0, 1, None, 1, 0, None, 0, None, 1, 1, None, 4), 0),     # n == 0
])
def test_gesv_argument_checks(args, expect):
    assert lib.batchlu_gesv(*args, stream=0, raise_on_error=False) == expect


def test_error_raises_in_binding():
    with pytest.raises(lib.BatchLUError):
        lib.batchlu_getrf(0, -1, FAKE, 4, 16, FAKE, 4, FAKE, 1, stream=0)


@pytest.mark.parametrize("t,op,n,nrhs,tier", [
    (lib.R32, 2, 16, 1, lib.TIER_TINY),
    (lib.R32, 2, 32, 8, lib.TIER_TINY),
    (lib.R32, 0, 1, 0, lib.TIER_TINY),
    (lib.C64, 2, 64, 16, lib.TIER_CTA),
    (lib.R64, 0, 33, 0, lib.TIER_CTA),
    (lib.C128, 0, 32, 0, lib.TIER_TINY),
])
def test_selector(t, op, n, nrhs, tier):
    assert lib.batchlu_select_tier(t, op, n, nrhs, 100) == tier


def test_tier_pin_refuses_instead_of_truncating():
    prev = lib.batchlu_set_tier(lib.TIER_TINY)
    try:
        assert lib.batchlu_select_tier(lib.R32, 0, 33, 0, 10) == -101
        assert lib.batchlu_getrf(lib.R32, 33, FAKE, 33, 33 * 33, FAKE, 33, FAKE, 1, stream=0,
                                 raise_on_error=False) == -101
    finally:
        lib.batchlu_set_tier(prev)


@pytest.mark.parametrize("t,op,n,nrhs,batch,tier", [
    # gesv, 16 right-hand sides, small batch: factor then solve (blocked)
    (lib.R64, 2, 64, 16, 64, lib.TIER_BLOCKED),
    (lib.R64, 2, 64, 16, 8192, lib.TIER_CTA),
    # complex double 33..64: the LDS-staged work-group tier at small batch
    (lib.C128, 2, 48, 1, 64, lib.TIER_CTA_LDS),
    (lib.C128, 2, 48, 1, 8192, lib.TIER_BLOCKED),
    # float n <= 8 with many right-hand sides: LDS tier up to batch 1024
    (lib.R32, 2, 8, 16, 1024, lib.TIER_CTA_LDS),
    (lib.R32, 2, 8, 16, 8192, lib.TIER_TINY),
    # complex float n = 32 with 16 right-hand sides: the register tier at
    # every batch
    (lib.C64, 2, 32, 16, 64, lib.TIER_TINY),
    # getrf keeps the register tiers at every batch
    (lib.R64, 0, 64, 0, 1, lib.TIER_CTA),
    (lib.C64, 0, 16, 0, 16, lib.TIER_TINY),
    # posv (op 4): double n >= 64 at small batch goes to the blocked driver
    (lib.R64, 4, 64, 1, 64, lib.TIER_BLOCKED),
    (lib.R64, 4, 64, 1, 4096, lib.TIER_CTA),
    (lib.C128, 4, 16, 16, 16, lib.TIER_BLOCKED),
    (lib.C128, 3, 16, 0, 16, lib.TIER_CTA),
])
def test_selector_uses_the_measured_crossovers(t, op, n, nrhs, batch, tier):
    """The selector keys on the batch and the number of right-hand sides as
    well as the type and order (crossovers measured by bench.py
    --tier-sweep)."""
    assert lib.batchlu_select_tier(t, op, n, nrhs, batch) == tier
