"""The C-ABI library: it loads, exports what include/rr.h declares, validates
its arguments before touching the GPU, and reports status strings.  No kernel
runs here (these tests need no GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import memory_bound_row_softmax_amd as rr
from _verify import check_bf16, check_f32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = rr.lib()
    names = _declared_functions()
    assert "rr_softmax_fwd" in names and "rr_cross_entropy_fwd" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rr.h but not exported"
    assert set(rr.EXPORTS) == set(names)


def test_status_strings():
    for s in range(6):
        assert rr.status_string(s).startswith("RR_")
    assert "unknown" in rr.status_string(99)
    assert rr.lib().rr_last_hip_error() == 0


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


# Calls below pass fake addresses: each must be rejected by validation before the
# library touches the device.  They are skipped where a GPU is visible, so that a
# validation bug can never launch a kernel on a fake address.
needs_no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation checks run on hosts without a GPU")

A, B, C = 1 << 40, 2 << 40, 3 << 40  # fake, far apart, never dereferenced


def test_zero_rows_is_a_no_op():
    assert rr.softmax_fwd_raw(0, 0, 0, 5, rr.RR_F32) == rr.RR_OK
    assert rr.rmsnorm_fwd_raw(0, 0, 0, 0, 0, 5, rr.RR_BF16, 1e-6) == rr.RR_OK
    assert rr.cross_entropy_fwd_raw(0, 0, 0, 0, 0, 5, rr.RR_F32) == rr.RR_OK
    assert rr.cross_entropy_fwd_bwd_raw(0, 0, 0, 0, 0, 0, 0, 5, rr.RR_BF16) == rr.RR_OK
    assert rr.softmax_bwd_raw(0, 0, 0, 0, 5, rr.RR_F32) == rr.RR_OK


@needs_no_gpu
@pytest.mark.parametrize("case", [
    ("null x", lambda: rr.softmax_fwd_raw(0, B, 4, 8, rr.RR_F32)),
    ("null y", lambda: rr.softmax_fwd_raw(A, 0, 4, 8, rr.RR_F32)),
    ("M < 0", lambda: rr.softmax_fwd_raw(A, B, -1, 8, rr.RR_F32)),
    ("N = 0", lambda: rr.softmax_fwd_raw(A, B, 4, 0, rr.RR_F32)),
    ("bad dtype", lambda: rr.softmax_fwd_raw(A, B, 4, 8, 7)),
    ("partial overlap", lambda: rr.softmax_fwd_raw(A, A + 16, 4, 8, rr.RR_F32)),
    ("rms null w", lambda: rr.rmsnorm_fwd_raw(A, 0, B, 0, 4, 8, rr.RR_F32, 1e-6)),
    ("rms eps < 0", lambda: rr.rmsnorm_fwd_raw(A, C, B, 0, 4, 8, rr.RR_F32, -1.0)),
    ("rms eps nan", lambda: rr.rmsnorm_fwd_raw(A, C, B, 0, 4, 8, rr.RR_F32, float("nan"))),
    ("rms eps inf", lambda: rr.rmsnorm_fwd_raw(A, C, B, 0, 4, 8, rr.RR_F32, float("inf"))),
    ("rms overlap", lambda: rr.rmsnorm_fwd_raw(A, C, A + 4, 0, 4, 8, rr.RR_F32, 1e-6)),
    ("xent null labels", lambda: rr.cross_entropy_fwd_raw(A, 0, B, 0, 4, 8, rr.RR_F32)),
    ("xent null loss", lambda: rr.cross_entropy_fwd_raw(A, C, 0, 0, 4, 8, rr.RR_F32)),
    ("xent N > int32", lambda: rr.cross_entropy_fwd_raw(A, C, B, 0, 1, 1 << 31, rr.RR_BF16)),
    ("xgrad null labels", lambda: rr.cross_entropy_fwd_bwd_raw(A, 0, C, C + 64, 0, B, 4, 8, rr.RR_F32)),
    ("xgrad null dloss", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, 0, C + 64, 0, B, 4, 8, rr.RR_F32)),
    ("xgrad null loss", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, C + 64, 0, 0, B, 4, 8, rr.RR_F32)),
    ("xgrad null dlogits", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, C + 64, C + 128, 0, 0, 4, 8,
                                                                rr.RR_F32)),
    ("xgrad overlap", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, C + 64, C + 128, 0, A + 4, 4, 8,
                                                           rr.RR_F32)),
    ("xgrad N > int32", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, C + 64, C + 128, 0, B, 1,
                                                             1 << 31, rr.RR_BF16)),
    ("xgrad M >= 2^30", lambda: rr.cross_entropy_fwd_bwd_raw(A, C, C + 64, C + 128, 0, B, 1 << 30,
                                                             8, rr.RR_BF16)),
    ("smbwd null dy", lambda: rr.softmax_bwd_raw(A, 0, B, 4, 8, rr.RR_F32)),
    ("smbwd null dx", lambda: rr.softmax_bwd_raw(A, C, 0, 4, 8, rr.RR_F32)),
    ("smbwd overlap y", lambda: rr.softmax_bwd_raw(A, C, A + 16, 4, 8, rr.RR_F32)),
    ("smbwd overlap dy", lambda: rr.softmax_bwd_raw(A, C, C - 16, 4, 8, rr.RR_F32)),
    ("rmsbwd null rstd", lambda: rr.rmsnorm_bwd_raw(A, C, A + 512, 0, B, C + 64, 4, 8, rr.RR_F32)),
    ("rmsbwd null dw", lambda: rr.rmsnorm_bwd_raw(A, C, A + 512, C + 64, B, 0, 4, 8, rr.RR_F32)),
    ("rmsbwd dw on dx", lambda: rr.rmsnorm_bwd_raw(A, C, A + 512, C + 64, B, B + 8, 4, 8,
                                                   rr.RR_F32)),
    ("rmsbwd dx overlap", lambda: rr.rmsnorm_bwd_raw(A, C, A + 512, C + 64, A + 4, C + 256, 4, 8,
                                                     rr.RR_F32)),
    ("size overflow", lambda: rr.softmax_fwd_raw(A, B, 1 << 62, 1 << 20, rr.RR_F32)),
    ("copy misaligned", lambda: rr.stream_copy_raw(A + 4, B, 64)),
    ("copy odd size", lambda: rr.stream_copy_raw(A, B, 40)),
    ("copy overlap", lambda: rr.stream_copy_raw(A, A + 16, 64)),
], ids=lambda c: c[0])
def test_invalid_arguments_are_rejected(case):
    assert case[1]() == rr.RR_ERR_INVALID_ARGUMENT


@needs_no_gpu
def test_too_long_rows_are_unsupported():
    # softmax and RMSNorm read rows past the on-chip capacity twice, up to 2^28 elements
    assert rr.softmax_fwd_raw(A, B, 2, (1 << 28) + 4, rr.RR_F32) == rr.RR_ERR_UNSUPPORTED
    # (a longer row than the on-chip plans hold, without a workspace)
    assert rr.softmax_fwd_raw(A, B, 2, (1 << 19) + 4, rr.RR_F32) == rr.RR_ERR_WORKSPACE
    # the softmax backward reads y and dy twice past the on-chip plans, up to 2^28
    assert rr.softmax_bwd_raw(A, C, B, 2, (1 << 20) + 4, rr.RR_F32) == rr.RR_ERR_WORKSPACE
    assert rr.softmax_bwd_raw(A, C, B, 2, (1 << 28) + 4, rr.RR_F32) == rr.RR_ERR_UNSUPPORTED
    # and so does the cross-entropy gradient
    assert rr.cross_entropy_fwd_bwd_raw(A, C, C + 4096, C + 8192, C + 12288, B, 2, (1 << 21) + 4,
                                        rr.RR_F32) == rr.RR_ERR_WORKSPACE
    assert rr.cross_entropy_fwd_bwd_raw(A, C, C + 4096, C + 8192, C + 12288, B, 2, (1 << 28) + 4,
                                        rr.RR_F32) == rr.RR_ERR_UNSUPPORTED


@needs_no_gpu
def test_missing_or_small_workspace():
    N = 131072
    need = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 64, N, rr.RR_F32, True)["ws_bytes"]
    assert 0 < need <= rr.workspace_bytes(rr.RR_OP_SOFTMAX, 64, N, rr.RR_F32)
    assert rr.softmax_fwd_raw(A, B, 64, N, rr.RR_F32) == rr.RR_ERR_WORKSPACE
    assert rr.softmax_fwd_raw(A, B, 64, N, rr.RR_F32, C, need - 1) == rr.RR_ERR_WORKSPACE
    assert rr.softmax_fwd_raw(A, B, 64, N, rr.RR_F32, C + 4, need) == rr.RR_ERR_WORKSPACE
    # a workspace that shares bytes with an operand
    assert rr.softmax_fwd_raw(A, B, 64, N, rr.RR_F32, B + 64 * N * 4 - 16, need) == \
        rr.RR_ERR_WORKSPACE
    assert rr.softmax_fwd_raw(A, B, 64, N, rr.RR_F32, A - need + 16, need) == rr.RR_ERR_WORKSPACE
    need_b = rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 64, N, rr.RR_F32, True)["ws_bytes"]
    assert need_b > 0
    assert rr.softmax_bwd_raw(A, C, B, 64, N, rr.RR_F32, C + 1024, need_b) == rr.RR_ERR_WORKSPACE


def test_plan_struct_layout_matches_header():
    # rr_plan_info: 7 ints, an int64 and a size_t
    assert ctypes.sizeof(rr.PlanInfo) == 7 * 4 + 4 + 8 + 8


# ---------------------------------------------------------------- verifier

def test_bf16_acceptance_is_one_ulp():
    ref = np.array([1.0 + 2.0**-9, 3.0, -0.3])
    # the two bracketing bf16 values of each reference pass, the next ones fail
    lo = np.array([0x3F80, 0x4040, 0xBE9A], dtype=np.uint16)
    hi = np.array([0x3F81, 0x4040, 0xBE99], dtype=np.uint16)
    check_bf16(lo, ref)
    check_bf16(hi, ref)
    with pytest.raises(AssertionError):
        check_bf16(np.array([0x3F82, 0x4040, 0xBE9A], dtype=np.uint16), ref)
    with pytest.raises(AssertionError):
        check_bf16(np.array([0x3F80, 0x4042, 0xBE9A], dtype=np.uint16), ref)


def test_f32_acceptance():
    ref = np.array([1.0, 1e-3, 1e-40, np.nan])
    check_f32(np.array([1.0 + 9e-6, 1e-3 * (1 - 9e-6), 0.0, np.nan]), ref)
    with pytest.raises(AssertionError):
        check_f32(np.array([1.0 + 2e-5, 1e-3, 0.0, np.nan]), ref)
    with pytest.raises(AssertionError):
        check_f32(np.array([1.0, 1e-3, 0.0, 0.0]), ref)
