"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function the header declares, its frame partition equals the oracle's for every
F up to 60, and argument errors come back as status codes without any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import hybrid_sparse_linear_chunked_amd as vdn
from oracle import vdn_oracle as orc
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "vdn_hybrid_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vdn.LIB_PATH):
        from hybrid_sparse_linear_chunked_amd import build
        build.build()
    return vdn.load()


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(vdn.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _ranges_to_list(a, b):
    return [] if a < 0 else list(range(a, b + 1))


@pytest.mark.parametrize("F", range(1, 61))
def test_schedule_matches_oracle_partition(lib, F):
    tab = vdn.schedule(F)
    covered = []
    for row in tab:
        q0, q1, ns = int(row[0]), int(row[1]), int(row[2])
        soft = []
        for x in range(ns):
            soft += _ranges_to_list(int(row[3 + 2 * x]), int(row[4 + 2 * x]))
        for x in range(ns, 3):
            assert row[3 + 2 * x] == -1 and row[4 + 2 * x] == -1
        fwd = _ranges_to_list(int(row[9]), int(row[10]))
        bwd = _ranges_to_list(int(row[11]), int(row[12]))
        for i in range(q0, q1 + 1):
            covered.append(i)
            assert soft == orc.softmax_frames(i, F), (F, i)
            assert fwd == orc.forward_frames(i, F), (F, i)
            assert bwd == orc.backward_frames(i, F), (F, i)
    assert covered == list(range(F))


def test_schedule_errors(lib):
    assert lib.vdn_schedule(0, None, 0) == vdn.ERR_INVALID_ARG
    assert lib.vdn_schedule(5, None, 3) == vdn.ERR_INVALID_ARG
    assert lib.vdn_schedule(20, None, 0) == 6


def test_workspace_bytes_rejects_bad_shapes(lib):
    assert lib.vdn_workspace_bytes(20, 16, 2, 32, 0) > 0
    assert lib.vdn_workspace_bytes(90, 4032, 24, 128, 1) > 0
    for args in [(0, 16, 2, 32, 0), (20, 0, 2, 32, 0), (20, 16, 0, 32, 0), (20, 16, 2, 48, 1),
                 (20, 16, 2, 32, 2), (20, 16, 2, 32, 3), (20, 16, 2, 32, -1)]:
        assert lib.vdn_workspace_bytes(*args) == 0, args


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.vdn_status_string(s)
    assert lib.vdn_last_hip_error() == 0


# Fake, aligned, non-null addresses: every call below must return during argument
# checks, before any device work.
A = 1 << 20


def test_argument_errors_return_before_launch(lib):
    F, N, H, d = 20, 16, 2, 32
    need = lib.vdn_workspace_bytes(F, N, H, d, 1)
    call = lib.vdn_hybrid_attn
    assert call(None, A, A, A, A, F, N, H, d, 1, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, None, A, F, N, H, d, 1, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, F, N, H, 48, 1, A, A, need, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, F, N, H, 32, 2, A, A, need, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, F, N, H, 32, 3, A, A, need, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, F, N, H, d, 4, A, A, need, None) == vdn.ERR_INVALID_ARG
    # the full-fp8 workspace holds the fp8-q.k one plus v's scale exponents
    assert lib.vdn_workspace_bytes(F, N, H, 64, 3) >= lib.vdn_workspace_bytes(F, N, H, 64, 2) > 0
    assert call(A, A, A, A, A, 0, N, H, d, 1, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, F, N, H, d, 7, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert call(A + 2, A, A, A, A, F, N, H, d, 1, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, F, N, H, d, 1, A, A + 16, need, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, F, N, H, d, 1, A, A, need - 1, None) == vdn.ERR_WORKSPACE
    assert lib.vdn_softmax_branch(A, A, A, F, N, H, d, 1, A, A, need - 1, None) == vdn.ERR_WORKSPACE
    assert lib.vdn_vda_states(A, A, None, F, N, H, d, 1, A, A, A, need, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_vda_linear(A, A, A, F, N, H, 64 + 1, 1, A, A, need, None) == vdn.ERR_UNSUPPORTED
    assert lib.vdn_fp8_quantize(A, F, N, H, 32, 1.0, A, A, None) == vdn.ERR_UNSUPPORTED
    assert lib.vdn_fp8_quantize(None, F, N, H, 64, 1.0, A, A, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_fp8_quantize(A, F, N, H, 64, 0.0, A, A, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_fp8_quantize(A, F, N, H, 64, float("inf"), A, A, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_last_hip_error() == 0


def test_mixed_and_projection_argument_errors(lib):
    # the extra-token and projection entry points reject bad arguments during their
    # checks, before any device work
    F, N, H, d, T, D = 20, 16, 2, 64, 10, 64
    need = lib.vdn_workspace_bytes(F, N, H, d, 1)
    need_x = lib.vdn_workspace_bytes_mixed(F, N, T, H, d, 1)
    assert lib.vdn_workspace_bytes_mixed(F, N, 0, H, d, 1) == need
    assert need_x > need
    assert lib.vdn_workspace_bytes_mixed(F, N, T, H, d, 0) == 0          # fp32 has no extra tokens
    assert lib.vdn_workspace_bytes_mixed(F, N, -1, H, d, 1) == 0
    call = lib.vdn_hybrid_attn_mixed
    assert call(A, A, A, A, A, F, N, T, H, d, 0, A, A, need_x, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, F, N, -1, H, d, 1, A, A, need_x, None) == vdn.ERR_INVALID_ARG
    assert call(A, None, A, A, A, F, N, T, H, d, 1, A, A, need_x, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, F, N, T, H, d, 1, A, A, need_x - 1, None) == vdn.ERR_WORKSPACE
    assert call(A, A, A, A, A, F, N, 1 << 30, H, d, 1, A, A, need_x, None) == vdn.ERR_UNSUPPORTED
    # the full-fp8 precision covers the plain layer only
    assert lib.vdn_workspace_bytes_mixed(F, N, T, H, d, vdn.PREC_FP8) == 0
    assert call(A, A, A, A, A, F, N, T, H, d, vdn.PREC_FP8, A, A, need_x, None) == vdn.ERR_UNSUPPORTED

    need_p = lib.vdn_workspace_bytes_proj(F, N, H, d, D, 1)
    assert need_p >= need + F * N * 2 * H * d * 2
    assert lib.vdn_workspace_bytes_proj(F, N, H, d, D, 0) == 0            # bf16 only
    assert lib.vdn_workspace_bytes_proj(F, N, H, d, 12, 1) == 0           # D a multiple of 8
    call = lib.vdn_hybrid_attn_proj
    assert call(A, A, A, A, A, A, F, N, H, d, D, 0, A, A, need_p, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, A, F, N, H, d, D, vdn.PREC_FP8, A, A, need_p, None) == vdn.ERR_UNSUPPORTED
    assert lib.vdn_workspace_bytes_proj(F, N, H, d, D, vdn.PREC_FP8) == 0
    assert call(A, A, A, A, A, A, F, N, H, d, 12, 1, A, A, need_p, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, None, F, N, H, d, D, 1, A, A, need_p, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, A + 8, F, N, H, d, D, 1, A, A, need_p, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, A, F, N, H, d, D, 1, A, A, need_p - 1, None) == vdn.ERR_WORKSPACE

    gemm = lib.vdn_out_proj
    assert gemm(A, A, 100, 96, 64, A, None) == vdn.ERR_UNSUPPORTED      # K a multiple of 64
    assert gemm(A, A, 100, 128, 60, A, None) == vdn.ERR_UNSUPPORTED     # N a multiple of 8
    assert gemm(A, A, 0, 128, 64, A, None) == vdn.ERR_INVALID_ARG
    assert gemm(None, A, 100, 128, 64, A, None) == vdn.ERR_INVALID_ARG
    assert gemm(A, A, 100, 128, 64, A + 4, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_last_hip_error() == 0


def test_noalloc_rejects_before_device_work(lib):
    # argument and size checks of the no-allocation entry point come before any
    # device work: too large a workspace, bad pointers and shapes return statuses
    call = lib.vdn_hybrid_attn_noalloc
    assert lib.vdn_workspace_bytes(45, 1024, 16, 128, 1) > vdn.NOALLOC_SCRATCH_BYTES
    assert lib.vdn_workspace_bytes(30, 256, 8, 64, 2) <= vdn.NOALLOC_SCRATCH_BYTES
    assert call(A, A, A, A, A, 45, 1024, 16, 128, 1, A, None) == vdn.ERR_TOO_LARGE
    assert call(A, A, A, A, A, 90, 4032, 24, 128, 2, A, None) == vdn.ERR_TOO_LARGE
    assert call(None, A, A, A, A, 20, 16, 2, 32, 0, A, None) == vdn.ERR_INVALID_ARG
    assert call(A, A, A, A, A, 20, 16, 2, 48, 1, A, None) == vdn.ERR_UNSUPPORTED
    assert call(A, A, A, A, A, 20, 16, 2, 32, 1, A + 8, None) == vdn.ERR_INVALID_ARG
    assert lib.vdn_last_hip_error() == 0
