"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before launching
anything (these paths make no HIP call, so they run without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmpack.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    from selective_state_space_varlen_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libssmpack.so is not built (python -m selective_state_space_varlen_amd.build)")
    return binding.load()


def test_header_lists_the_entry_points():
    names = declared_functions()
    for n in ("varlen_pack_indices", "conv1d_pack_fwd", "conv1d_pack_bwd", "selective_scan_pack_fwd",
              "selective_scan_pack_bwd", "selective_scan_pack_workspace_bytes", "conv1d_pack_bwd_workspace_bytes",
              "ssmp_status_string", "ssmp_abi_version", "selective_scan_pack_fwd_ex", "selective_scan_pack_bwd_ex",
              "varlen_pack_plan", "selective_scan_pack_fwd_states", "selective_scan_pack_bwd_states",
              "conv1d_pack_fwd_states", "conv1d_pack_bwd_states", "conv1d_pack_bwd_states_workspace_bytes",
              "selective_scan_pack_fwd_ck", "selective_scan_pack_bwd_ck", "selective_scan_pack_saved_bytes",
              "selective_scan_pack_fwd_scratch_bytes", "selective_scan_pack_bwd_scratch_bytes"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    from selective_state_space_varlen_amd import binding
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in ssmpack.h but not exported"
    assert sorted(binding.EXPORTED) == declared_functions()


def test_status_strings(lib):
    assert lib.ssmp_status_string(0) == b"ok"
    for s in range(1, 8):
        assert lib.ssmp_status_string(s) and lib.ssmp_status_string(s) != b"unknown status"
    assert lib.ssmp_status_string(99) == b"unknown status"
    assert lib.ssmp_abi_version() == 6


def test_workspace_sizes(lib):
    # checkpoints (the fp32 states of every 8th token) dominate the scan workspace
    T, D, N = 32768, 4096, 16
    ws = lib.selective_scan_pack_workspace_bytes(T, D, N)
    assert ws >= (T // 8) * D * N * 4
    assert lib.selective_scan_pack_workspace_bytes(0, D, N) == 0
    assert lib.conv1d_pack_bwd_workspace_bytes(T, D, 4) >= 5 * D * 4
    assert lib.conv1d_pack_bwd_workspace_bytes(0, D, 4) == 0
    # the conv backward with contexts adds one correction row set per sequence
    assert (lib.conv1d_pack_bwd_states_workspace_bytes(T, D, 4, 34)
            == lib.conv1d_pack_bwd_workspace_bytes(T, D, 4) + 34 * 5 * D * 4)


NULL = None


def test_host_validation(lib):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    # varlen_pack_indices: nseq < 1, T out of range, NULL cu_seqlens
    assert lib.varlen_pack_indices(fake, 0, 4, fake, NULL, NULL, NULL) == 2
    assert lib.varlen_pack_indices(fake, 1, -1, fake, NULL, NULL, NULL) == 2
    assert lib.varlen_pack_indices(fake, 1, 1 << 31, fake, NULL, NULL, NULL) == 2
    assert lib.varlen_pack_indices(NULL, 1, 4, fake, NULL, NULL, NULL) == 1
    assert lib.varlen_pack_indices(fake, 1, 4, NULL, NULL, NULL, NULL) == 1
    # conv: width, dtype, D, NULLs
    assert lib.conv1d_pack_fwd(fake, fake, NULL, fake, fake, 8, 4, 5, 1, 1, NULL) == 4
    assert lib.conv1d_pack_fwd(fake, fake, NULL, fake, fake, 8, 4, 0, 1, 1, NULL) == 4
    assert lib.conv1d_pack_fwd(fake, fake, NULL, fake, fake, 8, 4, 4, 7, 1, NULL) == 4
    assert lib.conv1d_pack_fwd(fake, fake, NULL, fake, fake, 8, 0, 4, 1, 1, NULL) == 2
    assert lib.conv1d_pack_fwd(NULL, fake, NULL, fake, fake, 8, 4, 4, 1, 1, NULL) == 1
    assert lib.conv1d_pack_bwd(fake, fake, NULL, fake, fake, fake, fake, NULL, NULL, 0, 8, 4, 4, 1, 1, NULL) == 6
    assert lib.conv1d_pack_bwd(fake, fake, NULL, fake, fake, fake, fake, NULL, fake, 4, 8, 4, 4, 1, 1, NULL) == 6
    # scan: d_state, dtype, NULLs, workspace
    args = [fake] * 9
    assert lib.selective_scan_pack_fwd(*args, fake, 1 << 30, 8, 4, 3, 1, NULL) == 4
    assert lib.selective_scan_pack_fwd(*args, fake, 1 << 30, 8, 4, 32, 1, NULL) == 4
    assert lib.selective_scan_pack_fwd(*args, fake, 1 << 30, 8, 4, 16, 2, NULL) == 4
    assert lib.selective_scan_pack_fwd(*args, fake, 1 << 30, -1, 4, 16, 1, NULL) == 2
    assert lib.selective_scan_pack_fwd(*args, NULL, 0, 8, 4, 16, 1, NULL) == 6
    assert lib.selective_scan_pack_fwd(*args, fake, 16, 8, 4, 16, 1, NULL) == 6
    nul_u = [NULL] + [fake] * 8
    assert lib.selective_scan_pack_fwd(*nul_u, fake, 1 << 30, 8, 4, 16, 1, NULL) == 1
    b = [fake] * 9 + [fake, 1 << 30] + [fake] * 7
    assert lib.selective_scan_pack_bwd(*b, 8, 4, 3, 1, NULL) == 4
    # dD must be given exactly when Dskip is
    b2 = [fake] * 5 + [NULL] + [fake] * 3 + [fake, 1 << 30] + [fake] * 7
    assert lib.selective_scan_pack_bwd(*b2, 8, 4, 16, 1, NULL) == 1


def test_host_validation_states(lib):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    # scan forward with states: a state pointer needs cu_seqlens and nseq >= 1
    f = [fake] * 9 + [fake, 1 << 30, 8, 4, 16, 1, NULL, 0, ctypes.c_float(0.0)]
    assert lib.selective_scan_pack_fwd_states(*f, NULL, 2, fake, NULL, NULL) == 1
    assert lib.selective_scan_pack_fwd_states(*f, NULL, 2, NULL, fake, NULL) == 1
    assert lib.selective_scan_pack_fwd_states(*f, fake, 0, fake, NULL, NULL) == 2
    # ... and the usual checks still come first
    f_bad_n = [fake] * 9 + [fake, 1 << 30, 8, 4, 3, 1, NULL, 0, ctypes.c_float(0.0)]
    assert lib.selective_scan_pack_fwd_states(*f_bad_n, fake, 2, fake, fake, NULL) == 4
    # scan backward with states
    b = [fake] * 9 + [fake, 1 << 30] + [fake] * 7 + [8, 4, 16, 1, NULL, 0, ctypes.c_float(0.0), NULL]
    assert lib.selective_scan_pack_bwd_states(*b, NULL, 2, fake, NULL, NULL, NULL) == 1
    assert lib.selective_scan_pack_bwd_states(*b, NULL, 2, NULL, NULL, fake, NULL) == 1
    assert lib.selective_scan_pack_bwd_states(*b, fake, 0, NULL, fake, NULL, NULL) == 2
    # the step-bias gradient must be given exactly when the step bias is
    b_bias = [fake] * 9 + [fake, 1 << 30] + [fake] * 7 + [8, 4, 16, 1, fake, 0, ctypes.c_float(0.0), NULL]
    assert lib.selective_scan_pack_bwd_states(*b_bias, fake, 2, fake, NULL, NULL, NULL) == 1
    # conv forward with contexts
    c = [fake, fake, NULL, fake, fake, 8, 4, 4, 1, 1]
    assert lib.conv1d_pack_fwd_states(*c, NULL, 2, fake, NULL, NULL) == 1
    assert lib.conv1d_pack_fwd_states(*c, fake, 0, NULL, fake, NULL) == 2
    assert lib.conv1d_pack_fwd_states(fake, fake, NULL, fake, fake, 8, 4, 5, 1, 1, fake, 2, fake, NULL, NULL) == 4
    # conv backward with contexts: cu_seqlens, nseq, and the larger workspace
    cb = [fake, fake, NULL, fake, fake, fake, fake, NULL]
    assert lib.conv1d_pack_bwd_states(*cb, fake, 1 << 30, 8, 4, 4, 1, 1, NULL, 2, fake, NULL, NULL, NULL) == 1
    assert lib.conv1d_pack_bwd_states(*cb, fake, 1 << 30, 8, 4, 4, 1, 1, fake, 0, fake, NULL, NULL, NULL) == 2
    small = lib.conv1d_pack_bwd_workspace_bytes(8, 4, 4)  # enough without contexts, too small with them
    assert lib.conv1d_pack_bwd_states(*cb, fake, small, 8, 4, 4, 1, 1, fake, 2, fake, NULL, NULL, NULL) == 6


def test_checkpoint_interval_sizes(lib):
    T, D, N = 32768, 4096, 16
    # kept states: one fp32 (D, N) slot per ckpt_interval tokens (256-byte rounded)
    for ci in (4, 8, 64, 256, 2048):
        assert lib.selective_scan_pack_saved_bytes(T, D, N, ci) == (T // ci) * D * N * 4
    assert lib.selective_scan_pack_saved_bytes(T + 1, D, N, 64) == (T // 64 + 1) * D * N * 4
    assert lib.selective_scan_pack_saved_bytes(T, D, N, 0) == 0
    for bad in (-4, 1, 2, 3, 6, 12, 4096):
        assert lib.selective_scan_pack_saved_bytes(T, D, N, bad) == 0
        assert lib.selective_scan_pack_bwd_scratch_bytes(T, D, N, bad) == 0
    # the forward's scratch is small next to the dense states; the backward's
    # holds states 8 tokens apart, replayed, unless the forward kept every
    # 4th or 8th
    fwd = lib.selective_scan_pack_fwd_scratch_bytes(T, D, N)
    dense = (T // 8) * D * N * 4
    assert 0 < fwd < dense // 4
    b8 = lib.selective_scan_pack_bwd_scratch_bytes(T, D, N, 8)
    assert lib.selective_scan_pack_bwd_scratch_bytes(T, D, N, 4) == b8
    for ci in (0, 16, 2048):
        assert lib.selective_scan_pack_bwd_scratch_bytes(T, D, N, ci) >= b8 + dense
    # the single workspace of the other entry points: kept states every 8 tokens, then the scratch
    assert lib.selective_scan_pack_workspace_bytes(T, D, N) == (lib.selective_scan_pack_saved_bytes(T, D, N, 8)
                                                                + max(fwd, b8))


def test_host_validation_checkpoint_interval(lib):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    big = 1 << 40
    f = [fake] * 9 + [8, 4, 16, 1, NULL, 0, ctypes.c_float(0.0), NULL, 0, NULL, NULL]
    for bad in (2, 12, 4096, -8):
        assert lib.selective_scan_pack_fwd_ck(*f, bad, fake, big, fake, big, NULL) == 2
    # a kept-state buffer is needed unless the interval is 0; the scratch always
    assert lib.selective_scan_pack_fwd_ck(*f, 8, NULL, 0, fake, big, NULL) == 6
    assert lib.selective_scan_pack_fwd_ck(*f, 8, fake, 16, fake, big, NULL) == 6
    assert lib.selective_scan_pack_fwd_ck(*f, 0, NULL, 0, NULL, 0, NULL) == 6
    assert lib.selective_scan_pack_fwd_ck(*f, 0, NULL, 0, fake, 16, NULL) == 6
    # argument checks come before the buffers
    f_bad_n = [fake] * 9 + [8, 4, 3, 1, NULL, 0, ctypes.c_float(0.0), NULL, 0, NULL, NULL]
    assert lib.selective_scan_pack_fwd_ck(*f_bad_n, 8, NULL, 0, NULL, 0, NULL) == 4
    b = [fake] * 16 + [8, 4, 16, 1, NULL, 0, ctypes.c_float(0.0), NULL, NULL, 0, NULL, NULL, NULL]
    for bad in (3, 4096):
        assert lib.selective_scan_pack_bwd_ck(*b, bad, fake, big, fake, big, NULL) == 2
    assert lib.selective_scan_pack_bwd_ck(*b, 16, NULL, 0, fake, big, NULL) == 6
    # with the interval 0 nothing was kept, but the scratch holds the replayed states
    small = lib.selective_scan_pack_bwd_scratch_bytes(8, 4, 16, 4)
    assert lib.selective_scan_pack_bwd_ck(*b, 0, NULL, 0, fake, small, NULL) == 6
    b_nodD = [fake] * 5 + [NULL] + [fake] * 10 + [8, 4, 16, 1, NULL, 0, ctypes.c_float(0.0), NULL, NULL, 0, NULL,
                                                  NULL, NULL]
    assert lib.selective_scan_pack_bwd_ck(*b_nodD, 4, fake, big, fake, big, NULL) == 1
