"""The C-ABI library loads and exports every function include/jfa.h declares;
host-only entry points behave without a GPU (no compute calls here)."""
import ctypes
import os
import subprocess

import pytest

from variable_length_attention_jfa_amd import jfa


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(jfa.LIB_PATH):
        pytest.skip("libjfa.so not built (run __graft_entry__.build())")
    return jfa.lib()


def test_exports_every_declared_function(L):
    names = jfa.declared_functions()
    assert len(names) >= 12
    nm = subprocess.run(["nm", "-D", "--defined-only", jfa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_binding_covers_the_header():
    assert set(jfa.declared_functions()) == set(jfa._SIGS)


def test_abi_version_matches_header(L):
    import re
    with open(jfa.HEADER_PATH) as fh:
        ver = int(re.search(r"#define JFA_ABI_VERSION (\d+)", fh.read()).group(1))
    assert L.jfa_abi_version() == ver == jfa.ABI_VERSION


def test_host_only_queries(L):
    assert L.jfa_fwd_workspace_bytes(4, 2, 153, 153, 32, 0) > 0
    assert L.jfa_fwd_workspace_bytes(4, 2, 153, 153, 48, 0) == 0
    assert L.jfa_bwd_workspace_bytes(-1, 2, 10, 10, 64, 0) == 0
    assert L.jfa_bwd_workspace_bytes(64, 8, 31132, 31132, 64, 0) > 31132 * 8 * 8
    assert L.jfa_fwd_workspace_bytes(4, 65535, 10, 10, 64, 0) > 0
    assert L.jfa_fwd_workspace_bytes(4, 65536, 10, 10, 64, 0) == 0  # beyond JFA_MAX_HEADS
    assert L.jfa_bwd_workspace_bytes(4, 0, 10, 10, 64, 0) == 0
    for kernel in (jfa.KERNEL_FWD, jfa.KERNEL_BWD_DKDV, jfa.KERNEL_BWD_DQ, jfa.KERNEL_BWD_SQ, jfa.KERNEL_FWD_SQ):
        tm, tn = jfa.tile_config(kernel, 128)
        assert tm % 32 == 0 and tn % 32 == 0 and tm > 0 and tn > 0
    for kernel in jfa.SQ_KERNELS:
        assert jfa.tile_config(kernel, 64) == (64, 1024)  # short-query rows, keys per chunk
    # the forward workspace holds the short-query partials: [64, D] fp32 rows per chunk of 1024 keys
    assert L.jfa_fwd_workspace_bytes(128, 8, 4281, 617399, 128, 0) > (617399 // 1024) * 8 * 64 * 128 * 4
    with pytest.raises(jfa.JFAError):
        jfa.tile_config(7, 128)
    assert L.jfa_status_string(2) == b"workspace missing, misaligned or too small"


def test_invalid_arguments_rejected_on_host(L):
    # bad sizes are rejected before any device call
    st = L.jfa_fwd(None, None, None, None, None, -1, 1, 64, 0, 0, 0, None, 0, None, None, None, 0, None)
    assert st == 1
    assert b"invalid sizes" in L.jfa_last_error()
    st = L.jfa_bwd(None, None, None, None, None, None, None, None, 4, 0, 64, 0, 0, 0, None, 0, None, None, None, None,
                   None, 0, None)
    assert st == 1
    st = L.jfa_fwd(None, None, None, None, None, 2, 2, 64, 0, 0, 0, None, 0, None, None, None, 0, None)
    assert st == 1 and b"offsets" in L.jfa_last_error()
    dummy = ctypes.c_void_p(4096)
    st = L.jfa_fwd(dummy, dummy, dummy, dummy, dummy, 2, 2, 64, 10, 10, 0, None, 0, dummy, dummy, None, 0, None)
    assert st == 2
    # a negative key-count bound is an invalid argument
    st = L.jfa_fwd(dummy, dummy, dummy, dummy, dummy, 2, 2, 64, 10, 10, -1, None, 0, dummy, dummy, dummy, 1 << 20, None)
    assert st == 1 and b"max_kv_len" in L.jfa_last_error()


def test_bias_gradient_needs_bias(L):
    dummy = ctypes.c_void_p(4096)
    fdummy = ctypes.c_void_p(4096)
    st = L.jfa_bwd(dummy, dummy, dummy, dummy, fdummy, dummy, dummy, dummy, 2, 2, 64, 10, 10, 0, None, 0, dummy, dummy,
                   dummy, fdummy, dummy, 1 << 20, None)
    assert st == 1 and b"dbias needs a bias" in L.jfa_last_error()


def test_padded_baseline_host_checks(L):
    # workspace of the padded-dense baseline covers either pass at the padded totals
    n = L.jfa_padded_workspace_bytes(64, 8, 1024, 1024, 64)
    assert n >= L.jfa_bwd_workspace_bytes(64, 8, 64 * 1024, 64 * 1024, 64, 0)
    assert n >= L.jfa_fwd_workspace_bytes(64, 8, 64 * 1024, 64 * 1024, 64, 0)
    assert L.jfa_padded_workspace_bytes(8192, 1, 1 << 18, 1, 64) == 0  # B * q_slot = 2^31
    assert L.jfa_padded_workspace_bytes(4, 2, -1, 8, 64) == 0
    assert L.jfa_padded_workspace_bytes(4, 2, 8, 8, 48) == 0
    dummy = ctypes.c_void_p(4096)
    st = L.jfa_fwd_padded(dummy, dummy, dummy, dummy, 2, -1, 8, 2, 64, None, 0, dummy, dummy, dummy, 1 << 20, None)
    assert st == 1 and b"invalid sizes" in L.jfa_last_error()
    st = L.jfa_fwd_padded(dummy, dummy, dummy, None, 2, 8, 8, 2, 64, None, 0, dummy, dummy, dummy, 1 << 20, None)
    assert st == 1 and b"kv_lens" in L.jfa_last_error()
    ws = ctypes.c_void_p(4096 * 16)
    st = L.jfa_bwd_padded(dummy, dummy, dummy, dummy, dummy, dummy, dummy, 2, 8, 8, 2, 64, None, 0, dummy, dummy, dummy,
                          ws, 64, None)
    assert st == 2 and b"workspace too small" in L.jfa_last_error()
    st = L.jfa_bwd_padded(dummy, dummy, dummy, dummy, dummy, dummy, None, 2, 8, 8, 2, 64, None, 0, dummy, dummy, dummy,
                          ws, 1 << 20, None)
    assert st == 1 and b"kv_lens" in L.jfa_last_error()
