"""Error propagation from a failed launch (CPU).  libmha_fault.so is libmha
built with its fault-injection hook (MHA_FAULT_INJECTION): mha_fault_inject(n)
makes the next n kernel launches fail before they reach the HIP runtime, so
valid calls report MHA_ERR_HIP on a machine without a GPU, and the binding
turns that status into an MHAError."""

import ctypes
import os

import pytest

from head_attention_forward_amd import _abi
from head_attention_forward_amd import _binding as bnd
from head_attention_forward_amd import build as hbuild

HIP = -7
FAKE = ctypes.c_void_p(0x10000)
FAKE2 = ctypes.c_void_p(0x20000)


@pytest.fixture(scope="module")
def LF():
    if not os.path.exists(hbuild.FAULT_LIB_PATH):
        hbuild.build(fault=True)
    L = ctypes.CDLL(hbuild.FAULT_LIB_PATH)
    for name, (res, args) in _abi.SIG.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    L.mha_fault_inject.restype = None
    L.mha_fault_inject.argtypes = [ctypes.c_int]
    return L


def test_injected_launch_failure_is_reported(LF):
    LF.mha_fault_inject(1)
    st = LF.sdpa_forward(FAKE, FAKE, FAKE, FAKE2, 2, 2, 8, 8, 64, 64, 0.125, 0, None, bnd.DTYPE_BF16, None)
    assert st == HIP
    # the whole block: its first launch fails, the call stops there
    ws_bytes = LF.mha_workspace_bytes(2, 8, 8, 2, 64, 64, bnd.DTYPE_BF16)
    LF.mha_fault_inject(1)
    st = LF.mha_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, 2, 8, 8, 64, 2, 64, 64, 0, None,
                        bnd.DTYPE_BF16, FAKE, ws_bytes, None)
    assert st == HIP
    # an argument error is still reported as such (checks come first)
    LF.mha_fault_inject(1)
    assert LF.sdpa_forward(None, FAKE, FAKE, FAKE2, 2, 2, 8, 8, 64, 64, 0.125, 0, None,
                           bnd.DTYPE_BF16, None) == -1
    LF.mha_fault_inject(0)


def test_binding_raises_on_a_launch_failure(LF, monkeypatch):
    monkeypatch.setattr(bnd, "_lib", LF)
    LF.mha_fault_inject(1)
    st = LF.sdpa_backward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, FAKE2, FAKE2, 1, 1, 8, 8,
                                  64, 64, 0.125, 0, None, bnd.DTYPE_BF16, None)
    LF.mha_fault_inject(0)
    # the allocation-free entry looks its array up first (no device here: MHA_ERR_HIP either way)
    assert st == HIP
    LF.mha_fault_inject(1)
    st = LF.sdpa_forward(FAKE, FAKE, FAKE, FAKE2, 1, 1, 8, 8, 64, 64, 0.125, 0, None, bnd.DTYPE_BF16, None)
    with pytest.raises(bnd.MHAError) as e:
        bnd._check("sdpa_forward", st)
    assert e.value.status == HIP
    assert "MHA_ERR_HIP" in str(e.value) and "HIP launch failed" in str(e.value)


def test_normal_build_has_no_hook():
    L = ctypes.CDLL(bnd.LIB_PATH)
    assert not hasattr(L, "mha_fault_inject")
