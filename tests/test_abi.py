"""CPU checks of the C ABI: the library loads, exports every function include/lsnf4.h declares,
and its host-computed NF4 codebook equals the oracle's bit for bit (the two are computed by
independent code: the library by bisection + Newton on erfc in C++, the oracle with the
stdlib's inverse normal CDF)."""

import ctypes
import os
import re

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import lib
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsnf4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("nf4_pack", "nf4_dequant", "lora_linear_fwd", "lora_linear_bwd",
                 "layer_pool_prefetch", "layer_pool_acquire", "layer_pool_release"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = lib.load()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in lsnf4.h but not exported"
    assert set(declared_functions()) == set(lib.EXPORTS)


def test_abi_version():
    assert lib.load().lsn_abi_version() == 1


def test_codebook_matches_oracle_bitwise():
    q, m = lib.codebook()
    np.testing.assert_array_equal(q.view(np.uint32), nf4.codebook().view(np.uint32))
    np.testing.assert_array_equal(m.view(np.uint32), nf4.code_thresholds().view(np.uint32))


def test_workspace_sizes_are_sane():
    L = lib.load()
    assert L.nf4_pack_ws_bytes(896, 896) >= 896 * 896 // 64 * 4
    assert L.nf4_pack_ws_bytes(0, 64) == 0


def test_argument_errors_without_gpu():
    """Validation runs before any device call, so it works (and must fail) on the CPU."""
    L = lib.load()
    st = L.nf4_pack(None, 3, 100, None, None, None, None, None, 0, None)
    assert st == lib.LSN_E_ARG
    assert b"cols % 64" in L.lsn_last_error()
    d = lib.NF4Desc(896, 896, None, None, None, 0.0)
    assert L.nf4_dequant(ctypes.byref(d), None, 0, None) == lib.LSN_E_ARG
    with pytest.raises(lib.LsnError):
        lib.check(L.nf4_dequant(None, None, 0, None))


def test_glue_argument_errors_without_gpu():
    """The glue entry points reject bad shapes before touching the device."""
    L = lib.load()
    assert L.rmsnorm_fwd(4, 12, None, None, 1e-5, None, None, None) == lib.LSN_E_ARG
    assert b"multiple of 8" in L.lsn_last_error()
    assert L.rmsnorm_bwd(0, 64, None, None, None, None, None, 0, None) == lib.LSN_E_ARG
    assert L.rope_apply(1, 1, 3, None, 3, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert L.rope_apply(1, 1, 1026, None, 1026, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert L.rope_apply(2, 2, 64, None, 100, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert b"ld" in L.lsn_last_error()
    assert L.swiglu_fwd(7, None, None, None, None) == lib.LSN_E_ARG
    assert L.swiglu_bwd(16, None, None, None, None, None, None) == lib.LSN_E_ARG
