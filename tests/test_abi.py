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
    assert L.rmsnorm_bwd(0, 64, None, None, None, None, None, 0, None, None) == lib.LSN_E_ARG
    assert L.rope_apply(1, 1, 3, None, 3, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert L.rope_apply(1, 1, 1026, None, 1026, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert L.rope_apply(2, 2, 64, None, 100, None, 10000.0, 0, None) == lib.LSN_E_ARG
    assert b"ld" in L.lsn_last_error()
    assert L.swiglu_fwd(7, None, None, None, None) == lib.LSN_E_ARG
    assert L.swiglu_bwd(16, None, None, None, None, None, None) == lib.LSN_E_ARG


def test_attention_argument_errors_without_gpu():
    """Shape, stride and overlap checks of the attention entry points run before any device
    call: column ranges of one fused buffer are accepted (the call then stops at the device
    check), overlapping ones are refused."""
    L = lib.load()
    base = 1 << 20                      # a fake, 16-byte aligned device address (never dereferenced)
    T, nq, nkv, d = 8, 4, 2, 64
    W = (nq + 2 * nkv) * d
    q, k, v = base, base + 2 * nq * d, base + 2 * (nq + nkv) * d
    o, lse = base + 2 * T * W + 4096, base + 4 * T * W + 8192
    args = lambda hd, oo: (2, 4, nq, nkv, hd, q, W, k, W, v, W, 0.125, oo, nq * d, lse, None)  # noqa: E731
    assert L.attention_fwd(*args(96, o)) == lib.LSN_E_ARG
    assert b"head_dim" in L.lsn_last_error()
    assert L.attention_fwd(*args(d, q)) == lib.LSN_E_ARG          # o on top of q
    assert L.attention_fwd(*args(d, o)) not in (lib.LSN_OK, lib.LSN_E_ARG)   # valid: reaches the device check
    g = base + 6 * T * W + 16384       # fused gradient buffer: dq, dk, dv column ranges
    dq, dk, dv = g, g + 2 * nq * d, g + 2 * (nq + nkv) * d
    ws = g + 2 * T * W + 4096
    bwd = lambda a, b_, c_: (2, 4, nq, nkv, d, q, W, k, W, v, W, o, nq * d, lse, o + 2 * T * nq * d + 256,  # noqa: E731
                             nq * d, 0.125, a, W, b_, W, c_, W, ws, 1 << 20, None)
    assert L.attention_bwd(*bwd(dq, dk, dv)) not in (lib.LSN_OK, lib.LSN_E_ARG)
    assert L.attention_bwd(*bwd(dq, dq + 64, dv)) == lib.LSN_E_ARG     # dk overlaps dq's columns
    assert b"overlap" in L.lsn_last_error()
    # the row dots (rounded up to 256 bytes), and with an even number of query heads per key/value
    # head the dk, dv partial sums of the two halves of them
    assert L.attention_bwd_ws_bytes(2, 4, nq, nkv, d) == 256 + 4 * (2 * 4) * nkv * d * 4
    assert L.attention_bwd_ws_bytes(2, 4, 3, 1, d) == 256
    assert L.attention_bwd_ws_bytes(2, 100, 3, 1, d) == (2 * 100 * 3 * 4 + 255) // 256 * 256
    assert L.attention_bwd_ws_bytes(2, 4, 4, 3, d) == 0


def test_lora_argument_errors_without_gpu():
    """The LoRA entry points refuse an empty token batch, a reduction or output width that is
    not a multiple of 64 and an unsupported rank before any device call (the pointers here are
    never dereferenced)."""
    L = lib.load()
    p = 1 << 20   # a 16-byte aligned stand-in address

    def desc(T, K, N, r):
        return lib.LoraLinearDesc(T, K, N, r, 2.0, lib.WeightDesc(lib.W_BF16, lib.NF4Desc(), p), p, p)

    for (T, K, N, r), msg in (((0, 128, 128, 16), b"T >= 1"), ((64, 100, 128, 16), b"multiples of 64"),
                              ((64, 128, 96, 16), b"multiples of 64"), ((64, 128, 128, 12), b"rank r")):
        d = desc(T, K, N, r)
        assert L.lora_linear_fwd(ctypes.byref(d), lib.ADAPTERS_ON, p, p, p, p, 1 << 30, None) == lib.LSN_E_ARG
        assert msg in L.lsn_last_error()
        assert L.lora_linear_bwd(ctypes.byref(d), p, p, p, p, lib.DX_BF16_SET, p, p, lib.GRAD_SET, p, 1 << 30,
                                 None) == lib.LSN_E_ARG
        assert msg in L.lsn_last_error()
        assert L.lora_linear_bwd_noalloc(ctypes.byref(d), p, p, p, p, lib.DX_BF16_SET, p, p, lib.GRAD_SET,
                                         None) == lib.LSN_E_ARG
        assert msg in L.lsn_last_error()
    assert L.lora_down(0, 128, p, 1, (ctypes.c_void_p * 1)(p), (ctypes.c_int32 * 1)(16),
                       (ctypes.c_void_p * 1)(p), None) == lib.LSN_E_ARG
    assert b"T >= 1" in L.lsn_last_error()
