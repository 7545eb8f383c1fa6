"""lora_linear_bwd_noalloc, the backward on the library's static per-GPU workspace (for callers
that cannot allocate), against lora_linear_bwd with a caller workspace on the same inputs: the
same kernels in the same order, so dX, dA and dB must be identical bits. Two calls in a row, the
second on a smaller shape (the static array still holds the first call's partial sums), with
NF4 and bf16 weights and every dX / gradient mode; a shape whose workspace exceeds the static
array is refused before any device work."""

import pytest

from layer_streamed_nf4_dequant_amd import lib
from lora_cases import Case

pytestmark = pytest.mark.gpu


def _eq(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _outputs(c: Case, dx_mode):
    """dX (fp32 for the fp32 modes, starting from the case's dX_init) and dA, dB (starting from
    the case's g_init, which GRAD_ADD accumulates onto)."""
    import torch
    if dx_mode == lib.DX_BF16_SET:
        dX = torch.empty((c.T, c.K), dtype=torch.bfloat16, device="cuda")
    else:
        dX = torch.from_numpy(c.dX_init).cuda()
    g0 = torch.from_numpy(c.g_init).cuda()
    return dX, g0[: c.r * c.K].view(c.r, c.K).clone(), g0[c.r * c.K:].view(c.N, c.r).clone()


def _both(c: Case, U, dx_mode, grad_mode):
    """(with a caller workspace, no-alloc) outputs from the same initial values."""
    import torch
    ref = _outputs(c, dx_mode)
    lib.lora_linear_bwd(c.desc(), c.Xd, c.dYd, U, *ref, dx_mode=dx_mode, grad_mode=grad_mode, ws=c.ws)
    got = _outputs(c, dx_mode)
    lib.lora_linear_bwd_noalloc(c.desc(), c.Xd, c.dYd, U, *got, dx_mode=dx_mode, grad_mode=grad_mode)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("base", ["nf4", "bf16"])
def test_noalloc_backward_equals_workspace_backward(gpu, base):
    import torch
    # (T, K, N, r, dX mode, gradient mode): the second call is smaller than the first
    calls = [(1000, 1344, 2048, 32, lib.DX_F32_SET, lib.GRAD_SET),
             (300, 256, 192, 16, lib.DX_BF16_SET, lib.GRAD_ADD)]
    if base == "nf4":
        calls.append((129, 128, 128, 8, lib.DX_F32_ADD, lib.GRAD_SET))
    for T, K, N, r, dx_mode, grad_mode in calls:
        print(f"case: noalloc backward base={base} T={T} K={K} N={N} r={r} dx_mode={dx_mode} "
              f"grad_mode={grad_mode}", flush=True)
        assert lib.ws_bytes(T, K, N, r) <= lib.noalloc_max_ws_bytes()
        c = Case(T, K, N, r=r, base=base, tag="noalloc")
        _, U = c.gpu_fwd()
        torch.cuda.synchronize()
        (dX0, dA0, dB0), (dX1, dA1, dB1) = _both(c, U, dx_mode, grad_mode)
        assert _eq(dX0, dX1) and _eq(dA0, dA1) and _eq(dB0, dB1)


def test_noalloc_refuses_a_shape_beyond_its_workspace(gpu):
    import torch
    T, K, N, r = 8192, 14336, 14336, 32
    assert lib.ws_bytes(T, K, N, r) > lib.noalloc_max_ws_bytes()
    print(f"case: noalloc refusal T={T} K={K} N={N} r={r}", flush=True)
    X = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    A = torch.empty((r, K), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((N, r), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    desc = lib.linear_desc(T, K, N, r, 2.0, W, A, B)
    with pytest.raises(lib.LsnError) as e:
        lib.lora_linear_bwd_noalloc(desc, X, dY, U, dX, dA, dB)
    assert e.value.status == lib.LSN_E_ARG and "static" in str(e.value)
