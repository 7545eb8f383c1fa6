"""The forward of an NF4 linear with the weight decoded inside the direct-load GEMM (each K-step's
NF4 block per W row unpacked into the LDS stage beside the matrix-core work). It must hand the
matrix cores exactly the bf16 operand that nf4_dequant writes, in the same tiles and order, so the
results are bit-identical to the same GEMM on the staged bf16 weight: checked over K-step counts
that reach the pipeline's prologue and both parities of its unrolled loop (1, 2, 3, 15, 16, 64
steps), ragged rows and columns, both adapter modes, the grouped launch with its residual and
rotary epilogues, the full 8B projection shapes, and the path taken when the arrays are not
aligned for it. (The oracle parity of the NF4 forward is in test_gpu_lora.py.)"""

from __future__ import annotations

import pytest

from layer_streamed_nf4_dequant_amd import lib
from lora_cases import Case

pytestmark = pytest.mark.gpu


def _eq(a, b):
    import torch
    return a.shape == b.shape and torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("T,K,N", [(256, 64, 256), (300, 128, 512), (257, 192, 512), (512, 960, 768),
                                   (200, 1024, 1344), (1024, 4096, 1024)])
@pytest.mark.parametrize("adapters", [True, False])
def test_nf4_forward_equals_staged(gpu, T, K, N, adapters):
    import torch
    print(f"case: nf4 direct forward T={T} K={K} N={N} adapters={adapters}", flush=True)
    c = Case(T, K, N, tag="nf4direct")
    w16 = lib.nf4_dequant(c.Wd, "bf16")
    Y1, U1 = c.gpu_fwd(adapters=adapters)
    Y2, U2 = c.gpu_fwd(adapters=adapters, W=w16)
    torch.cuda.synchronize()
    assert _eq(Y1, Y2)
    if adapters:
        assert _eq(U1, U2)


def _seeded_nf4(N, K, seed):
    """A seeded normal W[N][K] packed to NF4 on the device (the comparison is GPU against GPU, so
    no oracle-side copy is needed), and its staged bf16 dequantisation."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    w = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
    p = lib.nf4_pack(w)
    return p, lib.nf4_dequant(p, "bf16")


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 14336), (14336, 4096)])
def test_full_size_nf4_forward_equals_staged(gpu, K, N):
    """The 8B projection shapes at T = 4096 (q, gate, down): the whole output bit for bit."""
    import torch
    T, r = 4096, 16
    print(f"case: full-size nf4 direct forward T={T} K={K} N={N}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(7 + K + N)
    X = (torch.randn((T, K), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    A = (torch.randn((r, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    B = (torch.randn((N, r), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    p, w16 = _seeded_nf4(N, K, 11 + N)
    ws = torch.empty(max(lib.ws_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
    out = []
    for W in (p, w16):
        Y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
        lib.lora_linear_fwd(lib.linear_desc(T, K, N, r, 2.0, W, A, B), X, Y, U, adapters=True, ws=ws)
        out.append(Y)
    torch.cuda.synchronize()
    assert _eq(out[0], out[1])


def test_grouped_nf4_epilogues_equal_staged(gpu):
    """A layer's q, k, v (rotated in the epilogue) and a member with a residual, all NF4 in one
    grouped launch, against the same launch on the staged bf16 weights."""
    import torch
    T, K, r, d = 300, 512, 16, 128
    Ns = [512, 128, 128, 256]
    cs = [Case(T, K, N, r=r, tag=f"nf4grp{i}") for i, N in enumerate(Ns)]
    X = cs[0].Xd
    print(f"case: grouped nf4 direct with epilogues T={T} K={K} N={Ns}", flush=True)
    cst = lib.rope_table(1024, d, 10000.0)
    pos = (torch.arange(T, device="cuda", dtype=torch.int32) * 3 + 5) % 1024
    rope = lib.RopeDesc(cst.data_ptr(), 1024, d, pos.data_ptr())
    g = torch.Generator(device="cuda").manual_seed(3)
    R = torch.randn((T, Ns[3]), generator=g, device="cuda").to(torch.bfloat16)
    w16 = [lib.nf4_dequant(c.Wd, "bf16") for c in cs]     # (kept alive while the descriptors point at them)
    res = {}
    for kind in ("nf4", "bf16"):
        descs = [c.desc() if kind == "nf4" else c.desc(W=w) for c, w in zip(cs, w16)]
        Y = [torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
        U = [torch.empty((T, r), dtype=torch.bfloat16, device="cuda") for _ in Ns]
        lib.lora_linear_fwd_group_epi(descs, X, Y, U, adapters=True, residual=[None, None, None, R],
                                      rope_mask=0b011, rope=rope, ws=cs[0].ws)
        torch.cuda.synchronize()
        res[kind] = Y
    for a, b in zip(res["nf4"], res["bf16"]):
        assert _eq(a, b)


def test_unaligned_arrays_take_the_register_staged_kernel(gpu):
    """A quantised-constant array that is not 4-byte aligned cannot be staged by the direct loads:
    the forward then runs the register-staged NF4 kernel, with the same bits."""
    import torch
    T, K, N = 300, 512, 640
    print(f"case: nf4 forward with a misaligned constant array T={T} K={K} N={N}", flush=True)
    c = Case(T, K, N, tag="nf4misaligned")
    q = c.Wd.qabsmax
    buf = torch.empty(q.numel() + 16, dtype=torch.int8, device="cuda")
    shifted = buf[1:1 + q.numel()]
    shifted.copy_(q)
    assert shifted.data_ptr() % 4 == 1
    Wm = lib.NF4Tensor(c.Wd.rows, c.Wd.cols, c.Wd.codes, shifted, c.Wd.absmax2, c.Wd.mean)
    Y1, U1 = c.gpu_fwd()
    Y2, U2 = c.gpu_fwd(W=Wm)
    torch.cuda.synchronize()
    assert _eq(Y1, Y2) and _eq(U1, U2)
