"""GPU parity of the LoRA linear (forward, recomputed forward, backward) against the oracle,
through the C ABI, plus the exact invariants that hold on the GPU itself:
  * fused NF4-dequant-in-LDS GEMM == bf16 GEMM on the standalone-dequantised W (bit-exact);
  * B = 0 == adapters off (bit-exact); recompute == forward (bit-exact); two runs bit-equal.
Tolerances (relative L2 over the whole tensor, fp64): Y, dX 5e-3; dA, dB 1e-2.
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import lib
from lora_cases import Case, assert_close, to_np
from oracle import lora as olora
from oracle.nf4 import bf16_to_f32 as onf4_f32

pytestmark = pytest.mark.gpu


def _eq(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _full_parity(c: Case, transposed=False):
    """transposed: the backward reads W^T [K][N] (LSN_W_BF16_T) instead of W."""
    import torch
    Y, U = c.gpu_fwd()
    if transposed:
        dX, dA, dB = c.gpu_bwd(U, W=c.w_transposed(), transposed=True)
    else:
        dX, dA, dB = c.gpu_bwd(U)
    torch.cuda.synchronize()
    Yo, Uo = c.oracle_fwd()
    dXo, dAo, dBo, Go = c.oracle_bwd()
    errs = {
        "U": assert_close("U", to_np(U), Uo),
        "Y": assert_close("Y", to_np(Y), Yo),
        "dX": assert_close("dX", to_np(dX), dXo),
        # dA/dB were initialised to g0 but grad_mode SET overwrites them
        "dA": assert_close("dA", to_np(dA), dAo),
        "dB": assert_close("dB", to_np(dB), dBo),
    }
    print({k: f"{v:.2e}" for k, v in errs.items()})
    return Y, U, dX, dA, dB


@pytest.mark.parametrize("transposed", [False, True], ids=["W", "WT"])
@pytest.mark.parametrize("base", ["nf4", "bf16"])
def test_single_linear_parity(gpu, base, transposed):
    print(f"case: single linear T=512 K=N=896 r=16 base={base} transposed={transposed}", flush=True)
    _full_parity(Case(512, 896, 896, base=base, tag="single"), transposed)


@pytest.mark.parametrize("transposed", [False, True], ids=["W", "WT"])
@pytest.mark.parametrize("T,K,N,r", [(300, 256, 192, 16), (1, 128, 128, 8), (777, 512, 1344, 32),
                                     (256, 64, 256, 24), (2048, 896, 128, 16)])
def test_ragged_and_rank_shapes(gpu, T, K, N, r, transposed):
    print(f"case: T={T} K={K} N={N} r={r} transposed={transposed}", flush=True)
    _full_parity(Case(T, K, N, r=r, tag="ragged"), transposed)


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 192, 16), (777, 512, 1344, 32), (256, 64, 256, 24),
                                     (2048, 896, 128, 16), (513, 960, 896, 8), (1, 128, 64, 16)])
def test_bf16_w_backward_equals_transposed_layout(gpu, T, K, N, r):
    """The backward on a bf16 W [N][K] reads it reduction-major (LDS transpose reads) and must hand
    the matrix cores the same fragments as W^T [K][N]: dX, dA and dB bit-identical in both dX
    modes (ragged T, K and N tiles, K = 64, every rank), and dX within tolerance of the oracle."""
    import torch
    c = Case(T, K, N, r=r, base="bf16", tag="wlayout")
    print(f"case: W vs W^T backward T={T} K={K} N={N} r={r}", flush=True)
    Y, U = c.gpu_fwd()
    wt = c.w_transposed()
    for dx_mode, grad_mode in ((lib.DX_BF16_SET, lib.GRAD_SET), (lib.DX_F32_ADD, lib.GRAD_ADD)):
        got = c.gpu_bwd(U, dx_mode=dx_mode, grad_mode=grad_mode)
        want = c.gpu_bwd(U, dx_mode=dx_mode, grad_mode=grad_mode, W=wt, transposed=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dX", "dA", "dB"), got, want):
            assert _eq(a, b), (name, dx_mode)
    dX, dA, dB = c.gpu_bwd(U)
    torch.cuda.synchronize()
    dXo, dAo, dBo, _ = c.oracle_bwd()
    assert_close("dX", to_np(dX), dXo)
    assert_close("dA", to_np(dA), dAo)
    assert_close("dB", to_np(dB), dBo)


@pytest.mark.parametrize("transposed", [False, True], ids=["W", "WT"])
def test_accumulate_modes(gpu, transposed):
    import torch
    c = Case(384, 512, 320, tag="accum")
    print(f"case: accumulate modes T=384 K=512 N=320 transposed={transposed}", flush=True)
    Y, U = c.gpu_fwd()
    if transposed:
        dX, dA, dB = c.gpu_bwd(U, dx_mode=lib.DX_F32_ADD, grad_mode=lib.GRAD_ADD, W=c.w_transposed(),
                               transposed=True)
    else:
        dX, dA, dB = c.gpu_bwd(U, dx_mode=lib.DX_F32_ADD, grad_mode=lib.GRAD_ADD)
    torch.cuda.synchronize()
    dXo, dAo, dBo, _ = c.oracle_bwd()
    r, K = c.r, c.K
    # the increment added into the fp32 buffer must match dY W + s G A to the dX tolerance
    assert_close("dX", to_np(dX).astype(np.float64) - c.dX_init, dXo)
    assert_close("dA", to_np(dA).astype(np.float64) - c.g_init[: r * K].reshape(r, K), dAo)
    assert_close("dB", to_np(dB).astype(np.float64) - c.g_init[r * K:].reshape(c.N, r), dBo)


@pytest.mark.parametrize("base,transposed", [("nf4", False), ("bf16", False), ("bf16", True)])
def test_f32_store_mode_equals_add_into_zeros(gpu, base, transposed):
    """LSN_DX_F32_SET writes what LSN_DX_F32_ADD adds into a zeroed buffer (single linear, and a
    group of three whose members share X), with identical LoRA gradients."""
    import torch
    c = Case(300, 512, 320, base=base, tag="f32set")
    print(f"case: fp32 store mode base={base} transposed={transposed}", flush=True)
    Y, U = c.gpu_fwd()
    W = c.w_transposed() if transposed else None
    desc = c.desc(W, transposed)
    outs = {}
    for mode in (lib.DX_F32_SET, lib.DX_F32_ADD):
        dX = torch.full((c.T, c.K), 7.0 if mode == lib.DX_F32_SET else 0.0, dtype=torch.float32, device="cuda")
        dA = torch.empty((c.r, c.K), dtype=torch.float32, device="cuda")
        dB = torch.empty((c.N, c.r), dtype=torch.float32, device="cuda")
        lib.lora_linear_bwd(desc, c.Xd, c.dYd, U, dX, dA, dB, dx_mode=mode, ws=c.ws)
        outs[mode] = (dX, dA, dB)
    torch.cuda.synchronize()
    for a, b in zip(outs[lib.DX_F32_SET], outs[lib.DX_F32_ADD]):
        assert torch.equal(a, b)
    cs = [Case(300, 512, N, base=base, tag=f"f32setg{i}") for i, N in enumerate((320, 128, 448))]
    X = cs[0].Xd
    Us = []
    for m in cs:
        Ym = torch.empty((300, m.N), dtype=torch.bfloat16, device="cuda")
        Um = torch.empty((300, 16), dtype=torch.bfloat16, device="cuda")
        lib.lora_linear_fwd(m.desc(), X, Ym, Um, adapters=True, ws=m.ws)
        Us.append(Um)
    wts = [m.w_transposed() for m in cs] if transposed else [None] * len(cs)   # kept alive: descs hold pointers
    descs = [m.desc(wt, True) if transposed else m.desc() for m, wt in zip(cs, wts)]
    ws = torch.empty(lib.group_ws_bytes(descs), dtype=torch.uint8, device="cuda")
    res = {}
    for mode in (lib.DX_F32_SET, lib.DX_F32_ADD):
        dX = torch.full((300, 512), -3.0 if mode == lib.DX_F32_SET else 0.0, dtype=torch.float32, device="cuda")
        dA = [torch.empty((16, 512), dtype=torch.float32, device="cuda") for _ in cs]
        dB = [torch.empty((m.N, 16), dtype=torch.float32, device="cuda") for m in cs]
        lib.lora_linear_bwd_group(descs, X, [m.dYd for m in cs], Us, dX, dA, dB, dx_mode=mode, ws=ws)
        res[mode] = (dX, dA, dB)
    torch.cuda.synchronize()
    assert torch.equal(res[lib.DX_F32_SET][0], res[lib.DX_F32_ADD][0])
    for a, b in zip(res[lib.DX_F32_SET][1] + res[lib.DX_F32_SET][2], res[lib.DX_F32_ADD][1] + res[lib.DX_F32_ADD][2]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,K,N", [(512, 896, 896), (300, 1024, 640)])
def test_fused_nf4_equals_bf16_gemm_on_dequantised_weights(gpu, T, K, N):
    """The dequant-into-LDS path must hand the matrix cores exactly the bf16 W that the
    standalone dequantisation writes: same tiles, same order, so identical bits."""
    import torch
    c = Case(T, K, N, tag="fused")
    print(f"case: fused vs bf16 T={T} K={K} N={N}", flush=True)
    w16 = lib.nf4_dequant(c.Wd, "bf16")
    Y1, U1 = c.gpu_fwd()
    Y2, U2 = c.gpu_fwd(W=w16)
    dX1, dA1, dB1 = c.gpu_bwd(U1)
    dX2, dA2, dB2 = c.gpu_bwd(U2, W=w16)
    torch.cuda.synchronize()
    for a, b in ((Y1, Y2), (U1, U2), (dX1, dX2), (dA1, dA2), (dB1, dB2)):
        assert _eq(a, b)


@pytest.mark.parametrize("scale", [1.5, 0.75, 4.0])
def test_scale_not_one_or_two(gpu, scale):
    """Scales other than the configurations' 2 (alpha = 24, 12 or 64 at r = 16): the oracle's s U B^T
    against the GEMMs' (bf16(s U)) B^T, the dequant-into-LDS GEMM bit-identical to the bf16 one on
    the dequantised weights, and the bf16 path with a power-of-two s bit-identical to scaling by
    hand: s = 4 on (U, B) equals s = 1 on (4 U, B), 4 U being exact in bf16."""
    import torch
    print(f"case: scale {scale}", flush=True)
    c = Case(300, 512, 640, scale=scale, tag="scale")
    _full_parity(c)
    w16 = lib.nf4_dequant(c.Wd, "bf16")
    Y1, U1 = c.gpu_fwd()
    Y2, U2 = c.gpu_fwd(W=w16)
    dX1, dA1, dB1 = c.gpu_bwd(U1)
    dX2, dA2, dB2 = c.gpu_bwd(U2, W=w16)
    torch.cuda.synchronize()
    for a, b in ((Y1, Y2), (U1, U2), (dX1, dX2), (dA1, dA2), (dB1, dB2)):
        assert _eq(a, b)
    if scale == 4.0:
        Y3 = torch.empty_like(Y2)
        U4 = (U2.float() * 4.0).to(torch.bfloat16)
        d1 = lib.linear_desc(c.T, c.K, c.N, c.r, 1.0, w16, c.Ad, c.Bd)
        lib.lora_linear_fwd(d1, c.Xd, Y3, U4, adapters=lib.ADAPTERS_U_READY, ws=c.ws)
        torch.cuda.synchronize()
        assert _eq(Y2, Y3)


@pytest.mark.parametrize("base", ["nf4", "bf16"])
def test_grouped_forward_equals_single_forwards(gpu, base):
    """Five linears sharing one input (a decoder layer's q, k, v, gate, up at small widths),
    with ragged T: the grouped forward is bit-identical to one call per linear, and matches
    the oracle."""
    import torch
    T, K, r = 300, 512, 16
    Ns = [512, 128, 128, 1344, 1344]
    cs = [Case(T, K, N, r=r, base=base, tag=f"group{i}") for i, N in enumerate(Ns)]
    X = cs[0].Xd
    print(f"case: grouped forward T={T} K={K} N={Ns} base={base}", flush=True)
    for mode in (lib.ADAPTERS_ON, lib.ADAPTERS_OFF):
        Yg = [torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
        Ug = [torch.empty((T, r), dtype=torch.bfloat16, device="cuda") for _ in Ns]
        lib.lora_linear_fwd_group([c.desc() for c in cs], X, Yg, Ug, adapters=mode, ws=cs[0].ws)
        for c, y, u in zip(cs, Yg, Ug):
            Y1 = torch.empty_like(y)
            U1 = torch.empty_like(u)
            lib.lora_linear_fwd(c.desc(), X, Y1, U1, adapters=mode, ws=c.ws)
            torch.cuda.synchronize()
            assert _eq(y, Y1)
            if mode == lib.ADAPTERS_ON:
                assert _eq(u, U1)
            Yo, _ = olora.forward(onf4_f32(cs[0].X), onf4_f32(c.W_hat_bits), onf4_f32(c.A),
                                  onf4_f32(c.B), c.s, mode == lib.ADAPTERS_ON)
            assert_close("Y", to_np(y), Yo)
    with pytest.raises(lib.LsnError):          # members must share K
        bad = Case(T, 256, 128, r=r, base=base, tag="group-bad")
        lib.lora_linear_fwd_group([cs[0].desc(), bad.desc()], X, Yg[:2], Ug[:2], ws=cs[0].ws)
    with pytest.raises(lib.LsnError):          # a Y overlapping X
        lib.lora_linear_fwd_group([cs[0].desc(), cs[1].desc()], X, [Yg[0], X], Ug[:2], ws=cs[0].ws)


@pytest.mark.parametrize("T,r", [(300, 16), (129, 32)])
@pytest.mark.parametrize("base", ["nf4", "bf16"])
def test_grouped_backward(gpu, base, T, r):
    """Five linears sharing X (ragged T, mixed N): the grouped backward gives each member's dA,
    dB bit-identical to its own backward, and dX equal to the sum of the members' dX (one GEMM
    over the concatenated N for bf16 weights, bit-identical for W and W^T; member order for
    NF4 weights), matching the oracle; the fp32 accumulate mode adds onto what dX held. (All
    members' G in one launch, all dA/dB partials in one launch, all reductions in one launch.)"""
    import torch
    K = 512
    Ns = [512, 128, 128, 1344, 1344]
    cs = [Case(T, K, N, r=r, base=base, tag=f"gbwd{i}") for i, N in enumerate(Ns)]
    X = cs[0].Xd
    print(f"case: grouped backward T={T} K={K} N={Ns} r={r} base={base}", flush=True)
    Us = []
    for c in cs:
        Y = torch.empty((T, c.N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
        lib.lora_linear_fwd(c.desc(), X, Y, U, adapters=True, ws=c.ws)
        Us.append(U)
    wts = [c.w_transposed() for c in cs]
    descs = [c.desc(wt, transposed=True) for c, wt in zip(cs, wts)]
    ws = torch.empty(lib.group_ws_bytes(descs), dtype=torch.uint8, device="cuda")
    dX0 = torch.from_numpy(cs[0].dX_init).cuda()
    dX = dX0.clone()
    dA = [torch.empty((r, K), dtype=torch.float32, device="cuda") for _ in cs]
    dB = [torch.empty((c.N, r), dtype=torch.float32, device="cuda") for c in cs]
    lib.lora_linear_bwd_group(descs, X, [c.dYd for c in cs], Us, dX, dA, dB, dx_mode=lib.DX_F32_ADD, ws=ws)
    dX16 = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA2 = [torch.empty_like(a) for a in dA]
    dB2 = [torch.empty_like(b) for b in dB]
    lib.lora_linear_bwd_group(descs, X, [c.dYd for c in cs], Us, dX16, dA2, dB2, dx_mode=lib.DX_BF16_SET, ws=ws)
    # members one by one
    dX_seq = dX0.clone()
    for c, wt, U, a, b in zip(cs, wts, Us, dA2, dB2):
        a1, b1 = torch.empty_like(a), torch.empty_like(b)
        lib.lora_linear_bwd(c.desc(wt, transposed=True), X, c.dYd, U, dX_seq, a1, b1, dx_mode=lib.DX_F32_ADD,
                            ws=c.ws)
        torch.cuda.synchronize()
        assert _eq(a, a1) and _eq(b, b1)
    torch.cuda.synchronize()
    for a, a2, b, b2 in zip(dA, dA2, dB, dB2):
        assert _eq(a, a2) and _eq(b, b2)
    want = np.zeros((T, K))
    for c in cs:
        dXo, dAo, dBo, _ = olora.backward(onf4_f32(cs[0].X), onf4_f32(c.dY), onf4_f32(c.W_hat_bits),
                                         onf4_f32(c.A), onf4_f32(c.B), c.s)
        want += dXo
    assert_close("dX", to_np(dX).astype(np.float64) - cs[0].dX_init, want)
    assert_close("dX", to_np(dX16), want)
    assert_close("dX", to_np(dX_seq).astype(np.float64) - cs[0].dX_init, want)
    # the fused sum differs from the member-order sum only by fp32 rounding
    assert olora.rel_l2(to_np(dX).astype(np.float64), to_np(dX_seq).astype(np.float64)) < 1e-6
    # weights as given (W [N][K]): bf16 members run the same single GEMM, reading W reduction-
    # major, with the transposed layout's bits; NF4 members run one after another, bit-identical
    # to separate calls
    dXn = dX0.clone()
    dA3 = [torch.empty_like(a) for a in dA]
    dB3 = [torch.empty_like(b) for b in dB]
    lib.lora_linear_bwd_group([c.desc() for c in cs], X, [c.dYd for c in cs], Us, dXn, dA3, dB3,
                              dx_mode=lib.DX_F32_ADD, ws=ws)
    if base == "bf16":
        dX16n = torch.empty_like(dX16)
        lib.lora_linear_bwd_group([c.desc() for c in cs], X, [c.dYd for c in cs], Us, dX16n, dA3, dB3,
                                  dx_mode=lib.DX_BF16_SET, ws=ws)
        torch.cuda.synchronize()
        assert _eq(dXn, dX) and _eq(dX16n, dX16)
        for a, a3, b, b3 in zip(dA, dA3, dB, dB3):
            assert _eq(a, a3) and _eq(b, b3)
        with pytest.raises(lib.LsnError):      # mixed layouts: no single GEMM, so no bf16 sum
            lib.lora_linear_bwd_group([descs[0]] + [c.desc() for c in cs[1:]], X, [c.dYd for c in cs], Us,
                                      dX16n, dA3, dB3, dx_mode=lib.DX_BF16_SET, ws=ws)
    else:
        dXm = dX0.clone()
        for c, U in zip(cs, Us):
            a1 = torch.empty((r, K), dtype=torch.float32, device="cuda")
            b1 = torch.empty((c.N, r), dtype=torch.float32, device="cuda")
            lib.lora_linear_bwd(c.desc(), X, c.dYd, U, dXm, a1, b1, dx_mode=lib.DX_F32_ADD, ws=c.ws)
        torch.cuda.synchronize()
        assert _eq(dXn, dXm)
        with pytest.raises(lib.LsnError):      # bf16 dX over several NF4 members
            lib.lora_linear_bwd_group([c.desc() for c in cs], X, [c.dYd for c in cs], Us, dX16, dA3, dB3,
                                      dx_mode=lib.DX_BF16_SET, ws=ws)
    with pytest.raises(lib.LsnError):          # workspace too small
        lib.lora_linear_bwd_group(descs, X, [c.dYd for c in cs], Us, dX, dA, dB, ws=ws[:1024])
    with pytest.raises(lib.LsnError):          # an output overlapping an input
        lib.lora_linear_bwd_group(descs, X, [c.dYd for c in cs], Us, dX, [dA[0], dA[1], dA[2], dA[3], dB[4]], dB,
                                  ws=ws)


def test_b_zero_equals_adapters_off_and_recompute_equals_forward(gpu):
    import torch
    c = Case(512, 896, 896, B_zero=True, tag="bzero")
    print("case: B=0 vs adapters off", flush=True)
    Y_on, _ = c.gpu_fwd(adapters=True)
    Y_off, _ = c.gpu_fwd(adapters=False)
    Y_again, _ = c.gpu_fwd(adapters=True)
    torch.cuda.synchronize()
    assert _eq(Y_on, Y_off) and _eq(Y_on, Y_again)
    Yo, _ = c.oracle_fwd(adapters=False)
    assert_close("Y", to_np(Y_off), Yo)


def test_runs_are_bit_identical(gpu):
    import torch
    c = Case(640, 1024, 2048, tag="det")
    print("case: determinism T=640 K=1024 N=2048", flush=True)
    outs1 = list(c.gpu_fwd()) + list(c.gpu_bwd(c.gpu_fwd()[1]))
    outs2 = list(c.gpu_fwd()) + list(c.gpu_bwd(c.gpu_fwd()[1]))
    torch.cuda.synchronize()
    for a, b in zip(outs1, outs2):
        assert _eq(a, b)


def test_argument_validation(gpu):
    import torch
    c = Case(64, 128, 128, tag="args")
    Y = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((64, 16), dtype=torch.bfloat16, device="cuda")
    bad = lib.linear_desc(64, 100, 128, 16, 2.0, c.Wd, c.Ad, c.Bd)
    with pytest.raises(lib.LsnError):
        lib.lora_linear_fwd(bad, c.Xd, Y, U, ws=c.ws)
    with pytest.raises(lib.LsnError):          # output overlapping an input
        lib.lora_linear_fwd(c.desc(), c.Xd, c.Xd, U, ws=c.ws)
    with pytest.raises(lib.LsnError):          # rank not a multiple of 8
        lib.lora_linear_fwd(lib.linear_desc(64, 128, 128, 12, 2.0, c.Wd, c.Ad, c.Bd), c.Xd, Y, U, ws=c.ws)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    dX = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((16, 128), dtype=torch.float32, device="cuda")
    dB = torch.empty((128, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.LsnError):
        lib.lora_linear_bwd(c.desc(), c.Xd, c.dYd, U, dX, dA, dB, ws=small)
    with pytest.raises(lib.LsnError) as e:     # the transposed layout is for the backward only
        lib.lora_linear_fwd(c.desc(c.w_transposed(), transposed=True), c.Xd, Y, U, ws=c.ws)
    assert e.value.status == lib.LSN_E_ARG


@pytest.mark.parametrize("label,T,K,N", [("8B gate", 4096, 4096, 14336), ("8B down", 4096, 14336, 4096),
                                         ("72B q/o", 2048, 8192, 8192), ("72B k/v", 2048, 8192, 1024),
                                         ("72B gate/up", 2048, 8192, 29568), ("72B down", 2048, 29568, 8192)])
def test_full_size_sampled_parity(gpu, label, T, K, N):
    """Full-size projections (every distinct shape of the 8B and 72B layers) in the launch
    configuration the stack uses, against the oracle: Y and dX on sampled rows (a row of each
    depends only on the same row of X or dY), dA and dB on sampled columns over all T rows. The
    oracle's references come from olora.forward / olora.backward called on the sampled slices:
    a row slice of X and dY gives those rows of Y and dX; a column slice of dY and B (with the
    matching rows of W) leaves U = X A^T whole and gives those columns of dB; a column slice of
    X, A and W leaves G = dY B whole and gives those columns of dA."""
    import torch
    print(f"case: {label} T={T} K={K} N={N}", flush=True)
    c = Case(T, K, N, tag="full")
    Y, U = c.gpu_fwd()
    dX, dA, dB = c.gpu_bwd(U, W=c.w_transposed(), transposed=True)
    dX_w, dA_w, dB_w = c.gpu_bwd(U, W=lib.nf4_dequant(c.Wd, "bf16"))   # the stack's backward path
    dX_nn, dA_nn, dB_nn = c.gpu_bwd(U)
    torch.cuda.synchronize()
    # the LoRA gradients do not involve W: every backward path runs the same kernels for them;
    # the staged W [N][K] and W^T [K][N] give the same dX bits
    assert _eq(dA, dA_nn) and _eq(dB, dB_nn) and _eq(dA, dA_w) and _eq(dB, dB_w)
    assert _eq(dX, dX_w)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(T, 48, replace=False))
    cols_n = np.sort(rng.choice(N, 64, replace=False))
    cols_k = np.sort(rng.choice(K, 64, replace=False))
    X, dY = onf4_f32(c.X), onf4_f32(c.dY)
    Wh = onf4_f32(c.W_hat_bits)
    A, B = onf4_f32(c.A), onf4_f32(c.B)
    Yo, _ = olora.forward(X[rows], Wh, A, B, c.s)
    assert_close("Y", to_np(Y)[rows], Yo)
    dXo, _, _, _ = olora.backward(X[rows], dY[rows], Wh, A, B, c.s)
    assert_close("dX", to_np(dX)[rows], dXo)
    assert_close("dX", to_np(dX_nn)[rows], dXo)
    _, _, dBo, _ = olora.backward(X, dY[:, cols_n], Wh[cols_n], A, B[cols_n], c.s)
    assert_close("dB", to_np(dB)[cols_n], dBo)
    _, dAo, _, _ = olora.backward(X[:, cols_k], dY, Wh[:, cols_k], A[:, cols_k], B, c.s)
    assert_close("dA", to_np(dA)[:, cols_k], dAo)
