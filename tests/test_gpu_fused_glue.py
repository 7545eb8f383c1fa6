"""GPU parity of the projections (and attention's backward) with the decoder-layer glue applied in
their epilogues, through the C ABI:

  * rope_table against the rotation angles the oracle computes;
  * lora_linear_fwd_group_epi (rotary embedding of q and k, residual adds after o and down),
    lora_linear_fwd_swiglu (gate, up and the SwiGLU in one launch), lora_linear_bwd_swiglu (the
    down projection's backward with the SwiGLU's backward in its epilogue) and attention_bwd_rope
    (dq, dk rotated back as they are stored): each bit for bit against the unfused sequence it
    replaces (the projection or attention entry point, then the standalone glue kernel), and
    against the oracle (the LoRA linear / attention oracle composed with the glue oracle, the
    stored activations rounded to bf16 at the same points), rel-L2 5e-3 for outputs and input
    gradients, 1e-2 for adapter gradients as the other projection tests;
  * a decoder training step with the glue fused equals the step with the separate glue kernels,
    bit for bit (loss, every dA and dB).

Shapes span several 256-row tiles with a ragged last one (T = 300), a ragged 128-column pair tile
for the SwiGLU (N = 192), NF4 and bf16 weights (the fused-dequant GEMM and the staged one).
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import inputs, lib
from oracle import attention as oatt
from oracle import glue as og
from oracle import lora as olora
from oracle import nf4 as onf4

from lora_cases import Case, assert_close, bf16_dev, f32, to_np

pytestmark = pytest.mark.gpu


def r16(a):
    """Storage rounding: fp64 -> fp32 -> bf16 (nearest even) -> value."""
    return onf4.bf16_to_f32(onf4.bf16_rne(np.asarray(a, dtype=np.float32))).astype(np.float64)


def _eq(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
    return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))


def _assert_eq(name, a, b):
    import torch
    if not _eq(a, b):
        ia = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
        ib = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        bad = (ia != ib).nonzero()
        raise AssertionError(f"{name}: {bad.shape[0]} elements differ, first at {bad[0].tolist()}")


def _positions(T, p0, seed):
    pos = (p0 + np.arange(T)).astype(np.int32)
    rng = np.random.default_rng(seed)
    pos[rng.integers(0, T, size=T // 10)] = 0
    return pos


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d,theta,n_pos", [(128, 500000.0, 8192), (64, 1000000.0, 2049), (16, 10000.0, 3)])
def test_rope_table_matches_oracle_angles(gpu, d, theta, n_pos):
    """cs[p][i] = (cos, sin) of p theta^(-2i/d): the fp32 angle fl32(p fl32(f_i)) is within
    |a| 2^-23 of the exact one, and sincosf within a few ulp, so |cs - exact| <= 1.2e-7 |a| + 6e-7."""
    print(f"case: rope_table d={d} n_pos={n_pos}", flush=True)
    cs = lib.rope_table(n_pos, d, theta).cpu().numpy().astype(np.float64)
    a = og.rope_angles(np.arange(n_pos), d, theta)
    bound = 1.2e-7 * np.abs(a) + 6e-7
    for name, got, ref in (("cos", cs[..., 0], np.cos(a)), ("sin", cs[..., 1], np.sin(a))):
        err = np.abs(got - ref)
        assert (err <= bound).all(), f"{name}: worst {err.max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}"


# ---------------------------------------------------------------------------------------------
ROPE_GROUPS = [  # T, K, head_dim, n_q, n_kv, theta, first position
    (300, 256, 128, 4, 2, 500000.0, 0),
    (300, 256, 64, 6, 2, 1000000.0, 1500),
    (64, 512, 128, 2, 1, 500000.0, 7),
]


@pytest.mark.parametrize("base", ["bf16", "nf4"])
@pytest.mark.parametrize("T,K,d,nq,nkv,theta,p0", ROPE_GROUPS)
def test_group_rope_epilogue(gpu, T, K, d, nq, nkv, theta, p0, base):
    """q and k leave the grouped projection rotated, v untouched: bit-identical to
    lora_linear_fwd_group then rope_apply on q and k; matches the oracle's rotation of the
    rounded projection outputs."""
    import torch
    print(f"case: group rope T={T} K={K} d={d} nq={nq} nkv={nkv} base={base}", flush=True)
    Ns = [nq * d, nkv * d, nkv * d]
    cs = [Case(T, K, N, base=base, tag=f"rope{i}-{d}") for i, N in enumerate(Ns)]
    X = cs[0].Xd
    pos = _positions(T, p0, T + d)
    n_pos = int(pos.max()) + 1
    posd = torch.from_numpy(pos).cuda()
    tab = lib.rope_table(n_pos, d, theta)
    rope = lib.rope_desc(tab, n_pos, d, posd)
    for mode in (lib.ADAPTERS_ON, lib.ADAPTERS_OFF):
        Yf = [torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
        Uf = [torch.empty((T, 16), dtype=torch.bfloat16, device="cuda") for _ in Ns]
        lib.lora_linear_fwd_group_epi([c.desc() for c in cs], X, Yf, Uf, adapters=mode, rope_mask=0b011, rope=rope,
                                      ws=cs[0].ws)
        Yu = [torch.empty_like(y) for y in Yf]
        Uu = [torch.empty_like(u) for u in Uf]
        lib.lora_linear_fwd_group([c.desc() for c in cs], X, Yu, Uu, adapters=mode, ws=cs[0].ws)
        lib.rope_apply(Yu[0], posd, nq, d, theta)
        lib.rope_apply(Yu[1], posd, nkv, d, theta)
        torch.cuda.synchronize()
        for name, a, b in zip("qkv", Yf, Yu):
            _assert_eq(name, a, b)
        for c, y, nh in zip(cs, Yf, (nq, nkv, None)):
            ref = r16(olora.forward(f32(cs[0].X), f32(c.W_hat_bits), f32(c.A), f32(c.B), c.s,
                                    mode == lib.ADAPTERS_ON)[0])
            if nh is not None:
                ref = og.rope(ref, pos, nh, d, theta)
            assert_close("Y", to_np(y), ref)


def test_group_rope_epilogue_validation(gpu):
    import torch
    T, K, d = 64, 256, 128
    cs = [Case(T, K, N, base="bf16", tag=f"ropev{i}") for i, N in enumerate((256, 192))]
    posd = torch.zeros(T, dtype=torch.int32, device="cuda")
    tab = lib.rope_table(4, d, 10000.0)
    Y = [torch.empty((T, c.N), dtype=torch.bfloat16, device="cuda") for c in cs]
    with pytest.raises(lib.LsnError):     # 192 columns are not whole heads of 128
        lib.lora_linear_fwd_group_epi([c.desc() for c in cs], cs[0].Xd, Y, adapters=False, rope_mask=0b10,
                                      rope=lib.rope_desc(tab, 4, d, posd))
    with pytest.raises(lib.LsnError):     # head width 96 is not a fused-epilogue width
        lib.lora_linear_fwd_group_epi([cs[0].desc()], cs[0].Xd, Y[:1], adapters=False, rope_mask=0b1,
                                      rope=lib.rope_desc(tab, 4, 96, posd))
    with pytest.raises(lib.LsnError):     # rope_mask names a member past n
        lib.lora_linear_fwd_group_epi([cs[0].desc()], cs[0].Xd, Y[:1], adapters=False, rope_mask=0b10,
                                      rope=lib.rope_desc(tab, 4, d, posd))
    with pytest.raises(lib.LsnError):     # a residual and a rotation on one member
        lib.lora_linear_fwd_group_epi([cs[0].desc()], cs[0].Xd, Y[:1], adapters=False, residual=[Y[1]],
                                      rope_mask=0b1, rope=lib.rope_desc(tab, 4, d, posd))


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("base", ["bf16", "nf4"])
@pytest.mark.parametrize("in_place", [False, True], ids=["separate", "in-place"])
def test_group_residual_epilogue(gpu, base, in_place):
    """Y_g = bf16(R_g + P_g) for members with a residual (the o and down projections' residual
    adds), the others plain: bit-identical to the projection then add_bf16; Y may be R."""
    import torch
    T, K = 300, 512
    Ns = [512, 256]
    print(f"case: group residual T={T} K={K} N={Ns} base={base} in_place={in_place}", flush=True)
    cs = [Case(T, K, N, base=base, tag=f"res{i}") for i, N in enumerate(Ns)]
    X = cs[0].Xd
    Rb = inputs.act_bf16(T, Ns[0], 0, "residual", T, Ns[0])
    for mode in (lib.ADAPTERS_ON, lib.ADAPTERS_OFF):
        R = bf16_dev(Rb, torch)
        Yf = [R if in_place else torch.empty((T, Ns[0]), dtype=torch.bfloat16, device="cuda"),
              torch.empty((T, Ns[1]), dtype=torch.bfloat16, device="cuda")]
        Uf = [torch.empty((T, 16), dtype=torch.bfloat16, device="cuda") for _ in Ns]
        lib.lora_linear_fwd_group_epi([c.desc() for c in cs], X, Yf, Uf, adapters=mode, residual=[R, None],
                                      ws=cs[0].ws)
        Yu = [torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
        lib.lora_linear_fwd_group([c.desc() for c in cs], X, Yu, [torch.empty_like(u) for u in Uf], adapters=mode,
                                  ws=cs[0].ws)
        lib.add_bf16(bf16_dev(Rb, torch), Yu[0], Yu[0])
        torch.cuda.synchronize()
        _assert_eq("Y residual", Yf[0], Yu[0])
        _assert_eq("Y plain", Yf[1], Yu[1])
        c = cs[0]
        P = r16(olora.forward(f32(c.X), f32(c.W_hat_bits), f32(c.A), f32(c.B), c.s, mode == lib.ADAPTERS_ON)[0])
        assert_close("Y", to_np(Yf[0]), r16(f32(Rb) + P))
    with pytest.raises(lib.LsnError):     # a residual that partially overlaps its output
        Rw = torch.empty((T + 1, Ns[0]), dtype=torch.bfloat16, device="cuda")
        lib.lora_linear_fwd_group_epi([cs[0].desc()], X, [Rw[1:]], adapters=False, residual=[Rw[:T]])


# ---------------------------------------------------------------------------------------------
SWIGLU_SHAPES = [(300, 256, 192), (300, 512, 1344), (1, 256, 128)]


@pytest.mark.parametrize("base", ["bf16", "nf4"])
@pytest.mark.parametrize("T,K,N", SWIGLU_SHAPES)
def test_swiglu_forward_epilogue(gpu, T, K, N, base):
    """M = silu(gate) up with gate and up in one launch (128 columns of each per tile):
    bit-identical to the grouped gate/up projections then swiglu_fwd; gate and up stored when
    given (and, with bf16 weights, not when they are not)."""
    import torch
    print(f"case: swiglu forward T={T} K={K} N={N} base={base}", flush=True)
    cg, cu = Case(T, K, N, base=base, tag="sw-gate"), Case(T, K, N, base=base, tag="sw-up")
    X = cg.Xd
    for mode in (lib.ADAPTERS_ON, lib.ADAPTERS_OFF):
        G, Up, M = (torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        Ug, Uu = (torch.empty((T, 16), dtype=torch.bfloat16, device="cuda") for _ in range(2))
        lib.lora_linear_fwd_swiglu(cg.desc(), cu.desc(), X, M, gate=G, up=Up, Ug=Ug, Uu=Uu, adapters=mode)
        G2, Up2, M2 = (torch.empty_like(G) for _ in range(3))
        Ug2, Uu2 = torch.empty_like(Ug), torch.empty_like(Uu)
        lib.lora_linear_fwd_group([cg.desc(), cu.desc()], X, [G2, Up2], [Ug2, Uu2], adapters=mode)
        lib.swiglu_fwd(G2, Up2, M2)
        torch.cuda.synchronize()
        _assert_eq("gate", G, G2)
        _assert_eq("up", Up, Up2)
        _assert_eq("m", M, M2)
        if mode == lib.ADAPTERS_ON:
            _assert_eq("Ug", Ug, Ug2)
            _assert_eq("Uu", Uu, Uu2)
        if base == "bf16":
            M3 = torch.empty_like(M)
            lib.lora_linear_fwd_swiglu(cg.desc(), cu.desc(), X, M3, Ug=Ug, Uu=Uu,
                                       adapters=lib.ADAPTERS_U_READY if mode == lib.ADAPTERS_ON else mode)
            torch.cuda.synchronize()
            _assert_eq("m without gate/up", M3, M)
        on = mode == lib.ADAPTERS_ON
        g = r16(olora.forward(f32(cg.X), f32(cg.W_hat_bits), f32(cg.A), f32(cg.B), cg.s, on)[0])
        u = r16(olora.forward(f32(cg.X), f32(cu.W_hat_bits), f32(cu.A), f32(cu.B), cu.s, on)[0])
        assert_close("Y", to_np(M), og.swiglu(g, u))
    if base == "nf4":
        with pytest.raises(lib.LsnError):     # NF4 weights need gate and up to be given
            lib.lora_linear_fwd_swiglu(cg.desc(), cu.desc(), X, M, adapters=False)


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["bf16", "bf16_t", "nf4"])
@pytest.mark.parametrize("T,I,H", [(300, 1344, 256), (129, 192, 512)])
def test_swiglu_backward_epilogue(gpu, T, I, H, layout):
    """The down projection's backward with the SwiGLU's backward in its dX epilogue: dgate, dup,
    dA, dB bit-identical to lora_linear_bwd (bf16 dX) then swiglu_bwd; matches the oracle."""
    import torch
    print(f"case: swiglu backward T={T} I={I} H={H} layout={layout}", flush=True)
    base = "nf4" if layout == "nf4" else "bf16"
    c = Case(T, I, H, base=base, tag="sw-down")
    gb = inputs.act_bf16(T, I, 0, "sw-bwd", "gate", T, I)
    ub = inputs.act_bf16(T, I, 0, "sw-bwd", "up", T, I)
    gate, up = bf16_dev(gb, torch), bf16_dev(ub, torch)
    transposed = layout == "bf16_t"
    W = c.w_transposed() if transposed else None
    desc = c.desc(W, transposed)
    U = torch.empty((T, 16), dtype=torch.bfloat16, device="cuda")
    lib.lora_down(c.Xd, [c.Ad], [U])
    for grad_mode in (lib.GRAD_SET, lib.GRAD_ADD):
        g0 = torch.from_numpy(c.g_init).cuda()
        dA1 = g0[: c.r * c.K].view(c.r, c.K).clone()
        dB1 = g0[c.r * c.K:].view(c.N, c.r).clone()
        dA2, dB2 = dA1.clone(), dB1.clone()
        dg1, du1 = torch.empty_like(gate), torch.empty_like(gate)
        lib.lora_linear_bwd_swiglu(desc, c.Xd, c.dYd, U, gate, up, dg1, du1, dA1, dB1, grad_mode=grad_mode, ws=c.ws)
        dm = torch.empty_like(gate)
        dg2, du2 = torch.empty_like(gate), torch.empty_like(gate)
        lib.lora_linear_bwd(desc, c.Xd, c.dYd, U, dm, dA2, dB2, dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode,
                            ws=c.ws)
        lib.swiglu_bwd(gate, up, dm, dg2, du2)
        torch.cuda.synchronize()
        for name, a, b in (("dgate", dg1, dg2), ("dup", du1, du2), ("dA", dA1, dA2), ("dB", dB1, dB2)):
            _assert_eq(name, a, b)
    dX, dA, dB, _ = c.oracle_bwd()
    dg_ref, du_ref = og.swiglu_bwd(f32(gb), f32(ub), r16(dX))
    assert_close("dX", to_np(dg1), dg_ref)
    assert_close("dX", to_np(du1), du_ref)
    g0 = c.g_init.astype(np.float64)
    assert_close("dA", to_np(dA1), g0[: c.r * c.K].reshape(c.r, c.K) + dA)
    assert_close("dB", to_np(dB1), g0[c.r * c.K:].reshape(c.N, c.r) + dB)


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_seq,S,nq,nkv,d,theta", [(2, 200, 4, 2, 128, 500000.0), (3, 130, 6, 2, 64, 1e6),
                                                    (1, 64, 2, 2, 128, 10000.0)])
def test_attention_backward_rope_epilogue(gpu, n_seq, S, nq, nkv, d, theta):
    """dq and dk rotated back as they are stored: bit-identical to attention_bwd then
    rope_apply(inverse) on dq and dk; the unrotated gradients match the oracle."""
    import torch
    print(f"case: attention bwd rope n_seq={n_seq} S={S} nq={nq} nkv={nkv} d={d}", flush=True)
    T = n_seq * S
    key = ("attn-rope", n_seq, S, nq, nkv, d)
    qb, kb, vb = (inputs.act_bf16(T, n * d, 0, *key, nm) for nm, n in (("q", nq), ("k", nkv), ("v", nkv)))
    q, k, v = (bf16_dev(b, torch) for b in (qb, kb, vb))
    dOb = inputs.act_bf16(T, nq * d, 0, *key, "dO")
    dO = bf16_dev(dOb, torch)
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, nq), dtype=torch.float32, device="cuda")
    lib.attention_fwd(q, k, v, o, lse, n_seq, nq, nkv, d)
    pos = (np.arange(T) % S).astype(np.int32)
    posd = torch.from_numpy(pos).cuda()
    tab = lib.rope_table(S, d, theta)
    ws = torch.empty(lib.attention_bwd_ws_bytes(n_seq, S, nq, nkv, d), dtype=torch.uint8, device="cuda")
    outs = [[torch.empty((T, n * d), dtype=torch.bfloat16, device="cuda") for n in (nq, nkv, nkv)] for _ in range(2)]
    lib.attention_bwd_rope(q, k, v, o, lse, dO, *outs[0], ws, n_seq, nq, nkv, d, lib.rope_desc(tab, S, d, posd))
    lib.attention_bwd(q, k, v, o, lse, dO, *outs[1], ws, n_seq, nq, nkv, d)
    lib.rope_apply(outs[1][0], posd, nq, d, theta, inverse=True)
    lib.rope_apply(outs[1][1], posd, nkv, d, theta, inverse=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), outs[0], outs[1]):
        _assert_eq(name, a, b)
    dq, dk, dv = oatt.backward(f32(qb), f32(kb), f32(vb), f32(dOb), n_seq, nq, nkv, d)
    for name, got, ref, nh in (("dq", outs[0][0], og.rope(r16(dq), pos, nq, d, theta, inverse=True), nq),
                               ("dk", outs[0][1], og.rope(r16(dk), pos, nkv, d, theta, inverse=True), nkv),
                               ("dv", outs[0][2], dv, None)):
        err = olora.rel_l2(to_np(got), ref)
        assert err <= 1e-2, f"{name}: rel L2 {err:.3e}"


# ---------------------------------------------------------------------------------------------
def test_decoder_step_fused_glue_equals_separate_kernels(gpu):
    """A training step (two layers, streamed) with the glue in the epilogues equals the same step
    with the separate glue kernels: loss, final hidden state and every dA, dB bit for bit."""
    import torch
    from layer_streamed_nf4_dequant_amd.configs import StackConfig
    from layer_streamed_nf4_dequant_amd.decoder import DecoderModel
    cfg = StackConfig("tiny-decoder", layers=2, hidden=256, kv=128, inter=640, T=600, head_dim=64, seq_len=300)
    print("case: decoder fused glue vs separate kernels", flush=True)
    res = []
    for fuse in (True, False):
        m = DecoderModel(cfg, 1024, seed=3, fuse_glue=fuse)
        m.step("streamed", check_recompute=True)
        assert all(bool(t) for t in m.recompute_ok)
        res.append((m.loss.clone(), m.x[m.L].clone(), [t.clone() for l in m.dA for t in l],
                    [t.clone() for l in m.dB for t in l]))
        m.close()
        del m
    (l1, x1, a1, b1), (l2, x2, a2, b2) = res
    _assert_eq("loss", l1, l2)
    _assert_eq("final hidden", x1, x2)
    for i, (a, b) in enumerate(zip(a1, a2)):
        _assert_eq(f"dA[{i}]", a, b)
    for i, (a, b) in enumerate(zip(b1, b2)):
        _assert_eq(f"dB[{i}]", a, b)
