"""GPU parity of the decoder-layer glue (RMSNorm, rotary embedding, SwiGLU; forward and backward)
against the fp64 oracle, through the C ABI, and a chained MLP block (RMSNorm -> gate/up LoRA
projections on NF4 bases -> SwiGLU -> down projection, forward and backward, with the residual
gradient) against the same chain composed from the oracle.

Per-element bounds for the glue kernels: a bf16 output is the fp32 value rounded to nearest,
so |got - ref| <= 2^-8 |ref| plus the fp32 arithmetic error, bounded below for each formula.
The chain is checked by relative L2 (outputs 5e-3, adapter gradients 1e-2): the oracle rounds
the stored activations to bf16 at the same points but does its products in fp64.
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import inputs, lib
from oracle import glue as og
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -8   # bf16 rounding bound, relative


def f32(bits):
    return onf4.bf16_to_f32(bits)


def bf16_round(a):
    """The oracle's storage rounding: fp64 -> fp32 -> bf16 (nearest even) -> value."""
    return f32(onf4.bf16_rne(np.asarray(a, dtype=np.float32)))


def dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def assert_within(name, got, ref, bound):
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} elements beyond the bound; worst at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)}: got "
                           f"{got.flat[np.argmax(err - bound)]} want {ref.flat[np.argmax(err - bound)]}")


def activations(T, H, seed, *key):
    """bf16 rows of N(0,1) with some rows scaled down to 1e-3 (where eps matters), some up by 30,
    and one all-zero row."""
    x = inputs.host_normal((T, H), 1.0, seed, *key, "x")
    scale = np.ones((T, 1), np.float32)
    scale[1::7] = 1e-3
    scale[3::11] = 30.0
    x = x * scale
    if T > 5:
        x[5] = 0.0
    return inputs.to_bf16_bits(x)


def gain(H, seed, *key):
    return inputs.to_bf16_bits(1.0 + inputs.host_normal((H,), 0.1, seed, *key, "gain"))


# one workgroup per row of 64, 128 or 256 threads (the row's 16-byte chunks rounded up to waves)
RMS_SHAPES = [(1, 8, 1e-5), (300, 896, 1e-6), (257, 4096, 1e-5), (7, 2056, 1e-5), (64, 5120, 1e-6),
              (33, 1024, 1e-5), (5, 520, 1e-6), (9, 512, 1e-5)]


@pytest.mark.parametrize("T,H,eps", RMS_SHAPES)
def test_rmsnorm_fwd_parity(gpu, T, H, eps):
    import torch
    print(f"case: rmsnorm_fwd T={T} H={H} eps={eps}", flush=True)
    xb, gb = activations(T, H, 0, "rms", T, H), gain(H, 0, "rms", H)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    lib.rmsnorm_fwd(dev_bf16(xb, torch), dev_bf16(gb, torch), eps, y, rstd)
    torch.cuda.synchronize()
    x, g = f32(xb), f32(gb)
    ref = og.rmsnorm(x, g, eps)
    assert_within("y", host(y), ref, (U8 + 2e-5) * np.abs(ref))
    r_ref = 1.0 / og.rms(x, eps)
    assert_within("rstd", host(rstd), r_ref, 4e-6 * r_ref)


@pytest.mark.parametrize("accumulate", [False, True], ids=["set", "add"])
@pytest.mark.parametrize("T,H,eps", RMS_SHAPES)
def test_rmsnorm_bwd_parity(gpu, T, H, eps, accumulate):
    import torch
    print(f"case: rmsnorm_bwd T={T} H={H} eps={eps} accumulate={accumulate}", flush=True)
    key = ("rmsb", T, H)
    xb, gb = activations(T, H, 0, *key), gain(H, 0, *key)
    dy = inputs.host_normal((T, H), 1.0, 0, *key, "dy")
    dx0 = inputs.host_normal((T, H), 1.0, 0, *key, "dx0")
    xd, gd = dev_bf16(xb, torch), dev_bf16(gb, torch)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    lib.rmsnorm_fwd(xd, gd, eps, y, rstd)
    dx = torch.from_numpy(dx0.copy()).cuda() if accumulate else torch.full((T, H), float("nan"), device="cuda")
    dx16 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    lib.rmsnorm_bwd(xd, gd, rstd, torch.from_numpy(dy).cuda(), dx, accumulate=accumulate, dx_bf16=dx16)
    torch.cuda.synchronize()
    # the bf16 copy is the stored fp32 gradient rounded to nearest even
    np.testing.assert_array_equal(bits(dx16).view(np.uint16), onf4.bf16_rne(dx.cpu().numpy()))
    x, g, dy64 = f32(xb), f32(gb), dy.astype(np.float64)
    ref = og.rmsnorm_bwd(x, g, dy64, eps) + (dx0 if accumulate else 0.0)
    # fp32 error: the first term to a few ulps, the row sum to ~30 ulps of the sum of |terms|
    r = 1.0 / og.rms(x, eps)[:, None]
    t2 = np.abs(x) * r ** 3 * np.abs(g * dy64 * x).sum(axis=-1, keepdims=True) / H
    bound = 3e-5 * (r * np.abs(g * dy64) + t2) + (1e-6 * np.abs(ref) if accumulate else 0.0) + 1e-30
    assert_within("dx", host(dx), ref, bound)


ROPE_CASES = [  # n_q, n_kv, head_dim, theta, T, first position, extra columns per row
    (32, 8, 128, 500000.0, 300, 0, 0),        # vector form: q one row per workgroup, k four rows
    (14, 2, 64, 1000000.0, 129, 7000, 0),     # a last workgroup with fewer rows than the others
    (4, 4, 512, 10000.0, 33, 123, 0),
    (40, 8, 128, 500000.0, 3000, 0, 0),       # more head chunks per row than threads: two rounds
    (1, 1, 512, 10000.0, 9, 3, 0),            # rows per workgroup capped by the LDS for their angles
    (1, 1, 2, 10000.0, 1, 8191, 0),           # scalar form (head width 2)
    (3, 1, 16, 10000.0, 17, 5, 4),            # scalar form (row stride not a multiple of 8)
]


def _rope_bound(ref, x_pairs_abs, pos):
    E = (pos[:, None] * 2.5e-7 + 1e-6) * x_pairs_abs
    return U8 * (np.abs(ref) + E) + E + 1e-30


def _pair_abs(x, n_heads, d):
    x = np.abs(x).reshape(x.shape[0], n_heads, d)
    h = d // 2
    s = x[..., :h] + x[..., h:]
    return np.concatenate([s, s], axis=-1).reshape(x.shape[0], n_heads * d)


@pytest.mark.parametrize("inverse", [False, True], ids=["fwd", "inverse"])
@pytest.mark.parametrize("nq,nkv,d,theta,T,p0,pad", ROPE_CASES)
def test_rope_parity_on_fused_qkv(gpu, nq, nkv, d, theta, T, p0, pad, inverse):
    """q and k are rotated in place inside a fused [T][(nq + 2 nkv) d] projection output by two
    calls on column offsets; v (and q's and k's neighbours) stay bit-identical."""
    import torch
    print(f"case: rope nq={nq} nkv={nkv} d={d} T={T} p0={p0} pad={pad} inverse={inverse}", flush=True)
    W = (nq + 2 * nkv) * d + pad
    xb = inputs.act_bf16(T, W, 0, "rope", nq, nkv, d, T)
    pos = (p0 + np.arange(T)).astype(np.int32)
    if T > 2:
        pos[T // 2] = 0
    xd = dev_bf16(xb, torch)
    posd = torch.from_numpy(pos).cuda()
    lib.rope_apply(xd[:, : nq * d], posd, nq, d, theta, inverse)
    lib.rope_apply(xd[:, nq * d:(nq + nkv) * d], posd, nkv, d, theta, inverse)
    torch.cuda.synchronize()
    got = host(xd)
    x = f32(xb)
    for name, c0, nh in (("q", 0, nq), ("k", nq * d, nkv)):
        xs = x[:, c0:c0 + nh * d]
        ref = og.rope(xs, pos, nh, d, theta, inverse)
        assert_within(name, got[:, c0:c0 + nh * d], ref, _rope_bound(ref, _pair_abs(xs, nh, d), pos.astype(np.float64)))
    v0 = (nq + nkv) * d
    np.testing.assert_array_equal(bits(xd)[:, v0:], xb.view(np.int16)[:, v0:])


def _swiglu_inputs(n, seed, *key):
    g = inputs.host_normal((n,), 2.0, seed, *key, "g")
    special = [0.0, -0.0, 1.0, -1.0, -1.278, 30.0, -30.0, 88.0, -88.0, 100.0, -100.0, 300.0, -300.0,
               1e-3, -1e-3, 5.0]
    g[:min(n, 16)] = special[:min(n, 16)]
    u = inputs.host_normal((n,), 1.0, seed, *key, "u")
    dm = inputs.host_normal((n,), 1.0, seed, *key, "dm")
    return tuple(inputs.to_bf16_bits(a) for a in (g, u, dm))


@pytest.mark.parametrize("n", [8, 4864 * 37, 14336 * 5 + 8])
def test_swiglu_parity(gpu, n):
    import torch
    print(f"case: swiglu n={n}", flush=True)
    gb, ub, dmb = _swiglu_inputs(n, 0, "swiglu", n)
    gd, ud, dmd = (dev_bf16(a, torch) for a in (gb, ub, dmb))
    m = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dg, du = torch.empty_like(m), torch.empty_like(m)
    lib.swiglu_fwd(gd, ud, m)
    lib.swiglu_bwd(gd, ud, dmd, dg, du)
    torch.cuda.synchronize()
    g, u, dm = f32(gb), f32(ub), f32(dmb)
    ref = og.swiglu(g, u)
    assert_within("m", host(m), ref, (U8 + 1e-6) * np.abs(ref) + 1e-30)
    dg_ref, du_ref = og.swiglu_bwd(g, u, dm)
    s = og.sigmoid(g)
    E = 1e-5 * np.abs(dm * u * s) * (1.0 + np.abs(g))
    assert_within("dg", host(dg), dg_ref, U8 * (np.abs(dg_ref) + E) + E + 1e-30)
    assert_within("du", host(du), du_ref, (U8 + 1e-6) * np.abs(du_ref) + 1e-30)


def test_glue_bitwise_reproducible(gpu):
    """Two runs of every glue kernel on the same inputs give the same bits."""
    import torch
    T, H, n = 257, 4096, 4864 * 37
    xb, gb = activations(T, H, 1, "rep"), gain(H, 1, "rep")
    dy = torch.from_numpy(inputs.host_normal((T, H), 1.0, 1, "rep", "dy")).cuda()
    sg, su, sdm = (dev_bf16(a, torch) for a in _swiglu_inputs(n, 1, "rep"))
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        xd, gd = dev_bf16(xb, torch), dev_bf16(gb, torch)
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        rstd = torch.empty(T, dtype=torch.float32, device="cuda")
        dx = torch.empty((T, H), dtype=torch.float32, device="cuda")
        lib.rmsnorm_fwd(xd, gd, 1e-5, y, rstd)
        lib.rmsnorm_bwd(xd, gd, rstd, dy, dx)
        lib.rope_apply(xd, pos, 32, 128, 500000.0)
        m, dg, du = (torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(3))
        lib.swiglu_fwd(sg, su, m)
        lib.swiglu_bwd(sg, su, sdm, dg, du)
        torch.cuda.synchronize()
        outs.append([bits(t) for t in (y, rstd, dx, xd, m, dg, du)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


class MlpBlock:
    """One gated MLP block of a decoder layer on NF4 bases with LoRA adapters on all three
    projections: xn = RMSNorm(x), m = silu(xn Wg'^T) * (xn Wu'^T), d = m Wd'^T, out = x + d,
    where W' x = W x + s B A x."""

    def __init__(self, T, H, I, r=16, s=2.0, eps=1e-5, seed=0):
        import torch
        self.T, self.H, self.I, self.r, self.s, self.eps = T, H, I, r, s, eps
        key = ("mlp", T, H, I, r)
        self.x = activations(T, H, seed, *key)
        self.g = gain(H, seed, *key)
        self.dout = inputs.act_bf16(T, H, seed, *key, "dout")
        self.proj = {}
        for name, K, N in (("gate", H, I), ("up", H, I), ("down", I, H)):
            W = inputs.weight_f32(N, K, seed, *key, name)
            self.proj[name] = {
                "K": K, "N": N,
                "W_hat": f32(onf4.dequant_bf16(onf4.pack(W))),
                "A": inputs.lora_A_bf16(r, K, seed, *key, name),
                "B": inputs.lora_B_bf16(N, r, seed, *key, name),
                "Wd": lib.nf4_pack(torch.from_numpy(W).cuda()),
            }

    def oracle(self):
        P, s = self.proj, self.s
        x, g = f32(self.x), f32(self.g)

        def fwd(p, X):
            return olora.forward(X, p["W_hat"], f32(p["A"]), f32(p["B"]), s)[0]

        def bwd(p, X, dY):
            dX, dA, dB, _ = olora.backward(X, dY, p["W_hat"], f32(p["A"]), f32(p["B"]), s)
            return dX, dA, dB

        xn = bf16_round(og.rmsnorm(x, g, self.eps))
        gate, up = bf16_round(fwd(P["gate"], xn)), bf16_round(fwd(P["up"], xn))
        m = bf16_round(og.swiglu(gate, up))
        d = fwd(P["down"], m)
        dout = f32(self.dout)
        dm, dA_d, dB_d = bwd(P["down"], m, dout)
        dgt, dup = og.swiglu_bwd(gate, up, bf16_round(dm))
        dxg, dA_g, dB_g = bwd(P["gate"], xn, bf16_round(dgt))
        dxu, dA_u, dB_u = bwd(P["up"], xn, bf16_round(dup))
        dx = dout + og.rmsnorm_bwd(x, g, dxg + dxu, self.eps)
        return {"d": d, "dx": dx, "dA_gate": dA_g, "dB_gate": dB_g, "dA_up": dA_u, "dB_up": dB_u,
                "dA_down": dA_d, "dB_down": dB_d}

    def gpu(self):
        import torch
        T, H, I, r = self.T, self.H, self.I, self.r
        bf = dict(dtype=torch.bfloat16, device="cuda")
        P = self.proj
        dev = {n: (dev_bf16(p["A"], torch), dev_bf16(p["B"], torch)) for n, p in P.items()}
        desc = {n: lib.linear_desc(T, p["K"], p["N"], r, self.s, p["Wd"], *dev[n]) for n, p in P.items()}
        ws = torch.empty(max(lib.group_ws_bytes([desc["gate"], desc["up"]]), lib.ws_bytes(T, I, H, r), 256),
                         dtype=torch.uint8, device="cuda")
        x, g, dout = dev_bf16(self.x, torch), dev_bf16(self.g, torch), dev_bf16(self.dout, torch)
        # forward
        xn, rstd = torch.empty((T, H), **bf), torch.empty(T, dtype=torch.float32, device="cuda")
        lib.rmsnorm_fwd(x, g, self.eps, xn, rstd)
        gate, up = torch.empty((T, I), **bf), torch.empty((T, I), **bf)
        Ug, Uu, Ud = (torch.empty((T, r), **bf) for _ in range(3))
        lib.lora_linear_fwd_group([desc["gate"], desc["up"]], xn, [gate, up], [Ug, Uu], ws=ws)
        m = torch.empty((T, I), **bf)
        lib.swiglu_fwd(gate, up, m)
        d = torch.empty((T, H), **bf)
        lib.lora_linear_fwd(desc["down"], m, d, Ud, ws=ws)
        # backward
        grads = {n: (torch.empty((r, p["K"]), dtype=torch.float32, device="cuda"),
                     torch.empty((p["N"], r), dtype=torch.float32, device="cuda")) for n, p in P.items()}
        dm = torch.empty((T, I), **bf)
        lib.lora_linear_bwd(desc["down"], m, dout, Ud, dm, *grads["down"], dx_mode=lib.DX_BF16_SET,
                            grad_mode=lib.GRAD_SET, ws=ws)
        dgt, dup = torch.empty((T, I), **bf), torch.empty((T, I), **bf)
        lib.swiglu_bwd(gate, up, dm, dgt, dup)
        dxn = torch.empty((T, H), dtype=torch.float32, device="cuda")
        lib.lora_linear_bwd_group([desc["gate"], desc["up"]], xn, [dgt, dup], [Ug, Uu], dxn,
                                  [grads["gate"][0], grads["up"][0]], [grads["gate"][1], grads["up"][1]],
                                  dx_mode=lib.DX_F32_SET, grad_mode=lib.GRAD_SET, ws=ws)
        dx = dout.float()          # the residual branch's gradient
        lib.rmsnorm_bwd(x, g, rstd, dxn, dx, accumulate=True)
        torch.cuda.synchronize()
        out = {"d": d, "dx": dx}
        for n in P:
            out[f"dA_{n}"], out[f"dB_{n}"] = grads[n]
        return {k: host(v) for k, v in out.items()}


@pytest.mark.parametrize("T,H,I", [(300, 256, 704), (129, 896, 4864)])
def test_mlp_block_chain_parity(gpu, T, H, I):
    print(f"case: MLP block chain T={T} H={H} I={I}", flush=True)
    blk = MlpBlock(T, H, I)
    got, want = blk.gpu(), blk.oracle()
    errs = {}
    for k in want:
        tol = 5e-3 if k in ("d", "dx") else 1e-2
        errs[k] = olora.rel_l2(got[k], want[k])
        assert errs[k] <= tol, f"{k}: rel L2 {errs[k]:.3e} > {tol:.0e}"
    print({k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("n", [8, 4096 * 7 + 8])
def test_residual_add_and_conversions_bit_exact(gpu, n):
    """add_bf16 is bf16(fl32(a + b)); fp32 -> bf16 rounds to nearest even; bf16 -> fp32 is exact.
    Also in place (out = a)."""
    import torch
    a = inputs.to_bf16_bits(inputs.host_normal((n,), 3.0, 0, "add", n, "a"))
    b = inputs.to_bf16_bits(inputs.host_normal((n,), 1e-3, 0, "add", n, "b"))   # large exponent gaps
    want = onf4.bf16_rne(f32(a) + f32(b))                  # fp32 sum, then one rounding
    ad, bd = dev_bf16(a, torch), dev_bf16(b, torch)
    out = torch.empty_like(ad)
    lib.add_bf16(ad, bd, out)
    lib.add_bf16(ad, bd, ad)                               # in place
    x = inputs.host_normal((n,), 10.0, 0, "cvt", n)
    xd = torch.from_numpy(x).cuda()
    xb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    lib.convert(xd, xb)
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    lib.convert(xb, back)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out).view(np.uint16), want)
    np.testing.assert_array_equal(bits(ad).view(np.uint16), want)
    np.testing.assert_array_equal(bits(xb).view(np.uint16), onf4.bf16_rne(x))
    np.testing.assert_array_equal(back.cpu().numpy(), f32(onf4.bf16_rne(x)))
