"""GPU parity of causal grouped-query attention (forward and backward) against the fp64 oracle,
through the C ABI.

q, k and v are column ranges of one fused projection output [T][(n_q + 2 n_kv) d], as the fused
projection leaves them; dq, dk and dv are written into column ranges of one fused gradient.
Tolerances: o rel-L2 5e-3 (bf16 probabilities and output), lse abs 2e-4 (fp32 sums), dq, dk, dv
rel-L2 1e-2 (bf16 probabilities and score gradients). Results are bit-identical across calls.
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import inputs, lib
from oracle import attention as oatt
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


def f32(bits):
    return onf4.bf16_to_f32(bits)


def dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


class AttnCase:
    def __init__(self, n_seq, S, n_q, n_kv, d, q_scale=1.0, seed=0):
        import torch
        self.n_seq, self.S, self.n_q, self.n_kv, self.d = n_seq, S, n_q, n_kv, d
        T = n_seq * S
        self.T = T
        key = ("attn", n_seq, S, n_q, n_kv, d, q_scale)
        W = (n_q + 2 * n_kv) * d
        x = inputs.host_normal((T, W), 1.0, seed, *key, "qkv")
        x[:, : n_q * d] *= np.float32(q_scale)
        self.qkv = inputs.to_bf16_bits(x)
        self.dO = inputs.act_bf16(T, n_q * d, seed, *key, "dO")
        self.qkvd = dev_bf16(self.qkv, torch)
        self.dOd = dev_bf16(self.dO, torch)

    def slices(self, t):
        nq, nkv, d = self.n_q, self.n_kv, self.d
        return t[:, : nq * d], t[:, nq * d:(nq + nkv) * d], t[:, (nq + nkv) * d:]

    def host_qkv(self):
        return self.slices(f32(self.qkv))

    def gpu_fwd(self, pad=8):
        import torch
        q, k, v = self.slices(self.qkvd)
        # o lives in a wider buffer whose extra columns must stay untouched
        obuf = torch.full((self.T, self.n_q * self.d + pad), 7.0, dtype=torch.bfloat16, device="cuda")
        o = obuf[:, : self.n_q * self.d]
        lse = torch.empty((self.T, self.n_q), dtype=torch.float32, device="cuda")
        lib.attention_fwd(q, k, v, o, lse, self.n_seq, self.n_q, self.n_kv, self.d)
        return obuf, o, lse

    def gpu_bwd(self, o, lse):
        import torch
        q, k, v = self.slices(self.qkvd)
        g = torch.full_like(self.qkvd, float("nan"))
        dq, dk, dv = self.slices(g)
        ws = torch.empty(lib.attention_bwd_ws_bytes(self.n_seq, self.S, self.n_q, self.n_kv, self.d), dtype=torch.uint8, device="cuda")
        lib.attention_bwd(q, k, v, o, lse, self.dOd, dq, dk, dv, ws, self.n_seq, self.n_q, self.n_kv, self.d)
        return g


CASES = [  # n_seq, S, n_q, n_kv, head_dim, query scale
    (1, 64, 1, 1, 64, 1.0),        # one block
    (2, 100, 4, 2, 64, 1.0),       # ragged tail (2 blocks, 36 rows in the last)
    (3, 130, 8, 2, 128, 1.0),      # 3 blocks, groups of 4 query heads
    (1, 1, 2, 1, 128, 1.0),        # a single row
    (2, 257, 14, 2, 64, 1.0),      # Qwen2.5-0.5B heads, one row past 4 blocks
    (1, 512, 32, 8, 128, 1.0),     # Llama-3.1-8B heads
    (2, 192, 4, 1, 128, 4.0),      # sharp softmax (scores with std 4)
]


@pytest.mark.parametrize("n_seq,S,n_q,n_kv,d,qs", CASES)
def test_attention_parity(gpu, n_seq, S, n_q, n_kv, d, qs):
    import torch
    print(f"case: attention n_seq={n_seq} S={S} n_q={n_q} n_kv={n_kv} d={d} q_scale={qs}", flush=True)
    c = AttnCase(n_seq, S, n_q, n_kv, d, qs)
    obuf, o, lse = c.gpu_fwd()
    g = c.gpu_bwd(o, lse)
    torch.cuda.synchronize()
    q, k, v = c.host_qkv()
    O_ref, L_ref = oatt.forward(q, k, v, n_seq, n_q, n_kv, d)
    err_o = olora.rel_l2(host(o), O_ref)
    assert err_o <= 5e-3, f"o rel L2 {err_o:.2e}"
    assert np.abs(lse.cpu().numpy() - L_ref).max() <= 2e-4
    assert torch.equal(obuf[:, n_q * d:].float().cpu(), torch.full((c.T, 8), 7.0))
    dq_ref, dk_ref, dv_ref = oatt.backward(q, k, v, f32(c.dO), n_seq, n_q, n_kv, d)
    dq, dk, dv = (host(t) for t in c.slices(g))
    errs = {n: olora.rel_l2(a, b) for n, a, b in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref))}
    print({n: f"{e:.2e}" for n, e in errs.items()}, f"o {err_o:.2e}")
    for n, e in errs.items():
        assert e <= 1e-2, f"{n}: rel L2 {e:.2e}"


def test_attention_growing_row_maxima(gpu):
    """Scores that climb along the keys: over the first half of the sequence each 64-key block
    lifts a row's maximum by about 3 in log2 units, which the forward absorbs without rescaling
    its output (the probabilities stay below 2^8 until the maximum has moved by more than 8),
    and over the second half by about 12 per block, a rescale at every block. o and lse against
    the oracle at the usual bars, and dV = P^T dO, whose probabilities the backward rebuilds from
    that lse. (dQ and dK are not compared on this input: its keys are nearly parallel and grow
    along the sequence, so dQ = scale dS K is a difference of terms about 3000 times its size,
    and rounding dS to bf16 for the matrix cores alone moves it by 6% rel-L2 in an fp64
    computation.)"""
    import torch
    n_seq, S, n_q, n_kv, d = 1, 640, 2, 1, 64
    print(f"case: attention with growing row maxima S={S} n_q={n_q} d={d}", flush=True)
    c = AttnCase(n_seq, S, n_q, n_kv, d, seed=11)
    key = ("attn growing maxima",)
    u = inputs.host_normal((d,), 1.0, 11, *key, "u").astype(np.float64)
    u /= np.linalg.norm(u)
    j = np.arange(S, dtype=np.float64)
    # log2-domain growth per block: 64 * slope * |q.u| * scale * log2(e), with |q.u| = 8 and
    # scale = 1/8: about 92 * slope
    f = np.where(j < 320, 0.0325 * j, 0.0325 * 320 + 0.13 * (j - 320))
    q = np.tile(8.0 * u, (S, n_q))
    k = f[:, None] * u[None, :] + inputs.host_normal((S, d), 0.05, 11, *key, "k")
    v = inputs.host_normal((S, d), 1.0, 11, *key, "v")
    c.qkv = inputs.to_bf16_bits(np.concatenate([q, k, v], axis=1).astype(np.float32))
    c.qkvd = dev_bf16(c.qkv, torch)
    obuf, o, lse = c.gpu_fwd()
    g = c.gpu_bwd(o, lse)
    torch.cuda.synchronize()
    qh, kh, vh = c.host_qkv()
    O_ref, L_ref = oatt.forward(qh, kh, vh, n_seq, n_q, n_kv, d)
    err_o = olora.rel_l2(host(o), O_ref)
    assert L_ref.max() > 40.0          # the scores did climb (lse in natural-log units)
    assert err_o <= 5e-3, f"o rel L2 {err_o:.2e}"
    assert np.abs(lse.cpu().numpy() - L_ref).max() <= 2e-4
    _, _, dv_ref = oatt.backward(qh, kh, vh, f32(c.dO), n_seq, n_q, n_kv, d)
    e = olora.rel_l2(host(c.slices(g)[2]), dv_ref)
    print(f"o {err_o:.2e} dv {e:.2e}")
    assert e <= 1e-2, f"dv: rel L2 {e:.2e}"


def test_attention_bitwise_reproducible(gpu):
    import torch
    c = AttnCase(2, 257, 8, 2, 128, 1.0, seed=3)
    runs = []
    for _ in range(2):
        obuf, o, lse = c.gpu_fwd()
        g = c.gpu_bwd(o, lse)
        torch.cuda.synchronize()
        runs.append((obuf.view(torch.int16).cpu(), lse.view(torch.int32).cpu(), g.view(torch.int16).cpu()))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_attention_full_size_sampled_heads(gpu):
    """Llama-3.1-8B attention at the 8B-shaped workload's 2 sequences of 2048 rows (32 query / 8
    key-value heads of 128): the outputs of sampled sequences and key/value groups against the
    oracle run on just those rows and heads."""
    import torch
    n_seq, S, n_q, n_kv, d = 2, 2048, 32, 8, 128
    print("case: attention full size 2 x 2048, 32/8 heads, sampled", flush=True)
    c = AttnCase(n_seq, S, n_q, n_kv, d, 1.0, seed=5)
    obuf, o, lse = c.gpu_fwd()
    g = c.gpu_bwd(o, lse)
    torch.cuda.synchronize()
    q, k, v = c.host_qkv()
    grp = n_q // n_kv
    O, L = host(o), lse.cpu().numpy()
    dq, dk, dv = (host(t) for t in c.slices(g))
    dO = f32(c.dO)
    for b, gk in ((0, 0), (1, 7), (1, 4)):
        rows = slice(b * S, (b + 1) * S)
        qh = slice(gk * grp * d, (gk + 1) * grp * d)
        kh = slice(gk * d, (gk + 1) * d)
        O_ref, L_ref = oatt.forward(q[rows, qh], k[rows, kh], v[rows, kh], 1, grp, 1, d)
        assert olora.rel_l2(O[rows, qh], O_ref) <= 5e-3
        assert np.abs(L[rows, gk * grp:(gk + 1) * grp] - L_ref).max() <= 2e-4
        dq_ref, dk_ref, dv_ref = oatt.backward(q[rows, qh], k[rows, kh], v[rows, kh], dO[rows, qh], 1, grp, 1, d)
        for name, got, ref in (("dq", dq[rows, qh], dq_ref), ("dk", dk[rows, kh], dk_ref), ("dv", dv[rows, kh], dv_ref)):
            e = olora.rel_l2(got, ref)
            assert e <= 1e-2, f"seq {b} group {gk} {name}: rel L2 {e:.2e}"
