"""The decoder-layer training step (embedding, L decoder layers of RMSNorm / LoRA projections on
a streamed NF4 base / RoPE / causal grouped-query attention / SwiGLU, final norm, LM head and
cross-entropy, backward with per-layer recompute):

  * against the same chain composed from the oracle (fp64 products, the stored activations
    rounded to bf16 at the same points) on a tiny two-layer model: per-row loss and every LoRA
    gradient;
  * streamed == resident bit for bit (loss, final hidden state, every dA and dB), each layer's
    recompute equal to its forward, at the Qwen2.5-0.5B shape with four layers;
  * two micro-batches of the same rows give exactly twice every gradient;
  * the GEMMs dequantising NF4 tiles into LDS agree with the staged dequant to fp32 rounding;
  * the adapters-off reference sweep changes no training state and equals the step with B = 0.
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import lib
from layer_streamed_nf4_dequant_amd.configs import C3, StackConfig
from layer_streamed_nf4_dequant_amd.decoder import DecoderModel
from oracle import attention as oatt
from oracle import ce as oce
from oracle import glue as og
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

TINY = StackConfig("tiny-decoder", layers=2, hidden=256, kv=128, inter=512, T=192, head_dim=64, seq_len=96)
QWEN4 = StackConfig("qwen2.5-0.5b-shape", layers=24, hidden=896, kv=128, inter=4864, T=2048, head_dim=64,
                    seq_len=1024)


def r16(a):
    """Storage rounding: fp64 -> fp32 -> bf16 (nearest even) -> value."""
    return onf4.bf16_to_f32(onf4.bf16_rne(np.asarray(a, dtype=np.float32))).astype(np.float64)


def hb(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def oracle_step(m: DecoderModel):
    """The training step of the model's inputs composed from the oracle."""
    cfg, L, eps, theta = m.cfg, m.L, m.eps, m.theta
    n_seq, nq, nkv, d, s = m.n_seq, m.nq, m.nkv, m.d, cfg.scale
    ids, labels, pos = (t.cpu().numpy() for t in (m.ids, m.labels, m.positions))
    W_hat = [{n: onf4.bf16_to_f32(onf4.dequant_bf16(onf4.pack(m.base_weight(l, n).cpu().numpy())))
              for n in m.names} for l in range(L)]
    A = [{n: hb(m.A[l][m.j[n]]) for n in m.names} for l in range(L)]
    B = [{n: hb(m.B[l][m.j[n]]) for n in m.names} for l in range(L)]
    g1, g2, gf = [hb(t) for t in m.g1], [hb(t) for t in m.g2], hb(m.g_final)

    def fwd(l, n, X):
        return r16(olora.forward(X, W_hat[l][n], A[l][n], B[l][n], s)[0])

    def bwd(l, n, X, dY):
        dX, dA, dB, _ = olora.backward(X, dY, W_hat[l][n], A[l][n], B[l][n], s)
        return dX, dA, dB

    x = oce.embed(ids, hb(m.E))
    saved = []
    for l in range(L):
        n1 = r16(og.rmsnorm(x, g1[l], eps))
        q = r16(og.rope(fwd(l, "q", n1), pos, nq, d, theta))
        k = r16(og.rope(fwd(l, "k", n1), pos, nkv, d, theta))
        v = fwd(l, "v", n1)
        o = r16(oatt.forward(q, k, v, n_seq, nq, nkv, d)[0])
        h = r16(x + fwd(l, "o", o))
        n2 = r16(og.rmsnorm(h, g2[l], eps))
        gate, up = fwd(l, "gate", n2), fwd(l, "up", n2)
        mm = r16(og.swiglu(gate, up))
        y = r16(h + fwd(l, "down", mm))
        saved.append((x, n1, q, k, v, o, h, n2, gate, up, mm))
        x = y
    nf = r16(og.rmsnorm(x, gf, eps))
    # an ignored row has no loss and no gradient: the head runs on the counted rows alone
    counted = labels >= 0
    loss, dh = np.zeros(nf.shape[0]), np.zeros_like(nf)
    loss[counted], _, dh[counted] = oce.cross_entropy(nf[counted], hb(m.W_head), labels[counted],
                                                      1.0 / m.n_counted)
    dy = og.rmsnorm_bwd(x, gf, r16(dh), eps)
    grads = {}
    for l in reversed(range(L)):
        x, n1, q, k, v, o, h, n2, gate, up, mm = saved[l]
        dm, grads[(l, "down", "A")], grads[(l, "down", "B")] = bwd(l, "down", mm, r16(dy))
        dg, du = og.swiglu_bwd(gate, up, r16(dm))
        dn2 = 0.0
        for n, dY in (("gate", r16(dg)), ("up", r16(du))):
            dX, grads[(l, n, "A")], grads[(l, n, "B")] = bwd(l, n, n2, dY)
            dn2 = dn2 + dX
        dh = dy + og.rmsnorm_bwd(h, g2[l], dn2, eps)
        do, grads[(l, "o", "A")], grads[(l, "o", "B")] = bwd(l, "o", o, r16(dh))
        dq, dk, dv = oatt.backward(q, k, v, r16(do), n_seq, nq, nkv, d)
        dq = r16(og.rope(r16(dq), pos, nq, d, theta, inverse=True))
        dk = r16(og.rope(r16(dk), pos, nkv, d, theta, inverse=True))
        dn1 = 0.0
        for n, dY in (("q", dq), ("k", dk), ("v", r16(dv))):
            dX, grads[(l, n, "A")], grads[(l, n, "B")] = bwd(l, n, n1, dY)
            dn1 = dn1 + dX
        dy = dh + og.rmsnorm_bwd(x, g1[l], dn1, eps)
    return loss, grads


def test_decoder_step_matches_oracle_chain(gpu):
    print("case: tiny decoder (2 layers, H 256, 4/2 heads of 64, 2 x 96 rows, V 512) vs oracle", flush=True)
    m = DecoderModel(TINY, vocab=512, modes=("resident",))
    m.step("resident")
    loss_gpu = hb(m.loss)
    grads_gpu = {(l, n, w): hb((m.dA if w == "A" else m.dB)[l][m.j[n]]) for l in range(m.L) for n in m.names
                 for w in "AB"}
    loss_ref, grads_ref = oracle_step(m)
    counted = m.labels.cpu().numpy() >= 0
    e_loss = olora.rel_l2(loss_gpu[counted], loss_ref[counted])
    assert e_loss <= 1e-3, f"loss rel L2 {e_loss:.2e}"
    assert np.all(loss_gpu[~counted] == 0.0)
    worst = 0.0
    for key, ref in grads_ref.items():
        e = olora.rel_l2(grads_gpu[key], ref)
        worst = max(worst, e)
        assert e <= 1e-2, f"{key}: rel L2 {e:.2e}"
    print(f"loss rel L2 {e_loss:.2e}, worst gradient rel L2 {worst:.2e}")
    m.close()


QWEN2 = StackConfig("qwen2.5-0.5b-shape", layers=2, hidden=896, kv=128, inter=4864, T=2048, head_dim=64,
                    seq_len=1024)


@pytest.mark.timeout(600)
def test_decoder_step_matches_oracle_chain_qwen_width(gpu):
    """The same chain at the Qwen2.5-0.5B width (hidden 896, 14 query and 2 key/value heads of 64,
    MLP 4864, 2 x 1024-row sequences, vocabulary 151936) with two layers; the loss is taken on a
    seeded sample of 96 rows (the rest ignored), so the oracle's LM head runs on those rows only."""
    print("case: Qwen2.5-0.5B-width decoder (2 layers, H 896, 14/2 heads of 64, 2 x 1024 rows, "
          "V 151936, 96 labelled rows) vs oracle", flush=True)
    m = DecoderModel(QWEN2, vocab=151936, modes=("streamed",), label_rows=96)
    assert m.n_counted == 96
    m.step("streamed")
    loss_gpu = hb(m.loss)
    grads_gpu = {(l, n, w): hb((m.dA if w == "A" else m.dB)[l][m.j[n]]) for l in range(m.L) for n in m.names
                 for w in "AB"}
    loss_ref, grads_ref = oracle_step(m)
    counted = m.labels.cpu().numpy() >= 0
    e_loss = olora.rel_l2(loss_gpu[counted], loss_ref[counted])
    assert e_loss <= 1e-3, f"loss rel L2 {e_loss:.2e}"
    assert np.all(loss_gpu[~counted] == 0.0)
    worst = 0.0
    for key, ref in grads_ref.items():
        e = olora.rel_l2(grads_gpu[key], ref)
        worst = max(worst, e)
        assert e <= 1e-2, f"{key}: rel L2 {e:.2e}"
    print(f"loss rel L2 {e_loss:.2e}, worst gradient rel L2 {worst:.2e}")
    m.close()


def _snapshot(m):
    import torch
    out = [m.loss.view(torch.int32).clone(), m.x[m.L].view(torch.int16).clone()]
    for l in range(m.L):
        out += [t.view(torch.int32).clone() for t in m.dA[l] + m.dB[l]]
    return out


@pytest.mark.parametrize("cfg,vocab,layers", [(QWEN4, 151936, 4), (QWEN4, 151936, None), (C3, 128256, None)],
                         ids=["qwen0.5b-4-layers", "qwen0.5b-24-layers", "llama8b-32-layers"])
def test_decoder_streamed_equals_resident_and_recompute(gpu, cfg, vocab, layers):
    import torch
    print(f"case: decoder {cfg.name}, {layers or cfg.layers} layers, V {vocab}, streamed vs resident", flush=True)
    m = DecoderModel(cfg, vocab=vocab, layers=layers, modes=("streamed", "resident"))
    m.step("resident", check_recompute=True)
    assert all(bool(f) for f in m.recompute_ok)
    ref = _snapshot(m)
    for t in m.dA[0] + m.dB[0]:
        t.fill_(float("nan"))
    m.step("streamed", check_recompute=True)
    assert all(bool(f) for f in m.recompute_ok)
    got = _snapshot(m)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), f"tensor {i} differs between streamed and resident"
    assert np.isfinite(m.mean_loss()) and abs(m.mean_loss() - np.log(vocab)) < 1.5
    stats = m.pool.stats()
    assert stats["bytes_copied"] == 2 * m.L * m.image_bytes
    m.close()


def test_decoder_gradient_accumulation(gpu):
    import torch
    m = DecoderModel(TINY, vocab=512, modes=("streamed",))
    m.step("streamed")
    one = [t.clone() for l in range(m.L) for t in m.dA[l] + m.dB[l]]
    m.step("streamed", micro_batches=2)
    two = [t for l in range(m.L) for t in m.dA[l] + m.dB[l]]
    for a, b in zip(one, two):
        assert torch.equal(2 * a, b)
    m.close()



def test_decoder_fused_dequant_matches_staged(gpu):
    """The GEMMs that dequantise NF4 tiles into LDS ("fused") against the staged dequant: the
    forward GEMMs and every single-projection backward see the same bf16 operands, so the
    forward (and the loss) is identical; only the grouped backward's input-gradient sum runs in
    another order (member by member). That fp32 rounding difference can flip the bf16 rounding
    of an activation gradient further down (one element by 2^-8), and such flips travel through
    the layers below. Measured (deterministic, the same on every box): the top layer's gate, up
    and down gradients, computed before the first differing sum, are bit-identical; its q, k, v
    and o gradients differ by 1e-6 to 4e-4 and the bottom layer's by up to 7.4e-4 rel-L2. The
    bar is 2e-3 (a fifth of the oracle bar)."""
    import torch
    res = {}
    for dq in ("staged", "fused"):
        m = DecoderModel(TINY, vocab=512, modes=("resident",), dequant=dq)
        m.step("resident")
        res[dq] = (hb(m.loss), [hb(t) for l in range(m.L) for t in m.dA[l] + m.dB[l]])
        m.close()
    assert np.array_equal(res["fused"][0], res["staged"][0])
    errs = [olora.rel_l2(a, b) for a, b in zip(res["fused"][1], res["staged"][1])]
    # per layer (bottom first), the dA then dB of q, k, v, o, gate, up, down: the top layer's
    # down/gate/up gradients come before the first differing sum and agree bit for bit
    n = len(errs) // TINY.layers
    for l in range(TINY.layers):
        print(f"  layer {l}: dA/dB rel-L2 fused vs staged " + " ".join(f"{e:.1e}" for e in errs[l * n:(l + 1) * n]),
              flush=True)
    top = errs[(TINY.layers - 1) * n:]
    assert all(top[j] == 0.0 for j in (4, 5, 6, 11, 12, 13))   # gate, up, down: dA and dB
    assert max(errs) <= 2e-3
    torch.cuda.synchronize()


def test_decoder_reference_sweep(gpu):
    """The adapters-off reference sweep (DPO-style objectives): it changes no training state,
    streamed == resident on its per-row loss, it matches the oracle chain with the adapters'
    contribution removed, and with every B zeroed the adapted step's loss equals it bit for bit."""
    import torch
    m = DecoderModel(TINY, vocab=512, modes=("streamed", "resident"))
    m.step("streamed")
    plain = _snapshot(m)
    m.step("streamed", reference=True)
    for a, b in zip(plain, _snapshot(m)):
        assert torch.equal(a, b)
    ref = m.loss_ref.clone()
    m.step("resident", reference=True)
    assert torch.equal(m.loss_ref.view(torch.int32), ref.view(torch.int32))
    for l in range(m.L):
        for t in m.B[l]:
            t.zero_()
    m.step("resident")
    assert torch.equal(m.loss.view(torch.int32), ref.view(torch.int32))
    loss_oracle, _ = oracle_step(m)      # B = 0: the oracle's adapters add nothing
    counted = m.labels.cpu().numpy() >= 0
    assert olora.rel_l2(hb(ref)[counted], loss_oracle[counted]) <= 1e-3
    m.close()
