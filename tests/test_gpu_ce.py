"""GPU parity of the resident ends through the C ABI: cross-entropy through the frozen LM head
(chunked over rows) against the oracle, bit-identical across chunk sizes, at the Llama-3.1-8B
head's full size on sampled rows, and the embedding lookup bit-exact. Tolerances: loss within
2e-5 relative per row (fp32 logits over bf16 inputs); dh relative L2 5e-3 (the logit gradients
are rounded to bf16 before the product, as dX's inputs are)."""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import inputs, lib
from lora_cases import to_np
from oracle import ce as oce
from oracle import lora as olora
from oracle.nf4 import bf16_to_f32

pytestmark = pytest.mark.gpu


def _case(T, H, V, seed=0, ignored=()):
    import torch
    key = ("ce", T, H, V)
    h_bits = inputs.act_bf16(T, H, seed, *key, "h")
    w_bits = inputs.to_bf16_bits(inputs.host_normal((V, H), 0.02, seed, *key, "W"))
    labels = inputs.host_rng(seed, *key, "labels").integers(0, V, T).astype(np.int32)
    for i, v in ignored:
        labels[i] = v
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    return h_bits, w_bits, labels, dev(h_bits), dev(w_bits), torch.from_numpy(labels).cuda()


def _run(h, W, lab, scale, chunk):
    import torch
    T, H = h.shape
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    dh = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lib.lm_head_ce_ws_bytes(chunk, H, W.shape[0]), dtype=torch.uint8, device="cuda")
    lib.lm_head_ce(h, W, lab, scale, loss, dh, chunk, ws)
    torch.cuda.synchronize()
    return loss, dh


@pytest.mark.parametrize("T,H,V", [(300, 256, 1088), (64, 64, 64), (129, 512, 4096)])
def test_ce_matches_oracle_and_is_chunk_invariant(gpu, T, H, V):
    import torch
    print(f"case: lm_head_ce T={T} H={H} V={V}", flush=True)
    h_bits, w_bits, labels, h, W, lab = _case(T, H, V, ignored=[(1, -100), (T - 1, V + 5)])
    n = int(((labels >= 0) & (labels < V)).sum())
    loss, dh = _run(h, W, lab, 1.0 / n, chunk=T)
    lo, _, dho = oce.cross_entropy(bf16_to_f32(h_bits), bf16_to_f32(w_bits), labels, 1.0 / n)
    got = to_np(loss).astype(np.float64)
    assert got[1] == 0 and got[T - 1] == 0 and np.all(to_np(dh)[[1, T - 1]] == 0)
    np.testing.assert_allclose(got, lo, rtol=2e-5, atol=1e-6)
    err = olora.rel_l2(to_np(dh), dho)
    print(f"  dh rel-L2 {err:.2e}", flush=True)
    assert err < 5e-3
    for chunk in (1, 17, 64, 4 * T):
        l2, d2 = _run(h, W, lab, 1.0 / n, chunk)
        assert torch.equal(l2.view(torch.int32), loss.view(torch.int32)), chunk
        assert torch.equal(d2.view(torch.int16), dh.view(torch.int16)), chunk


def test_ce_full_size_llama_head_sampled_rows(gpu):
    """T = 4096 rows through the Llama-3.1-8B head (H = 4096, V = 128256) in chunks of 512,
    checked on sampled rows (every row's loss and dh depend on that row alone)."""
    import torch
    T, H, V = 4096, 4096, 128256
    print(f"case: lm_head_ce full size T={T} H={H} V={V}", flush=True)
    h_bits, w_bits, labels, h, W, lab = _case(T, H, V)
    loss, dh = _run(h, W, lab, 1.0 / T, chunk=512)
    rows = np.sort(inputs.host_rng(0, "ce rows").choice(T, 12, replace=False))
    lo, _, dho = oce.cross_entropy(bf16_to_f32(h_bits[rows]), bf16_to_f32(w_bits), labels[rows], 1.0 / T)
    np.testing.assert_allclose(to_np(loss).astype(np.float64)[rows], lo, rtol=2e-5, atol=1e-6)
    err = olora.rel_l2(to_np(dh)[rows], dho)
    print(f"  dh rel-L2 on sampled rows {err:.2e}", flush=True)
    assert err < 5e-3
    assert np.isfinite(to_np(loss)).all()


def test_ce_argument_validation(gpu):
    import torch
    _, _, _, h, W, lab = _case(64, 64, 128)
    loss = torch.empty(64, dtype=torch.float32, device="cuda")
    dh = torch.empty((64, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lib.lm_head_ce_ws_bytes(64, 64, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.LsnError):          # workspace too small
        lib.lm_head_ce(h, W, lab, 1.0, loss, dh, 64, ws[:1024])
    with pytest.raises(lib.LsnError):          # dh overlapping h
        lib.lm_head_ce(h, W, lab, 1.0, loss, h, 64, ws)
    with pytest.raises(lib.LsnError) as e:     # H not a multiple of 64
        lib.lm_head_ce(h[:, :48].contiguous(), W[:, :48].contiguous(), lab, 1.0, loss, dh, 64, ws)
    assert e.value.status == lib.LSN_E_ARG


def test_embedding_gather_is_a_row_copy(gpu):
    import torch
    V, H, T = 1000, 4096, 257
    E = inputs.device_normal((V, H), 0.02, 0, "emb", "E", dtype=torch.bfloat16)
    ids_np = inputs.host_rng(0, "emb", "ids").integers(0, V, T).astype(np.int32)
    ids_np[[3, 100]] = [-1, V]
    ids = torch.from_numpy(ids_np).cuda()
    X = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.embedding_gather(ids, E, X, bad)
    torch.cuda.synchronize()
    want = oce.embed(ids_np, E.view(torch.int16).cpu().numpy())
    assert np.array_equal(X.view(torch.int16).cpu().numpy(), want)
    assert int(bad.item()) == 2
