"""The exactness protocol on the GPU: the streamed stack must be bit-identical to a resident run
of the same numerics, forward outputs and every LoRA gradient tensor checked separately
("Exact Layer Streaming", Abstract; Soup v0.73.0 benchmarks README, reading conventions), with
same-process controls: planted pool defects must break the backward while the forward stays
exact, and the aliasing audit must flag them. The stack's parity with the oracle is in
test_gpu_stack_oracle.py.
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import configs, inputs, lib
from layer_streamed_nf4_dequant_amd.configs import PROJ_INPUT
from layer_streamed_nf4_dequant_amd.stack import Stack

pytestmark = pytest.mark.gpu


def snapshot(st):
    import torch
    torch.cuda.synchronize()
    checks = {k: int(v.item()) for k, v in st.checks.items()}
    grads = [[(a.clone(), b.clone()) for a, b in zip(dA, dB)] for dA, dB in zip(st.dA, st.dB)]
    st.checks = {}
    return checks, grads


def compare(ref, got):
    """Returns (forward_equal, recompute_equal, dx_equal, n_grad_tensors_equal, n_grad_tensors)."""
    import torch
    (rc, rg), (gc, gg) = ref, got
    fwd = all(rc[k] == gc[k] for k in rc if k[0] == "fwd")
    re = all(rc[k] == gc[k] for k in rc if k[0] == "re")
    dx = all(rc[k] == gc[k] for k in rc if k[0] == "dx")
    eq = n = 0
    for lr, lg in zip(rg, gg):
        for (a1, b1), (a2, b2) in zip(lr, lg):
            eq += int(torch.equal(a1.view(torch.int32), a2.view(torch.int32)))
            eq += int(torch.equal(b1.view(torch.int32), b2.view(torch.int32)))
            n += 2
    return fwd, re, dx, eq, n


def recompute_matches_forward(checks, L, n_proj):
    return all(checks[("fwd", l, j)] == checks[("re", l, j)] for l in range(L) for j in range(n_proj))


def test_toy_8b_shapes_exactness_and_controls(gpu):
    """Three 8B-shaped layers: streamed (2, 1 and 3 slots; KEEP_AT_TURN; audit on; from pinned
    host memory and from a file through the pool's file tier) equals resident bit for bit; each
    planted defect leaves the forward exact but breaks gradients, and the audit reports it."""
    cfg = configs.C3
    print("case: 3-layer 8B-shaped toy", flush=True)
    st = Stack(cfg, modes=("streamed", "resident"), record=True, layers=3)
    st.step("resident")
    ref = snapshot(st)
    assert recompute_matches_forward(ref[0], 3, 7)
    variants = [("2 slots", 0, None, "ram"), ("1 slot", 0, 1, "ram"), ("3 slots", 0, 3, "ram"),
                ("keep at turn", lib.POOL_KEEP_AT_TURN, 2, "ram"), ("audit", lib.POOL_AUDIT, 2, "ram"),
                ("file", 0, 2, "file"), ("file, audit", lib.POOL_AUDIT, 2, "file"),
                ("file, 1 slot, keep at turn", lib.POOL_KEEP_AT_TURN, 1, "file"),
                ("file, O_DIRECT", 0, 2, "file direct"), ("file, O_DIRECT, audit", lib.POOL_AUDIT, 2, "file direct")]
    for name, flags, n_slots, source in variants:
        print(f"  variant {name}", flush=True)
        direct = source == "file direct"
        if direct and not _direct_io_supported(st):
            print("    (skipped: no O_DIRECT on this file system)", flush=True)
            continue
        st.reset_pool(flags, n_slots, source.split()[0], direct=direct)
        st.step("streamed")
        if flags & lib.POOL_AUDIT:
            st.pool.audit()
        fwd, re, dx, eq, n = compare(ref, snapshot(st))
        assert fwd and re and dx and eq == n, (name, fwd, re, dx, eq, n)
    for name, fault, source in (("stale re-fetch", lib.FAULT_STALE_REFETCH, "ram"),
                                ("wrong slot", lib.FAULT_WRONG_SLOT, "ram"),
                                ("stale re-fetch, file", lib.FAULT_STALE_REFETCH, "file")):
        print(f"  control {name}", flush=True)
        st.reset_pool(fault, 2, source)
        st.step("streamed")
        got = snapshot(st)
        fwd, re, dx, eq, n = compare(ref, got)
        assert fwd, f"{name}: the forward must stay exact"
        assert eq < n and not re and not dx, \
            f"{name}: the planted defect must break the backward ({eq}/{n} gradient tensors equal)"
        assert not recompute_matches_forward(got[0], 3, 7)
        st.reset_pool(fault | lib.POOL_AUDIT, 2, source)
        st.step("streamed")
        with pytest.raises(lib.LsnError) as e:
            st.pool.audit()
        assert e.value.status == lib.LSN_E_AUDIT
        snapshot(st)
    st.close()


def _direct_io_supported(st) -> bool:
    import os
    path = st.write_image_file()
    try:
        fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
    except OSError:
        return False
    os.close(fd)
    return True


def test_auto_source_streams_from_the_file_tier(gpu):
    """source="auto" with a host budget too small for the pinned images: the stack keeps its base
    in the file tier (no pinned images), and the streamed step equals the resident one bit for bit."""
    cfg = configs.C3
    L = 4
    print(f"case: {L}-layer 8B-shaped toy, auto source with a small host budget", flush=True)
    from layer_streamed_nf4_dequant_amd.stack import predict_host_bytes
    f = predict_host_bytes(cfg, "file", layers=L)
    budget = f["pinned"] + f["setup_extra"]          # enough for the file tier, not for L pinned images
    assert budget < predict_host_bytes(cfg, "ram", layers=L)["pinned"]
    st = Stack(cfg, modes=("streamed", "resident"), record=True, layers=L, source="auto", host_budget=budget)
    assert st.source == "file" and st.host_images is None and st.image_file is not None
    st.step("resident")
    ref = snapshot(st)
    st.step("streamed")
    fwd, re, dx, eq, n = compare(ref, snapshot(st))
    assert fwd and re and dx and eq == n == 2 * 7 * L
    assert st.pool.stats()["copies"] == 2 * L
    st.close()


def test_staged_w_equals_staged_transposed(gpu):
    """Three 8B-shaped layers: the backward on the staged W [N][K] (the dX GEMM reads it
    reduction-major) and on a staged W^T [K][N] give identical bits: forward, recompute and dX
    checksums and every LoRA gradient tensor."""
    cfg = configs.C3
    print("case: 3-layer 8B-shaped toy, staged W vs staged W^T", flush=True)
    runs = []
    for dequant in ("staged", "staged_t"):
        st = Stack(cfg, modes=("resident",), record=True, layers=3, dequant=dequant)
        st.step("resident")
        runs.append(snapshot(st))
        st.close()
    fwd, re, dx, eq, n = compare(runs[0], runs[1])
    assert fwd and re and dx and eq == n == 2 * 7 * 3, (fwd, re, dx, eq, n)


def test_gradient_accumulation_over_micro_batches(gpu):
    """Three 8B-shaped layers, two micro-batches per step ("Exact Layer Streaming", Abstract:
    accumulation is per-token I/O-neutral): the first micro-batch sets dA, dB and the second adds
    into them; the stack's inputs repeat, so every gradient is exactly twice a single pass's.
    Streamed equals resident, and the pool copies every layer twice per micro-batch."""
    import torch
    cfg = configs.C3
    print("case: 3-layer 8B-shaped toy, two micro-batches", flush=True)
    st = Stack(cfg, modes=("streamed", "resident"), layers=3)
    st.step("resident")
    single = snapshot(st)[1]
    st.step("resident", micro_batches=2)
    double = snapshot(st)[1]
    for l1, l2 in zip(single, double):
        for (a1, b1), (a2, b2) in zip(l1, l2):
            assert torch.equal(a2, 2 * a1) and torch.equal(b2, 2 * b1)
    st.reset_pool(0, 2)
    st.step("streamed", micro_batches=2)
    streamed = snapshot(st)[1]
    for l1, l2 in zip(double, streamed):
        for (a1, b1), (a2, b2) in zip(l1, l2):
            assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
            assert torch.equal(b1.view(torch.int32), b2.view(torch.int32))
    assert st.pool.stats()["copies"] == 2 * 2 * 3
    st.close()


def test_reference_pass_adapters_off(gpu):
    """The DPO-style reference sweep ("An 8B Fine-Tune Now Fits in 4 GB of VRAM": the streamed
    base with the adapters off is the reference model): three 8B-shaped layers. The sweep changes
    no training state (every forward, recompute, dX checksum and every LoRA gradient equals a step
    without it); streamed equals resident on the reference outputs too; the pool copies each
    layer three times per step; and the reference outputs of k and o match the oracle's
    adapters-off forward on sampled rows."""
    import torch
    from oracle import lora as olora
    from oracle import nf4 as onf4
    cfg = configs.C3
    print("case: 3-layer 8B-shaped toy, reference sweep", flush=True)
    st = Stack(cfg, modes=("streamed", "resident"), record=True, layers=3)
    st.step("resident")
    plain = snapshot(st)
    st.step("resident", reference=True)
    with_ref = snapshot(st)
    fwd, re, dx, eq, n = compare(plain, with_ref)
    assert fwd and re and dx and eq == n == 2 * 7 * 3, (fwd, re, dx, eq, n)
    st.reset_pool(0, 2)
    st.step("streamed", reference=True)
    ref_out = [y.clone() for y in st.Yref]          # layer 2's reference outputs
    streamed = snapshot(st)
    fwd, re, dx, eq, n = compare(with_ref, streamed)
    assert fwd and re and dx and eq == n
    ref_keys = [k for k in with_ref[0] if k[0] == "ref"]
    assert len(ref_keys) == 3 * 7 and all(with_ref[0][k] == streamed[0][k] for k in ref_keys)
    assert st.pool.stats()["copies"] == 3 * 3
    rows = np.sort(np.random.default_rng(1).choice(cfg.T, 24, replace=False))
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for j, p in enumerate(st.layout):
        if p.name not in ("k", "o"):     # one projection per input width keeps the oracle's packing short
            continue
        W = inputs.device_normal((p.N, p.K), inputs.STD["W"], st.seed, cfg.name, 2, p.name, "W").cpu().numpy()
        Wh = onf4.bf16_to_f32(onf4.dequant_bf16(onf4.pack(W)))
        X = f(st.X[PROJ_INPUT[p.name]])[rows]
        Yo, _ = olora.forward(X, Wh, f(st.A[2][j]), f(st.B[2][j]), cfg.scale, False)
        got = ref_out[j].float().cpu().numpy()[rows]
        err = olora.rel_l2(got.astype(np.float64), Yo)
        assert err < 5e-3, (p.name, err)
    st.close()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["C2", "C4", "C3", "C5"])
def test_streamed_equals_resident_full_stack(gpu, name):
    cfg = configs.CONFIGS[name]
    print(f"case: {cfg.name} ({cfg.layers} layers) streamed vs resident", flush=True)
    st = Stack(cfg, modes=("streamed", "resident"), record=True)
    st.step("resident")
    ref = snapshot(st)
    st.step("streamed")
    got = snapshot(st)
    fwd, re, dx, eq, n = compare(ref, got)
    ledger = {"config": cfg.name, "base": cfg.base, "MiB_per_layer": round(st.image_bytes / 2 ** 20, 1),
              "forward_exact": fwd, "recompute_exact": re, "dX_exact": dx,
              "lora_grad_tensors_exact": f"{eq}/{n}"}
    print("ledger", ledger, flush=True)
    assert fwd and re and dx and eq == n == 2 * 7 * cfg.layers
    assert recompute_matches_forward(got[0], cfg.layers, 7)
    stats = st.pool.stats()
    assert stats["copies"] == 2 * cfg.layers and stats["misses"] == 0
    st.close()
