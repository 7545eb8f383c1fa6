"""Micro-benchmarks of kernels that sit beside the streamed projection step: the decoder-layer
glue (RMSNorm, rotary embedding, SwiGLU; standalone and in the projections' epilogues), the
forward GEMM decoding NF4 weights itself against staging plus the bf16 GEMM, and causal
attention, at a stack configuration's token count, widths and heads.

    python -m layer_streamed_nf4_dequant_amd.microbench [--config C3] [--iters 20]
    python -m layer_streamed_nf4_dequant_amd.microbench --decoder [--config C3] [--steps 3]

prints one JSON object: per kernel, microseconds per call (HIP events around a replayed HIP graph
of back-to-back calls) and the algorithmic HBM rate against the 8 TB/s peak. bench.py reports
the same figure beside its headline line.

The figures free their buffers into torch's cache and do not hand them back to the driver
(torch.cuda.empty_cache): after a release of 12 GB that way, the projection stack's next steps
ran up to 18% slower for about a second (165 -> 194 ms per streamed step, measured on MI355X),
which skewed whatever was timed next. The device has room to keep them.
"""

from __future__ import annotations

import argparse
import json
import os


def _time_calls(fn, iters: int, graph: bool = True):
    """Microseconds per call of `iters` back-to-back calls, timed with HIP events. With graph=True
    the calls are captured into one HIP graph and replayed, so host launch cost does not show;
    returns None if the capture fails."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    run = None
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(iters):
                    fn()
            run = g.replay
        except Exception:
            torch.cuda.synchronize()
            return None
    else:
        def run():
            for _ in range(iters):
                fn()
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def glue_figure(cfg, iters: int = 20):
    """The decoder-layer glue kernels at the workload's T and widths, each timed with HIP events
    over `iters` back-to-back calls replayed from a HIP graph: microseconds per call and the
    algorithmic HBM rate (bytes each call must move, stated per kernel below) as a fraction of
    the 8 TB/s peak."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, H, I, KV = cfg.T, cfg.hidden, cfg.inter, cfg.kv
    d = cfg.head_dim
    nq, nkv = H // d, KV // d
    bf = dict(dtype=torch.bfloat16)
    x = inputs.device_normal((T, H), 1.0, 0, "bench glue", "x", **bf)
    g = inputs.device_normal((H,), 0.1, 0, "bench glue", "g", **bf)
    y = torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    dy = inputs.device_normal((T, H), 1.0, 0, "bench glue", "dy")
    dx = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    qk = inputs.device_normal((T, (nq + nkv) * d), 1.0, 0, "bench glue", "qk", **bf)
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    gt = inputs.device_normal((T, I), 2.0, 0, "bench glue", "gate", **bf)
    up = inputs.device_normal((T, I), 1.0, 0, "bench glue", "up", **bf)
    dm = inputs.device_normal((T, I), 1.0, 0, "bench glue", "dm", **bf)
    m, dgt, dup = torch.empty_like(gt), torch.empty_like(gt), torch.empty_like(gt)
    jobs = {
        # x read, y written (bf16), rstd written, gain read
        "rmsnorm_fwd": (lambda: lib.rmsnorm_fwd(x, g, 1e-5, y, rstd), 4 * T * H + 4 * T + 2 * H),
        # x (bf16) and dy (fp32) read, dx (fp32) read and written (accumulating), rstd and gain read
        "rmsnorm_bwd_accumulate": (lambda: lib.rmsnorm_bwd(x, g, rstd, dy, dx, accumulate=True),
                                   14 * T * H + 4 * T + 2 * H),
        # q and k heads read and written in place (the backward is the same kernel)
        "rope_q_and_k": (lambda: (lib.rope_apply(qk[:, : nq * d], pos, nq, d, 500000.0),
                                  lib.rope_apply(qk[:, nq * d:], pos, nkv, d, 500000.0)),
                         4 * T * (nq + nkv) * d),
        "swiglu_fwd": (lambda: lib.swiglu_fwd(gt, up, m), 6 * T * I),   # g, u read; m written
        "swiglu_bwd": (lambda: lib.swiglu_bwd(gt, up, dm, dgt, dup), 10 * T * I),  # g, u, dm read; dg, du written
    }
    out = {"tokens": T, "hidden": H, "inter": I, "heads": [nq, nkv, d], "timing": "graph"}
    for name, (fn, nbytes) in jobs.items():
        us = _time_calls(fn, iters)
        if us is None:
            out["timing"] = "eager"
            us = _time_calls(fn, iters, graph=False)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 1), "bytes": nbytes, "GBs": round(gbs, 1), "frac": round(gbs / 8000.0, 3)}
    del x, g, y, rstd, dy, dx, qk, pos, gt, up, dm, m, dgt, dup
    return out


def fused_glue_figure(cfg, iters: int = 10):
    """The glue the decoder step runs in its projections' epilogues, at the workload's shapes with
    bf16 (staged) weights: per fused call, its time, the plain projection's time and the
    standalone glue kernel's time (HIP events over replayed HIP graphs), and what the fusion saves
    (plain + glue - fused, microseconds per call)."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, H, I, KV, r, d = cfg.T, cfg.hidden, cfg.inter, cfg.kv, cfg.r, cfg.head_dim
    nq, nkv = H // d, KV // d
    theta = 500000.0
    bf = dict(dtype=torch.bfloat16)
    key = ("bench fused glue", cfg.name)

    def lin(K, N, name):
        W = inputs.device_normal((N, K), 0.02, 0, *key, name, "W", **bf)
        A = inputs.device_normal((r, K), 0.01, 0, *key, name, "A", **bf)
        B = inputs.device_normal((N, r), 0.01, 0, *key, name, "B", **bf)
        return (W, A, B), lib.linear_desc(T, K, N, r, cfg.scale, W, A, B)

    X = inputs.device_normal((T, H), 1.0, 0, *key, "X", **bf)
    Xi = inputs.device_normal((T, I), 1.0, 0, *key, "Xi", **bf)
    dY = inputs.device_normal((T, H), 1.0, 0, *key, "dY", **bf)
    keep, D = [], {}
    for name, K, N in (("q", H, H), ("k", H, KV), ("v", H, KV), ("o", H, H), ("gate", H, I), ("up", H, I),
                       ("down", I, H)):
        t, D[name] = lin(K, N, name)
        keep.append(t)
    U = [inputs.device_normal((T, r), 1.0, 0, *key, "U", j, **bf) for j in range(7)]
    q, k, v, o = (torch.empty((T, n), **bf, device="cuda") for n in (H, KV, KV, H))
    gate, up, m, dm, dg, du = (torch.empty((T, I), **bf, device="cuda") for _ in range(6))
    res = inputs.device_normal((T, H), 1.0, 0, *key, "residual", **bf)
    pos = torch.arange(T, dtype=torch.int32, device="cuda") % cfg.seq_len
    tab = lib.rope_table(cfg.seq_len, d, theta)
    rope = lib.rope_desc(tab, cfg.seq_len, d, pos)
    dA = torch.empty((r, I), dtype=torch.float32, device="cuda")
    dB = torch.empty((H, r), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.ws_bytes(T, I, H, r), dtype=torch.uint8, device="cuda")
    RD = lib.ADAPTERS_U_READY
    cases = {
        "rope_in_qkv": (
            lambda: lib.lora_linear_fwd_group_epi([D["q"], D["k"], D["v"]], X, [q, k, v], U[:3], adapters=RD,
                                                  rope_mask=0b011, rope=rope),
            lambda: lib.lora_linear_fwd_group([D["q"], D["k"], D["v"]], X, [q, k, v], U[:3], adapters=RD),
            lambda: (lib.rope_apply(q, pos, nq, d, theta), lib.rope_apply(k, pos, nkv, d, theta))),
        "residual_in_o": (
            lambda: lib.lora_linear_fwd_group_epi([D["o"]], X, [o], U[3:4], adapters=RD, residual=[res]),
            lambda: lib.lora_linear_fwd_group([D["o"]], X, [o], U[3:4], adapters=RD),
            lambda: lib.add_bf16(res, o, q)),
        "swiglu_in_gate_up_m_only": (
            lambda: lib.lora_linear_fwd_swiglu(D["gate"], D["up"], X, m, Ug=U[4], Uu=U[5], adapters=RD),
            lambda: lib.lora_linear_fwd_group([D["gate"], D["up"]], X, [gate, up], U[4:6], adapters=RD),
            lambda: lib.swiglu_fwd(gate, up, m)),
        "swiglu_in_gate_up_stored": (
            lambda: lib.lora_linear_fwd_swiglu(D["gate"], D["up"], X, m, gate=gate, up=up, Ug=U[4], Uu=U[5],
                                               adapters=RD),
            lambda: lib.lora_linear_fwd_group([D["gate"], D["up"]], X, [gate, up], U[4:6], adapters=RD),
            lambda: lib.swiglu_fwd(gate, up, m)),
        "swiglu_bwd_in_down_dx": (
            lambda: lib.lora_linear_bwd_swiglu(D["down"], Xi, dY, U[6], gate, up, dg, du, dA, dB, ws=ws),
            lambda: lib.lora_linear_bwd(D["down"], Xi, dY, U[6], dm, dA, dB, ws=ws),
            lambda: lib.swiglu_bwd(gate, up, dm, dg, du)),
    }
    out = {"timing": "graph"}
    for name, fns in cases.items():
        t = []
        for fn in fns:
            us = _time_calls(fn, iters)
            if us is None:
                out["timing"] = "eager"
                us = _time_calls(fn, iters, graph=False)
            t.append(us)
        out[name] = {"fused_us": round(t[0], 1), "plain_us": round(t[1], 1), "glue_kernel_us": round(t[2], 1),
                     "saved_us": round(t[1] + t[2] - t[0], 1)}
    del keep, X, Xi, dY, U, q, k, v, o, gate, up, m, dm, dg, du, res, pos, tab, dA, dB, ws
    return out


def nf4_gemm_figure(cfg, iters: int = 10):
    """The forward launches of one layer with NF4 base weights, two ways: the weights staged by
    nf4_dequant (one launch for the layer's weights of the launch) and then the bf16 GEMM, against
    the GEMM that decodes each K-step's NF4 blocks into LDS itself. Per launch (the grouped
    q/k/v/gate/up, o, down): microseconds (HIP events over replayed HIP graphs) and the GEMM's
    TFLOP/s (2 T K N + 2 T r N per member)."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, H, I, KV, r = cfg.T, cfg.hidden, cfg.inter, cfg.kv, cfg.r
    bf = dict(dtype=torch.bfloat16)
    key = ("bench nf4 gemm", cfg.name)
    launches = {"qkv_gate_up": (H, [("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I)]),
                "o": (H, [("o", H)]), "down": (I, [("down", H)])}
    out = {"timing": "graph"}
    for lname, (K, members) in launches.items():
        X = inputs.device_normal((T, K), 1.0, 0, *key, lname, "X", **bf)
        nf, st, w16s, ys, us, keep = [], [], [], [], [], []
        for name, N in members:
            Wf = inputs.device_normal((N, K), 0.02, 0, *key, name, "W", dtype=torch.float32)
            P = lib.nf4_pack(Wf)
            del Wf
            A = inputs.device_normal((r, K), 0.01, 0, *key, name, "A", **bf)
            B = inputs.device_normal((N, r), 0.01, 0, *key, name, "B", **bf)
            w16 = torch.empty((N, K), **bf, device="cuda")
            keep += [P, A, B]
            w16s.append(w16)
            nf.append(lib.linear_desc(T, K, N, r, cfg.scale, P, A, B))
            st.append(lib.linear_desc(T, K, N, r, cfg.scale, w16, A, B))
            ys.append(torch.empty((T, N), **bf, device="cuda"))
            us.append(inputs.device_normal((T, r), 1.0, 0, *key, name, "U", **bf))
        pdescs = [P.desc() for P in keep[0::3]]
        RD = lib.ADAPTERS_U_READY
        fns = {
            "nf4_in_gemm": lambda: lib.lora_linear_fwd_group(nf, X, ys, us, adapters=RD),
            "dequant": lambda: lib.nf4_dequant_batch(pdescs, w16s, "bf16"),
            "bf16_gemm": lambda: lib.lora_linear_fwd_group(st, X, ys, us, adapters=RD),
        }
        t = {}
        for name, fn in fns.items():
            us_ = _time_calls(fn, iters)
            if us_ is None:
                out["timing"] = "eager"
                us_ = _time_calls(fn, iters, graph=False)
            t[name] = us_
        flop = sum(2 * T * K * N + 2 * T * r * N for _, N in members)
        out[lname] = {"nf4_in_gemm_us": round(t["nf4_in_gemm"], 1),
                      "staged_us": round(t["dequant"] + t["bf16_gemm"], 1),
                      "dequant_us": round(t["dequant"], 1), "bf16_gemm_us": round(t["bf16_gemm"], 1),
                      "nf4_in_gemm_TFLOPs": round(flop / t["nf4_in_gemm"] / 1e6, 1),
                      "bf16_gemm_TFLOPs": round(flop / t["bf16_gemm"] / 1e6, 1)}
        del X, nf, st, w16s, ys, us, keep, pdescs
    return out


def attention_figure(cfg, iters: int = 10):
    """Causal grouped-query attention at the configuration's T rows as T / seq_len sequences, its
    heads and head width: microseconds per forward and per backward call (graph-replayed) and
    the algorithmic rate against the 2.5 PFLOP/s bf16 peak. Algorithmic FLOPs: the forward's
    two products over the causal half, 2 n_seq n_q S^2 d; the backward's five (scores
    recomputed, dP, dV, dQ, dK), 2.5 times that."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, S, d = cfg.T, cfg.seq_len, cfg.head_dim
    n_seq, nq, nkv = T // S, cfg.hidden // d, cfg.kv // d
    W = (nq + 2 * nkv) * d
    qkv = inputs.device_normal((T, W), 1.0, 0, "bench attention", "qkv", dtype=torch.bfloat16)
    q, k, v = qkv[:, : nq * d], qkv[:, nq * d:(nq + nkv) * d], qkv[:, (nq + nkv) * d:]
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, nq), dtype=torch.float32, device="cuda")
    dO = inputs.device_normal((T, nq * d), 1.0, 0, "bench attention", "dO", dtype=torch.bfloat16)
    g = torch.empty_like(qkv)
    dq, dk, dv = g[:, : nq * d], g[:, nq * d:(nq + nkv) * d], g[:, (nq + nkv) * d:]
    ws = torch.empty(lib.attention_bwd_ws_bytes(n_seq, S, nq, nkv, d), dtype=torch.uint8, device="cuda")
    fwd = lambda: lib.attention_fwd(q, k, v, o, lse, n_seq, nq, nkv, d)  # noqa: E731
    bwd = lambda: lib.attention_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws, n_seq, nq, nkv, d)  # noqa: E731
    flops_f = 2 * n_seq * nq * S * S * d
    out = {"tokens": T, "seq_len": S, "sequences": n_seq, "heads": [nq, nkv, d], "timing": "graph"}
    for name, fn, fl in (("forward", fwd, flops_f), ("backward", bwd, flops_f * 5 // 2)):
        us = _time_calls(fn, iters)
        if us is None:
            out["timing"] = "eager"
            us = _time_calls(fn, iters, graph=False)
        tf = fl / (us * 1e-6) / 1e12
        out[name] = {"us": round(us, 1), "flops": fl, "TFLOPs": round(tf, 1), "frac": round(tf / 2500.0, 3)}
    del qkv, o, lse, dO, g, ws
    return out


def decoder_figure(cfg, vocab: int = 128256, steps: int = 3, modes=("streamed", "resident")):
    """The whole decoder training step (embedding, every layer's glue, attention and seven LoRA
    projections on the NF4 base, final norm, LM-head cross-entropy, backward with per-layer
    recompute) at the configuration's shape with a Llama-3.1 vocabulary: tokens/s over `steps`
    timed steps after one warm-up, streamed through the 2-slot pool, with every layer resident
    (same kernels, no copies), and streamed with the adapters-off reference sweep in front (the
    reference model of DPO-style objectives: one more read of every layer per step)."""
    import time

    import torch
    from layer_streamed_nf4_dequant_amd.decoder import DecoderModel, predict_decoder_bytes
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ref = "streamed" in modes
    m = DecoderModel(cfg, vocab=vocab, modes=tuple(modes), reference=ref)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    out = {"layers": m.L, "vocab": vocab, "tokens_per_step": cfg.T, "seq_len": cfg.seq_len}
    runs = [(mode, mode, False) for mode in modes]
    if "streamed" in modes:
        runs.append(("streamed_with_reference_sweep", "streamed", True))
    for name, mode, ref in runs:
        m.step(mode, reference=ref)
        torch.cuda.synchronize()
        copied0 = m.pool.stats()["bytes_copied"] if mode == "streamed" else 0
        t0 = time.perf_counter()
        for _ in range(steps):
            m.step(mode, reference=ref)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        out[name] = {"tokens_per_s": round(cfg.T * steps / wall, 1), "ms_per_step": round(wall * 1e3 / steps, 1)}
        if mode == "streamed":
            out[name]["layer_reads_per_step"] = round((m.pool.stats()["bytes_copied"] - copied0)
                                                      / (steps * m.image_bytes), 2)
    if "streamed" in modes:
        # the host link as the streamed steps saw it: four of the model's pinned layer images into
        # the slots on its copy stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(m.copy_stream):
            e0.record(m.copy_stream)
            for i in range(4):
                m.slots[i % len(m.slots)][:m.image_bytes].copy_(m.host_images[i], non_blocking=True)
            e1.record(m.copy_stream)
        e1.synchronize()
        out["h2d_GBs"] = round(4 * m.image_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    out["mean_loss"] = round(m.mean_loss(), 4)
    # the fit predictor: the device memory the steps above held against the prediction
    out["peak_hbm_GB"] = round((torch.cuda.max_memory_allocated() - before) / 1e9, 4)
    out["predicted_peak_hbm_GB"] = round(predict_decoder_bytes(cfg, vocab, modes=tuple(modes),
                                                               reference=ref)["total"] / 1e9, 4)
    m.close()
    del m
    return out


def gemm_vs_hipblaslt(cfg, iters: int = 5):
    """Our forward GEMM (bf16 weights, with the LoRA term) against hipBLASLt (torch.matmul on the
    same X and W, no LoRA term) on the q (H -> H), gate (H -> inter) and down (inter -> H) shapes
    at the configuration's T, for kernel traces and byte counters of the two side by side. A
    1 GiB device-to-device copy runs first (a plain copy kernel of known size, to scale the
    hardware byte counters). Each product runs `iters` times back to back, ours first; returns
    per shape the two mean times in microseconds (HIP events) and TFLOP/s."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, H, I, r = cfg.T, cfg.hidden, cfg.inter, cfg.r
    bf = dict(dtype=torch.bfloat16)
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    torch.empty_like(src).copy_(src)
    del src
    key = ("gemm vs hipblaslt", cfg.name)
    out = {}
    for name, K, N in (("q", H, H), ("gate", H, I), ("down", I, H)):
        X = inputs.device_normal((T, K), 1.0, 0, *key, name, "X", **bf)
        W = inputs.device_normal((N, K), 0.02, 0, *key, name, "W", **bf)
        A = inputs.device_normal((r, K), 0.01, 0, *key, name, "A", **bf)
        B = inputs.device_normal((N, r), 0.01, 0, *key, name, "B", **bf)
        U = inputs.device_normal((T, r), 1.0, 0, *key, name, "U", **bf)
        Y = torch.empty((T, N), **bf, device="cuda")
        desc = lib.linear_desc(T, K, N, r, 2.0, W, A, B)
        Wt = W.t()
        res = {}
        for who, fn in (("ours", lambda: lib.lora_linear_fwd(desc, X, Y, U, adapters=lib.ADAPTERS_U_READY)),
                        ("hipblaslt", lambda: torch.matmul(X, Wt))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / iters
            flop = 2 * T * K * N + (2 * T * r * N if who == "ours" else 0)
            res[who] = {"us": round(us, 1), "TFLOPs": round(flop / (us * 1e-6) / 1e12, 1)}
        out[f"{name} {K}->{N}"] = res
        del X, W, A, B, U, Y, desc, Wt
    return out


def main() -> None:
    from layer_streamed_nf4_dequant_amd import configs
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="C3")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--decoder", action="store_true",
                    help="time the whole decoder training step (streamed, then resident) instead")
    ap.add_argument("--steps", type=int, default=3, help="timed decoder steps per mode")
    ap.add_argument("--gemm-vs-hipblaslt", action="store_true",
                    help="run the forward GEMM and hipBLASLt on the q, gate and down shapes instead")
    args = ap.parse_args()
    cfg = getattr(configs, args.config)
    if args.gemm_vs_hipblaslt:
        print(json.dumps({"gemm_vs_hipblaslt": gemm_vs_hipblaslt(cfg)}), flush=True)
    elif args.decoder:
        print(json.dumps({"decoder_step": decoder_figure(cfg, steps=args.steps)}), flush=True)
    else:
        print(json.dumps({"glue": glue_figure(cfg, args.iters), "fused_glue": fused_glue_figure(cfg),
                          "nf4_gemm": nf4_gemm_figure(cfg), "attention": attention_figure(cfg)}), flush=True)


def hw_queues_for_streaming(minimum: int = 16) -> None:
    """At least `minimum` hardware queues for this process (GPU_MAX_HW_QUEUES; must run before
    the first HIP call). The layer pools' copy streams must not share a hardware queue with work
    the compute streams wait on: the marker that signals a copy's completion then blocks the
    compute kernels queued behind it until the copy ends, and copies stop overlapping compute.
    With 4 queues per process and torch's pool of streams, the decoder step's copy stream did
    land on such a queue when two streams (the projection stack's) existed before it: 335 ms
    per streamed step instead of 208."""
    have = int(os.environ.get("GPU_MAX_HW_QUEUES", "0") or 0)
    if have < minimum:
        os.environ["GPU_MAX_HW_QUEUES"] = str(minimum)


if __name__ == "__main__":
    hw_queues_for_streaming()
    main()
