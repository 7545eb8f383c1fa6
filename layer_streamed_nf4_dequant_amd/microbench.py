"""Micro-benchmarks of kernels that sit beside the streamed projection step: the decoder-layer
glue (RMSNorm, rotary embedding, SwiGLU) and causal attention, at a stack configuration's token
count, widths and heads.

    python -m layer_streamed_nf4_dequant_amd.microbench [--config C3] [--iters 20]
    python -m layer_streamed_nf4_dequant_amd.microbench --decoder [--config C3] [--steps 3]

prints one JSON object: per kernel, microseconds per call (HIP events around a replayed HIP graph
of back-to-back calls) and the algorithmic HBM rate against the 8 TB/s peak. bench.py reports
the same figure beside its headline line.
"""

from __future__ import annotations

import argparse
import json


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
    torch.cuda.empty_cache()
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
    ws = torch.empty(lib.attention_bwd_ws_bytes(n_seq, S, nq), dtype=torch.uint8, device="cuda")
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
    torch.cuda.empty_cache()
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
    from layer_streamed_nf4_dequant_amd.decoder import DecoderModel
    m = DecoderModel(cfg, vocab=vocab, modes=tuple(modes))
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
    out["mean_loss"] = round(m.mean_loss(), 4)
    m.close()
    del m
    torch.cuda.empty_cache()
    return out


def main() -> None:
    from layer_streamed_nf4_dequant_amd import configs
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="C3")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--decoder", action="store_true",
                    help="time the whole decoder training step (streamed, then resident) instead")
    ap.add_argument("--steps", type=int, default=3, help="timed decoder steps per mode")
    args = ap.parse_args()
    cfg = getattr(configs, args.config)
    if args.decoder:
        print(json.dumps({"decoder_step": decoder_figure(cfg, steps=args.steps)}), flush=True)
    else:
        print(json.dumps({"glue": glue_figure(cfg, args.iters), "attention": attention_figure(cfg)}), flush=True)


if __name__ == "__main__":
    main()
