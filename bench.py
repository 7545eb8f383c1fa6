"""Benchmark: training tokens/s through the 8B-shaped NF4 LoRA projection stack on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode streamed|resident|no_h2d]
                    [--config C3] [--no-cpu-baseline]

Workload (Llama-3.1-8B projection shapes): 32 decoder layers, hidden 4096, q/o 4096x4096,
k/v 4096->1024, gate/up 4096->14336, down 14336->4096, NF4 base with double-quantised
absmax, LoRA r=16 alpha=32 on all seven projections, T = 4096 token rows (2 x 2048), bf16
activations; the base streams from pinned host memory through a 2-slot device pool. One step
= forward over all layers, then per layer (in reverse) the re-fetch, the recomputed forward and
the backward (dX, dA, dB). Inputs are seeded synthetic tensors resident in HBM (the base in
pinned host memory, as the method keeps it) before the timed region starts.

Prints one JSON line. `value` = T * steps / wall time of the K timed steps. `roofline` is the
dominant kernel, the forward/recompute GEMM (k_gemm_direct on the staged bf16 W, LoRA term in its
prologue): achieved = algorithmic FLOPs of its launches in the timed steps / their summed
durations, measured with HIP events recorded around every launch on the compute stream; traffic =
the calibrated byte counters of the same launches from the committed profile summary. `cpu_baseline` times the CPU oracle on a
bounded sample (one layer, a subset of token rows) and scales it to the workload.

The figures after the headline free their buffers into torch's cache, never back to the driver:
memory handed back (torch.cuda.empty_cache) slowed the next second of kernels by up to 18%.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "training tokens/sec through 8B-shaped NF4 LoRA stack; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_direct_llama8b_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "layer_streamed_nf4_dequant_amd", "csrc", "gemm.hip")


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary
    (its `traffic_bytes_per_launch:` line), provided the summary was taken on the current kernel
    source (its `gemm_source_sha256:` line matches); null otherwise."""
    import hashlib
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    fields = dict(line.strip("` ").split(": ", 1) for line in text.splitlines()
                  if line.strip("` ").startswith(("traffic_bytes_per_launch: ", "gemm_source_sha256: ")))
    if fields.get("gemm_source_sha256") != sha:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def clock_sampler():
    """Samples the GPU's current sclk and mclk (the sysfs pp_dpm_* entry marked '*') and its
    power reading every 250 ms in a thread while the timed steps run (no child process; each
    sysfs clock read queries the power-management firmware, and sampling every 50 ms cost the
    timed steps about 0.8%). Returns
    a stop function giving the medians, or None where sysfs has no such files."""
    import glob
    import re
    import threading
    dev = next((d for d in sorted(glob.glob("/sys/class/drm/card*/device"))
                if os.path.exists(os.path.join(d, "pp_dpm_sclk"))), None)
    if dev is None:
        return None
    power = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_average")) +
                   glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")))
    samples = {"sclk_MHz": [], "mclk_MHz": [], "power_W": []}
    stop = threading.Event()

    def current(name):
        try:
            with open(os.path.join(dev, name)) as f:
                for ln in f:
                    if ln.strip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", ln)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def run():
        while not stop.is_set():
            for key, name in (("sclk_MHz", "pp_dpm_sclk"), ("mclk_MHz", "pp_dpm_mclk")):
                v = current(name)
                if v is not None:
                    samples[key].append(v)
            if power:
                try:
                    with open(power[0]) as f:
                        samples["power_W"].append(int(f.read()) / 1e6)
                except (OSError, ValueError):
                    pass
            stop.wait(0.25)

    th = threading.Thread(target=run, daemon=True)
    th.start()

    def finish():
        stop.set()
        th.join(timeout=5)
        out = {k: sorted(v)[len(v) // 2] for k, v in samples.items() if v}
        if out:
            out["samples"] = max(len(v) for v in samples.values())
            out["source"] = os.path.basename(os.path.dirname(dev)) + " sysfs"
        return out or None
    return finish


def lm_head_figure(cfg, vocab: int = 128256, chunk: int = 2048, iters: int = 5):
    """The resident LM head's cross-entropy (lm_head_ce) at the workload's T and hidden width with
    a Llama-3.1 vocabulary: time per call, its two GEMMs' rate (4 T V H FLOPs per call), and the
    workspace per logit element of a chunk."""
    import torch
    from layer_streamed_nf4_dequant_amd import inputs, lib
    T, H, V = cfg.T, cfg.hidden, vocab
    h = inputs.device_normal((T, H), 1.0, 0, "bench ce", "h", dtype=torch.bfloat16)
    W = inputs.device_normal((V, H), 0.02, 0, "bench ce", "W", dtype=torch.bfloat16)
    labels = torch.randint(0, V, (T,), generator=inputs.device_generator(0, "bench ce", "labels"),
                           device="cuda", dtype=torch.int32)
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    dh = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws_bytes = lib.lm_head_ce_ws_bytes(chunk, H, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lib.lm_head_ce(h, W, labels, 1.0 / T, loss, dh, chunk, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        lib.lm_head_ce(h, W, labels, 1.0 / T, loss, dh, chunk, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    out = {"vocab": V, "hidden": H, "tokens": T, "chunk_rows": chunk, "ms_per_call": round(ms, 3),
           "gemm_tflops": round(4 * T * V * H / (ms * 1e-3) / 1e12, 1),
           "workspace_bytes_per_logit_element": round(ws_bytes / (chunk * V), 3),
           "logits_bytes_per_logit_element": 6,
           "mean_loss": round(float(loss.mean()), 4)}
    del h, W, labels, loss, dh, ws
    return out


def hipblaslt_ceiling(cfg, iters: int = 10):
    """Same-session reference: torch.matmul (hipBLASLt) bf16 X W^T at the stack's projection shapes
    and T, TFLOP/s per (K, N) (no LoRA term): the forward shapes and the input-gradient shapes
    (dY [T][N] times W: a product of shape (N, K))."""
    import torch
    res = {}
    seen = set()
    shapes = [(n, K, N) for n, K, N in cfg.projections()] + [(f"d{n}", N, K) for n, K, N in cfg.projections()]
    for name, K, N in shapes:
        if (K, N) in seen:
            continue
        seen.add((K, N))
        g = torch.Generator(device="cuda").manual_seed(0)
        X = torch.randn((cfg.T, K), device="cuda", generator=g).to(torch.bfloat16)
        W = torch.randn((N, K), device="cuda", generator=g).to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(X, W.t())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            torch.matmul(X, W.t())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        res[f"{name} {K}->{N}"] = round(2 * cfg.T * K * N / (ms * 1e-3) / 1e12, 1)
        del X, W
    return res


def device_copy_rate(nbytes: int = 1 << 30, iters: int = 10) -> dict:
    """Same-session reference for the HBM-bound kernels: a device-to-device copy of `nbytes`
    (torch copy_, the runtime's blit kernel), counted as nbytes read plus nbytes written."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"GBs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_copy": 2 * nbytes,
            "what": "torch copy_ of 1 GiB on the device (the runtime's blit kernel), read + written"}


def cpu_baseline(cfg, seed: int = 0, rows: int | None = 32, layers: int = 1, n_max: int | None = None):
    """Oracle (numpy, fp64 LoRA + fp32 NF4) on `layers` layers of the workload: the NF4 dequant of
    all 7 projections twice (forward and backward visit; none for a bf16 base) plus forward,
    recomputed forward and backward on `rows` token rows (None: all T). With n_max, each
    projection is cut to its first n_max output rows and its times are scaled by N / n_max.
    Derived tokens/s = T / ((L / layers) * (t_dequant + (T / rows) * t_rows)); a full step when
    layers = L, rows = None and n_max = None."""
    import numpy as np
    from layer_streamed_nf4_dequant_amd import inputs
    from oracle import lora as olora
    from oracle import nf4 as onf4

    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(seed)
    n_rows = cfg.T if rows is None else rows
    t_deq = 0.0
    t_rows = 0.0
    deq_bytes = 0.0
    for _ in range(layers):
        for name, K, N in cfg.projections():
            Ns = N if n_max is None else min(N, n_max)
            scale = N / Ns
            W = rng.standard_normal((Ns, K), dtype=np.float32) * np.float32(0.02)
            if cfg.base == "nf4":
                p = onf4.pack(W)
                del W
                t0 = time.perf_counter()
                Wh = onf4.bf16_to_f32(onf4.dequant_bf16(p))          # forward visit
                Wh = onf4.bf16_to_f32(onf4.dequant_bf16(p))          # backward visit (re-dequantised)
                t_deq += (time.perf_counter() - t0) * scale
                deq_bytes += 2 * (K * N * 0.5 + K * N / 64 + 4 * K * N / 16384 + 2 * K * N)
            else:
                Wh = onf4.bf16_to_f32(onf4.bf16_rne(W))              # the bf16 base as stored
                del W
            A = onf4.bf16_to_f32(inputs.to_bf16_bits(rng.uniform(-K ** -0.5, K ** -0.5, (cfg.r, K)).astype(np.float32)))
            B = onf4.bf16_to_f32(inputs.to_bf16_bits((rng.standard_normal((Ns, cfg.r)) * 0.01).astype(np.float32)))
            X = onf4.bf16_to_f32(inputs.to_bf16_bits(rng.standard_normal((n_rows, K), dtype=np.float32)))
            dY = onf4.bf16_to_f32(inputs.to_bf16_bits(rng.standard_normal((n_rows, Ns), dtype=np.float32)))
            t0 = time.perf_counter()
            olora.forward(X, Wh, A, B, cfg.scale)                # forward
            olora.forward(X, Wh, A, B, cfg.scale)                # recomputed forward
            olora.backward(X, dY, Wh, A, B, cfg.scale)           # backward
            t_rows += (time.perf_counter() - t0) * scale
            del Wh
    per_layer_full_T = (t_deq + (cfg.T / n_rows) * t_rows) / layers
    tok_s = cfg.T / (cfg.layers * per_layer_full_T)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    full = layers == cfg.layers and rows is None and n_max is None
    sample = (f"{layers} of {cfg.layers} layers, {n_rows} of {cfg.T} token rows"
              + (f", each projection cut to its first {n_max} output rows (times scaled by N / {n_max})" if n_max else "")
              + (f": NF4 dequant of all {len(cfg.projections())} projections twice ({t_deq:.2f} s)" if cfg.base == "nf4"
                 else ": no dequant (bf16 base)")
              + f" + fp64 fwd/recompute/bwd on the sampled rows ({t_rows:.2f} s)"
              + ("; a timed full step" if full else "; derived tokens/s = T / (L / layers * (t_dequant + T/rows * t_rows))"))
    out = {"value": round(tok_s, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model, "timed_full_step": full, "sample": sample}
    if deq_bytes:
        out["dequant_GBs"] = round(deq_bytes / t_deq / 1e9, 3)
    return out


def direct_io_dir():
    """A directory whose file system accepts O_DIRECT reads: the temporary directory, else the
    repository root (None if neither does)."""
    import tempfile
    for d in (tempfile.gettempdir(), ROOT):
        path = None
        try:
            fd, path = tempfile.mkstemp(dir=d, prefix="lsnf4_direct_probe_")
            os.write(fd, bytes(8192))
            os.close(fd)
            fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
            os.close(fd)
            return d
        except OSError:
            continue
        finally:
            if path is not None and os.path.exists(path):
                os.remove(path)
    return None


def fs_type(path) -> str | None:
    """The mount's file system type and device for `path` (from /proc/mounts)."""
    import tempfile
    path = os.path.realpath(path or tempfile.gettempdir())
    best = None
    try:
        with open("/proc/mounts") as f:
            for ln in f:
                dev, mnt, fs = ln.split()[:3]
                if (path == mnt or path.startswith(mnt.rstrip("/") + "/")) and (best is None or len(mnt) > len(best[1])):
                    best = (dev, mnt, fs)
    except OSError:
        return None
    return None if best is None else f"{best[2]} on {best[0]} at {best[1]}"


def timed_steps(stack, mode: str, steps: int) -> float:
    """tokens/s of `steps` steps in `mode` after one untimed step (wall clock, synchronised)."""
    import torch
    stack.step(mode)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step(mode)
    torch.cuda.synchronize()
    return stack.cfg.T * steps / (time.perf_counter() - t0)


# the CPU oracle's sample per configuration (kept to a few seconds each; see cpu_baseline)
ORACLE_SAMPLE = {"C1": dict(rows=None, layers=1), "C2": dict(rows=None, layers=2),
                 "C4": dict(rows=32, layers=1), "C5": dict(rows=32, layers=1, n_max=1024)}


def config_figures(names=("C1", "C2", "C4", "C5"), steps: int = 3, cpu: bool = True):
    """The other seeded configurations: tokens/s of the streamed, resident and no-H2D steps (same
    kernels and pool as the headline), the streamed/resident ratio, and the CPU oracle on a
    bounded sample of each."""
    import torch
    from layer_streamed_nf4_dequant_amd import configs
    from layer_streamed_nf4_dequant_amd.stack import Stack
    out = {}
    for name in names:
        cfg = configs.CONFIGS[name]
        print(f"[bench] config {name} ({cfg.name}): {cfg.layers} layers, T={cfg.T}", flush=True)
        modes = ("streamed", "resident", "no_h2d")
        st = Stack(cfg, modes=modes)
        res = {m: round(timed_steps(st, m, steps), 1) for m in modes}
        st.close()
        del st
        fig = {"workload": cfg.name, "layers": cfg.layers, "tokens_per_step": cfg.T, "base": cfg.base,
               "steps_timed": steps, "tokens_per_s": res,
               "streamed_over_resident": round(res["streamed"] / res["resident"], 4),
               "flops_per_step": cfg.flops_per_step(),
               "streamed_tflops": round(cfg.flops_per_step() * res["streamed"] / cfg.T / 1e12, 1)}
        if cpu:
            fig["cpu_oracle"] = cpu_baseline(cfg, **ORACLE_SAMPLE[name])
        print(f"[bench] config {name}: {fig['tokens_per_s']}", flush=True)
        out[name] = fig
    return out


def _stats(values):
    v = sorted(values)
    return {"mean": round(sum(v) / len(v), 2), "median": round(v[len(v) // 2], 2),
            "p90": round(v[min(len(v) - 1, int(0.9 * len(v)))], 2), "max": round(v[-1], 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--mode", default="streamed", choices=["streamed", "resident", "no_h2d"])
    ap.add_argument("--config", default="C3")
    ap.add_argument("--dequant", default="staged", choices=["staged", "staged_t", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-modes", action="store_true",
                    help="skip the resident and no-H2D comparison timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other seeded configurations (C1, C2, C4, C5)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, run one device-to-device copy of MIB MiB (a plain copy kernel of "
                         "known size, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the stack streams one GPU's layers; no sharding across GPUs is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from layer_streamed_nf4_dequant_amd import configs, lib
    from layer_streamed_nf4_dequant_amd.microbench import (attention_figure, decoder_figure, fused_glue_figure,
                                                           glue_figure, nf4_gemm_figure)
    from layer_streamed_nf4_dequant_amd.stack import Stack

    lib.load()
    cfg = configs.CONFIGS[args.config]
    print(f"[bench] setting up {cfg.name}: {cfg.layers} layers, T={cfg.T}, mode={args.mode}", flush=True)
    t0 = time.perf_counter()
    modes = (args.mode,) if args.no_other_modes else tuple(dict.fromkeys((args.mode, "streamed", "resident", "no_h2d")))
    stack = Stack(cfg, modes=modes, dequant=args.dequant)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t0:.1f} s; image {stack.image_bytes / 1e6:.2f} MB/layer",
          flush=True)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        ms = stack.step(args.mode)
        print(f"[bench] warmup {i}: {ms:.1f} ms", flush=True)

    # the staging kernels are timed in a pass of their own below when that pass runs (their events
    # in the streamed pass would also count copy waits); the GEMM events stay in the timed steps
    dequant_separately = not args.no_other_modes and stack.slots is not None and stack.dequant != "fused"
    gemm_events, dequant_events = [], []
    torch.cuda.reset_peak_memory_stats()
    torch.cuda.synchronize()
    clocks_done = clock_sampler()
    t_start = time.perf_counter()
    step_ms = []
    for i in range(args.steps):
        step_ms.append(stack.step(args.mode, gemm_events=gemm_events, dequant_events=dequant_events))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    peak_alloc = torch.cuda.max_memory_allocated()
    pool = stack.pool.stats() if stack.pool is not None else None   # before any pool reset below
    clocks = clocks_done() if clocks_done else None
    print(f"[bench] {args.steps} steps: {wall * 1e3 / args.steps:.1f} ms/step (events median "
          f"{sorted(step_ms)[len(step_ms) // 2]:.1f} ms)", flush=True)

    # dominant kernel: the fused forward GEMM launches of the timed steps
    dur_ms, flops = 0.0, 0
    per_class = {}
    for js, e0, e1 in gemm_events:
        ms = e0.elapsed_time(e1)
        dur_ms += ms
        f = 0
        for j in js:
            _, K, N = cfg.projections()[j]
            f += 2 * cfg.T * K * N + 2 * cfg.T * cfg.r * N
        flops += f
        name = "+".join(cfg.projections()[j][0] for j in js)
        c = per_class.setdefault(name, {"us": [], "flops": f})
        c["us"].append(ms * 1e3)
    n_launch = len(gemm_events)
    launches = {}
    for name, c in per_class.items():
        st_ = _stats(c["us"])
        st_["calls"] = len(c["us"])
        st_["tflops_at_mean"] = round(c["flops"] / (st_["mean"] * 1e-6) / 1e12, 1)
        launches[name] = st_
    achieved = flops / (dur_ms * 1e-3) / 1e12 if dur_ms > 0 else 0.0
    if cfg.base == "nf4" and stack.dequant == "fused":
        kernel = "k_gemm<NT,NF4> (fused NF4 dequant-into-LDS + bf16 MFMA + LoRA prologue)"
    else:
        kernel = "k_gemm_direct (bf16 MFMA + LoRA prologue; W dequantised per visit by k_dequant)"
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_from_profiles(),
                "kernel": kernel, "launches": n_launch,
                "avg_launch_us": round(dur_ms * 1e3 / max(n_launch, 1), 2),
                "per_launch_us": launches,
                "timed_in": f"{args.mode} timed steps (HIP events around every forward/recompute GEMM launch)"}

    # The staging events of the streamed pass start behind the compute stream's wait for the layer's
    # copy, and a HIP event takes its time stamp from the command before it, so in a copy-bound phase
    # they also count the wait. The headline dequant figure is therefore taken in a pass over layer
    # images already in the pool slots (same kernels, same bytes, no copies), when that pass exists;
    # the streamed step's own events are reported beside it.
    n_params = sum(K * N for _, K, N in cfg.projections())
    nf4_b = cfg.nf4_bytes_per_layer()

    def dequant_figure(events):
        """Algorithmic bytes per staged visit (read the NF4 image, write bf16 W; with staged_t the
        backward visit also writes bf16 W^T) over the summed event durations, per visit kind too."""
        if not events:
            return None
        d_ms = sum(e0.elapsed_time(e1) for _, e0, e1 in events)
        d_bytes = sum((2 if with_t else 1) * (nf4_b + 2 * n_params) for (_, with_t), _, _ in events)
        gbs = d_bytes / (d_ms * 1e-3) / 1e9
        per_kernel = {}
        for visit in ("fwd", "bwd"):
            ev = [(with_t, e0.elapsed_time(e1)) for (v, with_t), e0, e1 in events if v == visit]
            if not ev:
                continue
            b = sum((2 if with_t else 1) * (nf4_b + 2 * n_params) for with_t, _ in ev)
            g = b / (sum(ms for _, ms in ev) * 1e-3) / 1e9
            name = "k_dequant + k_dequant_t" if any(w for w, _ in ev) else "k_dequant"
            label = "forward" if visit == "fwd" else "backward"
            per_kernel[f"{name} ({label} visits)"] = {"achieved": round(g, 1), "frac": round(g / PEAK_HBM_GBS, 4)}
        return {"achieved": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "visits": len(events),
                "avg_visit_us": round(d_ms * 1e3 / len(events), 2), "by_visit": per_kernel}

    in_step = dequant_figure(dequant_events)
    head = in_step
    dequant_source = f"{args.mode} timed steps (events may include waits for layer copies)"
    if dequant_separately:
        stack.step("no_h2d")
        no_h2d_events = []
        for _ in range(max(2, args.steps // 2)):
            stack.step("no_h2d", dequant_events=no_h2d_events)
        torch.cuda.synchronize()
        head = dequant_figure(no_h2d_events)
        dequant_source = "no_h2d pass (layer images already in the pool slots; no copy waits)"
    dequant = None
    if head is not None:
        kernels = ("k_dequant + k_dequant_t" if stack.dequant == "staged_t" else "k_dequant") + " (per-visit staging)"
        dequant = {"bound": "hbm", "achieved": head["achieved"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": head["frac"], "kernels": kernels, "bytes_per_param": round(nf4_b / n_params + 2, 4),
                   "visits": head["visits"], "avg_visit_us": head["avg_visit_us"], "by_visit": head["by_visit"],
                   "timed_in": dequant_source}
        if dequant_separately and in_step is not None:
            dequant["in_timed_steps"] = dict(in_step, timed_in=f"{args.mode} timed steps (events may include "
                                                                 "waits for layer copies)")

    other = {}
    if not args.no_other_modes:
        for m in ("resident", "no_h2d"):
            if m == args.mode:
                continue
            stack.step(m)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = max(3, args.steps // 2)
            for _ in range(n):
                stack.step(m)
            torch.cuda.synchronize()
            other[m] = round(cfg.T * n / (time.perf_counter() - t0), 1)
            print(f"[bench] {m}: {other[m]} tokens/s", flush=True)
        # the whole decoder training step (its own model and pool), before the file tier below
        # fills the page cache with the stack's image file
        if cfg.base == "nf4" and not cfg.single:
            other["decoder_step"] = decoder_figure(cfg)
            print(f"[bench] decoder step: {other['decoder_step']}", flush=True)
        if stack.pool is not None:
            # the pool reusing the layers still in a slot at the forward/backward and step
            # boundaries (LSN_POOL_KEEP_AT_TURN) instead of copying every visit
            stack.reset_pool(lib.POOL_KEEP_AT_TURN)
            stack.step("streamed")
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = max(3, args.steps // 2)
            for _ in range(n):
                stack.step("streamed")
            torch.cuda.synchronize()
            other["streamed_keep_at_turn"] = round(cfg.T * n / (time.perf_counter() - t0), 1)
            print(f"[bench] streamed, keep at turn: {other['streamed_keep_at_turn']} tokens/s", flush=True)
            # the same with an 8-slot pool (7 layers in flight ahead of the compute, 7 kept at each
            # turn; 0.9 GB of slots at the 8B shape): how much of the streaming overhead a slightly
            # larger pool removes
            if cfg.layers >= 16:
                stack.reset_pool(lib.POOL_KEEP_AT_TURN, n_slots=8)
                c0 = stack.pool.stats()["copies"]
                other["streamed_keep_at_turn_8_slots"] = round(timed_steps(stack, "streamed", n), 1)
                other["streamed_keep_at_turn_8_slots_copies_per_step"] = round(
                    (stack.pool.stats()["copies"] - c0) / (n + 1), 1)
                print(f"[bench] streamed, keep at turn, 8 slots: {other['streamed_keep_at_turn_8_slots']} tokens/s "
                      f"({other['streamed_keep_at_turn_8_slots_copies_per_step']} copies per step)", flush=True)
                stack.reset_pool(0, n_slots=cfg.pool_slots)
            else:
                stack.reset_pool(0)
            # a DPO-style step: the frozen reference model's forward (one more streamed sweep with
            # the adapters off) before the training step
            torch.cuda.reset_peak_memory_stats()
            stack.step("streamed", reference=True)
            torch.cuda.synchronize()
            c0 = stack.pool.stats()["copies"]
            t0 = time.perf_counter()
            for _ in range(n):
                stack.step("streamed", reference=True)
            torch.cuda.synchronize()
            other["streamed_with_reference_sweep"] = round(cfg.T * n / (time.perf_counter() - t0), 1)
            other["reference_sweep_layer_reads_ratio"] = round((stack.pool.stats()["copies"] - c0) / n / (2 * stack.L), 3)
            other["reference_sweep_peak_hbm_ratio"] = round(torch.cuda.max_memory_allocated() / peak_alloc, 3)
            print(f"[bench] streamed with the reference sweep: {other['streamed_with_reference_sweep']} tokens/s",
                  flush=True)
            # gradient accumulation: two micro-batches per step (each streams every layer twice)
            stack.step("streamed", micro_batches=2)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                stack.step("streamed", micro_batches=2)
            torch.cuda.synchronize()
            other["streamed_2_micro_batches"] = round(2 * cfg.T * n / (time.perf_counter() - t0), 1)
            print(f"[bench] streamed, 2 micro-batches per step: {other['streamed_2_micro_batches']} tokens/s",
                  flush=True)
            # the layers streamed from one file through the pool's file tier: buffered reads (the
            # file was just written, so they come from the page cache: a RAM-speed read), then
            # O_DIRECT reads (past the page cache: the storage device's rate), where the file
            # system allows them
            stack.image_dir = direct_io_dir()
            for key, direct in (("streamed_from_file_page_cached", False), ("streamed_from_file_direct", True)):
                try:
                    stack.reset_pool(0, source="file", direct=direct)
                except lib.LsnError as e:
                    other[key] = f"unavailable: {e}"
                    continue
                other[key] = round(timed_steps(stack, "streamed", n), 1)
                print(f"[bench] {key}: {other[key]} tokens/s", flush=True)
            other["file_tier_directory_fs"] = fs_type(stack.image_dir)
            stack.reset_pool(0, source="ram")
            if stack.source == "ram":
                stack.drop_image_file()
        if stack.slots is not None:
            other["h2d_GBs"] = round(stack.h2d_rate(), 1)
        other["lm_head_ce"] = lm_head_figure(cfg)
        print(f"[bench] lm_head_ce: {other['lm_head_ce']}", flush=True)
        other["glue"] = glue_figure(cfg)   # layer_streamed_nf4_dequant_amd/microbench.py
        print(f"[bench] glue: {other['glue']}", flush=True)
        if not cfg.single:
            other["fused_glue"] = fused_glue_figure(cfg)
            print(f"[bench] fused glue: {other['fused_glue']}", flush=True)
        if cfg.base == "nf4" and not cfg.single:
            other["nf4_in_gemm"] = nf4_gemm_figure(cfg)
            print(f"[bench] nf4 decoded in the GEMM vs staged: {other['nf4_in_gemm']}", flush=True)
        other["attention"] = attention_figure(cfg)
        print(f"[bench] attention: {other['attention']}", flush=True)

    tokens = cfg.T * args.steps
    value = tokens / wall
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} NF4-LoRA projection stack" if cfg.base == "nf4"
                   else f"{cfg.name} LoRA projection stack",
                   "layers": cfg.layers, "tokens_per_step": cfg.T, "hidden": cfg.hidden, "kv": cfg.kv,
                   "inter": cfg.inter, "lora_rank": cfg.r, "lora_alpha": cfg.alpha, "base": cfg.base,
                   "mode": args.mode, "pool_slots": cfg.pool_slots, "dequant": stack.dequant,
                   "flops_per_step": cfg.flops_per_step(),
                   "stack_tflops": round(cfg.flops_per_step() / (wall / args.steps) / 1e12, 1),
                   "h2d_bytes_per_step": (pool["bytes_copied"] // (args.steps + args.warmup)) if pool else 0},
        "roofline": roofline,
    }
    if dequant is not None:
        out["dequant"] = dequant
    if other:
        out["other_modes_tokens_per_s"] = other
    # context for the numbers above (same session)
    context = {"events_median_ms_per_step": round(sorted(step_ms)[len(step_ms) // 2], 2),
               "peak_hbm_allocated_GB_during_timed_steps": round(peak_alloc / 1e9, 2)}
    if clocks:
        context["gpu_clocks_during_timed_steps"] = clocks
    if not args.no_other_modes:
        rates = hipblaslt_ceiling(cfg)
        context["hipblaslt_bf16_tflops_same_shapes"] = rates
        # the pages' protocol: the step against its same-session GEMM ceiling, i.e. the time the
        # step's base GEMMs (forward, recompute and dX, no LoRA term) would take at hipBLASLt's
        # rate for each shape, over the measured step time
        by_shape = {tuple(int(x) for x in k.split(" ")[1].split("->")): v for k, v in rates.items()}
        t_ceiling = cfg.layers * sum(2 * 2 * cfg.T * K * N / (by_shape[(K, N)] * 1e12) +
                                     2 * cfg.T * K * N / (by_shape[(N, K)] * 1e12)
                                     for _, K, N in cfg.projections())
        context["step_fraction_of_gemm_ceiling"] = {
            "value": round(t_ceiling / (wall / args.steps), 4), "ceiling_ms": round(t_ceiling * 1e3, 2),
            "step_ms": round(wall * 1e3 / args.steps, 2),
            "definition": "time of the step's base GEMMs at the same-session hipBLASLt rate per shape / step time"}
        copy = device_copy_rate()
        if dequant is not None:
            copy["dequant_over_copy"] = round(dequant["achieved"] / copy["GBs"], 4)
        context["device_copy_reference"] = copy
    out["context"] = context
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg)
    stack.close()
    del stack
    if not args.no_other_modes and not args.no_configs and args.config == "C3":
        out["configs"] = config_figures(cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


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
