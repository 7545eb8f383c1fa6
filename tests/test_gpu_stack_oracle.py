"""The projection stack against the oracle, through the launches a streamed training step makes
(the grouped q/k/v/gate/up forward GEMM, the grouped backward whose input gradients run as one
GEMM over the members' concatenated reductions, the single o and down launches, the pool), on
the seeded inputs of every stacked configuration:

  * the 0.5B-shaped stack (24 layers) and the 3B-shaped bf16-base stack (36 layers) with the
    whole backward chain composed from the oracle: down's upstream gradient is the oracle's dX of
    o one layer up, gate's and up's is the oracle's dX of down one layer up, both rounded to bf16
    where the stack stores them. Every layer of the 0.5B stack and layers {0, 1, 17, 34, 35} of
    the 3B stack are compared in full: Y and the recomputed Y of all seven projections on
    sampled rows, every dA and dB, and dX_h, dX_o, dX_d;
  * the 8B-shaped (32 layers) and 72B-shaped (80 layers) stacks on sampled layers, where the
    chain would cost the oracle the whole stack's fp64 products: Y and the recomputed Y of all
    seven projections on sampled rows, dA and dB of q, k, v and o (their upstream gradients are
    seeded at every layer) and dX of o; at the top layer, where every upstream gradient is
    seeded, also dA and dB of gate, up and down, dX of down and the summed dX_h.

Tolerances (relative L2 over the compared values, fp64): Y and dX 5e-3, dA and dB 1e-2 (the
acceptance bar of the method's exactness claim restated for an fp32-accumulating bf16 GEMM).
The oracle sees only the seeded inputs (W drawn by the same generator, X, dY, A, B); no value
the HIP path produced enters it.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import configs, inputs
from layer_streamed_nf4_dequant_amd.configs import PROJ_INPUT
from layer_streamed_nf4_dequant_amd.stack import Stack
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

TOL = {"Y": 5e-3, "dX": 5e-3, "dA": 1e-2, "dB": 1e-2}


def f64(t):
    """A device tensor's exact values as fp64 numpy."""
    if str(t.dtype) == "torch.bfloat16":
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def r16(a):
    """The stack's bf16 storage of an fp32-accumulated result: round to fp32, then to bf16."""
    return onf4.bf16_to_f32(onf4.bf16_rne(np.asarray(a, dtype=np.float32))).astype(np.float64)


class Capture:
    """on_visit hook for Stack.step: copies the outputs of the chosen layers before the next
    layer overwrites them (sampled rows of Y and of the recomputed Y, the whole input gradients)."""

    def __init__(self, st, layers, rows):
        import torch
        self.st, self.layers = st, set(layers)
        self.rows = torch.as_tensor(rows, device="cuda")
        torch.cuda.synchronize()              # rows is used on the stack's compute stream
        self.data = {}

    def __call__(self, visit, l):
        if l not in self.layers:
            return
        st = self.st
        if visit == "fwd":
            self.data[("Y", l)] = [y.index_select(0, self.rows) for y in st.Y]
        else:
            self.data[("Yre", l)] = [y.index_select(0, self.rows) for y in st.Yre]
            self.data[("dX_h", l)] = st.dX_h.clone()
            self.data[("dX_o", l)] = st.dX_o_pp[l % 2].clone()
            self.data[("dX_d", l)] = st.dX_d_pp[l % 2].clone()


def oracle_w_hat(cfg, st, l, names):
    """The oracle's bf16 base operand of the named projections of layer l, from the seeded fp32 W
    (NF4: pack, then dequantise; bf16 base: round to nearest even), one thread per projection."""
    Ws = {p.name: inputs.device_normal((p.N, p.K), inputs.STD["W"], st.seed, cfg.name, l, p.name, "W").cpu().numpy()
          for p in st.layout if p.name in names}

    def one(W):
        if cfg.base == "nf4":
            return onf4.bf16_to_f32(onf4.dequant_bf16(onf4.pack(W)))
        return onf4.bf16_to_f32(onf4.bf16_rne(W))

    with ThreadPoolExecutor(len(Ws)) as ex:
        return dict(zip(Ws, ex.map(one, Ws.values())))


class OracleLayer:
    """Oracle forward on sampled rows and (where the upstream gradient is known) the backward of
    the projections of one layer on the stack's own seeded inputs."""

    def __init__(self, cfg, st, X):
        self.cfg, self.st, self.X = cfg, st, X

    def run(self, l, rows, dY_of, names):
        st, cfg = self.st, self.cfg
        W_hat = oracle_w_hat(cfg, st, l, names)
        out = {}
        for j, p in enumerate(st.layout):
            if p.name not in names:
                continue
            X = self.X[PROJ_INPUT[p.name]]
            A, B = f64(st.A[l][j]), f64(st.B[l][j])
            if rows is not None:
                out[(p.name, "Y")] = olora.forward(X[rows], W_hat[p.name], A, B, cfg.scale)[0]
            dY = dY_of(p.name)
            if dY is not None:
                dX, dA, dB, _ = olora.backward(X, dY, W_hat[p.name], A, B, cfg.scale)
                out[(p.name, "dX")], out[(p.name, "dA")], out[(p.name, "dB")] = dX, dA, dB
        return out


class Checker:
    def __init__(self):
        self.worst = {}
        self.n = 0

    def __call__(self, what, kind, got, want):
        e = olora.rel_l2(got, want)
        self.n += 1
        self.worst[kind] = max(self.worst.get(kind, 0.0), e)
        assert e <= TOL[kind], f"{what}: rel L2 {e:.3e} > {TOL[kind]:.0e}"


def _setup(name, layers):
    import torch
    cfg = configs.CONFIGS[name]
    st = Stack(cfg, modes=("streamed",))
    rows = np.sort(np.random.default_rng(7).choice(cfg.T, 48, replace=False))
    checked = range(cfg.layers) if layers is None else layers
    cap = Capture(st, checked, rows)
    st.step("streamed", on_visit=cap)
    torch.cuda.synchronize()
    X = {w: f64(st.X[w]) for w in ("h", "o", "d")}
    return cfg, st, rows, list(checked), cap.data, OracleLayer(cfg, st, X)


def _check_layer(chk, st, l, rows, got, o, backward_names):
    """Y and the recomputed Y of every projection on the sampled rows; dA, dB of the projections
    whose backward the oracle ran."""
    for j, p in enumerate(st.layout):
        want = o[(p.name, "Y")]
        chk(f"layer {l} {p.name} Y", "Y", f64(got[("Y", l)][j]), want)
        chk(f"layer {l} {p.name} recomputed Y", "Y", f64(got[("Yre", l)][j]), want)
        if p.name in backward_names:
            chk(f"layer {l} {p.name} dA", "dA", f64(st.dA[l][j]), o[(p.name, "dA")])
            chk(f"layer {l} {p.name} dB", "dB", f64(st.dB[l][j]), o[(p.name, "dB")])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers", [("C2", None), ("C4", (0, 1, 17, 34, 35))],
                         ids=["qwen0.5b-all-24-layers", "qwen3b-bf16-5-layers"])
def test_stack_with_oracle_chain(gpu, name, layers):
    print(f"case: {name} streamed, oracle chain, layers checked {layers or 'all'}", flush=True)
    cfg, st, rows, checked, got, orc = _setup(name, layers)
    chk = Checker()
    names_all = [p.name for p in st.layout]
    above = None                       # the oracle's (dX of o, dX of down) one layer up, as stored (bf16)
    for l in reversed(range(cfg.layers)):
        def dY_of(n):
            if above is not None and n == "down":
                return above[0]
            if above is not None and n in ("gate", "up"):
                return above[1]
            return f64(st.dY[names_all.index(n)])
        full = l in checked
        o = orc.run(l, rows if full else None, dY_of, names_all if full else ("o", "down"))
        if full:
            _check_layer(chk, st, l, rows, got, o, names_all)
            dX_h = sum(o[(n, "dX")] for n in names_all if PROJ_INPUT[n] == "h")
            chk(f"layer {l} dX_h", "dX", f64(got[("dX_h", l)]), dX_h)
            chk(f"layer {l} dX_o", "dX", f64(got[("dX_o", l)]), o[("o", "dX")])
            chk(f"layer {l} dX_d", "dX", f64(got[("dX_d", l)]), o[("down", "dX")])
        above = (r16(o[("o", "dX")]), r16(o[("down", "dX")]))
    print(f"{chk.n} tensors compared; worst rel L2 {({k: f'{v:.2e}' for k, v in chk.worst.items()})}")
    st.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers", [("C3", (0, 15, 31)), ("C5", (0, 79))],
                         ids=["llama8b-layers-0-15-31", "qwen72b-layers-0-79"])
def test_stack_sampled_layers(gpu, name, layers):
    print(f"case: {name} streamed, layers checked {layers}", flush=True)
    cfg, st, rows, checked, got, orc = _setup(name, layers)
    chk = Checker()
    top = cfg.layers - 1
    names_all = [p.name for p in st.layout]
    for l in checked:
        seeded = names_all if l == top else ["q", "k", "v", "o"]
        o = orc.run(l, rows, lambda n: f64(st.dY[names_all.index(n)]) if n in seeded else None, names_all)
        _check_layer(chk, st, l, rows, got, o, seeded)
        chk(f"layer {l} dX_o", "dX", f64(got[("dX_o", l)]), o[("o", "dX")])
        if l == top:
            chk(f"layer {l} dX_d", "dX", f64(got[("dX_d", l)]), o[("down", "dX")])
            dX_h = sum(o[(n, "dX")] for n in names_all if PROJ_INPUT[n] == "h")
            chk(f"layer {l} dX_h", "dX", f64(got[("dX_h", l)]), dX_h)
        print(f"  layer {l} done", flush=True)
    print(f"{chk.n} tensors compared; worst rel L2 {({k: f'{v:.2e}' for k, v in chk.worst.items()})}")
    st.close()
