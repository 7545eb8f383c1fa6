"""Workload shapes: a single LoRA linear and four decoder-stack shapes.

Each stack adapts the seven projections of every decoder layer (q, k, v, o, gate, up, down)
with rank-16 LoRA (alpha 32), on an NF4 base (or, for the 3B shape, an un-quantised bf16
base), streamed through a 2-slot device pool.  Shapes follow the models the pages train
("Exact Layer Streaming", Abstract: Llama-3.1-8B in NF4, Qwen2.5-3B with a bf16 base, the
0.5B resident baseline, and gating up to 72B; Soup v0.73.0 benchmarks README, record index).
"""

from __future__ import annotations

from dataclasses import dataclass

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
# which shared input each projection reads: h = attention input, o = attention output,
# d = MLP intermediate
PROJ_INPUT = {"q": "h", "k": "h", "v": "h", "o": "o", "gate": "h", "up": "h", "down": "d"}


@dataclass(frozen=True)
class StackConfig:
    name: str
    layers: int
    hidden: int
    kv: int          # k/v output width
    inter: int       # MLP intermediate width
    T: int           # token rows per step (batch x sequence, flattened)
    r: int = 16
    alpha: float = 32.0
    base: str = "nf4"         # "nf4" or "bf16"
    pool_slots: int = 2
    single: bool = False      # single linear (no stack)
    head_dim: int = 128       # attention head width (q has hidden/head_dim heads, k and v kv/head_dim)
    seq_len: int = 1024       # rows per sequence: the T rows are T/seq_len packed sequences

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    def projections(self):
        """[(name, K_in, N_out)] for one layer."""
        if self.single:
            return [("q", self.hidden, self.hidden)]
        h, kv, it = self.hidden, self.kv, self.inter
        return [("q", h, h), ("k", h, kv), ("v", h, kv), ("o", h, h),
                ("gate", h, it), ("up", h, it), ("down", it, h)]

    def input_width(self, which: str) -> int:
        return {"h": self.hidden, "o": self.hidden, "d": self.inter}[which]

    def params_per_layer(self) -> int:
        return sum(k * n for _, k, n in self.projections())

    def nf4_bytes_per_layer(self) -> int:
        """Packed bytes of one layer's base: codes + int8 absmax + fp32 second-level scales."""
        n = self.params_per_layer()
        return n // 2 + n // 64 + 4 * (n // 16384)

    def flops_per_step(self) -> int:
        """Algorithmic FLOPs of one step (forward, recomputed forward, backward).

        Base: 6*T*K*N per projection (two forward GEMMs and the dX GEMM; the base is frozen,
        so there is no weight-gradient GEMM).  LoRA: 8*T*r*(K+N) per projection (U and U B^T
        in each forward, G and G A in dX, dB and dA).
        """
        total = 0
        for _, k, n in self.projections():
            total += 6 * self.T * k * n + 8 * self.T * self.r * (k + n)
        return total * self.layers


C1 = StackConfig("single-linear-896", layers=1, hidden=896, kv=896, inter=896, T=512, single=True,
                 pool_slots=1, head_dim=64)
C2 = StackConfig("qwen2.5-0.5b-shape", layers=24, hidden=896, kv=128, inter=4864, T=2048, head_dim=64)
C3 = StackConfig("llama-3.1-8b-shape", layers=32, hidden=4096, kv=1024, inter=14336, T=4096, seq_len=2048)
C4 = StackConfig("qwen2.5-3b-shape-bf16", layers=36, hidden=2048, kv=256, inter=11008, T=2048,
                 base="bf16")
C5 = StackConfig("qwen2.5-72b-shape", layers=80, hidden=8192, kv=1024, inter=29568, T=2048)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}
