"""A decoder-only language model trained with LoRA on a layer-streamed NF4 base: the seven
adapted projections of every layer with the glue between them, the resident embedding and LM
head, and cross-entropy on next-token labels, forward and backward.

"Exact Layer Streaming", Abstract, and "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the decoder
layers stream through a small pool of device slots from host RAM; only the adapters, their
gradients, the embedding and the output head stay resident ("Can You Fine-Tune a 27B Model on a
Laptop?", transcript @7:42-7:55); each layer is read twice per step, forward and the backward's
recompute (transcript @7:32). The layer is the Llama-3.1 / Qwen2.5 decoder layer, whose formulas
the pages do not print (the published definitions):

    n1 = RMSNorm(x; g1);  q, k, v = LoRA projections of n1;  RoPE on q and k
    a  = o-projection( causal grouped-query attention(q, k, v) );  h = x + a
    n2 = RMSNorm(h; g2);  m = silu(gate(n2)) * up(n2);  y = h + down(m)

The residual stream and every stored activation are bf16; the residual stream's gradient is
fp32. The step checkpoints only each layer's input x_l; the backward visit of layer l re-reads
its base, recomputes the layer from x_l (its output is compared bit for bit with x_{l+1}, a free
aliasing check), and runs the backward through it. Every operation is a call through the C ABI
(layer_streamed_nf4_dequant_amd.lib); torch allocates memory, provides streams and times them.
"""

from __future__ import annotations

import numpy as np

from . import inputs, lib
from .configs import StackConfig
from .stack import layer_layout

EPS = 1e-5
THETA = 500000.0


class DecoderModel:
    """Frozen NF4 base (streamed or resident), LoRA adapters on all seven projections, resident
    embedding / final norm / LM head, packed sequences of cfg.seq_len rows."""

    def __init__(self, cfg: StackConfig, vocab: int, layers: int | None = None, seed: int = 0,
                 modes=("streamed",), dequant: str = "staged", eps: float = EPS, theta: float = THETA,
                 ce_chunk: int = 2048):
        import torch
        self.torch = torch
        self.cfg, self.V, self.seed = cfg, vocab, seed
        self.L = cfg.layers if layers is None else layers
        self.eps, self.theta = eps, theta
        T, H, I, r, d = cfg.T, cfg.hidden, cfg.inter, cfg.r, cfg.head_dim
        if T % cfg.seq_len or H % d or cfg.kv % d or cfg.base != "nf4" or cfg.single:
            raise ValueError("DecoderModel needs an NF4 stack with T a multiple of seq_len and whole heads")
        if dequant not in ("staged", "fused"):
            raise ValueError(dequant)
        self.dequant = dequant
        self.n_seq, self.nq, self.nkv, self.d = T // cfg.seq_len, H // d, cfg.kv // d, d
        self.dev = torch.device("cuda")
        self.compute = torch.cuda.Stream()
        self.copy_stream = torch.cuda.Stream()
        self.layout, self.image_bytes = layer_layout(cfg)
        self.names = [p.name for p in self.layout]
        self.j = {n: i for i, n in enumerate(self.names)}
        bf16, f32 = torch.bfloat16, torch.float32
        dev = self.dev
        key0 = ("decoder", cfg.name, vocab)

        # ---- frozen base: per-layer NF4 images in pinned host memory (and on the device) ----
        self.means = np.zeros((self.L, len(self.layout)), dtype=np.float32)
        self.host_images, self.resident = [], ([] if "resident" in modes else None)
        for l in range(self.L):
            dev_img = torch.zeros(self.image_bytes, dtype=torch.uint8, device=dev)
            for j, p in enumerate(self.layout):
                w = self.base_weight(l, p.name)
                n = p.K * p.N
                ws = torch.empty(lib.load().nf4_pack_ws_bytes(p.N, p.K), dtype=torch.uint8, device=dev)
                self.means[l, j] = lib.nf4_pack_into(
                    w, dev_img[p.codes:p.codes + n // 2], dev_img[p.qabsmax:p.qabsmax + n // 64].view(torch.int8),
                    dev_img[p.absmax2:p.absmax2 + 4 * (n // 16384)].view(f32), ws)
                del w, ws
            img = torch.empty(self.image_bytes, dtype=torch.uint8, pin_memory=True)
            img.copy_(dev_img)
            self.host_images.append(img)
            if self.resident is not None:
                self.resident.append(dev_img)
            else:
                del dev_img
        torch.cuda.synchronize()

        # ---- resident frozen parts and trainable adapters (seeded, synthetic) ----
        self.E = inputs.device_normal((vocab, H), 1.0, seed, *key0, "E", dtype=bf16)
        self.W_head = inputs.device_normal((vocab, H), 0.02, seed, *key0, "head", dtype=bf16)
        self.g_final = self._gain(H, "g_final")
        self.g1 = [self._gain(H, "g1", l) for l in range(self.L)]
        self.g2 = [self._gain(H, "g2", l) for l in range(self.L)]
        self.A, self.B, self.dA, self.dB = [], [], [], []
        for l in range(self.L):
            key = ("decoder", cfg.name, l)
            self.A.append([inputs.device_uniform((r, p.K), 1.0 / np.sqrt(p.K), seed, *key, p.name, "A", dtype=bf16)
                           for p in self.layout])
            self.B.append([inputs.device_normal((p.N, r), inputs.STD["B"], seed, *key, p.name, "B", dtype=bf16)
                           for p in self.layout])
            self.dA.append([torch.zeros((r, p.K), dtype=f32, device=dev) for p in self.layout])
            self.dB.append([torch.zeros((p.N, r), dtype=f32, device=dev) for p in self.layout])

        # ---- tokens: packed sequences, next-token labels (the last row of a sequence ignored) ----
        ids = torch.randint(0, vocab, (T,), generator=inputs.device_generator(seed, *key0, "ids"), device=dev,
                            dtype=torch.int32)
        self.ids = ids
        lab = torch.roll(ids, -1)
        lab[cfg.seq_len - 1::cfg.seq_len] = -1
        self.labels = lab.contiguous()
        self.n_counted = T - self.n_seq
        self.positions = (torch.arange(T, device=dev, dtype=torch.int32) % cfg.seq_len).contiguous()

        # ---- activations and gradients ----
        e = lambda shape, dt=bf16: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        self.x = [e((T, H)) for _ in range(self.L + 1)]          # checkpoints: layer inputs, final hidden
        self.y_re = e((T, H))                                    # the recompute's layer output
        self.n1, self.n2, self.h, self.a, self.dproj = e((T, H)), e((T, H)), e((T, H)), e((T, H)), e((T, H))
        self.rstd1, self.rstd2, self.rstd_f = e((T,), f32), e((T,), f32), e((T,), f32)
        self.q, self.k, self.v = e((T, H)), e((T, cfg.kv)), e((T, cfg.kv))
        self.o_att, self.lse = e((T, H)), e((T, self.nq), f32)
        self.gate, self.up, self.m = e((T, I)), e((T, I)), e((T, I))
        self.U = [e((T, r)) for _ in self.layout]
        self.dy, self.dn = e((T, H), f32), e((T, H), f32)
        self.dy_b, self.dh_b, self.do_att = e((T, H)), e((T, H)), e((T, H))
        self.dm, self.dgate, self.dup = e((T, I)), e((T, I)), e((T, I))
        self.dq, self.dk, self.dv = e((T, H)), e((T, cfg.kv)), e((T, cfg.kv))
        self.n_f, self.dn_f = e((T, H)), e((T, H))
        self.loss = e((T,), f32)
        self.ce_chunk = ce_chunk
        descs = [lib.LoraLinearDesc(T, p.K, p.N, r, cfg.scale, lib.WeightDesc(), None, None) for p in self.layout]
        ws = max(lib.ws_bytes(T, p.K, p.N, r) for p in self.layout)
        ws = max(ws, lib.group_ws_bytes(descs[0:3]), lib.group_ws_bytes(descs[4:6]))
        self.ws = e((ws,), torch.uint8)
        self.ws_att = e((lib.attention_bwd_ws_bytes(self.n_seq, cfg.seq_len, self.nq),), torch.uint8)
        self.ws_ce = e((lib.lm_head_ce_ws_bytes(ce_chunk, H, vocab),), torch.uint8)
        self.w_stage = [e((p.N, p.K)) for p in self.layout] if dequant == "staged" else None
        self.recompute_ok = []
        self.x_ref = self.loss_ref = None

        # ---- pool ----
        self.pool, self.slots = None, None
        if "streamed" in modes:
            self.slots = [torch.empty(self.image_bytes, dtype=torch.uint8, device=dev) for _ in range(cfg.pool_slots)]
            self.pool = lib.LayerPool([t.data_ptr() for t in self.slots], self.image_bytes, self.L,
                                      self.copy_stream.cuda_stream, 0)
            for l in range(self.L):
                self.pool.register(l, self.host_images[l].data_ptr(), self.image_bytes)
        torch.cuda.synchronize()

    # -------------------------------------------------------------------------------------------
    def base_weight(self, l: int, name: str):
        """The fp32 base weight W [N][K] of projection `name` in layer l, as the seeded generator
        draws it (on the device) before packing."""
        p = self.layout[self.j[name]]
        return inputs.device_normal((p.N, p.K), inputs.STD["W"], self.seed, "decoder", self.cfg.name, l, p.name, "W")

    def _gain(self, H, *key):
        t = inputs.device_normal((H,), 0.1, self.seed, "decoder", self.cfg.name, *key)
        return (t + 1.0).to(self.torch.bfloat16)

    def _desc(self, base: int, l: int, name: str) -> lib.LoraLinearDesc:
        j = self.j[name]
        p, cfg = self.layout[j], self.cfg
        if self.dequant == "staged":
            w = lib.WeightDesc(lib.W_BF16, lib.NF4Desc(), self.w_stage[j].data_ptr())
        else:
            w = lib.WeightDesc(lib.W_NF4, lib.NF4Desc(p.N, p.K, base + p.codes, base + p.qabsmax, base + p.absmax2,
                                                      float(self.means[l, j])), None)
        return lib.LoraLinearDesc(cfg.T, p.K, p.N, cfg.r, cfg.scale, w, self.A[l][j].data_ptr(),
                                  self.B[l][j].data_ptr())

    def _stage(self, base: int, l: int, s):
        if self.dequant != "staged":
            return
        descs = [lib.NF4Desc(p.N, p.K, base + p.codes, base + p.qabsmax, base + p.absmax2, float(self.means[l, j]))
                 for j, p in enumerate(self.layout)]
        lib.nf4_dequant_batch(descs, self.w_stage, "bf16", stream=s)

    def _base(self, mode: str, l: int, sh, forward: bool) -> int:
        if mode == "streamed":
            ahead = len(self.slots) - 1
            nxt = range(l, min(self.L, l + 1 + ahead)) if forward else range(l, max(-1, l - 1 - ahead), -1)
            for a in nxt:
                self.pool.prefetch(a)
            return self.pool.acquire(l, sh)
        return self.resident[l].data_ptr()

    # -------------------------------------------------------------------------------------------
    def _layer_fwd(self, base: int, l: int, x, y, s, adapters: bool = True):
        """y = layer l applied to x (keeps the intermediates the backward needs). adapters=False:
        the frozen base alone (the reference model), U untouched."""
        J, U = self.j, self.U
        mode = lib.ADAPTERS_U_READY if adapters else lib.ADAPTERS_OFF
        lib.rmsnorm_fwd(x, self.g1[l], self.eps, self.n1, self.rstd1, stream=s)
        qkv = ("q", "k", "v")
        if adapters:
            lib.lora_down(self.n1, [self.A[l][J[n]] for n in qkv], [U[J[n]] for n in qkv], stream=s)
        lib.lora_linear_fwd_group([self._desc(base, l, n) for n in qkv], self.n1, [self.q, self.k, self.v],
                                  [U[J[n]] for n in qkv] if adapters else None, adapters=mode, ws=self.ws, stream=s)
        lib.rope_apply(self.q, self.positions, self.nq, self.d, self.theta, stream=s)
        lib.rope_apply(self.k, self.positions, self.nkv, self.d, self.theta, stream=s)
        lib.attention_fwd(self.q, self.k, self.v, self.o_att, self.lse, self.n_seq, self.nq, self.nkv, self.d,
                          stream=s)
        lib.lora_linear_fwd(self._desc(base, l, "o"), self.o_att, self.a, U[J["o"]] if adapters else None,
                            adapters=adapters, ws=self.ws, stream=s)
        lib.add_bf16(x, self.a, self.h, stream=s)
        lib.rmsnorm_fwd(self.h, self.g2[l], self.eps, self.n2, self.rstd2, stream=s)
        gu = ("gate", "up")
        if adapters:
            lib.lora_down(self.n2, [self.A[l][J[n]] for n in gu], [U[J[n]] for n in gu], stream=s)
        lib.lora_linear_fwd_group([self._desc(base, l, n) for n in gu], self.n2, [self.gate, self.up],
                                  [U[J[n]] for n in gu] if adapters else None, adapters=mode, ws=self.ws, stream=s)
        lib.swiglu_fwd(self.gate, self.up, self.m, stream=s)
        lib.lora_linear_fwd(self._desc(base, l, "down"), self.m, self.dproj, U[J["down"]] if adapters else None,
                            adapters=adapters, ws=self.ws, stream=s)
        lib.add_bf16(self.h, self.dproj, y, stream=s)

    def _layer_bwd(self, base: int, l: int, x, s, grad_mode: int):
        """self.dy (fp32, the gradient of the layer's output; self.dy_b its bf16 copy) becomes the
        gradient of its input x (and self.dy_b that one's bf16 copy); dA, dB of the layer's seven
        projections are set (GRAD_SET) or added to (GRAD_ADD)."""
        J, U, dA, dB = self.j, self.U, self.dA[l], self.dB[l]
        lib.lora_linear_bwd(self._desc(base, l, "down"), self.m, self.dy_b, U[J["down"]], self.dm, dA[J["down"]],
                            dB[J["down"]], dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        lib.swiglu_bwd(self.gate, self.up, self.dm, self.dgate, self.dup, stream=s)
        gu = ("gate", "up")
        lib.lora_linear_bwd_group([self._desc(base, l, n) for n in gu], self.n2, [self.dgate, self.dup],
                                  [U[J[n]] for n in gu], self.dn, [dA[J[n]] for n in gu], [dB[J[n]] for n in gu],
                                  dx_mode=lib.DX_F32_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        lib.rmsnorm_bwd(self.h, self.g2[l], self.rstd2, self.dn, self.dy, accumulate=True, dx_bf16=self.dh_b,
                        stream=s)                                                                   # dy = dh
        lib.lora_linear_bwd(self._desc(base, l, "o"), self.o_att, self.dh_b, U[J["o"]], self.do_att, dA[J["o"]],
                            dB[J["o"]], dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        lib.attention_bwd(self.q, self.k, self.v, self.o_att, self.lse, self.do_att, self.dq, self.dk, self.dv,
                          self.ws_att, self.n_seq, self.nq, self.nkv, self.d, stream=s)
        lib.rope_apply(self.dq, self.positions, self.nq, self.d, self.theta, inverse=True, stream=s)
        lib.rope_apply(self.dk, self.positions, self.nkv, self.d, self.theta, inverse=True, stream=s)
        qkv = ("q", "k", "v")
        lib.lora_linear_bwd_group([self._desc(base, l, n) for n in qkv], self.n1, [self.dq, self.dk, self.dv],
                                  [U[J[n]] for n in qkv], self.dn, [dA[J[n]] for n in qkv], [dB[J[n]] for n in qkv],
                                  dx_mode=lib.DX_F32_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        lib.rmsnorm_bwd(x, self.g1[l], self.rstd1, self.dn, self.dy, accumulate=True, dx_bf16=self.dy_b,
                        stream=s)                                                                   # dy = dx

    # -------------------------------------------------------------------------------------------
    def step(self, mode: str = "streamed", micro_batches: int = 1, check_recompute: bool = False,
             reference: bool = False) -> float:
        """One training step (forward, loss, backward with per-layer recompute); returns its time in
        ms on the compute stream. The mean loss over counted rows is self.mean_loss().
        micro_batches=k: k passes over the same rows, the first setting dA, dB, the others adding.
        check_recompute: compare each recomputed layer output with the forward's checkpoint of the
        next layer's input, bit for bit (device flags in self.recompute_ok; waits for nothing).
        reference=True first streams every layer once more with the adapters off (the frozen
        reference model of DPO-style objectives, "An 8B Fine-Tune Now Fits in 4 GB of VRAM": no
        second copy of the weights, more layer reads) and leaves its per-row loss in
        self.loss_ref (the reference log-likelihood of each label is -loss_ref). It changes no
        training state."""
        if mode == "streamed" and self.pool is None or mode == "resident" and self.resident is None \
                or mode not in ("streamed", "resident"):
            raise ValueError(f"mode {mode!r} was not built for this model")
        torch = self.torch
        s = self.compute
        sh = s.cuda_stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.recompute_ok = []
        with torch.cuda.stream(s):
            e0.record(s)
            if reference:
                self._reference_sweep(mode, s)
            for mb in range(micro_batches):
                grad_mode = lib.GRAD_SET if mb == 0 else lib.GRAD_ADD
                lib.embedding_gather(self.ids, self.E, self.x[0], stream=s)
                for l in range(self.L):
                    base = self._base(mode, l, sh, forward=True)
                    self._stage(base, l, s)
                    self._layer_fwd(base, l, self.x[l], self.x[l + 1], s)
                    if mode == "streamed":
                        self.pool.release(l, sh)
                # final norm, LM head and cross-entropy (mean over counted rows)
                xL = self.x[self.L]
                lib.rmsnorm_fwd(xL, self.g_final, self.eps, self.n_f, self.rstd_f, stream=s)
                lib.lm_head_ce(self.n_f, self.W_head, self.labels, 1.0 / self.n_counted, self.loss, self.dn_f,
                               self.ce_chunk, self.ws_ce, stream=s)
                lib.convert(self.dn_f, self.dn, stream=s)
                lib.rmsnorm_bwd(xL, self.g_final, self.rstd_f, self.dn, self.dy, accumulate=False,
                                dx_bf16=self.dy_b, stream=s)
                for l in reversed(range(self.L)):
                    base = self._base(mode, l, sh, forward=False)
                    self._stage(base, l, s)
                    self._layer_fwd(base, l, self.x[l], self.y_re, s)            # recompute
                    if check_recompute:
                        self.recompute_ok.append((self.y_re.view(torch.int16) == self.x[l + 1].view(torch.int16)).all())
                    self._layer_bwd(base, l, self.x[l], s, grad_mode)
                    if mode == "streamed":
                        self.pool.release(l, sh)
            e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1)

    def _reference_sweep(self, mode: str, s):
        sh = s.cuda_stream
        torch = self.torch
        if self.x_ref is None:
            self.x_ref = [torch.empty_like(self.x[0]) for _ in range(2)]
            self.loss_ref = torch.empty_like(self.loss)
        lib.embedding_gather(self.ids, self.E, self.x_ref[0], stream=s)
        for l in range(self.L):
            base = self._base(mode, l, sh, forward=True)
            self._stage(base, l, s)
            self._layer_fwd(base, l, self.x_ref[l % 2], self.x_ref[(l + 1) % 2], s, adapters=False)
            if mode == "streamed":
                self.pool.release(l, sh)
        xL = self.x_ref[self.L % 2]
        lib.rmsnorm_fwd(xL, self.g_final, self.eps, self.n_f, self.rstd_f, stream=s)
        lib.lm_head_ce(self.n_f, self.W_head, self.labels, 1.0 / self.n_counted, self.loss_ref, self.dn_f,
                       self.ce_chunk, self.ws_ce, stream=s)

    def mean_loss(self) -> float:
        return float(self.loss.sum() / self.n_counted)

    def close(self):
        if self.pool is not None:
            self.pool.close()
            self.pool = None
