"""A decoder-only language model trained with LoRA on a layer-streamed NF4 base: the seven
adapted projections of every layer with the glue between them, the resident embedding and LM
head, and cross-entropy on next-token labels, forward and backward.

"Exact Layer Streaming", Abstract, and "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the decoder
layers stream through a small pool of device slots from host RAM; only the adapters, their
gradients, the embedding and the output head stay resident ("Can You Fine-Tune a 27B Model on a
Laptop?", transcript @7:42-7:55); every layer crosses the host link two times in a step, for the
forward and again for the backward's recompute (transcript @7:32). The layer is the Llama-3.1 / Qwen2.5 decoder layer, whose formulas
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
from .stack import arena_offsets, layer_layout, make_pool

EPS = 1e-5
THETA = 500000.0


def activation_shapes(cfg: StackConfig, layers: int, nq: int, fuse_glue: bool = True) -> dict:
    """Per-visit activations and gradients of the decoder step (one set, reused by every layer):
    name -> (shape, dtype). With the glue fused into the projections' epilogues the o and down
    outputs before the residual add and the SwiGLU output's gradient are never stored."""
    T, H, I, kv = cfg.T, cfg.hidden, cfg.inter, cfg.kv
    th, ti, tk = (T, H), (T, I), (T, kv)
    out = {n: (th, "bf16") for n in ("y_re", "n1", "n2", "h", "q", "o_att", "dy_b", "dh_b", "do_att", "dq",
                                     "n_f", "dn_f") + (() if fuse_glue else ("a", "dproj"))}
    out.update({n: (tk, "bf16") for n in ("k", "v", "dk", "dv")})
    out.update({n: (ti, "bf16") for n in ("gate", "up", "m", "dgate", "dup") + (() if fuse_glue else ("dm",))})
    out.update({n: ((T,), "f32") for n in ("rstd1", "rstd2", "rstd_f", "loss")})
    out.update({"lse": ((T, nq), "f32"), "dy": (th, "f32"), "dn": (th, "f32")})
    return out


def decoder_workspaces(cfg: StackConfig, vocab: int, ce_chunk: int) -> dict:
    """Device workspace bytes of the step's library calls: the projections' backward (single and
    grouped), attention's backward and the chunked LM-head cross-entropy."""
    T, r = cfg.T, cfg.r
    layout, _ = layer_layout(cfg)
    descs = [lib.LoraLinearDesc(T, p.K, p.N, r, cfg.scale, lib.WeightDesc(), None, None) for p in layout]
    ws = max(lib.ws_bytes(T, p.K, p.N, r) for p in layout)
    ws = max(ws, lib.group_ws_bytes(descs[0:3]), lib.group_ws_bytes(descs[4:6]))
    n_seq, nq = T // cfg.seq_len, cfg.hidden // cfg.head_dim
    return {"ws": ws, "ws_att": lib.attention_bwd_ws_bytes(n_seq, cfg.seq_len, nq, cfg.kv // cfg.head_dim, cfg.head_dim),
            "ws_ce": lib.lm_head_ce_ws_bytes(ce_chunk, cfg.hidden, vocab)}


def decoder_buffer_plan(cfg: StackConfig, vocab: int, layers: int | None = None, modes=("streamed",),
                        dequant: str = "staged", ce_chunk: int = 2048, reference: bool = False,
                        fuse_glue: bool = True) -> list:
    """Every device buffer a decoder training step uses, in arena order: [(key, part, nbytes)]."""
    L = cfg.layers if layers is None else layers
    layout, image = layer_layout(cfg)
    T, H, r = cfg.T, cfg.hidden, cfg.r
    nq = H // cfg.head_dim
    sz = {"bf16": 2, "f32": 4, "u8": 1}
    plan = [(("E",), "embedding_and_head", vocab * H * 2), (("head",), "embedding_and_head", vocab * H * 2),
            (("g_final",), "norm_gains", H * 2)]
    for l in range(L):
        plan += [(("g1", l), "norm_gains", H * 2), (("g2", l), "norm_gains", H * 2)]
        for j, p in enumerate(layout):
            plan += [(("A", l, j), "adapters", r * p.K * 2), (("B", l, j), "adapters", p.N * r * 2),
                     (("dA", l, j), "adapter_grads", r * p.K * 4), (("dB", l, j), "adapter_grads", p.N * r * 4)]
    plan += [((k,), "tokens", T * 4) for k in ("ids", "labels", "positions")]
    plan += [(("rope_cs",), "tokens", cfg.seq_len * cfg.head_dim * 4)]
    plan += [(("x", i), "layer_checkpoints", T * H * 2) for i in range(L + 1)]
    for key, (shape, dt) in activation_shapes(cfg, L, nq, fuse_glue).items():
        plan.append(((key,), "activations", int(np.prod(shape)) * sz[dt]))
    plan += [(("U", j), "activations", T * r * 2) for j, _ in enumerate(layout)]
    plan += [((k,), "workspaces", n) for k, n in decoder_workspaces(cfg, vocab, ce_chunk).items()]
    if dequant == "staged":
        plan += [(("w_stage", j), "staging", p.N * p.K * 2) for j, p in enumerate(layout)]
    if reference:
        plan += [(("x_ref", i), "reference", T * H * 2) for i in range(2)] + [(("loss_ref",), "reference", T * 4)]
    if "streamed" in modes:
        plan += [(("slot", i), "pool_slots", image) for i in range(cfg.pool_slots)]
    if "resident" in modes:
        plan += [(("resident", l), "resident_images", image) for l in range(L)]
    return plan


def predict_decoder_bytes(cfg: StackConfig, vocab: int, layers: int | None = None, modes=("streamed",),
                          dequant: str = "staged", ce_chunk: int = 2048, reference: bool = False,
                          fuse_glue: bool = True) -> dict:
    """Peak device memory of a decoder training step, from the shapes alone ("Soup v0.73.0
    benchmarks README", record index: a peak-VRAM predictor whose fit decision refuses): the step
    allocates nothing beyond its arena, so the step's peak is the arena. Also returned: the
    set-up's largest extra temporaries (the embedding or head drawn in fp32 and rounded to bf16,
    or one base weight in fp32 with its layer image and the packing workspace), which the fit
    decision adds. Returns the parts, their "total" and "setup_extra"."""
    plan = decoder_buffer_plan(cfg, vocab, layers, modes, dequant, ce_chunk, reference, fuse_glue)
    parts = {}
    for _, part, nbytes in plan:
        parts[part] = parts.get(part, 0) + nbytes
    _, parts["total"] = arena_offsets(plan)
    layout, image = layer_layout(cfg)
    big = max(layout, key=lambda p: p.K * p.N)
    pack = (allocator_block_bytes(big.K * big.N * 4) + allocator_block_bytes(lib.load().nf4_pack_ws_bytes(big.N, big.K))
            + (allocator_block_bytes(image) if "resident" not in modes else 0))
    emb = allocator_block_bytes(vocab * cfg.hidden * 4) + allocator_block_bytes(vocab * cfg.hidden * 2)
    parts["setup_extra"] = max(emb, pack)
    return parts


def allocator_block_bytes(n: int) -> int:
    """Bytes torch's caching allocator books for a fresh n-byte device allocation: the size
    rounded to 512 B; a large one gets a segment of whole 2 MiB, and when less than 1 MiB of that
    segment would remain the block keeps all of it (the remainder is too small to split off)."""
    size = (n + 511) // 512 * 512
    if size <= (1 << 20):
        return size
    seg = (size + (2 << 20) - 1) // (2 << 20) * (2 << 20)
    return seg if seg - size < (1 << 20) else size


class DecoderModel:
    """Frozen NF4 base (streamed or resident), LoRA adapters on all seven projections, resident
    embedding / final norm / LM head, packed sequences of cfg.seq_len rows.

    Streaming overlaps a layer's copy (on the copy stream) with the compute of the layers before
    it only while the two streams sit on different hardware queues of the process: a copy's
    completion marker on a queue shared with compute work blocks the kernels queued behind it.
    HIP maps streams onto GPU_MAX_HW_QUEUES queues (4 by default); a process that creates many
    streams should raise it (bench.py and the microbenchmarks take 16) before its first HIP call."""

    def __init__(self, cfg: StackConfig, vocab: int, layers: int | None = None, seed: int = 0,
                 modes=("streamed",), dequant: str = "staged", eps: float = EPS, theta: float = THETA,
                 ce_chunk: int = 2048, label_rows: int | None = None, hbm_budget: int | None = None,
                 reference: bool = False, fuse_glue: bool = True):
        """label_rows: keep the next-token label on only this many rows (a seeded sample of the
        rows that have one) and ignore the rest, so that the loss, and the gradient flowing back
        from it, come from a sample of positions. hbm_budget: device bytes the model may take
        (default: the free memory the device reports); the predicted arena plus the set-up's
        temporaries (predict_decoder_bytes) must fit, else MemoryError before anything is
        allocated. reference: also place the reference sweep's buffers in the arena (otherwise
        the first reference step allocates them). fuse_glue: the rotary embedding, the residual
        adds and the SwiGLU (forward and backward) run in the epilogues of the projections and
        of attention's backward (the same bits as the separate glue kernels, which
        fuse_glue=False runs)."""
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
        self.fuse = bool(fuse_glue)
        self.n_seq, self.nq, self.nkv, self.d = T // cfg.seq_len, H // d, cfg.kv // d, d
        self.dev = torch.device("cuda")
        self.layout, self.image_bytes = layer_layout(cfg)
        self.names = [p.name for p in self.layout]
        self.j = {n: i for i, n in enumerate(self.names)}
        bf16, f32 = torch.bfloat16, torch.float32
        dev = self.dev
        key0 = ("decoder", cfg.name, vocab)
        self.ce_chunk = ce_chunk

        # ---- the fit decision, then every step buffer carved from one arena allocated first ----
        pred = predict_decoder_bytes(cfg, vocab, self.L, modes, dequant, ce_chunk, reference, self.fuse)
        need = pred["total"] + pred["setup_extra"]
        budget = hbm_budget if hbm_budget is not None else torch.cuda.mem_get_info()[0]
        if need > budget:
            raise MemoryError(f"{cfg.name} decoder: needs {need} B of device memory (predicted: {pred['total']} B "
                              f"arena + {pred['setup_extra']} B during set-up), {budget} B available: refused")
        self.compute = torch.cuda.Stream()
        self.copy_stream = torch.cuda.Stream()
        plan = decoder_buffer_plan(cfg, vocab, self.L, modes, dequant, ce_chunk, reference, self.fuse)
        offsets, arena_bytes = arena_offsets(plan)
        self.arena = torch.empty(arena_bytes, dtype=torch.uint8, device=dev)
        sizes = {key: nbytes for key, _, nbytes in plan}

        def buf(key, shape, dtype):
            o = offsets[key]
            return self.arena[o:o + sizes[key]].view(dtype).view(shape)

        # ---- frozen base: per-layer NF4 images in pinned host memory (and on the device) ----
        self.means = np.zeros((self.L, len(self.layout)), dtype=np.float32)
        self.host_images, self.resident = [], ([] if "resident" in modes else None)
        big = max(self.layout, key=lambda p: p.K * p.N)
        ws_pack = torch.empty(lib.load().nf4_pack_ws_bytes(big.N, big.K), dtype=torch.uint8, device=dev)
        for l in range(self.L):
            if self.resident is not None:
                dev_img = buf(("resident", l), (self.image_bytes,), torch.uint8)
                dev_img.zero_()
            else:
                dev_img = torch.zeros(self.image_bytes, dtype=torch.uint8, device=dev)
            for j, p in enumerate(self.layout):
                w = self.base_weight(l, p.name)
                n = p.K * p.N
                self.means[l, j] = lib.nf4_pack_into(
                    w, dev_img[p.codes:p.codes + n // 2], dev_img[p.qabsmax:p.qabsmax + n // 64].view(torch.int8),
                    dev_img[p.absmax2:p.absmax2 + 4 * (n // 16384)].view(f32), ws_pack)
                del w
            img = torch.empty(self.image_bytes, dtype=torch.uint8, pin_memory=True)
            img.copy_(dev_img)
            self.host_images.append(img)
            if self.resident is not None:
                self.resident.append(dev_img)
            else:
                del dev_img
        del ws_pack
        torch.cuda.synchronize()

        # ---- resident frozen parts and trainable adapters (seeded, synthetic) ----
        self.E = buf(("E",), (vocab, H), bf16)
        self.E.copy_(inputs.device_normal((vocab, H), 1.0, seed, *key0, "E", dtype=bf16))
        self.W_head = buf(("head",), (vocab, H), bf16)
        self.W_head.copy_(inputs.device_normal((vocab, H), 0.02, seed, *key0, "head", dtype=bf16))
        self.g_final = buf(("g_final",), (H,), bf16)
        self.g_final.copy_(self._gain(H, "g_final"))
        self.g1, self.g2 = [], []
        for l in range(self.L):
            self.g1.append(buf(("g1", l), (H,), bf16))
            self.g1[-1].copy_(self._gain(H, "g1", l))
            self.g2.append(buf(("g2", l), (H,), bf16))
            self.g2[-1].copy_(self._gain(H, "g2", l))
        self.A, self.B, self.dA, self.dB = [], [], [], []
        for l in range(self.L):
            key = ("decoder", cfg.name, l)
            Al, Bl = [], []
            for j, p in enumerate(self.layout):
                Al.append(buf(("A", l, j), (r, p.K), bf16))
                Al[-1].copy_(inputs.device_uniform((r, p.K), 1.0 / np.sqrt(p.K), seed, *key, p.name, "A", dtype=bf16))
                Bl.append(buf(("B", l, j), (p.N, r), bf16))
                Bl[-1].copy_(inputs.device_normal((p.N, r), inputs.STD["B"], seed, *key, p.name, "B", dtype=bf16))
            self.A.append(Al)
            self.B.append(Bl)
            self.dA.append([buf(("dA", l, j), (r, p.K), f32).zero_() for j, p in enumerate(self.layout)])
            self.dB.append([buf(("dB", l, j), (p.N, r), f32).zero_() for j, p in enumerate(self.layout)])

        # ---- tokens: packed sequences, next-token labels (the last row of a sequence ignored) ----
        ids = torch.randint(0, vocab, (T,), generator=inputs.device_generator(seed, *key0, "ids"), device=dev,
                            dtype=torch.int32)
        lab = torch.roll(ids, -1)
        lab[cfg.seq_len - 1::cfg.seq_len] = -1
        if label_rows is not None:
            order = torch.randperm(T, generator=inputs.device_generator(seed, *key0, "label rows"), device=dev)
            has = order[lab[order] >= 0][:label_rows]
            keep = torch.zeros(T, dtype=torch.bool, device=dev)
            keep[has] = True
            lab = torch.where(keep, lab, torch.full_like(lab, -1))
        self.ids = buf(("ids",), (T,), torch.int32)
        self.ids.copy_(ids)
        self.labels = buf(("labels",), (T,), torch.int32)
        self.labels.copy_(lab)
        del ids, lab
        self.n_counted = int((self.labels >= 0).sum())
        self.positions = buf(("positions",), (T,), torch.int32)
        self.positions.copy_(torch.arange(T, device=dev, dtype=torch.int32) % cfg.seq_len)
        self.rope_cs = buf(("rope_cs",), (cfg.seq_len, d // 2, 2), f32)
        lib.rope_table(cfg.seq_len, d, theta, out=self.rope_cs)
        self.rope = lib.rope_desc(self.rope_cs, cfg.seq_len, d, self.positions)

        # ---- activations and gradients ----
        for key, (shape, dt) in activation_shapes(cfg, self.L, self.nq, self.fuse).items():
            setattr(self, key, buf((key,), shape, {"bf16": bf16, "f32": f32, "u8": torch.uint8}[dt]))
        self.x = [buf(("x", i), (T, H), bf16) for i in range(self.L + 1)]   # layer inputs, final hidden
        self.U = [buf(("U", j), (T, r), bf16) for j, _ in enumerate(self.layout)]
        for key in ("ws", "ws_att", "ws_ce"):
            setattr(self, key, buf((key,), (sizes[(key,)],), torch.uint8))
        self.w_stage = ([buf(("w_stage", j), (p.N, p.K), bf16) for j, p in enumerate(self.layout)]
                        if dequant == "staged" else None)
        self.recompute_ok = []
        self.x_ref = self.loss_ref = None
        if reference:
            self.x_ref = [buf(("x_ref", i), (T, H), bf16) for i in range(2)]
            self.loss_ref = buf(("loss_ref",), (T,), f32)

        # ---- pool ----
        self.pool, self.slots = None, None
        if "streamed" in modes:
            self.slots = [buf(("slot", i), (self.image_bytes,), torch.uint8) for i in range(cfg.pool_slots)]
            self.pool = make_pool(self.slots, self.image_bytes, self.L, self.copy_stream, 0)
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
    def _layer_fwd(self, base: int, l: int, x, y, s, adapters: bool = True, keep: bool = True):
        """y = layer l applied to x (keeps the intermediates the backward needs). adapters=False:
        the frozen base alone (the reference model), U untouched. keep=False: a forward whose
        backward recomputes the layer; the MLP's gate and up outputs need not be stored."""
        J, U = self.j, self.U
        mode = lib.ADAPTERS_U_READY if adapters else lib.ADAPTERS_OFF
        d = lambda n: self._desc(base, l, n)  # noqa: E731
        us = lambda names: [U[J[n]] for n in names] if adapters else None  # noqa: E731
        lib.rmsnorm_fwd(x, self.g1[l], self.eps, self.n1, self.rstd1, stream=s)
        qkv = ("q", "k", "v")
        if adapters:
            lib.lora_down(self.n1, [self.A[l][J[n]] for n in qkv], us(qkv), stream=s)
        if self.fuse:
            # q and k leave the GEMM rotated
            lib.lora_linear_fwd_group_epi([d(n) for n in qkv], self.n1, [self.q, self.k, self.v], us(qkv),
                                          adapters=mode, rope_mask=0b011, rope=self.rope, ws=self.ws, stream=s)
        else:
            lib.lora_linear_fwd_group([d(n) for n in qkv], self.n1, [self.q, self.k, self.v], us(qkv),
                                      adapters=mode, ws=self.ws, stream=s)
            lib.rope_apply(self.q, self.positions, self.nq, self.d, self.theta, stream=s)
            lib.rope_apply(self.k, self.positions, self.nkv, self.d, self.theta, stream=s)
        lib.attention_fwd(self.q, self.k, self.v, self.o_att, self.lse, self.n_seq, self.nq, self.nkv, self.d,
                          stream=s)
        if self.fuse:
            # h = x + o-projection, added in the GEMM's epilogue
            # (U of o, and of down below, is computed by the call itself: ADAPTERS_ON)
            lib.lora_linear_fwd_group_epi([d("o")], self.o_att, [self.h], us(("o",)), adapters=adapters,
                                          residual=[x], ws=self.ws, stream=s)
        else:
            lib.lora_linear_fwd(d("o"), self.o_att, self.a, U[J["o"]] if adapters else None, adapters=adapters,
                                ws=self.ws, stream=s)
            lib.add_bf16(x, self.a, self.h, stream=s)
        lib.rmsnorm_fwd(self.h, self.g2[l], self.eps, self.n2, self.rstd2, stream=s)
        gu = ("gate", "up")
        if adapters:
            lib.lora_down(self.n2, [self.A[l][J[n]] for n in gu], us(gu), stream=s)
        if self.fuse:
            # m = silu(gate) up in the gate/up GEMM's epilogue (gate and up stored when kept)
            store = keep or self.dequant != "staged"
            Ug, Uu = us(gu) if adapters else (None, None)
            lib.lora_linear_fwd_swiglu(d("gate"), d("up"), self.n2, self.m, gate=self.gate if store else None,
                                       up=self.up if store else None, Ug=Ug, Uu=Uu, adapters=mode, ws=self.ws,
                                       stream=s)
            lib.lora_linear_fwd_group_epi([d("down")], self.m, [y], us(("down",)), adapters=adapters,
                                          residual=[self.h], ws=self.ws, stream=s)
        else:
            lib.lora_linear_fwd_group([d(n) for n in gu], self.n2, [self.gate, self.up], us(gu), adapters=mode,
                                      ws=self.ws, stream=s)
            lib.swiglu_fwd(self.gate, self.up, self.m, stream=s)
            lib.lora_linear_fwd(d("down"), self.m, self.dproj, U[J["down"]] if adapters else None,
                                adapters=adapters, ws=self.ws, stream=s)
            lib.add_bf16(self.h, self.dproj, y, stream=s)

    def _layer_bwd(self, base: int, l: int, x, s, grad_mode: int):
        """self.dy (fp32, the gradient of the layer's output; self.dy_b its bf16 copy) becomes the
        gradient of its input x (and self.dy_b that one's bf16 copy); dA, dB of the layer's seven
        projections are set (GRAD_SET) or added to (GRAD_ADD)."""
        J, U, dA, dB = self.j, self.U, self.dA[l], self.dB[l]
        d = lambda n: self._desc(base, l, n)  # noqa: E731
        jd = J["down"]
        if self.fuse:
            # the SwiGLU's backward in the down projection's dX epilogue
            lib.lora_linear_bwd_swiglu(d("down"), self.m, self.dy_b, U[jd], self.gate, self.up, self.dgate, self.dup,
                                       dA[jd], dB[jd], grad_mode=grad_mode, ws=self.ws, stream=s)
        else:
            lib.lora_linear_bwd(d("down"), self.m, self.dy_b, U[jd], self.dm, dA[jd], dB[jd],
                                dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
            lib.swiglu_bwd(self.gate, self.up, self.dm, self.dgate, self.dup, stream=s)
        gu = ("gate", "up")
        lib.lora_linear_bwd_group([d(n) for n in gu], self.n2, [self.dgate, self.dup],
                                  [U[J[n]] for n in gu], self.dn, [dA[J[n]] for n in gu], [dB[J[n]] for n in gu],
                                  dx_mode=lib.DX_F32_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        lib.rmsnorm_bwd(self.h, self.g2[l], self.rstd2, self.dn, self.dy, accumulate=True, dx_bf16=self.dh_b,
                        stream=s)                                                                   # dy = dh
        lib.lora_linear_bwd(d("o"), self.o_att, self.dh_b, U[J["o"]], self.do_att, dA[J["o"]],
                            dB[J["o"]], dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        if self.fuse:
            # dq and dk rotated back as attention's backward stores them
            lib.attention_bwd_rope(self.q, self.k, self.v, self.o_att, self.lse, self.do_att, self.dq, self.dk,
                                   self.dv, self.ws_att, self.n_seq, self.nq, self.nkv, self.d, self.rope, stream=s)
        else:
            lib.attention_bwd(self.q, self.k, self.v, self.o_att, self.lse, self.do_att, self.dq, self.dk, self.dv,
                              self.ws_att, self.n_seq, self.nq, self.nkv, self.d, stream=s)
            lib.rope_apply(self.dq, self.positions, self.nq, self.d, self.theta, inverse=True, stream=s)
            lib.rope_apply(self.dk, self.positions, self.nkv, self.d, self.theta, inverse=True, stream=s)
        qkv = ("q", "k", "v")
        lib.lora_linear_bwd_group([d(n) for n in qkv], self.n1, [self.dq, self.dk, self.dv],
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
                    self._layer_fwd(base, l, self.x[l], self.x[l + 1], s, keep=False)
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
            self._layer_fwd(base, l, self.x_ref[l % 2], self.x_ref[(l + 1) % 2], s, adapters=False, keep=False)
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
