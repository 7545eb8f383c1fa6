"""The layer-streamed projection stack: one training step's forward, recomputed forward and
backward through every adapted projection of every decoder layer, with the frozen base
streamed through a small device pool.

"Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @7:11-7:32: the
frozen base sits in host RAM, one decoder layer at a time is copied into a small on-card
buffer on a separate stream while the previous layer computes, and every layer crosses the
host link two times in a step (for the forward, and again for the backward's recompute). "Exact Layer Streaming", Abstract: the
streamed run must be bit-identical to a resident run of the same numerics, forward and every
LoRA gradient checked separately; the pages' own probe deletes every host-to-device byte.

Modes
  streamed  layers stream from pinned host images through the C-ABI layer pool (K slots)
  resident  every layer image lives in its own device buffer (byte-identical); no copies
  no_h2d    the pool's slots, but no copies at all: a timing probe (results are not valid)

Every kernel call goes through the C ABI (layer_streamed_nf4_dequant_amd.lib); torch only
allocates memory, provides streams and times them.

The synthetic stack (the projections are the path; attention, norms and the MLP activation
sit outside it here, and decoder.py runs them around the same kernels and pool): every layer
reads the same seeded inputs X_h (attention input, read by q, k,
v, gate, up), X_o (attention output, read by o) and X_d (MLP intermediate, read by down); W, A
and B are distinct per layer. Upstream gradients: q, k, v and o always get their own seeded
dY; the top layer's gate, up and down do too, but below it the backward is chained the way a
residual stream chains it, so that every layer's LoRA gradients depend on the base weights of
the layer above: for layer l < L-1, down's dY is dX_o of layer l+1 and gate's and up's dY is
dX_d of layer l+1 (both bf16, and both computed from seeded gradients, so the chain stays
bounded). A layer that read another layer's bytes therefore changes the forward outputs, the
input gradients and the LoRA gradients below it.
"""

from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

from . import inputs, lib
from .configs import PROJ_INPUT, StackConfig

ALIGN = 256


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


@dataclass
class ProjLayout:
    name: str
    K: int
    N: int
    off: int              # byte offset of the projection inside the layer image
    codes: int = 0        # offsets relative to the image (NF4)
    qabsmax: int = 0
    absmax2: int = 0
    w16: int = 0          # offset of the bf16 W (bf16 base)


def layer_layout(cfg: StackConfig) -> tuple[list[ProjLayout], int]:
    """Byte layout of one layer image: each projection's arrays at 256-byte aligned offsets."""
    projs, off = [], 0
    for name, K, N in cfg.projections():
        n = K * N
        p = ProjLayout(name, K, N, off)
        if cfg.base == "nf4":
            p.codes = off
            off = _align(off + n // 2)
            p.qabsmax = off
            off = _align(off + n // 64)
            p.absmax2 = off
            off = _align(off + 4 * (n // 16384))
        else:
            p.w16 = off
            off = _align(off + 2 * n)
        projs.append(p)
    return projs, _align(off)


MIB2 = 2 << 20
AUDIT_CAPACITY = 16384          # pool checksums between two audits (2 per layer visit)
FILE_ALIGN = 4096               # layer images in the file tier's file start on 4 KiB boundaries


def file_stride(image_bytes: int) -> int:
    """Bytes per layer in the file tier's file: the image padded to whole 4 KiB blocks (what an
    O_DIRECT read needs; a buffered read ignores the padding)."""
    return (image_bytes + FILE_ALIGN - 1) // FILE_ALIGN * FILE_ALIGN


def host_memory_available() -> int:
    """Host RAM the kernel reports as available for new allocations (MemAvailable)."""
    with open("/proc/meminfo") as f:
        for ln in f:
            if ln.startswith("MemAvailable:"):
                return int(ln.split()[1]) * 1024
    raise OSError("no MemAvailable in /proc/meminfo")


def predict_host_bytes(cfg: StackConfig, source: str, layers=None) -> dict:
    """Host memory and disk a stack's frozen base needs per tier: "ram" keeps every layer image in
    pinned host memory; "file" keeps them in one file (disk) and pins only the file tier's two
    bounce buffers (plus, during set-up, one layer image on its way to the file)."""
    L = cfg.layers if layers is None else layers
    _, image = layer_layout(cfg)
    if source == "ram":
        return {"pinned": L * image, "disk": 0}
    if source == "file":
        return {"pinned": 2 * file_stride(image), "setup_extra": image, "disk": L * file_stride(image)}
    raise ValueError(source)


def choose_source(cfg: StackConfig, source: str, host_budget: int | None = None, disk_free: int | None = None,
                  layers=None) -> str:
    """The host tier of the frozen base ("An 8B Fine-Tune Now Fits in 4 GB of VRAM", the adoption
    settings: the stream source picks RAM when the images fit and NVMe when they do not; "Soup
    v0.73.0 benchmarks README", reading conventions: a run that does not fit is stopped, not merely warned about).
    source "ram" or "file" is taken as given; "auto" picks "ram" when every pinned image fits
    the host budget (default: MemAvailable), else "file" when its bounce buffers fit the budget
    and the images fit the free disk space, else raises MemoryError before anything is
    allocated."""
    if source in ("ram", "file"):
        return source
    if source != "auto":
        raise ValueError(source)
    budget = host_memory_available() if host_budget is None else host_budget
    ram = predict_host_bytes(cfg, "ram", layers)
    if ram["pinned"] <= budget:
        return "ram"
    f = predict_host_bytes(cfg, "file", layers)
    if f["pinned"] + f["setup_extra"] <= budget and (disk_free is None or f["disk"] <= disk_free):
        return "file"
    raise MemoryError(f"{cfg.name}: the frozen base needs {ram['pinned']} B of pinned host memory, or "
                      f"{f['pinned'] + f['setup_extra']} B of host memory and {f['disk']} B of disk "
                      f"({budget} B of host memory and {disk_free} B of disk available): refused")


def make_pool(slots, slot_bytes: int, n_layers: int, copy_stream, flags: int):
    """A layer pool over the given device slots, with the caller-owned memory its flags need
    allocated here: the audit's checksum array (device, LSN_POOL_AUDIT), the file tier's two
    pinned bounce buffers (LSN_POOL_FILE_TIER) and, for O_DIRECT reads, two plain staging buffers
    (LSN_POOL_FILE_DIRECT). They stay referenced by the returned pool object for its lifetime."""
    import torch
    keep, audit, bounce, stage = [], None, None, None
    if flags & lib.POOL_AUDIT:
        sums = torch.zeros(AUDIT_CAPACITY, dtype=torch.int64, device="cuda")
        keep.append(sums)
        audit = (sums.data_ptr(), AUDIT_CAPACITY)
    if flags & lib.POOL_FILE_TIER:
        bufs = [torch.empty(slot_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        keep += bufs
        bounce = (bufs[0].data_ptr(), bufs[1].data_ptr())
    if flags & lib.POOL_FILE_DIRECT:
        # plain host memory, 4 KiB aligned, for the O_DIRECT reads (pinned memory cannot take them)
        st = []
        for _ in range(2):
            raw = np.empty(slot_bytes + FILE_ALIGN, dtype=np.uint8)
            st.append(raw[(-raw.ctypes.data) % FILE_ALIGN:][:slot_bytes])
        keep += st
        stage = (st[0].ctypes.data, st[1].ctypes.data)
    pool = lib.LayerPool([t.data_ptr() for t in slots], slot_bytes, n_layers, copy_stream.cuda_stream, flags,
                         audit_sums=audit, bounce=bounce, direct_stage=stage)
    pool.memory = keep
    return pool


def workspace_bytes(cfg: StackConfig) -> int:
    """The shared backward workspace the stack allocates (the largest single-linear need, or the
    grouped need of the linears that read X_h)."""
    T, r = cfg.T, cfg.r
    layout, _ = layer_layout(cfg)
    ws = max(lib.ws_bytes(T, p.K, p.N, r) for p in layout)
    hj = [p for p in layout if PROJ_INPUT[p.name] == "h"]
    if len(hj) > 1:
        probe = [lib.LoraLinearDesc(T, p.K, p.N, r, cfg.scale, lib.WeightDesc(), None, None) for p in hj]
        ws = max(ws, lib.group_ws_bytes(probe))
    return ws


def buffer_plan(cfg: StackConfig, modes=("streamed",), dequant: str = "staged", layers=None,
                reference: bool = False) -> list:
    """Every device buffer a training step uses, in arena order: [(key, part, nbytes)]. The stack
    carves them all from one arena allocated up front (the pages' pre-allocated device buffers),
    so a step allocates nothing."""
    L = cfg.layers if layers is None else layers
    layout, image = layer_layout(cfg)
    T, r = cfg.T, cfg.r
    if cfg.base != "nf4":
        dequant = "fused"
    plan = []
    for l in range(L):
        for j, p in enumerate(layout):
            plan += [(("A", l, j), "adapters", r * p.K * 2), (("B", l, j), "adapters", p.N * r * 2),
                     (("dA", l, j), "adapter_grads", r * p.K * 4), (("dB", l, j), "adapter_grads", p.N * r * 4)]
    plan += [(("X", w), "inputs", T * cfg.input_width(w) * 2) for w in ("h", "o", "d")]
    plan += [(("dY", j), "upstream_grads", T * p.N * 2) for j, p in enumerate(layout)]
    for name in ("Y", "Yre"):
        plan += [((name, j), "outputs", T * p.N * 2) for j, p in enumerate(layout)]
    plan += [(("U", j), "outputs", T * r * 2) for j, _ in enumerate(layout)]
    plan += [(("dX_h",), "input_grads", T * cfg.hidden * 4)]
    plan += [(("dX_o", i), "input_grads", T * cfg.hidden * 2) for i in range(2)]
    plan += [(("dX_d", i), "input_grads", T * cfg.inter * 2) for i in range(2)]
    plan += [(("ws",), "workspace", workspace_bytes(cfg))]
    if dequant in ("staged", "staged_t"):
        plan += [(("w_stage", j), "staging", p.N * p.K * 2) for j, p in enumerate(layout)]
    if dequant == "staged_t":
        plan += [(("w_stage_t", j), "staging", p.K * p.N * 2) for j, p in enumerate(layout)]
    if "streamed" in modes or "no_h2d" in modes:
        plan += [(("slot", i), "pool_slots", image) for i in range(cfg.pool_slots)]
    if "resident" in modes:
        plan += [(("resident", l), "resident_images", image) for l in range(L)]
    if reference:
        plan += [(("Yref", j), "reference_outputs", T * p.N * 2) for j, p in enumerate(layout)]
    return plan


def arena_offsets(plan) -> tuple[dict, int]:
    """Byte offset of every buffer (256-byte aligned) and the arena size (a whole number of
    2 MiB, the caching allocator's large-segment granule, so that it books exactly this size)."""
    off, at = {}, 0
    for key, _, nbytes in plan:
        at = _align(at)
        off[key] = at
        at += nbytes
    return off, (at + MIB2 - 1) // MIB2 * MIB2


def predict_device_bytes(cfg: StackConfig, modes=("streamed",), dequant: str = "staged", layers=None,
                         reference: bool = False) -> dict:
    """Peak device memory of a training step, from the shapes alone ("Soup v0.73.0 benchmarks
    README", record index: a peak-VRAM predictor, and a fit decision that refuses instead of
    warning). Every buffer a step uses lives in the stack's arena and a step allocates nothing
    more, so the step's peak is the arena: adapters and their gradients, the shared activations,
    upstream gradients and outputs, the workspace, the staging buffers, and the pool slots
    (streamed) or the resident images. Also returned: the set-up's extra temporaries (one
    weight generated in fp32, a layer image being packed, and the packing workspace), which the
    fit decision adds. Returns the parts, their "total" and "setup_extra"."""
    plan = buffer_plan(cfg, modes, dequant, layers, reference)
    parts = {}
    for _, part, nbytes in plan:
        parts[part] = parts.get(part, 0) + nbytes
    _, parts["total"] = arena_offsets(plan)
    layout, image = layer_layout(cfg)
    big = max(layout, key=lambda p: p.K * p.N)
    pack_ws = lib.load().nf4_pack_ws_bytes(big.N, big.K) if cfg.base == "nf4" else 0
    parts["setup_extra"] = big.K * big.N * 4 + (image if "resident" not in modes else 0) + pack_ws
    return parts


class Stack:
    """Owns the host images, device state and buffers of one configuration.

    Streaming overlaps a layer's copy (on the copy stream) with the compute of the layers before
    it only while the two streams sit on different hardware queues of the process: a copy's
    completion marker on a queue shared with compute work blocks the kernels queued behind it.
    HIP maps streams onto GPU_MAX_HW_QUEUES queues (4 by default); a process that creates many
    streams should raise it (bench.py and the microbenchmarks take 16) before its first HIP call."""

    def __init__(self, cfg: StackConfig, seed: int = 0, modes=("streamed",), audit: bool = False,
                 keep_at_turn: bool = False, fault: int = 0, record: bool = False, layers=None,
                 dequant: str = "staged", hbm_budget: int | None = None, reference: bool = False,
                 source: str = "ram", host_budget: int | None = None, image_dir: str | None = None):
        """hbm_budget: device bytes the stack may take; by default the free memory the device
        reports. The predicted arena plus the set-up's temporaries (predict_device_bytes) must
        fit, else MemoryError before anything is allocated. reference: also place the reference
        sweep's outputs in the arena (otherwise the first reference step allocates them).
        source: the host tier of the frozen base, "ram" (pinned images), "file" (one file read
        by the pool's file tier; nothing but its bounce buffers pinned) or "auto" (choose_source
        with host_budget, default MemAvailable); image_dir: where the file goes (default: a new
        temporary directory)."""
        import torch
        self.torch = torch
        self.cfg = cfg
        self.L = cfg.layers if layers is None else layers
        self.image_dir = image_dir
        disk_free = None
        if source == "auto":
            import shutil
            import tempfile
            disk_free = shutil.disk_usage(image_dir or tempfile.gettempdir()).free
        self.source = choose_source(cfg, source, host_budget, disk_free, self.L)
        pred = predict_device_bytes(cfg, modes, dequant, self.L, reference)
        need = pred["total"] + pred["setup_extra"]
        budget = hbm_budget if hbm_budget is not None else torch.cuda.mem_get_info()[0]
        if need > budget:
            raise MemoryError(f"{cfg.name}: the stack needs {need} B of device memory (predicted: "
                              f"{pred['total']} B arena + {pred['setup_extra']} B during set-up), "
                              f"{budget} B available: refused")
        self.seed = seed
        self.dev = torch.device("cuda")
        self.layout, self.image_bytes = layer_layout(cfg)
        self.record = record
        # "staged":   each visit dequantises every NF4 projection (nf4_dequant, HBM-bound) into
        #             bf16 staging buffers W [N][K] that all the visit's GEMMs read: the forward,
        #             the recompute and the dX product (a reduction over N, which reads W
        #             reduction-major);
        # "staged_t": as "staged", but the backward visit also stages W^T [K][N] and the dX
        #             product reads that (both operands N-contiguous);
        # "fused":    the GEMMs dequantise their W tiles straight into LDS (no staging buffer).
        # All three hand the matrix cores the same bf16 fragments: the forward outputs and every
        # single-projection backward are identical bits. The grouped backward of the projections
        # that share X_h sums their input gradients in a different order (staged: one GEMM over
        # their concatenated reduction; fused: member by member), so dX_h, and what depends on it,
        # agree across modes to fp32 rounding.
        if dequant not in ("staged", "staged_t", "fused"):
            raise ValueError(dequant)
        self.dequant = dequant if cfg.base == "nf4" else "fused"
        self.compute = torch.cuda.Stream()
        self.copy_stream = torch.cuda.Stream()
        T, r = cfg.T, cfg.r
        bf16 = torch.bfloat16

        # ---- the arena: every buffer a step uses, allocated once, first ----
        plan = buffer_plan(cfg, modes, self.dequant, self.L, reference)
        offsets, arena_bytes = arena_offsets(plan)
        self.arena = torch.empty(arena_bytes, dtype=torch.uint8, device=self.dev)
        sizes = {key: nbytes for key, _, nbytes in plan}

        def buf(key, shape, dtype):
            o = offsets[key]
            return self.arena[o:o + sizes[key]].view(dtype).view(shape)

        # ---- frozen base: generated on the device per layer, packed, kept in pinned host images
        # (source "ram") or written to the file tier's file (source "file")
        self.means = np.zeros((self.L, len(self.layout)), dtype=np.float32)
        self.host_images = [] if self.source == "ram" else None
        self.image_file = None
        out_file = self._open_image_file() if self.source == "file" else None
        self.resident = [] if "resident" in modes else None
        scratch_w = None
        for l in range(self.L):
            if self.resident is not None:
                dev_img = buf(("resident", l), (self.image_bytes,), torch.uint8)
                dev_img.zero_()
            else:
                dev_img = torch.zeros(self.image_bytes, dtype=torch.uint8, device=self.dev)
            for j, p in enumerate(self.layout):
                w = inputs.device_normal((p.N, p.K), inputs.STD["W"], seed, cfg.name, l, p.name, "W")
                if cfg.base == "nf4":
                    n = p.K * p.N
                    codes = dev_img[p.codes:p.codes + n // 2]
                    qabs = dev_img[p.qabsmax:p.qabsmax + n // 64].view(torch.int8)
                    abs2 = dev_img[p.absmax2:p.absmax2 + 4 * (n // 16384)].view(torch.float32)
                    nb = lib.load().nf4_pack_ws_bytes(p.N, p.K)
                    if scratch_w is None or scratch_w.numel() < nb:
                        scratch_w = torch.empty(nb, dtype=torch.uint8, device=self.dev)
                    self.means[l, j] = lib.nf4_pack_into(w, codes, qabs, abs2, scratch_w)
                else:
                    dev_img[p.w16:p.w16 + 2 * p.K * p.N].view(bf16).copy_(w.view(-1).to(bf16))
                del w
            if out_file is None:
                img = torch.empty(self.image_bytes, dtype=torch.uint8, pin_memory=True)
                img.copy_(dev_img)
                self.host_images.append(img)
            else:
                self._write_layer(out_file, dev_img.cpu().numpy())
            if self.resident is not None:
                self.resident.append(dev_img)
            else:
                del dev_img
        if out_file is not None:
            out_file.close()
        torch.cuda.synchronize()

        # ---- trainable adapters and their gradients (resident) ----
        self.A, self.B, self.dA, self.dB = [], [], [], []
        for l in range(self.L):
            Al, Bl, dAl, dBl = [], [], [], []
            for j, p in enumerate(self.layout):
                key = (cfg.name, l, p.name)
                Al.append(buf(("A", l, j), (r, p.K), bf16))
                Al[-1].copy_(inputs.device_uniform((r, p.K), 1.0 / np.sqrt(p.K), seed, *key, "A", dtype=bf16))
                Bl.append(buf(("B", l, j), (p.N, r), bf16))
                Bl[-1].copy_(inputs.device_normal((p.N, r), inputs.STD["B"], seed, *key, "B", dtype=bf16))
                dAl.append(buf(("dA", l, j), (r, p.K), torch.float32).zero_())
                dBl.append(buf(("dB", l, j), (p.N, r), torch.float32).zero_())
            self.A.append(Al)
            self.B.append(Bl)
            self.dA.append(dAl)
            self.dB.append(dBl)

        # ---- shared activations and upstream gradients ----
        self.X = {}
        for w in ("h", "o", "d"):
            self.X[w] = buf(("X", w), (T, cfg.input_width(w)), bf16)
            self.X[w].copy_(inputs.device_normal((T, cfg.input_width(w)), 1.0, seed, cfg.name, "X", w, dtype=bf16))
        self.dY = []
        for j, p in enumerate(self.layout):
            self.dY.append(buf(("dY", j), (T, p.N), bf16))
            self.dY[-1].copy_(inputs.device_normal((T, p.N), 1.0, seed, cfg.name, "dY", p.name, dtype=bf16))
        self.Y = [buf(("Y", j), (T, p.N), bf16) for j, p in enumerate(self.layout)]
        self.Yre = [buf(("Yre", j), (T, p.N), bf16) for j, p in enumerate(self.layout)]
        self.Yref = [buf(("Yref", j), (T, p.N), bf16) for j, p in enumerate(self.layout)] if reference else None
        self.U = [buf(("U", j), (T, r), bf16) for j, _ in enumerate(self.layout)]
        self.dX_h = buf(("dX_h",), (T, cfg.hidden), torch.float32).zero_()
        # dX_o and dX_d ping-pong by layer parity: layer l reads layer l+1's as upstream gradients
        self.dX_o_pp = [buf(("dX_o", i), (T, cfg.hidden), bf16) for i in range(2)]
        self.dX_d_pp = [buf(("dX_d", i), (T, cfg.inter), bf16) for i in range(2)]
        self.h_group = [j for j, p in enumerate(self.layout) if PROJ_INPUT[p.name] == "h"]
        self.ws = buf(("ws",), (sizes[("ws",)],), torch.uint8)
        self.w_stage = self.w_stage_t = None
        if self.dequant in ("staged", "staged_t"):
            self.w_stage = [buf(("w_stage", j), (p.N, p.K), bf16) for j, p in enumerate(self.layout)]
        if self.dequant == "staged_t":
            self.w_stage_t = [buf(("w_stage_t", j), (p.K, p.N), bf16) for j, p in enumerate(self.layout)]

        # ---- pool (streamed) or fixed slots (no_h2d) ----
        self.pool = None
        self.slots = None
        if "streamed" in modes or "no_h2d" in modes:
            self.slots = [buf(("slot", i), (self.image_bytes,), torch.uint8) for i in range(cfg.pool_slots)]
        if "streamed" in modes:
            flags = (lib.POOL_AUDIT if audit else 0) | (lib.POOL_KEEP_AT_TURN if keep_at_turn else 0) | fault
            self.reset_pool(flags)
        self.checks = {}
        torch.cuda.synchronize()

    def reset_pool(self, flags: int = 0, n_slots: int | None = None, source: str | None = None,
                   direct: bool = False):
        """(Re)create the layer pool with the given flags and slot count over the same images.
        source "ram": the pinned host images; "file": the same bytes in one file (the pool's
        file tier reads them; written on first use from the pinned images when the stack keeps
        them, see write_image_file); None: the stack's own tier. direct: the file tier reads with
        O_DIRECT (past the page cache: a read of the storage device)."""
        torch = self.torch
        torch.cuda.synchronize()
        if self.pool is not None:
            self.pool.close()
            self.pool = None
        if n_slots is not None and n_slots != len(self.slots):
            self.slots = [torch.empty(self.image_bytes, dtype=torch.uint8, device=self.dev)
                          for _ in range(n_slots)]
        source = self.source if source is None else source
        if source == "file":
            path = self.write_image_file()
            flags |= lib.POOL_FILE_TIER | (lib.POOL_FILE_DIRECT if direct else 0)
        elif source != "ram" or self.host_images is None:
            raise ValueError(f"source {source!r} is not available for this stack (its tier: {self.source})")
        # O_DIRECT reads whole 4 KiB blocks into the bounce buffers and slots are 4 KiB multiples
        slot_bytes = file_stride(self.image_bytes) if direct else self.image_bytes
        if direct and any(t.numel() < slot_bytes or t.data_ptr() % FILE_ALIGN for t in self.slots):
            self.slots = [torch.empty(slot_bytes + FILE_ALIGN, dtype=torch.uint8, device=self.dev)
                          for _ in self.slots]
            self.slots = [t[(-t.data_ptr()) % FILE_ALIGN:][:slot_bytes] for t in self.slots]
        self.pool = make_pool(self.slots, slot_bytes, self.L, self.copy_stream, flags)
        stride = file_stride(self.image_bytes)
        for l in range(self.L):
            if source == "file":
                self.pool.register_file(l, path, l * stride, self.image_bytes)
            else:
                self.pool.register(l, self.host_images[l].data_ptr(), self.image_bytes)

    def _open_image_file(self):
        import tempfile
        d = tempfile.mkdtemp(prefix="lsnf4_images_", dir=self.image_dir)
        self.image_file = os.path.join(d, "layers.bin")
        return open(self.image_file, "wb")

    def _write_layer(self, f, img: np.ndarray) -> None:
        """Appends one layer image and its padding to whole 4 KiB blocks."""
        f.write(memoryview(img))
        pad = file_stride(img.size) - img.size
        if pad:
            f.write(bytes(pad))

    def write_image_file(self) -> str:
        """The file tier's file: the layer images, each at a 4 KiB aligned offset (l * stride,
        the image padded to whole 4 KiB blocks), in `image_dir` (else a new temporary directory);
        written from the pinned images on first use, or at set-up when the stack keeps no pinned
        images. Removed by close()."""
        if self.image_file is None:
            with self._open_image_file() as f:
                for img in self.host_images:
                    self._write_layer(f, img.numpy())
        return self.image_file

    # ------------------------------------------------------------------------------------------
    def _nf4_desc(self, base: int, l: int, j: int) -> lib.NF4Desc:
        p = self.layout[j]
        return lib.NF4Desc(p.N, p.K, base + p.codes, base + p.qabsmax, base + p.absmax2, float(self.means[l, j]))

    def _stage(self, base: int, l: int, s, backward: bool = False):
        """Dequantise every projection of the layer image at `base` into the staging buffers
        (and, in "staged_t" mode on the backward visit, into the transposed ones too)."""
        descs = [self._nf4_desc(base, l, j) for j in range(len(self.layout))]
        lib.nf4_dequant_batch(descs, self.w_stage, "bf16", stream=s)
        if backward and self.dequant == "staged_t":
            lib.nf4_dequant_batch(descs, self.w_stage_t, "bf16_t", stream=s)

    def _desc(self, base: int, l: int, j: int, backward: bool = False) -> lib.LoraLinearDesc:
        p, cfg = self.layout[j], self.cfg
        if self.dequant in ("staged", "staged_t"):
            if backward and self.dequant == "staged_t":
                w = lib.WeightDesc(lib.W_BF16_T, lib.NF4Desc(), self.w_stage_t[j].data_ptr())
            else:
                w = lib.WeightDesc(lib.W_BF16, lib.NF4Desc(), self.w_stage[j].data_ptr())
            return lib.LoraLinearDesc(cfg.T, p.K, p.N, cfg.r, cfg.scale, w, self.A[l][j].data_ptr(),
                                      self.B[l][j].data_ptr())
        if cfg.base == "nf4":
            w = lib.WeightDesc(lib.W_NF4, lib.NF4Desc(p.N, p.K, base + p.codes, base + p.qabsmax,
                                                      base + p.absmax2, float(self.means[l, j])), None)
        else:
            w = lib.WeightDesc(lib.W_BF16, lib.NF4Desc(), base + p.w16)
        return lib.LoraLinearDesc(cfg.T, p.K, p.N, cfg.r, cfg.scale, w, self.A[l][j].data_ptr(),
                                  self.B[l][j].data_ptr())

    def _forward_layer(self, base: int, l: int, Y, s, gemm_events=None, adapters: bool = True):
        # per shared input (q, k, v, gate and up read X_h; o reads X_o; down reads X_d): the
        # adapters' down-projections in one pass over the input, then the projections' forward
        # GEMMs as one grouped launch (adapters off: the frozen base alone, Y = bf16(X W^T))
        for which in ("h", "o", "d"):
            js = [j for j, p in enumerate(self.layout) if PROJ_INPUT[p.name] == which]
            if not js:
                continue
            if adapters:
                lib.lora_down(self.X[which], [self.A[l][j] for j in js], [self.U[j] for j in js], stream=s)
            if gemm_events is not None:
                gemm_events.append((js, self.torch.cuda.Event(enable_timing=True),
                                    self.torch.cuda.Event(enable_timing=True)))
                gemm_events[-1][1].record(s)
            lib.lora_linear_fwd_group([self._desc(base, l, j) for j in js], self.X[which], [Y[j] for j in js],
                                      [self.U[j] for j in js], adapters=lib.ADAPTERS_U_READY if adapters else False,
                                      ws=self.ws, stream=s)
            if gemm_events is not None:
                gemm_events[-1][2].record(s)

    def upstream(self, l: int, j: int):
        """The upstream gradient dY of projection j in layer l (see the module docstring)."""
        name = self.layout[j].name
        if l < self.L - 1:
            if name == "down" and not self.cfg.single:
                return self.dX_o_pp[(l + 1) % 2]
            if name in ("gate", "up"):
                return self.dX_d_pp[(l + 1) % 2]
        return self.dY[j]

    @property
    def dX_o(self):
        return self.dX_o_pp[0]

    @property
    def dX_d(self):
        return self.dX_d_pp[0]

    def _backward_layer(self, base: int, l: int, s, grad_mode: int = lib.GRAD_SET):
        # q, k, v, gate and up read X_h: their input gradients add up in dX_h (fp32), as one
        # grouped backward (a single GEMM over their concatenated N when staged)
        hj = self.h_group
        lib.lora_linear_bwd_group([self._desc(base, l, j, backward=True) for j in hj], self.X["h"],
                                  [self.upstream(l, j) for j in hj], [self.U[j] for j in hj], self.dX_h,
                                  [self.dA[l][j] for j in hj], [self.dB[l][j] for j in hj],
                                  dx_mode=lib.DX_F32_SET, grad_mode=grad_mode, ws=self.ws, stream=s)
        for j, p in enumerate(self.layout):
            which = PROJ_INPUT[p.name]
            if which == "h":
                continue
            dX = self.dX_o_pp[l % 2] if which == "o" else self.dX_d_pp[l % 2]
            lib.lora_linear_bwd(self._desc(base, l, j, backward=True), self.X[which], self.upstream(l, j), self.U[j], dX,
                                self.dA[l][j], self.dB[l][j], dx_mode=lib.DX_BF16_SET, grad_mode=grad_mode,
                                ws=self.ws, stream=s)

    def _record(self, tag: str, l: int, tensors):
        """Position-weighted integer checksums of the outputs (exact, order-independent sums
        modulo 2^64), kept on the device."""
        torch = self.torch
        for j, t in enumerate(tensors):
            v = (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).reshape(-1)
            n = v.numel()
            if getattr(self, "_wvec", None) is None or self._wvec.numel() < n:
                self._wvec = torch.arange(1, n + 1, device=v.device, dtype=torch.int64)
            self.checks[(tag, l, j)] = (v.to(torch.int64) * self._wvec[:n]).sum()

    def step(self, mode: str = "streamed", gemm_events=None, dequant_events=None, wait: bool = True,
             reference: bool = False, micro_batches: int = 1, on_visit=None):
        """One training step of the projection stack; returns its time in ms (compute stream).
        gemm_events: optional list; (projections, start, end) HIP events around every forward
        GEMM launch (one per group of projections sharing an input) are appended to it.
        dequant_events: optional list; ((visit, with_transposed), start, end) around every visit's
        staging, visit "fwd" or "bwd", with_transposed when the visit also staged W^T.
        wait=False returns the step's (start, end) events without waiting for them, so the next
        step's first layer copies can be queued while this step's last visits still run.
        reference=True first runs the frozen reference model's forward: one more streamed sweep
        over every layer with the adapters off, into Yref ("An 8B Fine-Tune Now Fits in 4 GB of
        VRAM", the DPO paragraph: preference objectives take their frozen reference model from
        the same streamed base run without its adapters, so no second copy of the weights is
        needed, only more layer reads per step; here 3 per layer instead of 2).
        It changes no training state: the step's outputs and gradients are those of a step
        without it.
        micro_batches=k: gradient accumulation ("Exact Layer Streaming", Abstract: accumulation is
        per-token I/O-neutral): k forward/backward passes, each streaming every layer twice, the
        first setting dA, dB and the others adding into them (a step then trains on k x T
        tokens). The stack's inputs are the same for every micro-batch, so after k = 2 each
        gradient is exactly twice the single pass's (x + x is exact in fp32).
        on_visit: optional callable(visit, l), visit "fwd" or "bwd", called once the layer's work
        of that visit is queued on the compute stream (and is the current stream), before the
        layer is released: work it queues sees that visit's outputs (Y after "fwd"; Yre, dX_h
        and the layer's dX_o / dX_d after "bwd") before the next layer overwrites them."""
        torch = self.torch
        s = self.compute
        sh = s.cuda_stream
        L = self.L
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            start.record(s)
            # with K slots, up to K-1 layers are in flight ahead of the one being computed
            ahead = len(self.slots) - 1 if self.slots is not None else 0
            # ---- reference model (adapters off): layers 0 .. L-1 ----
            if reference:
                if self.Yref is None:          # not planned in the arena: allocated on first use
                    self.Yref = [torch.empty_like(y) for y in self.Y]
                for l in range(L):
                    base = self._visit_base(mode, l, sh, ahead, forward=True)
                    if self.dequant != "fused":
                        self._stage(base, l, s)
                    self._forward_layer(base, l, self.Yref, s, adapters=False)
                    if self.record:
                        self._record("ref", l, self.Yref)
                    if mode == "streamed":
                        self.pool.release(l, sh)
            for mb in range(micro_batches):
                grad_mode = lib.GRAD_SET if mb == 0 else lib.GRAD_ADD
                # ---- forward: layers 0 .. L-1 ----
                for l in range(L):
                    base = self._visit_base(mode, l, sh, ahead, forward=True)
                    if self.dequant != "fused":
                        self._timed(dequant_events, ("fwd", False), s, lambda: self._stage(base, l, s))
                    self._forward_layer(base, l, self.Y, s, gemm_events)
                    if self.record:
                        self._record("fwd", l, self.Y)
                    if on_visit is not None:
                        on_visit("fwd", l)
                    if mode == "streamed":
                        self.pool.release(l, sh)
                # ---- backward: layers L-1 .. 0, each re-read and recomputed ----
                for l in reversed(range(L)):
                    base = self._visit_base(mode, l, sh, ahead, forward=False)
                    if self.dequant != "fused":                               # re-dequantised per visit
                        self._timed(dequant_events, ("bwd", self.dequant == "staged_t"), s,
                                    lambda: self._stage(base, l, s, backward=True))
                    self._forward_layer(base, l, self.Yre, s, gemm_events)   # recompute
                    self._backward_layer(base, l, s, grad_mode)
                    if self.record:
                        self._record("re", l, self.Yre)
                        self._record("dx", l, [self.dX_h, self.dX_o_pp[l % 2], self.dX_d_pp[l % 2]])
                    if on_visit is not None:
                        on_visit("bwd", l)
                    if mode == "streamed":
                        self.pool.release(l, sh)
            end.record(s)
        if not wait:
            return start, end
        end.synchronize()
        return start.elapsed_time(end)

    def _visit_base(self, mode: str, l: int, sh, ahead: int, forward: bool) -> int:
        """Device address of layer l's image for this visit (streamed: prefetch the next layers in
        the sweep's direction and acquire l; the caller releases it)."""
        if mode == "streamed":
            nxt = range(l, min(self.L, l + 1 + ahead)) if forward else range(l, max(-1, l - 1 - ahead), -1)
            for a in nxt:
                self.pool.prefetch(a)
            return self.pool.acquire(l, sh)
        if mode == "resident":
            return self.resident[l].data_ptr()
        return self.slots[l % len(self.slots)].data_ptr()

    def _timed(self, events, tag, s, fn):
        if events is None:
            return fn()
        e0, e1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        events.append((tag, e0, e1))

    def h2d_rate(self, reps: int = 4) -> float:
        """Host-to-device bandwidth (GB/s) of one layer image into a slot on the copy stream."""
        torch = self.torch
        torch.cuda.synchronize()
        src = self.host_images
        if src is None:                          # file tier: one pinned buffer of an image's size
            src = [torch.empty(self.image_bytes, dtype=torch.uint8, pin_memory=True)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.copy_stream):
            e0.record(self.copy_stream)
            for i in range(reps):
                self.slots[i % len(self.slots)][:self.image_bytes].copy_(src[i % len(src)], non_blocking=True)
            e1.record(self.copy_stream)
        e1.synchronize()
        return reps * self.image_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9

    def grads(self):
        return self.dA, self.dB

    def drop_image_file(self):
        """Removes the file tier's file (written by write_image_file), when the pool no longer
        reads it (a stack whose own tier is the file keeps it)."""
        path = getattr(self, "image_file", None)
        if path is not None:
            os.remove(path)
            os.rmdir(os.path.dirname(path))
            self.image_file = None

    def close(self):
        if self.pool is not None:
            self.pool.close()
            self.pool = None
        self.drop_image_file()
