"""The fit decision ("Soup v0.73.0 benchmarks README", record index: a peak-VRAM predictor, and a
fit decision that refuses instead of warning): every buffer a step uses lives in one arena the
stack allocates up front, the predicted peak of a step is that arena, and a stack whose arena and
set-up temporaries exceed the budget is refused before anything is allocated. The GPU test checks
the prediction against the torch allocator's measured peak of real steps (the pages' predictor:
0.85% worst-case error)."""

import gc

import pytest

from layer_streamed_nf4_dequant_amd import configs, lib
from layer_streamed_nf4_dequant_amd.stack import (Stack, arena_offsets, buffer_plan, choose_source, file_stride,
                                                  layer_layout, predict_device_bytes, predict_host_bytes)


def test_prediction_parts_add_up_and_follow_the_modes():
    cfg = configs.C3
    p = predict_device_bytes(cfg)
    raw = sum(v for k, v in p.items() if k not in ("total", "setup_extra"))
    n_buffers = len(buffer_plan(cfg))
    # the arena: every buffer, each 256-byte aligned, rounded up to whole 2 MiB
    assert raw <= p["total"] < raw + 256 * n_buffers + (2 << 20) and p["total"] % (2 << 20) == 0
    _, image = layer_layout(cfg)
    assert p["pool_slots"] == 2 * image
    assert "resident_images" not in p and "reference_outputs" not in p
    r = predict_device_bytes(cfg, modes=("streamed", "resident"), reference=True)
    assert r["resident_images"] == cfg.layers * image
    assert r["reference_outputs"] == sum(cfg.T * n * 2 for _, _, n in cfg.projections())
    t = predict_device_bytes(cfg, dequant="staged_t")
    assert t["staging"] == 2 * p["staging"]
    # a bf16 base has no staging buffers
    assert "staging" not in predict_device_bytes(configs.C4)
    # adapters and their gradients scale with the layer count; the activations do not
    p3 = predict_device_bytes(cfg, layers=3)
    assert p3["adapters"] * cfg.layers == p["adapters"] * 3 and p3["inputs"] == p["inputs"]
    # the arena offsets are 256-byte aligned and do not overlap
    off, size = arena_offsets(buffer_plan(cfg, modes=("streamed", "resident"), reference=True))
    spans = sorted((o, o + n) for (key, _, n), o in zip(buffer_plan(cfg, modes=("streamed", "resident"),
                                                                       reference=True), off.values()))
    assert all(o % 256 == 0 for o, _ in spans)
    assert all(a_end <= b0 for (_, a_end), (b0, _) in zip(spans, spans[1:])) and spans[-1][1] <= size


def test_refused_before_allocating():
    pred = predict_device_bytes(configs.C3)
    with pytest.raises(MemoryError, match="refused"):
        Stack(configs.C3, hbm_budget=pred["total"] + pred["setup_extra"] - 1)


def test_auto_source_picks_ram_then_file_then_refuses():
    """The host tier ("stream source: auto"): pinned RAM when every image fits the host budget,
    else the file tier when its two bounce buffers and one set-up image fit and the images fit
    on disk, else a refusal (MemoryError) before anything is allocated."""
    cfg = configs.C3
    _, image = layer_layout(cfg)
    ram = predict_host_bytes(cfg, "ram")
    f = predict_host_bytes(cfg, "file")
    assert ram["pinned"] == cfg.layers * image
    assert f["pinned"] == 2 * file_stride(image) and f["disk"] == cfg.layers * file_stride(image)
    assert file_stride(image) % 4096 == 0 and 0 <= file_stride(image) - image < 4096
    assert choose_source(cfg, "auto", host_budget=ram["pinned"]) == "ram"
    assert choose_source(cfg, "auto", host_budget=ram["pinned"] - 1, disk_free=f["disk"]) == "file"
    with pytest.raises(MemoryError, match="refused"):
        choose_source(cfg, "auto", host_budget=ram["pinned"] - 1, disk_free=f["disk"] - 1)
    with pytest.raises(MemoryError, match="refused"):
        choose_source(cfg, "auto", host_budget=f["pinned"] + f["setup_extra"] - 1, disk_free=10 ** 15)
    assert choose_source(cfg, "file", host_budget=0) == "file"        # an explicit tier is taken as given
    with pytest.raises(MemoryError, match="refused"):                   # the stack refuses before allocating
        Stack(cfg, hbm_budget=10 ** 15, source="auto", host_budget=1)


@pytest.mark.gpu
@pytest.mark.parametrize("name,layers,modes,reference",
                         [("C3", 3, ("streamed",), False), ("C3", 3, ("streamed", "resident"), True),
                          ("C2", None, ("streamed",), True), ("C4", 4, ("streamed",), False)])
def test_predicted_peak_matches_measured(gpu, name, layers, modes, reference):
    import torch
    cfg = configs.CONFIGS[name]
    print(f"case: predictor {name} layers={layers} modes={modes} reference={reference}", flush=True)
    gc.collect()
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = Stack(cfg, modes=modes, layers=layers, reference=reference)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    for m in modes:
        st.step(m, reference=reference)
    torch.cuda.synchronize()
    measured = torch.cuda.max_memory_allocated() - before
    want = predict_device_bytes(cfg, modes, layers=layers, reference=reference)["total"]
    print(f"  predicted {want} B, measured {measured} B", flush=True)
    # the arena is the only allocation a step holds; the caching allocator may book it in a
    # cached block up to 1 MiB larger
    assert 0 <= measured - want <= (1 << 20)
    st.close()
    del st
    gc.collect()


def test_decoder_prediction_and_refusal():
    """The decoder step's arena: every buffer 256-byte aligned and disjoint, the parts adding up,
    and a model whose arena and set-up temporaries exceed the budget refused before allocating."""
    from layer_streamed_nf4_dequant_amd.decoder import DecoderModel, decoder_buffer_plan, predict_decoder_bytes
    cfg, V = configs.C3, 128256
    p = predict_decoder_bytes(cfg, V)
    plan = decoder_buffer_plan(cfg, V)
    raw = sum(n for _, _, n in plan)
    assert raw <= p["total"] < raw + 256 * len(plan) + (2 << 20) and p["total"] % (2 << 20) == 0
    assert p["embedding_and_head"] == 2 * V * cfg.hidden * 2
    assert p["layer_checkpoints"] == (cfg.layers + 1) * cfg.T * cfg.hidden * 2
    off, size = arena_offsets(plan)
    spans = sorted((off[k], off[k] + n) for k, _, n in plan)
    assert all(a_end <= b0 for (_, a_end), (b0, _) in zip(spans, spans[1:])) and spans[-1][1] <= size
    r = predict_decoder_bytes(cfg, V, modes=("streamed", "resident"), reference=True)
    _, image = layer_layout(cfg)
    assert r["resident_images"] == cfg.layers * image and r["reference"] == 2 * cfg.T * cfg.hidden * 2 + cfg.T * 4
    with pytest.raises(MemoryError, match="refused"):
        DecoderModel(cfg, vocab=V, hbm_budget=p["total"] + p["setup_extra"] - 1)


@pytest.mark.gpu
@pytest.mark.parametrize("name,vocab", [("C2", 151936), ("C3", 128256)])
def test_decoder_predicted_peak_matches_measured(gpu, name, vocab):
    """The decoder step allocates nothing beyond its arena: the measured peak of a streamed step
    equals the prediction (to the caching allocator's block slack, far inside the pages' 0.85%),
    and the set-up's peak stays within arena + predicted set-up temporaries."""
    import torch
    from layer_streamed_nf4_dequant_amd.decoder import DecoderModel, predict_decoder_bytes
    cfg = configs.CONFIGS[name]
    print(f"case: decoder predictor {cfg.name} ({cfg.layers} layers, V {vocab})", flush=True)
    gc.collect()
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    m = DecoderModel(cfg, vocab=vocab, modes=("streamed",))
    torch.cuda.synchronize()
    setup_peak = torch.cuda.max_memory_allocated() - before
    torch.cuda.reset_peak_memory_stats()
    m.step("streamed")
    torch.cuda.synchronize()
    measured = torch.cuda.max_memory_allocated() - before
    pred = predict_decoder_bytes(cfg, vocab)
    print(f"  predicted {pred['total']} B (+{pred['setup_extra']} B set-up), measured step {measured} B, "
          f"set-up {setup_peak} B", flush=True)
    assert 0 <= measured - pred["total"] <= (1 << 20)
    assert setup_peak <= pred["total"] + pred["setup_extra"] + (1 << 20)
    m.close()
    del m
    gc.collect()
