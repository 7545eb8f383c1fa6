"""GPU parity of NF4 pack and dequant against the oracle: bit-exact, full tensors.

The dequant tests feed the oracle's own packed arrays to the kernel, so dequant is checked
independently of the GPU pack. Shapes: the single 896x896 linear, the smallest legal tensor,
an 8B-shaped gate projection (14336x4096) and a 72B-shaped q projection (8192x8192).
"""

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import inputs, lib
from oracle import nf4

pytestmark = pytest.mark.gpu


def _to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_packed_on_device(p, torch):
    return lib.NF4Tensor(p["rows"], p["cols"], _to_dev(p["codes"], torch),
                         _to_dev(p["qabsmax"], torch), _to_dev(p["absmax2"], torch), float(p["mean"]))


def _check_pack(w_host, gpu_packed):
    p = nf4.pack(w_host)
    np.testing.assert_array_equal(gpu_packed.codes.cpu().numpy(), p["codes"])
    np.testing.assert_array_equal(gpu_packed.qabsmax.cpu().numpy(), p["qabsmax"])
    np.testing.assert_array_equal(gpu_packed.absmax2.cpu().numpy().view(np.uint32),
                                  p["absmax2"].view(np.uint32))
    assert np.float32(gpu_packed.mean).view(np.uint32) == np.float32(p["mean"]).view(np.uint32)
    return p


def _check_dequant(p, torch):
    dev = _oracle_packed_on_device(p, torch)
    got16 = lib.nf4_dequant(dev, "bf16")
    got32 = lib.nf4_dequant(dev, "f32")
    got16t = lib.nf4_dequant(dev, "bf16_t")
    torch.cuda.synchronize()
    want32 = nf4.dequant_f32(p)
    np.testing.assert_array_equal(got32.cpu().numpy().view(np.uint32), want32.view(np.uint32))
    want16 = nf4.bf16_rne(want32)
    np.testing.assert_array_equal(got16.view(torch.int16).cpu().numpy().view(np.uint16), want16)
    assert tuple(got16t.shape) == (p["cols"], p["rows"])
    np.testing.assert_array_equal(got16t.view(torch.int16).cpu().numpy().view(np.uint16), want16.T)


def test_pack_and_dequant_single_linear(gpu):
    import torch
    w = inputs.single_linear(0)["W"]
    print("case: single linear 896x896 seed 0", flush=True)
    gp = lib.nf4_pack(_to_dev(w, torch))
    p = _check_pack(w, gp)
    _check_dequant(p, torch)


def test_smallest_tensor_and_special_blocks(gpu):
    import torch
    rng = np.random.default_rng(11)
    w = rng.normal(0, 0.02, size=(256, 64)).astype(np.float32)
    w[5, :] = 0.0                                     # zero block -> codes 0x77
    w[9, :] = nf4.codebook()[rng.integers(0, 16, 64)] * np.float32(0.125)   # on-level block
    w[9, 0] = 0.125
    w[17, :] = 1e-30                                  # tiny values
    print("case: 256x64 special blocks", flush=True)
    gp = lib.nf4_pack(_to_dev(w, torch))
    p = _check_pack(w, gp)
    assert np.all(p["codes"][5 * 32:6 * 32] == 0x77)
    _check_dequant(p, torch)


def test_round_trip_exact_on_codebook_levels(gpu):
    import torch
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, size=(1024 * 512 // 64, 64)).astype(np.uint8)
    codes[:, 3] = 15
    w = (nf4.codebook()[codes] * np.float32(2.0 ** -6)).reshape(1024, 512)
    print("case: round trip 1024x512", flush=True)
    gp = lib.nf4_pack(_to_dev(w, torch))
    back = lib.nf4_dequant(gp, "f32")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32), w.view(np.uint32))


@pytest.mark.parametrize("shape,label", [((14336, 4096), "8B gate"), ((8192, 8192), "72B q")])
def test_pack_and_dequant_full_size(gpu, shape, label):
    import torch
    print(f"case: {label} {shape}", flush=True)
    w_dev = inputs.device_normal(shape, 0.02, 0, "nf4-parity", label)
    gp = lib.nf4_pack(w_dev)
    w_host = w_dev.cpu().numpy()
    p = _check_pack(w_host, gp)
    del w_host
    _check_dequant(p, torch)


@pytest.mark.parametrize("shape", [(136, 2048), (256, 320), (8, 2048)])
def test_transposed_dequant_ragged_tiles(gpu, shape):
    """Row and column counts that end inside a 128 x 256 tile of the transposed kernel."""
    import torch
    print(f"case: transposed dequant {shape}", flush=True)
    w = inputs.host_normal(shape, 0.02, 0, "nf4-t", shape)
    p = nf4.pack(w)
    _check_dequant(p, torch)


def test_transposed_dequant_needs_rows_multiple_of_8(gpu):
    import torch
    p = nf4.pack(inputs.host_normal((4, 4096), 0.02, 0, "nf4-t4"))
    dev = _oracle_packed_on_device(p, torch)
    with pytest.raises(lib.LsnError) as e:
        lib.nf4_dequant(dev, "bf16_t")
    assert e.value.status == lib.LSN_E_ARG


@pytest.mark.parametrize("layout", ["bf16", "f32", "bf16_t"])
def test_batched_dequant_equals_oracle_per_tensor(gpu, layout):
    """One launch over tensors of different shapes (a small layer's projections): every output
    equals the oracle bit for bit, in every layout."""
    import torch
    shapes = [(896, 896), (128, 896), (128, 896), (896, 896), (4864, 896), (4864, 896), (896, 4864)]
    print(f"case: batched dequant {layout}", flush=True)
    ps = [nf4.pack(inputs.host_normal(sh, 0.02, 0, "nf4-batch", i)) for i, sh in enumerate(shapes)]
    devs = [_oracle_packed_on_device(p, torch) for p in ps]
    dt = torch.float32 if layout == "f32" else torch.bfloat16
    outs = [torch.empty((p["cols"], p["rows"]) if layout == "bf16_t" else (p["rows"], p["cols"]), dtype=dt,
                        device="cuda") for p in ps]
    lib.nf4_dequant_batch([d.desc() for d in devs], outs, layout)
    torch.cuda.synchronize()
    for p, o in zip(ps, outs):
        want32 = nf4.dequant_f32(p)
        if layout == "f32":
            np.testing.assert_array_equal(o.cpu().numpy().view(np.uint32), want32.view(np.uint32))
        else:
            got = o.view(torch.int16).cpu().numpy().view(np.uint16)
            want = nf4.bf16_rne(want32)
            np.testing.assert_array_equal(got, want.T if layout == "bf16_t" else want)
    with pytest.raises(lib.LsnError) as e:          # two outputs overlapping
        lib.nf4_dequant_batch([devs[0].desc(), devs[3].desc()], [outs[0], outs[0]], layout)
    assert e.value.status == lib.LSN_E_ARG


def test_pack_rejects_non_finite(gpu):
    import torch
    w = torch.zeros((256, 64), dtype=torch.float32, device="cuda")
    w[3, 7] = float("nan")
    with pytest.raises(lib.LsnError) as e:
        lib.nf4_pack(w)
    assert e.value.status == lib.LSN_E_ARG


def test_dequant_is_deterministic_across_buffers(gpu):
    import torch
    w_dev = inputs.device_normal((4096, 1024), 0.02, 0, "nf4-det")
    gp = lib.nf4_pack(w_dev)
    a = lib.nf4_dequant(gp, "bf16")
    b = torch.empty_like(a)
    lib.nf4_dequant(gp, "bf16", out=b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
