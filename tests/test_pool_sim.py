"""The layer pool's state machine on the host-simulated backend (no GPU): slot choice, event
ordering rules, refusal, misuse errors, KEEP_AT_TURN reuse, the aliasing audit and the planted
faults the exactness gate's controls rely on."""

import ctypes

import numpy as np
import pytest

from layer_streamed_nf4_dequant_amd import lib

SLOT = 4096


def aligned(n):
    """A zeroed uint8 array of n bytes whose data starts on a 256-byte boundary."""
    raw = np.zeros(n + 256, dtype=np.uint8)
    off = (-raw.ctypes.data) % 256
    return raw[off:off + n]


def sim_pool(slots, n_layers, flags, keep):
    """A host-simulated pool over the given slots, with the caller-owned memory its flags need
    (a checksum array for the audit, two bounce buffers for the file tier) appended to keep."""
    audit = bounce = None
    if flags & lib.POOL_AUDIT:
        sums = np.zeros(1024, dtype=np.uint64)
        keep.append(sums)
        audit = (sums.ctypes.data, sums.size)
    if flags & lib.POOL_FILE_TIER:
        b = [aligned(SLOT), aligned(SLOT)]
        keep += b
        bounce = (b[0].ctypes.data, b[1].ctypes.data)
    return lib.LayerPool([s.ctypes.data for s in slots], SLOT, n_layers, None, flags | lib.POOL_HOST_SIM,
                         audit_sums=audit, bounce=bounce)


class SimPool:
    def __init__(self, n_slots=2, n_layers=4, flags=0, sizes=None):
        self.slots = [aligned(SLOT) for _ in range(n_slots)]
        self.images = []
        rng = np.random.default_rng(0)
        for l in range(n_layers):
            n = SLOT if sizes is None else sizes[l]
            self.images.append(rng.integers(0, 255, n, dtype=np.uint8))
        self.keep = []
        self.pool = sim_pool(self.slots, n_layers, flags, self.keep)
        for l, img in enumerate(self.images):
            self.pool.register(l, img.ctypes.data, img.size)

    def view(self, ptr, layer):
        n = self.images[layer].size
        return np.ctypeslib.as_array((ctypes.c_uint8 * n).from_address(ptr))

    def visit(self, layer):
        ptr = self.pool.acquire(layer, None)
        data = self.view(ptr, layer).copy()
        self.pool.release(layer, None)
        return data


def forward_backward(p: SimPool, n_layers: int):
    """One step's visiting order: forward 0..L-1, then backward L-1..0, prefetching one ahead."""
    seen = []
    p.pool.prefetch(0)
    for l in range(n_layers):
        if l + 1 < n_layers:
            p.pool.prefetch(l + 1)
        seen.append(("f", l, p.visit(l)))
    p.pool.prefetch(n_layers - 1)
    for l in reversed(range(n_layers)):
        if l > 0:
            p.pool.prefetch(l - 1)
        seen.append(("b", l, p.visit(l)))
    return seen


def test_every_visit_sees_its_own_layer_and_layers_are_read_twice():
    p = SimPool(n_slots=2, n_layers=5)
    for kind, l, data in forward_backward(p, 5):
        np.testing.assert_array_equal(data, p.images[l], err_msg=f"{kind} visit of layer {l}")
    st = p.pool.stats()
    assert st["copies"] == 10 and st["acquires"] == 10 and st["releases"] == 10
    assert st["misses"] == 0 and st["hits"] == 0
    assert st["bytes_copied"] == 10 * SLOT


def test_keep_at_turn_reuses_the_turnaround_layer():
    p = SimPool(n_slots=2, n_layers=5, flags=lib.POOL_KEEP_AT_TURN)
    for kind, l, data in forward_backward(p, 5):
        np.testing.assert_array_equal(data, p.images[l])
    st = p.pool.stats()
    assert st["hits"] >= 1 and st["copies"] < 10


def test_single_slot_pool_works_without_prefetch_ahead():
    p = SimPool(n_slots=1, n_layers=3)
    for l in (0, 1, 2, 2, 1, 0):
        np.testing.assert_array_equal(p.visit(l), p.images[l])
    assert p.pool.stats()["misses"] == 6


def test_prefetch_refuses_when_all_slots_busy():
    p = SimPool(n_slots=2, n_layers=4)
    p.pool.prefetch(0)
    p.pool.prefetch(1)
    with pytest.raises(lib.LsnError) as e:
        p.pool.prefetch(2)
    assert e.value.status == lib.LSN_E_STATE
    p.pool.acquire(0, None)
    with pytest.raises(lib.LsnError):
        p.pool.prefetch(2)           # slot 0 acquired, slot 1 pending
    p.pool.release(0, None)
    p.pool.prefetch(2)               # slot 0 is free again


def test_misuse_errors():
    p = SimPool(n_slots=2, n_layers=3)
    with pytest.raises(lib.LsnError) as e:
        p.pool.release(0, None)
    assert e.value.status == lib.LSN_E_STATE
    p.pool.acquire(1, None)
    with pytest.raises(lib.LsnError) as e:
        p.pool.acquire(1, None)
    assert e.value.status == lib.LSN_E_STATE
    with pytest.raises(lib.LsnError) as e:
        p.pool.prefetch(1)
    assert e.value.status == lib.LSN_E_STATE
    with pytest.raises(lib.LsnError) as e:
        p.pool.acquire(7, None)
    assert e.value.status == lib.LSN_E_ARG


def test_register_refuses_an_image_larger_than_a_slot():
    slots = [aligned(SLOT)]
    pool = lib.LayerPool([slots[0].ctypes.data], SLOT, 1, None, lib.POOL_HOST_SIM)
    big = np.zeros(2 * SLOT, dtype=np.uint8)
    with pytest.raises(lib.LsnError) as e:
        pool.register(0, big.ctypes.data, big.size)
    assert e.value.status == lib.LSN_E_NOFIT


def test_create_rejects_overlapping_or_misaligned_slots():
    buf = np.zeros(3 * SLOT + 512, dtype=np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    with pytest.raises(lib.LsnError):
        lib.LayerPool([base, base + 256], SLOT, 1, None, lib.POOL_HOST_SIM)
    with pytest.raises(lib.LsnError):
        lib.LayerPool([base + 8], SLOT, 1, None, lib.POOL_HOST_SIM)


def test_audit_passes_on_a_clean_step_and_poisons_released_slots():
    p = SimPool(n_slots=2, n_layers=4, flags=lib.POOL_AUDIT)
    forward_backward(p, 4)
    p.pool.audit()
    st = p.pool.stats()
    assert st["audit_checks"] == 16 and st["audit_failures"] == 0
    assert all(np.all(s == 0xFF) for s in p.slots), "released slots must be poisoned"


@pytest.mark.parametrize("fault", [lib.FAULT_STALE_REFETCH, lib.FAULT_WRONG_SLOT])
def test_planted_faults_corrupt_only_the_second_visit_and_the_audit_catches_them(fault):
    p = SimPool(n_slots=2, n_layers=4, flags=fault)
    seen = forward_backward(p, 4)
    fwd_ok = all(np.array_equal(d, p.images[l]) for k, l, d in seen if k == "f")
    bwd_ok = all(np.array_equal(d, p.images[l]) for k, l, d in seen if k == "b")
    assert fwd_ok and not bwd_ok
    q = SimPool(n_slots=2, n_layers=4, flags=fault | lib.POOL_AUDIT)
    forward_backward(q, 4)
    with pytest.raises(lib.LsnError) as e:
        q.pool.audit()
    assert e.value.status == lib.LSN_E_AUDIT
    assert q.pool.stats()["audit_failures"] > 0


# ---- file tier (LSN_POOL_FILE_TIER): the images are read from files by the pool's I/O thread ----

class FilePool(SimPool):
    """SimPool whose layers live in one file (each image at its own offset), read by the pool."""

    def __init__(self, tmp_path, n_slots=2, n_layers=4, flags=0, offset0=512):
        self.slots = [aligned(SLOT) for _ in range(n_slots)]
        rng = np.random.default_rng(1)
        self.images = [rng.integers(0, 255, SLOT, dtype=np.uint8) for _ in range(n_layers)]
        self.path = str(tmp_path / "base.bin")
        self.offsets = [offset0 + l * (SLOT + 256) for l in range(n_layers)]
        blob = np.zeros(self.offsets[-1] + SLOT, dtype=np.uint8)
        for off, img in zip(self.offsets, self.images):
            blob[off:off + SLOT] = img
        blob.tofile(self.path)
        self.keep = []
        self.pool = sim_pool(self.slots, n_layers, flags | lib.POOL_FILE_TIER, self.keep)
        for l, off in enumerate(self.offsets):
            self.pool.register_file(l, self.path, off, SLOT)


def test_file_tier_every_visit_sees_its_own_layer(tmp_path):
    p = FilePool(tmp_path, n_slots=2, n_layers=5)
    for kind, l, data in forward_backward(p, 5):
        np.testing.assert_array_equal(data, p.images[l], err_msg=f"{kind} visit of layer {l}")
    st = p.pool.stats()
    assert st["copies"] == 10 and st["bytes_copied"] == 10 * SLOT and st["misses"] == 0
    p.pool.close()


@pytest.mark.parametrize("n_slots", [2, 3])
def test_file_tier_other_slot_counts_and_keep_at_turn(tmp_path, n_slots):
    p = FilePool(tmp_path, n_slots=n_slots, n_layers=4, flags=lib.POOL_KEEP_AT_TURN)
    for kind, l, data in forward_backward(p, 4):
        np.testing.assert_array_equal(data, p.images[l], err_msg=f"{kind} visit of layer {l}")
    assert p.pool.stats()["hits"] >= 1
    p.pool.close()


def test_file_tier_single_slot_without_prefetch_ahead(tmp_path):
    p = FilePool(tmp_path, n_slots=1, n_layers=3)
    for l in (0, 1, 2, 2, 1, 0):
        np.testing.assert_array_equal(p.visit(l), p.images[l])
    assert p.pool.stats()["misses"] == 6
    p.pool.close()


def test_file_tier_audit_and_planted_fault(tmp_path):
    p = FilePool(tmp_path, n_layers=4, flags=lib.POOL_AUDIT)
    forward_backward(p, 4)
    p.pool.audit()                                   # clean run: every checksum matches the file
    q = FilePool(tmp_path, n_layers=4, flags=lib.POOL_AUDIT | lib.FAULT_STALE_REFETCH)
    forward_backward(q, 4)
    with pytest.raises(lib.LsnError) as e:
        q.pool.audit()
    assert e.value.status == lib.LSN_E_AUDIT
    p.pool.close()
    q.pool.close()


def test_file_tier_refusals(tmp_path):
    p = FilePool(tmp_path, n_layers=2)
    with pytest.raises(lib.LsnError) as e:           # missing file
        p.pool.register_file(0, str(tmp_path / "nope.bin"), 0, SLOT)
    assert e.value.status == lib.LSN_E_ARG
    with pytest.raises(lib.LsnError) as e:           # image past the end of the file
        p.pool.register_file(0, p.path, p.offsets[-1] + 256, SLOT)
    assert e.value.status == lib.LSN_E_ARG
    with pytest.raises(lib.LsnError) as e:           # larger than a slot
        p.pool.register_file(0, p.path, 0, 2 * SLOT)
    assert e.value.status == lib.LSN_E_NOFIT
    plain = SimPool(n_layers=2)                      # a pool without the file tier
    with pytest.raises(lib.LsnError) as e:
        plain.pool.register_file(0, p.path, 0, SLOT)
    assert e.value.status == lib.LSN_E_STATE
    p.pool.close()


def test_file_tier_read_error_is_reported_by_acquire(tmp_path):
    p = FilePool(tmp_path, n_layers=2)
    # shrink the file behind the pool's back: the read of layer 1 comes up short
    with open(p.path, "r+b") as f:
        f.truncate(p.offsets[1] + 16)
    p.pool.prefetch(1)
    with pytest.raises(lib.LsnError) as e:
        p.pool.acquire(1, None)
    assert e.value.status == lib.LSN_E_HIP and "end of file" in str(e.value)
    p.pool.close()


def test_create_needs_the_callers_audit_and_bounce_memory():
    slots = [aligned(SLOT)]
    for flags in (lib.POOL_AUDIT, lib.POOL_FILE_TIER):
        with pytest.raises(lib.LsnError) as e:           # flag set, no buffers
            lib.LayerPool([slots[0].ctypes.data], SLOT, 1, None, flags | lib.POOL_HOST_SIM)
        assert e.value.status == lib.LSN_E_ARG
    with pytest.raises(lib.LsnError):                    # checksum array inside a slot
        lib.LayerPool([slots[0].ctypes.data], SLOT, 1, None, lib.POOL_AUDIT | lib.POOL_HOST_SIM,
                      audit_sums=(slots[0].ctypes.data + 256, 8))
    with pytest.raises(lib.LsnError):                    # zero capacity
        sums = np.zeros(8, dtype=np.uint64)
        lib.LayerPool([slots[0].ctypes.data], SLOT, 1, None, lib.POOL_AUDIT | lib.POOL_HOST_SIM,
                      audit_sums=(sums.ctypes.data, 0))
    b = aligned(2 * SLOT)
    with pytest.raises(lib.LsnError):                    # the bounce buffers overlap
        lib.LayerPool([slots[0].ctypes.data], SLOT, 1, None, lib.POOL_FILE_TIER | lib.POOL_HOST_SIM,
                      bounce=(b.ctypes.data, b.ctypes.data + SLOT // 2))


def test_audit_capacity_is_the_callers():
    """Two checksums per visit: a capacity of 3 holds one visit, and the second visit's release
    overflows it (LSN_E_STATE) until the audit empties it."""
    slots = [aligned(SLOT), aligned(SLOT)]
    keep = []
    sums = np.zeros(3, dtype=np.uint64)
    pool = lib.LayerPool([s.ctypes.data for s in slots], SLOT, 2, None, lib.POOL_AUDIT | lib.POOL_HOST_SIM,
                         audit_sums=(sums.ctypes.data, 3))
    img = [np.full(SLOT, l + 1, dtype=np.uint8) for l in range(2)]
    keep += img
    for l in range(2):
        pool.register(l, img[l].ctypes.data, SLOT)
    pool.acquire(0, None)
    pool.release(0, None)
    pool.acquire(1, None)
    with pytest.raises(lib.LsnError) as e:
        pool.release(1, None)
    assert e.value.status == lib.LSN_E_STATE and "capacity" in str(e.value)
    pool.audit()
    assert np.all(sums == 0)                              # the audit zeroes what it read
    pool.close()


def test_register_again_replaces_the_image_and_refuses_while_in_flight():
    """A layer registered anew must not be served from a free slot that still holds its old bytes
    (KEEP_AT_TURN would otherwise reuse them without a copy); while the layer is prefetched or
    acquired, registering it again is refused."""
    p = SimPool(n_slots=2, n_layers=2, flags=lib.POOL_KEEP_AT_TURN)
    np.testing.assert_array_equal(p.visit(0), p.images[0])
    copies = p.pool.stats()["copies"]
    new = np.random.default_rng(9).integers(0, 255, SLOT, dtype=np.uint8)
    p.keep.append(new)
    p.pool.register(0, new.ctypes.data, SLOT)
    np.testing.assert_array_equal(p.visit(0), new)
    assert p.pool.stats()["copies"] == copies + 1         # a fresh copy, not a reuse
    p.pool.prefetch(1)
    with pytest.raises(lib.LsnError) as e:
        p.pool.register(1, new.ctypes.data, SLOT)
    assert e.value.status == lib.LSN_E_STATE
    p.pool.acquire(1, None)
    with pytest.raises(lib.LsnError) as e:
        p.pool.register(1, new.ctypes.data, SLOT)
    assert e.value.status == lib.LSN_E_STATE
    p.pool.release(1, None)
    np.testing.assert_array_equal(p.visit(1), p.images[1])


def test_file_tier_register_again_replaces_the_image(tmp_path):
    p = FilePool(tmp_path, n_slots=2, n_layers=2, flags=lib.POOL_KEEP_AT_TURN)
    np.testing.assert_array_equal(p.visit(0), p.images[0])
    p.pool.register_file(0, p.path, p.offsets[1], SLOT)   # layer 0 now names layer 1's bytes
    np.testing.assert_array_equal(p.visit(0), p.images[1])
    p.pool.close()


def aligned4k(n):
    raw = np.zeros(n + 4096, dtype=np.uint8)
    off = (-raw.ctypes.data) % 4096
    return raw[off:off + n]


def test_file_tier_direct_reads(tmp_path):
    """LSN_POOL_FILE_DIRECT: the fills read the file with O_DIRECT (4 KiB aligned offsets, each
    image's region padded to whole 4 KiB blocks); every visit still sees exactly its layer's bytes,
    the padding is never copied, and misaligned offsets or buffers are refused."""
    n_layers, img_bytes = 4, SLOT - 256          # the images do not fill a 4 KiB block: padding is read
    rng = np.random.default_rng(3)
    images = [rng.integers(0, 255, img_bytes, dtype=np.uint8) for _ in range(n_layers)]
    path = str(tmp_path / "direct.bin")
    blob = np.full(n_layers * SLOT + SLOT, 0xAB, dtype=np.uint8)   # padding bytes that must not appear
    offsets = [SLOT + l * SLOT for l in range(n_layers)]
    for off, img in zip(offsets, images):
        blob[off:off + img_bytes] = img
    blob.tofile(path)
    slots = [aligned4k(SLOT) for _ in range(2)]
    bounce = [aligned4k(SLOT) for _ in range(2)]
    stage = [aligned4k(SLOT) for _ in range(2)]
    flags = lib.POOL_HOST_SIM | lib.POOL_FILE_TIER | lib.POOL_FILE_DIRECT
    try:
        pool = lib.LayerPool([s.ctypes.data for s in slots], SLOT, n_layers, None, flags,
                             bounce=(bounce[0].ctypes.data, bounce[1].ctypes.data),
                             direct_stage=(stage[0].ctypes.data, stage[1].ctypes.data))
        pool.register_file(0, path, offsets[0], img_bytes)
    except lib.LsnError as e:
        if "O_DIRECT" in str(e):
            pytest.skip(f"the file system under {tmp_path} does not support O_DIRECT: {e}")
        raise
    for l in range(1, n_layers):
        pool.register_file(l, path, offsets[l], img_bytes)
    for s in slots:
        s[:] = 0
    for l in list(range(n_layers)) + list(reversed(range(n_layers))):
        ptr = pool.acquire(l, None)
        got = np.ctypeslib.as_array((ctypes.c_uint8 * SLOT).from_address(ptr)).copy()
        pool.release(l, None)
        np.testing.assert_array_equal(got[:img_bytes], images[l])
        assert not np.any(got[img_bytes:] == 0xAB), "the O_DIRECT padding must not be copied into a slot"
    with pytest.raises(lib.LsnError) as e:              # an offset that is not 4 KiB aligned
        pool.register_file(0, path, offsets[0] + 256, img_bytes)
    assert e.value.status == lib.LSN_E_ARG
    pool.close()
    with pytest.raises(lib.LsnError):                    # staging buffers not 4 KiB aligned
        lib.LayerPool([s.ctypes.data for s in slots], SLOT, n_layers, None, flags,
                      bounce=(bounce[0].ctypes.data, bounce[1].ctypes.data),
                      direct_stage=(stage[0].ctypes.data + 256, stage[1].ctypes.data))
    with pytest.raises(lib.LsnError):                    # no staging buffers
        lib.LayerPool([s.ctypes.data for s in slots], SLOT, n_layers, None, flags,
                      bounce=(bounce[0].ctypes.data, bounce[1].ctypes.data))
