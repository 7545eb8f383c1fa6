"""Pins for the NF4 oracle (oracle/nf4.py) against closed forms, invariants and brute force.

Each test checks the oracle against something other than itself: a different quantile/CDF
routine, an exactly representable round trip, a brute-force nearest-level search, torch's
bf16 conversion, or values worked out by hand.  No GPU, no product code.
"""

import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- codebook

def test_codebook_structure():
    q = nf4.codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0), "levels must be strictly increasing"
    assert q[0] == -1.0 and q[7] == 0.0 and q[15] == 1.0
    assert np.sum(q < 0) == 7 and np.sum(q > 0) == 8
    assert q[7].view(np.uint32) == 0, "the zero level is +0"


def test_codebook_levels_are_normal_quantiles():
    """Applying the forward normal CDF to the de-normalised levels recovers the evenly spaced
    probabilities of the construction (a different routine from the inverse used to build it)."""
    q = nf4.codebook().astype(np.float64)
    z_max = scipy.special.ndtri(nf4.P_MAX)
    p_pos = scipy.stats.norm.cdf(q[8:][::-1] * z_max)        # q15 .. q8
    p_neg = scipy.stats.norm.cdf(-q[:7] * z_max)              # q0 .. q6
    want_pos = nf4.P_MAX + np.arange(8) * (0.5 - nf4.P_MAX) / 8
    want_neg = nf4.P_MAX + np.arange(7) * (0.5 - nf4.P_MAX) / 7
    np.testing.assert_allclose(p_pos, want_pos, rtol=0, atol=1e-7)
    np.testing.assert_allclose(p_neg, want_neg, rtol=0, atol=1e-7)


def test_codebook_matches_independent_quantile_routine():
    """scipy's ndtri (Cephes) and the stdlib's inverse CDF agree after rounding to fp32."""
    pos = scipy.special.ndtri(np.linspace(nf4.P_MAX, 0.5, 9)[:-1])
    neg = -scipy.special.ndtri(np.linspace(nf4.P_MAX, 0.5, 8)[:-1])
    z = scipy.special.ndtri(nf4.P_MAX)
    alt = (np.sort(np.concatenate([neg, [0.0], pos])) / z).astype(np.float32)
    np.testing.assert_array_equal(alt.view(np.uint32), nf4.codebook().view(np.uint32))


def test_codebook_matches_golden():
    """Regression pin: the frozen table written by tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "nf4_codebook.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    levels = np.array([float.fromhex(r[1]) for r in rows if r[0] == "q"], dtype=np.float32)
    mids = np.array([float.fromhex(r[1]) for r in rows if r[0] == "m"], dtype=np.float32)
    np.testing.assert_array_equal(levels.view(np.uint32), nf4.codebook().view(np.uint32))
    np.testing.assert_array_equal(mids.view(np.uint32), nf4.code_thresholds().view(np.uint32))


def test_thresholds_are_midpoints():
    q = nf4.codebook().astype(np.float64)
    m = nf4.code_thresholds().astype(np.float64)
    assert np.all(q[:-1] < m) and np.all(m < q[1:])
    np.testing.assert_allclose(m, (q[:-1] + q[1:]) / 2, rtol=2 ** -23, atol=0)


# ---------------------------------------------------------------- first pass

def _block_with_unit_absmax(x):
    """A 64-element block whose absmax is exactly 1, so x = w / c_b = w exactly."""
    w = np.array(x, dtype=np.float32).reshape(-1, 64).copy()
    w[:, 0] = 1.0
    return w


def test_code_is_nearest_level_brute_force():
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, size=(256, 64)).astype(np.float32)
    w = _block_with_unit_absmax(x)
    codes, c = nf4.first_pass(w)
    assert np.all(c == 1.0)
    q = nf4.codebook().astype(np.float64)
    brute = np.argmin(np.abs(w.reshape(-1, 1).astype(np.float64) - q[None, :]), axis=1)
    m = nf4.code_thresholds().astype(np.float64)
    far = np.min(np.abs(w.reshape(-1, 1).astype(np.float64) - m[None, :]), axis=1) > 1e-6
    assert far.sum() > 16000
    np.testing.assert_array_equal(codes[far], brute[far])


def test_code_tie_goes_to_lower_level():
    m = nf4.code_thresholds()
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0
    w[0, 1:16] = m                                          # exact midpoints -> lower index
    w[0, 16:31] = np.nextafter(m, np.float32(np.inf))       # just above -> upper index
    codes, _ = nf4.first_pass(w)
    np.testing.assert_array_equal(codes[1:16], np.arange(15))
    np.testing.assert_array_equal(codes[16:31], np.arange(1, 16))
    assert codes[0] == 15


def test_nibble_order_high_nibble_is_even_element():
    codes = np.array([3, 12, 0, 15, 7, 7], dtype=np.uint8)
    np.testing.assert_array_equal(nf4.pack_nibbles(codes), [0x3C, 0x0F, 0x77])
    np.testing.assert_array_equal(nf4.unpack_nibbles([0x3C, 0x0F, 0x77]), codes)


def test_zero_block_packs_to_0x77_and_dequantises_to_zero():
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, size=(64, 256)).astype(np.float32)
    w[3, 64:128] = 0.0
    p = nf4.pack(w)
    row_bytes = 256 // 2
    blk = p["codes"][3 * row_bytes + 32: 3 * row_bytes + 64]
    assert np.all(blk == 0x77)
    deq = nf4.dequant_f32(p)
    assert np.all(deq[3, 64:128] == 0.0)


# ---------------------------------------------------------------- second pass

def test_int8_code_is_nearest_brute_force():
    rng = np.random.default_rng(3)
    # c_b values whose deviations from the mean cover the int8 range
    c = rng.uniform(0.01, 0.05, size=256 * 8).astype(np.float32)
    v, s2, mu = nf4.second_pass(c)
    d = (c - mu).reshape(-1, 256)
    y = (d / s2[:, None]).astype(np.float32).ravel().astype(np.float64)
    levels = np.arange(-127, 128) / 127.0
    brute = np.argmin(np.abs(y[:, None] - levels[None, :]), axis=1) - 127
    t = nf4.int8_thresholds().astype(np.float64)
    far = np.min(np.abs(y[:, None] - t[None, :]), axis=1) > 1e-6
    assert far.sum() > 2000
    np.testing.assert_array_equal(v.astype(np.int64)[far], brute[far])
    assert v.min() >= -127 and v.max() <= 127


def test_mean_is_exact_mean_rounded_to_fp32():
    """mu against math.fsum (an exactly rounded sum) on a modest array."""
    rng = np.random.default_rng(4)
    c = rng.uniform(0, 0.1, size=256 * 4).astype(np.float32)
    _, _, mu = nf4.second_pass(c)
    exact = math.fsum(float(x) for x in c) / c.size
    assert mu == np.float32(exact)


def test_decode_absmax_hand_values():
    """c' = code8[v] * s2 + mu with exactly representable operands."""
    qabs = np.zeros(256, dtype=np.int8)
    qabs[0], qabs[1], qabs[2] = 127, -127, 0
    c = nf4.decode_absmax(qabs, np.array([0.5], dtype=np.float32), np.float32(0.25))
    assert c[0] == 0.75 and c[1] == -0.25 and c[2] == 0.25


def test_dequant_hand_values():
    qabs = np.zeros(256, dtype=np.int8)
    qabs[0] = 127
    codes = np.full(256 * 64, 7, dtype=np.uint8)
    codes[0], codes[1], codes[2] = 15, 0, 7
    p = {"rows": 256, "cols": 64, "codes": nf4.pack_nibbles(codes), "qabsmax": qabs,
         "absmax2": np.array([0.5], dtype=np.float32), "mean": np.float32(0.25)}
    deq = nf4.dequant_f32(p)
    assert deq[0, 0] == 0.75 and deq[0, 1] == -0.75 and deq[0, 2] == 0.0
    assert np.all(deq[1:, :] == 0.0)


# ---------------------------------------------------------------- round trip and bounds

def test_round_trip_exact_on_codebook_levels():
    """W = q[code] * 2^-5 with a +-1 level in every block: every stage is exact, so the
    codes come back unchanged, mu = 2^-5, d = 0, s2 = 0, v = 0 and c' = 2^-5."""
    rng = np.random.default_rng(5)
    rows, cols = 128, 512
    codes = rng.integers(0, 16, size=(rows * cols // 64, 64)).astype(np.uint8)
    codes[:, 5] = rng.choice([0, 15], size=codes.shape[0])
    a = np.float32(2.0 ** -5)
    w = (nf4.codebook()[codes] * a).reshape(rows, cols)
    p = nf4.pack(w)
    np.testing.assert_array_equal(nf4.unpack_nibbles(p["codes"]), codes.ravel())
    assert p["mean"] == a and np.all(p["absmax2"] == 0) and np.all(p["qabsmax"] == 0)
    deq = nf4.dequant_f32(p)
    np.testing.assert_array_equal(deq.view(np.uint32), w.view(np.uint32))
    np.testing.assert_array_equal(nf4.dequant_bf16(p), nf4.bf16_rne(w))


def test_error_bound_on_normal_weights():
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, size=(256, 1024)).astype(np.float32)
    p = nf4.pack(w)
    deq = nf4.dequant_f32(p).astype(np.float64)
    c = np.abs(w.reshape(-1, 64)).max(axis=1).astype(np.float64)
    cp = nf4.decode_absmax(p["qabsmax"], p["absmax2"], p["mean"]).astype(np.float64)
    s2 = np.repeat(p["absmax2"].astype(np.float64), 256)
    # second pass: |c - c'| <= s2/254 plus fp32 rounding of the three steps
    assert np.all(np.abs(c - cp) <= s2 / 254 * (1 + 1e-6) + 4 * np.spacing(c.astype(np.float32)))
    q = nf4.codebook().astype(np.float64)
    half_gap = np.max(np.diff(q)) / 2
    err = np.abs(w.reshape(-1, 64) - deq.reshape(-1, 64))
    bound = c[:, None] * half_gap + np.abs(c - cp)[:, None] + 1e-9
    assert np.all(err <= bound)
    # and the quantisation is not vacuous: typical error is far below the bound
    assert err.mean() < 0.25 * bound.mean()


def test_pack_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(ValueError):
        nf4.pack(np.zeros((3, 100), dtype=np.float32))
    with pytest.raises(ValueError):
        nf4.pack(np.zeros((1, 64), dtype=np.float32))       # 64 elements, not a multiple of 16384
    w = np.zeros((256, 64), dtype=np.float32)
    w[1, 1] = np.inf
    with pytest.raises(ValueError):
        nf4.pack(w)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_matches_torch():
    import torch
    rng = np.random.default_rng(7)
    f = np.concatenate([
        rng.normal(0, 1, 20000).astype(np.float32),
        rng.normal(0, 1e-38, 2000).astype(np.float32),                  # denormals
        (rng.integers(0, 2 ** 16, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32),  # ties
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1e-45], dtype=np.float32),
    ])
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(nf4.bf16_rne(f), want)
    np.testing.assert_array_equal(nf4.bf16_to_f32(want), torch.from_numpy(f).to(
        torch.bfloat16).to(torch.float32).numpy())
