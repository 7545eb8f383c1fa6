"""Pins of the decoder-glue oracle (oracle/glue.py): closed forms (a constant row, position 0,
a zero gate), invariants (RoPE keeps each pair's length and composes by adding positions, its
inverse undoes it), and central finite differences of every backward."""

import numpy as np

from oracle import glue


def _fd(f, x, eps=1e-6):
    out = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        d = np.zeros_like(x)
        d[i] = eps
        out[i] = (f(x + d) - f(x - d)) / (2 * eps)
    return out


def test_rmsnorm_constant_row_and_scale_invariance():
    x = np.full((1, 8), 3.0)
    g = np.linspace(0.5, 2.0, 8)
    np.testing.assert_allclose(glue.rmsnorm(x, g, 0.0), g[None, :], rtol=1e-15)
    rng = np.random.default_rng(0)
    y = rng.normal(size=(3, 16))
    gg = rng.normal(size=16)
    np.testing.assert_allclose(glue.rmsnorm(7.5 * y, gg, 0.0), glue.rmsnorm(y, gg, 0.0), rtol=1e-13)


def test_rmsnorm_backward_matches_finite_differences():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 10))
    g = rng.normal(size=10)
    dy = rng.normal(size=(3, 10))
    eps = 1e-5
    num = _fd(lambda xx: (glue.rmsnorm(xx, g, eps) * dy).sum(), x)
    np.testing.assert_allclose(glue.rmsnorm_bwd(x, g, dy, eps), num, rtol=1e-6, atol=1e-9)


def test_rope_identity_at_zero_norms_composition_and_inverse():
    rng = np.random.default_rng(2)
    T, nh, d, theta = 5, 3, 8, 10000.0
    x = rng.normal(size=(T, nh * d))
    np.testing.assert_allclose(glue.rope(x, np.zeros(T), nh, d, theta), x, rtol=0, atol=1e-15)
    pos = np.arange(T) * 7
    y = glue.rope(x, pos, nh, d, theta)
    xr, yr = x.reshape(T, nh, d), y.reshape(T, nh, d)
    h = d // 2
    np.testing.assert_allclose(xr[..., :h] ** 2 + xr[..., h:] ** 2, yr[..., :h] ** 2 + yr[..., h:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(glue.rope(glue.rope(x, pos, nh, d, theta), pos + 3, nh, d, theta),
                               glue.rope(x, 2 * pos + 3, nh, d, theta), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(glue.rope(y, pos, nh, d, theta, inverse=True), x, rtol=1e-12, atol=1e-12)
    # the lowest pair turns by exactly pos radians (theta^0 = 1)
    np.testing.assert_allclose(yr[1, 0, 0], xr[1, 0, 0] * np.cos(7) - xr[1, 0, h] * np.sin(7), rtol=1e-14)


def test_rope_backward_is_the_inverse_rotation():
    rng = np.random.default_rng(3)
    T, nh, d, theta = 4, 2, 6, 500000.0
    x = rng.normal(size=(T, nh * d))
    dy = rng.normal(size=(T, nh * d))
    pos = np.array([0, 5, 9, 2047])
    num = _fd(lambda xx: (glue.rope(xx, pos, nh, d, theta) * dy).sum(), x)
    np.testing.assert_allclose(glue.rope(dy, pos, nh, d, theta, inverse=True), num, rtol=1e-6, atol=1e-9)


def test_swiglu_special_values_and_backward():
    u = np.array([1.5, -2.0, 3.0])
    np.testing.assert_allclose(glue.swiglu(np.zeros(3), u), 0.0, atol=0)
    np.testing.assert_allclose(glue.swiglu(np.full(3, 40.0), u), 40.0 * u, rtol=1e-15)   # silu(z) -> z
    np.testing.assert_allclose(glue.sigmoid(np.array([-800.0, 0.0, 800.0])), [0.0, 0.5, 1.0], atol=1e-300)
    rng = np.random.default_rng(4)
    g = rng.normal(size=(3, 7)) * 3
    uu = rng.normal(size=(3, 7))
    dm = rng.normal(size=(3, 7))
    dg, du = glue.swiglu_bwd(g, uu, dm)
    np.testing.assert_allclose(dg, _fd(lambda z: (glue.swiglu(z, uu) * dm).sum(), g), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(du, _fd(lambda z: (glue.swiglu(g, z) * dm).sum(), uu), rtol=1e-6, atol=1e-9)


def test_rope_pair_frequencies_closed_form():
    """The frequency of pair i is theta^(-2i/d). With theta = 10^4 and d = 8 the four pairs turn at
    1, 1/10, 1/100 and 1/1000 radians per position, so pair i at position 10^i is rotated by exactly
    one radian: a unit vector on the pair's first coordinate comes out as (cos 1, sin 1). A
    frequency of theta^(-i/d), or a pairing of neighbours (2i, 2i+1), fails this."""
    d, nh, theta = 8, 1, 10000.0
    h = d // 2
    for i in range(h):
        x = np.zeros((1, d))
        x[0, i] = 1.0
        y = glue.rope(x, np.array([10 ** i]), nh, d, theta)[0]
        want = np.zeros(d)
        want[i], want[i + h] = np.cos(1.0), np.sin(1.0)
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)
    # a second route to the angle: theta^(-2i/d) as exp(-(2i/d) ln theta), read back with atan2
    for d, theta in ((128, 500000.0), (64, 1000000.0)):
        for i in (d // 4, d // 2 - 1):
            x = np.zeros((1, d))
            x[0, i] = 1.0
            y = glue.rope(x, np.array([1]), 1, d, theta)[0]
            got = np.arctan2(y[i + d // 2], y[i])
            assert abs(got - np.exp(-(2.0 * i / d) * np.log(theta))) < 1e-15
