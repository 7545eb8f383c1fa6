"""Oracle for the decoder-layer glue around the seven projections, in fp64: RMSNorm, rotary
position embedding and the SwiGLU gate, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the product path.

Source: the pages train Llama-3.1-8B and Qwen2.5 models ("Exact Layer Streaming", Abstract;
"Soup v0.73.0 benchmarks README", record index) and name their decoder layers as the streamed unit
("An 8B Fine-Tune Now Fits in 4 GB of VRAM"); they print none of the layer's formulas.  These are
the published definitions of those models' layers, written from the definitions:

    RMSNorm   r_t = sqrt(mean_j x_tj^2 + eps),  y = x / r * g               (g frozen)
              dx = (g dy) / r - x * sum_j (g dy x)_tj / (H r^3)
    RoPE      per head of width d, pairs (i, i + d/2), angle a = pos * theta^(-2i/d):
              y_i = x_i cos a - x_{i+d/2} sin a,  y_{i+d/2} = x_{i+d/2} cos a + x_i sin a
              (the backward is the same rotation by -a)
    SwiGLU    m = silu(g) u,  silu(z) = z sigmoid(z)
              dg = dm u sigmoid(g) (1 + g (1 - sigmoid(g))),  du = dm silu(g)
"""

from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rms(x, eps: float) -> np.ndarray:
    x = _f64(x)
    return np.sqrt((x * x).mean(axis=-1) + eps)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x, g = _f64(x), _f64(g)
    return x / rms(x, eps)[:, None] * g


def rmsnorm_bwd(x, g, dy, eps: float) -> np.ndarray:
    x, g, dy = _f64(x), _f64(g), _f64(dy)
    r = rms(x, eps)[:, None]
    gy = g * dy
    H = x.shape[-1]
    return gy / r - x * (gy * x).sum(axis=-1, keepdims=True) / (H * r ** 3)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """[T, head_dim/2] angles pos * theta^(-2i/head_dim)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = float(theta) ** (-2.0 * i / head_dim)
    return _f64(positions)[:, None] * inv[None, :]


def rope(x, positions, n_heads: int, head_dim: int, theta: float, inverse: bool = False) -> np.ndarray:
    """x [T, n_heads * head_dim] -> rotated copy; inverse rotates by -angle (the backward)."""
    x = _f64(x).reshape(x.shape[0], n_heads, head_dim)
    a = rope_angles(positions, head_dim, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    if inverse:
        s = -s
    h = head_dim // 2
    x1, x2 = x[..., :h], x[..., h:]
    y = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return y.reshape(y.shape[0], n_heads * head_dim)


def sigmoid(z) -> np.ndarray:
    z = _f64(z)
    return 0.5 * (1.0 + np.tanh(0.5 * z))        # the same function as 1 / (1 + e^-z), overflow-free


def swiglu(g, u) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    return g * sigmoid(g) * u


def swiglu_bwd(g, u, dm):
    g, u, dm = _f64(g), _f64(u), _f64(dm)
    s = sigmoid(g)
    return dm * u * s * (1.0 + g * (1.0 - s)), dm * g * s
