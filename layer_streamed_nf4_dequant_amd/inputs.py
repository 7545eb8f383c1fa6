"""Seeded synthetic inputs, shared by the HIP path and the oracle's tests.

This module draws random tensors and nothing else: it holds none of the method's
arithmetic (no quantisation, no dequantisation, no LoRA).  Every tensor gets its own
stream keyed by (seed, config, layer, projection, kind), so a value never depends on the
order in which tensors are drawn.

Distributions (one per kind):
    W   ~ N(0, 0.02)  fp32   frozen base weight [N, K]   (std 0.02)
    A   ~ U(-1/sqrt(K), 1/sqrt(K)) -> bf16              LoRA down-projection [r, K]
    B   ~ N(0, 0.01) -> bf16                            LoRA up-projection [N, r]
    X   ~ N(0, 1) -> bf16                               activations [T, K]
    dY  ~ N(0, 1) -> bf16                               upstream gradient [T, N]
bf16 values are the round-to-nearest-even images of fp32 draws (torch's conversion), kept
as uint16 bit patterns on the host.

Host draws use numpy's PCG64; device draws (for shapes too large for the host) use torch's
Philox generator on the GPU, seeded from the same key.
"""

from __future__ import annotations

import hashlib

import numpy as np

KINDS = {"W": 0, "A": 1, "B": 2, "X": 3, "dY": 4, "misc": 5}
STD = {"W": 0.02, "B": 0.01, "X": 1.0, "dY": 1.0}


def key_seed(seed: int, *key) -> int:
    """A 63-bit integer seed derived from (seed, key...) by hashing its text form."""
    text = repr((int(seed),) + tuple(key)).encode()
    return int.from_bytes(hashlib.sha256(text).digest()[:8], "little") & ((1 << 63) - 1)


def host_rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(key_seed(seed, *key)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch's conversion) as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_normal(shape, std: float, seed: int, *key) -> np.ndarray:
    return (host_rng(seed, *key).standard_normal(shape, dtype=np.float32) * np.float32(std))


def host_uniform(shape, bound: float, seed: int, *key) -> np.ndarray:
    u = host_rng(seed, *key).random(shape, dtype=np.float32)
    return (u * np.float32(2.0) - np.float32(1.0)) * np.float32(bound)


def weight_f32(N: int, K: int, seed: int, *key) -> np.ndarray:
    return host_normal((N, K), STD["W"], seed, *key, "W")


def lora_A_bf16(r: int, K: int, seed: int, *key) -> np.ndarray:
    return to_bf16_bits(host_uniform((r, K), 1.0 / np.sqrt(K), seed, *key, "A"))


def lora_B_bf16(N: int, r: int, seed: int, *key) -> np.ndarray:
    return to_bf16_bits(host_normal((N, r), STD["B"], seed, *key, "B"))


def act_bf16(T: int, width: int, seed: int, *key) -> np.ndarray:
    return to_bf16_bits(host_normal((T, width), 1.0, seed, *key))


def single_linear(seed: int = 0, T: int = 512, K: int = 896, N: int = 896, r: int = 16) -> dict:
    """The single LoRA linear: W fp32, A, B, X, dY bf16 bit patterns."""
    key = ("single", T, K, N, r)
    return {
        "W": weight_f32(N, K, seed, *key),
        "A": lora_A_bf16(r, K, seed, *key),
        "B": lora_B_bf16(N, r, seed, *key),
        "X": act_bf16(T, K, seed, *key, "X"),
        "dY": act_bf16(T, N, seed, *key, "dY"),
    }


# ---- device draws (torch Philox) for large shapes ------------------------------------------

def device_generator(seed: int, *key):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(key_seed(seed, *key))
    return g


def device_normal(shape, std: float, seed: int, *key, dtype=None):
    """N(0, std) fp32 on the GPU, converted to `dtype` (e.g. torch.bfloat16) if given."""
    import torch
    t = torch.randn(shape, generator=device_generator(seed, *key), device="cuda",
                    dtype=torch.float32)
    t.mul_(std)
    return t if dtype is None else t.to(dtype)


def device_uniform(shape, bound: float, seed: int, *key, dtype=None):
    import torch
    t = torch.rand(shape, generator=device_generator(seed, *key), device="cuda",
                   dtype=torch.float32)
    t.mul_(2.0).sub_(1.0).mul_(bound)
    return t if dtype is None else t.to(dtype)
