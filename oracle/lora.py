"""Oracle for the LoRA linear on a frozen (dequantised) base, forward and backward, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the product path.

Source: "Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript
@1:25-1:58: the base is frozen (no gradient, no optimizer state) and a thin pair of
trainable matrices rides alongside each adapted layer.  The pages print no formula; this is
the standard LoRA linear with rank r, scale s = alpha / r, no bias and no dropout:

    U  = X A^T                     X [T,K], A [r,K]  ->  U [T,r]
    Y  = X W^T + s U B^T           W [N,K], B [N,r]  ->  Y [T,N]      (adapters off: Y = X W^T)
    G  = dY B                      dY [T,N]          ->  G [T,r]
    dX = dY W + s G A                                ->  dX [T,K]
    dB = s dY^T U                                    ->  dB [N,r]
    dA = s G^T X                                     ->  dA [r,K]

The same transcript (@7:32) has every layer fetched on two occasions in a step: for the
forward and again when the backward recomputes that layer's forward. The recompute applies
the same function to the same bytes, so the oracle has no separate recompute.

All inputs are the exact values of bf16 (or fp32) tensors, widened to fp64; products use
numpy's fp64 matmul as a library primitive.  Results are fp64, unrounded.
"""

from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def forward(X, W_hat, A, B, s: float, adapters: bool = True):
    """Returns (Y, U) in fp64.  With adapters off, Y = X W^T and U is None."""
    X, W_hat = _f64(X), _f64(W_hat)
    Y = X @ W_hat.T
    if not adapters:
        return Y, None
    A, B = _f64(A), _f64(B)
    U = X @ A.T
    Y = Y + float(s) * (U @ B.T)
    return Y, U


def backward(X, dY, W_hat, A, B, s: float):
    """Returns (dX, dA, dB, G) in fp64, for Y = X W^T + s (X A^T) B^T."""
    X, dY, W_hat, A, B = _f64(X), _f64(dY), _f64(W_hat), _f64(A), _f64(B)
    s = float(s)
    U = X @ A.T
    G = dY @ B
    dX = dY @ W_hat + s * (G @ A)
    dB = s * (dY.T @ U)
    dA = s * (G.T @ X)
    return dX, dA, dB, G


def rel_l2(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    got, ref = _f64(got).ravel(), _f64(ref).ravel()
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)
