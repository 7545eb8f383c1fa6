"""Oracle for the resident ends of the stack: the frozen embedding lookup and cross-entropy
through the frozen LM head, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the product path.

Source: "Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @7:42-7:55:
the embedding table and the output head stay resident and unquantised (and frozen: only the
adapters train); "Exact Layer Streaming", Abstract: the training objective's logits term.  The
pages print no formula; this is the standard token-level cross-entropy, written from its
definition:

    X_t      = E[id_t]                                  (lookup; no arithmetic)
    z        = h W^T                                    h [T,H], W [V,H]  ->  z [T,V]
    loss_t   = log sum_j exp(z_tj) - z_t,label_t        (0 for an ignored row)
    dz_tj    = scale * (softmax(z_t)_j - [j == label_t]) (0 for an ignored row)
    dh       = dz W                                     ->  dh [T,H]

so that with scale = 1/n, dh is the gradient of the mean loss over the n counted rows.  A row is
ignored when its label lies outside [0, V).  Products use numpy's fp64 matmul; the log-sum-exp
subtracts the row maximum before exponentiating (an exact identity that avoids overflow).
"""

from __future__ import annotations

import numpy as np


def embed(ids, E) -> np.ndarray:
    """X[t] = E[ids[t]]; ids outside [0, V) give zero rows."""
    ids = np.asarray(ids)
    E = np.asarray(E)
    ok = (ids >= 0) & (ids < E.shape[0])
    X = np.zeros((ids.shape[0], E.shape[1]), dtype=E.dtype)
    X[ok] = E[ids[ok]]
    return X


def logits(h, W) -> np.ndarray:
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def cross_entropy(h, W, labels, scale: float):
    """Returns (loss [T], dz [T,V], dh [T,H]) in fp64."""
    z = logits(h, W)
    T, V = z.shape
    labels = np.asarray(labels)
    counted = (labels >= 0) & (labels < V)
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    loss = np.zeros(T)
    rows = np.nonzero(counted)[0]
    loss[rows] = lse[rows] - z[rows, labels[rows]]
    p = np.exp(z - lse[:, None])
    dz = p.copy()
    dz[rows, labels[rows]] -= 1.0
    dz *= float(scale)
    dz[~counted] = 0.0
    dh = dz @ np.asarray(W, dtype=np.float64)
    return loss, dz, dh
