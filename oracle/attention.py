"""Oracle for causal multi-head attention with grouped key/value heads, forward and backward, in
fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the product path.

Source: the pages train Llama-3.1 and Qwen2.5 decoder layers ("Exact Layer Streaming", Abstract;
"An 8B Fine-Tune Now Fits in 4 GB of VRAM": the decoder layer is the streamed unit) and print no
attention formula. This is the published definition those models use, written out: causal
scaled dot-product attention where query head h reads key/value head h // (n_q / n_kv)
(consecutive query heads share a key/value head), on a batch of equal-length sequences packed
row after row (T = n_seq * S token rows; sequence b is rows b S .. b S + S - 1):

    s_ij  = scale * (q_i . k_j)            for j <= i in the same sequence (scale = 1/sqrt(d))
    lse_i = log sum_j exp(s_ij)
    P_ij  = exp(s_ij - lse_i)
    O_i   = sum_j P_ij v_j

Backward, for an upstream gradient dO:
    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j,   D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
with dK and dV of a shared key/value head summed over the query heads that read it.

Layouts: q [T][n_q d], k and v [T][n_kv d], head h in columns h d .. h d + d - 1; O like q;
lse [T][n_q].
"""

from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _heads(x, T, n, d):
    return _f64(x).reshape(T, n, d)


def _scores(qh, kh, scale):
    """[S, S] scaled scores of one sequence and head, -inf above the diagonal."""
    S = qh.shape[0]
    s = scale * (qh @ kh.T)
    s[np.triu_indices(S, k=1)] = -np.inf
    return s


def _lse(s):
    m = s.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]


def forward(q, k, v, n_seq: int, n_q: int, n_kv: int, d: int, scale: float | None = None):
    """Returns (O [T][n_q d], lse [T][n_q]) in fp64."""
    T = _f64(q).shape[0]
    S = T // n_seq
    assert S * n_seq == T and n_q % n_kv == 0
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    Q, K, V = _heads(q, T, n_q, d), _heads(k, T, n_kv, d), _heads(v, T, n_kv, d)
    O = np.zeros((T, n_q, d))
    L = np.zeros((T, n_q))
    group = n_q // n_kv
    for b in range(n_seq):
        r = slice(b * S, (b + 1) * S)
        for h in range(n_q):
            g = h // group
            s = _scores(Q[r, h], K[r, g], scale)
            lse = _lse(s)
            P = np.exp(s - lse[:, None])
            O[r, h] = P @ V[r, g]
            L[r, h] = lse
    return O.reshape(T, n_q * d), L


def backward(q, k, v, dO, n_seq: int, n_q: int, n_kv: int, d: int, scale: float | None = None):
    """Returns (dq, dk, dv) in fp64, the gradients of sum(O * dO)."""
    T = _f64(q).shape[0]
    S = T // n_seq
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    Q, K, V = _heads(q, T, n_q, d), _heads(k, T, n_kv, d), _heads(v, T, n_kv, d)
    G = _heads(dO, T, n_q, d)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    group = n_q // n_kv
    for b in range(n_seq):
        r = slice(b * S, (b + 1) * S)
        for h in range(n_q):
            g = h // group
            s = _scores(Q[r, h], K[r, g], scale)
            P = np.exp(s - _lse(s)[:, None])
            O = P @ V[r, g]
            dV[r, g] += P.T @ G[r, h]
            dP = G[r, h] @ V[r, g].T
            D = (G[r, h] * O).sum(axis=1)
            dS = P * (dP - D[:, None])
            dQ[r, h] = scale * (dS @ K[r, g])
            dK[r, g] += scale * (dS.T @ Q[r, h])
    return dQ.reshape(T, n_q * d), dK.reshape(T, n_kv * d), dV.reshape(T, n_kv * d)
