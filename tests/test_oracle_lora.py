"""Pins for the LoRA oracle (oracle/lora.py).

* gradients: fp64 central finite differences of L = <dY, Y>, which is affine in each of X, A
  and B separately, so the differences carry no truncation error;
* forward: special cases that reduce to a textbook GEMM (B = 0, adapters off, r = K with
  A = I) and the merged-weight identity Y = X (W + s B A)^T;
* products: a pure-Python triple loop on tiny non-square shapes.
Shapes are non-square everywhere so that a transposed operand cannot go unnoticed.
"""

import numpy as np

from oracle import lora

T, K, N, R, S = 5, 7, 6, 3, 1.75


def _rand(seed):
    rng = np.random.default_rng(seed)
    X = rng.normal(size=(T, K))
    W = rng.normal(size=(N, K))
    A = rng.normal(size=(R, K))
    B = rng.normal(size=(N, R))
    dY = rng.normal(size=(T, N))
    return X, W, A, B, dY


def _loss(X, W, A, B, dY):
    Y, _ = lora.forward(X, W, A, B, S)
    return float(np.sum(dY * Y))


def _fd(f, x, h=1e-3):
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_gradients_match_finite_differences():
    X, W, A, B, dY = _rand(0)
    dX, dA, dB, G = lora.backward(X, dY, W, A, B, S)
    fd_X = _fd(lambda x: _loss(x, W, A, B, dY), X)
    fd_A = _fd(lambda a: _loss(X, W, a, B, dY), A)
    fd_B = _fd(lambda b: _loss(X, W, A, b, dY), B)
    for got, want in ((dX, fd_X), (dA, fd_A), (dB, fd_B)):
        assert got.shape == want.shape
        assert lora.rel_l2(got, want) < 1e-8
    np.testing.assert_allclose(G, dY @ B, rtol=1e-14)


def test_b_zero_reproduces_base_exactly():
    X, W, A, B, _ = _rand(1)
    Y, U = lora.forward(X, W, A, np.zeros_like(B), S)
    assert np.array_equal(Y, X @ W.T)
    assert U.shape == (T, R)


def test_adapters_off_is_frozen_base():
    X, W, A, B, _ = _rand(2)
    Y, U = lora.forward(X, W, A, B, S, adapters=False)
    assert U is None and np.array_equal(Y, X @ W.T)


def test_merged_weight_identity():
    X, W, A, B, _ = _rand(3)
    Y, _ = lora.forward(X, W, A, B, S)
    np.testing.assert_allclose(Y, X @ (W + S * B @ A).T, rtol=1e-12, atol=1e-12)


def test_full_rank_identity_adapter_is_plain_gemm():
    rng = np.random.default_rng(4)
    X, W = rng.normal(size=(T, K)), rng.normal(size=(N, K))
    B = rng.normal(size=(N, K))
    Y, U = lora.forward(X, W, np.eye(K), B, S)
    assert np.array_equal(U, X)
    np.testing.assert_allclose(Y, X @ (W + S * B).T, rtol=1e-12, atol=1e-12)


def test_triple_loop_brute_force():
    X, W, A, B, dY = _rand(5)
    Y, U = lora.forward(X, W, A, B, S)
    dX, dA, dB, G = lora.backward(X, dY, W, A, B, S)
    Ub = [[sum(X[t][k] * A[j][k] for k in range(K)) for j in range(R)] for t in range(T)]
    Yb = [[sum(X[t][k] * W[n][k] for k in range(K)) + S * sum(Ub[t][j] * B[n][j] for j in range(R))
           for n in range(N)] for t in range(T)]
    Gb = [[sum(dY[t][n] * B[n][j] for n in range(N)) for j in range(R)] for t in range(T)]
    dXb = [[sum(dY[t][n] * W[n][k] for n in range(N)) + S * sum(Gb[t][j] * A[j][k] for j in range(R))
            for k in range(K)] for t in range(T)]
    dBb = [[S * sum(dY[t][n] * Ub[t][j] for t in range(T)) for j in range(R)] for n in range(N)]
    dAb = [[S * sum(Gb[t][j] * X[t][k] for t in range(T)) for k in range(K)] for j in range(R)]
    for got, want in ((U, Ub), (Y, Yb), (G, Gb), (dX, dXb), (dB, dBb), (dA, dAb)):
        np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


def test_rel_l2():
    ref = np.array([3.0, 4.0])
    assert lora.rel_l2(ref, ref) == 0.0
    assert abs(lora.rel_l2(ref + np.array([0.3, 0.4]), ref) - 0.1) < 1e-15
