"""Pins of the cross-entropy oracle (oracle/ce.py) against what the mathematics fixes: a uniform
head gives log V exactly and no hidden-state gradient, two classes reduce to the softplus, the
probabilities of a row sum to one, ignored rows contribute nothing, the hidden-state gradient
matches central finite differences of the mean loss, and the lookup is a plain row copy."""

import numpy as np

from oracle import ce


def test_uniform_head_gives_log_v_and_no_gradient():
    rng = np.random.default_rng(0)
    T, H, V = 5, 8, 37
    h = rng.normal(size=(T, H))
    W = np.zeros((V, H))
    labels = rng.integers(0, V, T)
    loss, dz, dh = ce.cross_entropy(h, W, labels, 1.0 / T)
    np.testing.assert_allclose(loss, np.log(V), rtol=0, atol=1e-15)
    assert np.all(dh == 0)
    # dz = (1/V - onehot) / T
    want = np.full((T, V), 1.0 / V)
    want[np.arange(T), labels] -= 1.0
    np.testing.assert_allclose(dz, want / T, rtol=0, atol=1e-16)


def test_two_classes_reduce_to_softplus():
    rng = np.random.default_rng(1)
    T, H = 6, 4
    h = rng.normal(size=(T, H))
    W = rng.normal(size=(2, H))
    labels = rng.integers(0, 2, T)
    loss, _, _ = ce.cross_entropy(h, W, labels, 1.0)
    z = h @ W.T
    other = z[np.arange(T), 1 - labels] - z[np.arange(T), labels]
    np.testing.assert_allclose(loss, np.log1p(np.exp(other)), rtol=1e-14)


def test_rows_sum_to_zero_gradient_and_ignored_rows_vanish():
    rng = np.random.default_rng(2)
    T, H, V = 7, 6, 11
    h = rng.normal(size=(T, H)) * 3
    W = rng.normal(size=(V, H))
    labels = rng.integers(0, V, T)
    labels[[1, 4]] = [-100, V]                  # ignored: negative, and past the vocabulary
    loss, dz, dh = ce.cross_entropy(h, W, labels, 0.5)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)   # softmax sums to one
    assert loss[1] == 0 and loss[4] == 0
    assert np.all(dz[[1, 4]] == 0) and np.all(dh[[1, 4]] == 0)
    assert np.all(loss[[0, 2, 3, 5, 6]] > 0)


def test_hidden_gradient_matches_finite_differences():
    rng = np.random.default_rng(3)
    T, H, V = 4, 5, 9
    h = rng.normal(size=(T, H))
    W = rng.normal(size=(V, H))
    labels = np.array([3, -1, 0, 8])
    n = 3                                       # counted rows
    _, _, dh = ce.cross_entropy(h, W, labels, 1.0 / n)

    def mean_loss(hh):
        return ce.cross_entropy(hh, W, labels, 1.0 / n)[0].sum() / n

    eps = 1e-6
    num = np.zeros_like(h)
    for i in range(T):
        for j in range(H):
            d = np.zeros_like(h)
            d[i, j] = eps
            num[i, j] = (mean_loss(h + d) - mean_loss(h - d)) / (2 * eps)
    np.testing.assert_allclose(dh, num, rtol=1e-6, atol=1e-9)


def test_large_logits_do_not_overflow():
    h = np.array([[1000.0, -1000.0]])
    W = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.5]])
    loss, dz, _ = ce.cross_entropy(h, W, np.array([0]), 1.0)
    assert np.isfinite(loss).all() and np.isfinite(dz).all()
    np.testing.assert_allclose(loss, 0.0, atol=1e-12)   # the label's logit dominates by 1000


def test_embed_copies_rows_and_zeroes_bad_ids():
    E = np.arange(20, dtype=np.float32).reshape(5, 4)
    X = ce.embed(np.array([4, 0, -1, 5, 2]), E)
    np.testing.assert_array_equal(X[0], E[4])
    np.testing.assert_array_equal(X[1], E[0])
    np.testing.assert_array_equal(X[4], E[2])
    assert np.all(X[2] == 0) and np.all(X[3] == 0)
