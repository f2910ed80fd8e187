"""Pins for the fp64 log-probability / entropy oracle (CPU only).

Each check ties oracle/logprob_entropy_oracle.py to something other than
itself: closed forms (uniform logits, two-token vocabulary, a point mass),
scipy's own log-softmax and entropy routines, bounds the definitions imply,
and central finite differences of the forward for every gradient.  A dropped
term (the one-hot, the +H inside the entropy gradient), a wrong sign or a
transposed weight fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import logprob_entropy_oracle as E


def _rng(seed):
    return np.random.default_rng(seed)


def _objective(z, y, g_lp, g_H):
    logp, H, _ = E.logprob_entropy(z, y)
    return float(np.sum(g_lp * logp + g_H * H))


# ----------------------------------------------------------------- forward

def test_uniform_logits():
    """Equal logits: H = log V and log p(y) = -log V for every y."""
    for V in (1, 2, 7, 1000):
        z = np.full((3, V), 1.7)
        y = np.array([0, V - 1, V // 2])
        logp, H, lse = E.logprob_entropy(z, y)
        assert np.allclose(H, math.log(V), rtol=0, atol=1e-12)
        assert np.allclose(logp, -math.log(V), rtol=0, atol=1e-12)
        assert np.allclose(lse, 1.7 + math.log(V), rtol=0, atol=1e-12)


def test_two_token_closed_form():
    """V = 2: p = sigmoid(z1 - z0), H = -p log p - (1-p) log(1-p),
    log p(1) = log sigmoid(z1 - z0), log p(0) = log sigmoid(z0 - z1)."""
    rng = _rng(1)
    z = rng.normal(0, 3, size=(50, 2))
    d = z[:, 1] - z[:, 0]
    p = 1.0 / (1.0 + np.exp(-d))
    for y, want in ((1, -np.log1p(np.exp(-d))), (0, -np.log1p(np.exp(d)))):
        logp, H, _ = E.logprob_entropy(z, np.full(50, y))
        assert np.allclose(logp, want, rtol=1e-12, atol=1e-14)
        assert np.allclose(H, -p * np.log(p) - (1 - p) * np.log(1 - p), rtol=1e-10, atol=1e-14)


def test_point_mass_limit():
    """One logit far above the rest: H -> 0 and log p(argmax) -> 0, while a
    non-argmax token gets log p = -(gap) to first order."""
    z = np.array([[0.0, 0.0, 60.0, 0.0]])
    logp, H, _ = E.logprob_entropy(z, np.array([2]))
    assert abs(logp[0]) < 1e-24 and 0 <= H[0] < 1e-23
    logp0, _, _ = E.logprob_entropy(z, np.array([0]))
    assert logp0[0] == pytest.approx(-60.0, abs=1e-12)


def test_matches_scipy_routines():
    """scipy's log_softmax and entropy compute the same textbook quantities."""
    rng = _rng(2)
    z = rng.normal(0, 2.5, size=(20, 97))
    y = rng.integers(0, 97, 20)
    logp, H, lse = E.logprob_entropy(z, y)
    ref_lp = scipy.special.log_softmax(z, axis=-1)
    assert np.allclose(logp, ref_lp[np.arange(20), y], rtol=1e-13, atol=1e-13)
    assert np.allclose(H, scipy.stats.entropy(np.exp(ref_lp), axis=-1), rtol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(z, axis=-1), rtol=1e-14)


def test_bounds_and_shift_invariance():
    rng = _rng(3)
    z = rng.normal(0, 4, size=(40, 33))
    y = rng.integers(0, 33, 40)
    logp, H, _ = E.logprob_entropy(z, y)
    assert np.all(H >= -1e-15) and np.all(H <= math.log(33) + 1e-12)
    assert np.all(logp <= 0)
    logp2, H2, _ = E.logprob_entropy(z + rng.normal(0, 100, size=(40, 1)), y)
    assert np.allclose(logp2, logp, atol=1e-11) and np.allclose(H2, H, atol=1e-11)


# ----------------------------------------------------------------- gradients

def test_dz_sums_to_zero_and_is_linear_in_g():
    """sum_v dz = g_lp (1 - sum p) - g_H (sum p log p + H) = 0 per row; dz is
    linear in (g_lp, g_H)."""
    rng = _rng(4)
    z = rng.normal(0, 2, size=(6, 41))
    y = rng.integers(0, 41, 6)
    g1, g2 = rng.normal(size=6), rng.normal(size=6)
    _, H, lse = E.logprob_entropy(z, y)
    a = E.logprob_entropy_dz(z, y, lse, H, g1, 0 * g1)
    b = E.logprob_entropy_dz(z, y, lse, H, 0 * g2, g2)
    both = E.logprob_entropy_dz(z, y, lse, H, g1, g2)
    assert np.allclose(both.sum(axis=1), 0, atol=1e-13)
    assert np.allclose(both, a + b, atol=1e-15)
    assert np.allclose(E.logprob_entropy_dz(z, y, lse, H, 3 * g1, 3 * g2), 3 * both, atol=1e-14)


def test_dz_central_differences():
    rng = _rng(5)
    z = rng.normal(0, 1.5, size=(3, 6))
    y = np.array([0, 5, 2])
    g_lp, g_H = rng.normal(size=3), rng.normal(size=3)
    _, H, lse = E.logprob_entropy(z, y)
    dz = E.logprob_entropy_dz(z, y, lse, H, g_lp, g_H)
    eps = 1e-6
    fd = np.zeros_like(z)
    for i in range(z.shape[0]):
        for v in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[i, v] += eps
            zm[i, v] -= eps
            fd[i, v] = (_objective(zp, y, g_lp, g_H) - _objective(zm, y, g_lp, g_H)) / (2 * eps)
    assert np.allclose(dz, fd, rtol=1e-7, atol=1e-9)


def test_column_subset_matches_full():
    """dz on a subset of the vocabulary columns (what a vocabulary chunk sees)
    equals those columns of the full dz, one-hot included."""
    rng = _rng(6)
    z = rng.normal(0, 2, size=(5, 30))
    y = np.array([3, 29, 0, 17, 17])
    _, H, lse = E.logprob_entropy(z, y)
    full = E.logprob_entropy_dz(z, y, lse, H, rng.normal(size=5), rng.normal(size=5))
    g_lp, g_H = rng.normal(size=5), rng.normal(size=5)
    full = E.logprob_entropy_dz(z, y, lse, H, g_lp, g_H)
    cols = np.array([0, 3, 16, 17, 29])
    part = E.logprob_entropy_dz(z[:, cols], y, lse, H, g_lp, g_H, cols=cols)
    assert np.array_equal(part, full[:, cols])


def test_dh_dW_central_differences():
    """dh = dz W and dW = dz^T h against central differences of the forward
    with respect to h and W (tiny shapes)."""
    rng = _rng(7)
    n, V, Hd = 3, 5, 4
    h = rng.normal(size=(n, Hd))
    W = rng.normal(0, 0.7, size=(V, Hd))
    y = np.array([4, 0, 2])
    g_lp, g_H = rng.normal(size=n), rng.normal(size=n)
    b = E.backward(h, W, y, g_lp, g_H)

    def F(hh, WW):
        logp, H, _ = E.forward(hh, WW, y)
        return float(np.sum(g_lp * logp + g_H * H))

    eps = 1e-6
    fd_h = np.zeros_like(h)
    for idx in np.ndindex(*h.shape):
        hp, hm = h.copy(), h.copy()
        hp[idx] += eps
        hm[idx] -= eps
        fd_h[idx] = (F(hp, W) - F(hm, W)) / (2 * eps)
    fd_W = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        fd_W[idx] = (F(h, Wp) - F(h, Wm)) / (2 * eps)
    assert np.allclose(b["dh"], fd_h, rtol=1e-7, atol=1e-9)
    assert np.allclose(b["dW"], fd_W, rtol=1e-7, atol=1e-9)


def test_dW_rows_and_row_chunking():
    """Selected dW rows equal the full dW's rows; row chunking changes nothing."""
    rng = _rng(8)
    h = rng.normal(size=(37, 8))
    W = rng.normal(0, 0.5, size=(23, 8))
    y = rng.integers(0, 23, 37)
    g_lp, g_H = rng.normal(size=37), rng.normal(size=37)
    full = E.backward(h, W, y, g_lp, g_H, row_chunk=5, want_dz=True)
    one = E.backward(h, W, y, g_lp, g_H, row_chunk=1000)
    assert np.allclose(full["dW"], one["dW"], atol=1e-13) and np.allclose(full["dh"], one["dh"], atol=1e-13)
    logp, H, lse = E.forward(h, W, y, row_chunk=7)
    vocab = np.array([0, 5, 22])
    assert np.allclose(E.dW_rows(h, W, y, vocab, lse, H, g_lp, g_H), full["dW"][vocab], atol=1e-13)
