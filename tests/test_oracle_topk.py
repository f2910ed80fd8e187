"""Pins of the top-k estimator oracle (oracle/topk_oracle.py) against what
the NeMo-RL page and the mathematics fix: the K = V limit is the exact
reverse KL and its gradient; the empty support is the sampled token's
log-probability gap; for every support the estimator and its gradient are
unbiased over the student's sampled token (exact enumeration); the support
part's gradient is the derivative of its value (central differences); dh
and dW follow from dz by the chain rule."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import topk_oracle as K


def _rng(seed):
    return np.random.default_rng(seed)


def _row(seed, V=9):
    r = _rng(seed)
    zs = r.normal(0, 1.5, V)
    zt = r.normal(0, 1.5, V)
    return zs, zt, scipy.special.log_softmax(zs), scipy.special.log_softmax(zt)


def _full_rkl_grad(zs, zt):
    """Gradient of sum_v p_s (log p_s - log p_t) in z_s by central differences."""
    def L(z):
        return scipy.stats.entropy(scipy.special.softmax(z), scipy.special.softmax(zt))
    g = np.zeros_like(zs)
    for j in range(zs.size):
        e = np.zeros_like(zs)
        e[j] = 1e-6
        g[j] = (L(zs + e) - L(zs - e)) / 2e-6
    return g


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_whole_vocabulary_support_is_the_reverse_kl(seed):
    zs, zt, lps, lpt = _row(seed)
    V = zs.size
    S = _rng(seed + 10).permutation(V)          # K = V, any order
    want_L = scipy.stats.entropy(np.exp(lps), np.exp(lpt))
    want_g = _full_rkl_grad(zs, zt)
    for y in range(V):                          # the tail is absent whatever was sampled
        L, g = K.estimator(lps, lpt[S], lpt[y], S, y)
        assert L == pytest.approx(want_L, rel=1e-12, abs=1e-14)
        assert np.allclose(g, want_g, rtol=1e-6, atol=1e-9)


def test_empty_support_is_the_sampled_token_gap():
    zs, zt, lps, lpt = _row(3)
    p = np.exp(lps)
    for y in range(zs.size):
        L, g = K.estimator(lps, np.zeros(0), lpt[y], np.zeros(0, np.int64), y)
        gap = lps[y] - lpt[y]
        assert L == pytest.approx(gap, rel=1e-13)
        e = np.zeros_like(p)
        e[y] = 1.0
        assert np.allclose(g, (gap + 1.0) * (e - p), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("Kk", [1, 3, 8])
def test_unbiased_over_the_sampled_token(Kk):
    """sum_y p_s(y) L_hat(y) = L and sum_y p_s(y) g_hat(y) = grad L for a support
    chosen without y."""
    zs, zt, lps, lpt = _row(20 + Kk)
    p = np.exp(lps)
    S = _rng(30 + Kk).choice(zs.size, Kk, replace=False)
    EL, Eg = 0.0, np.zeros_like(p)
    for y in range(zs.size):
        L, g = K.estimator(lps, lpt[S], lpt[y], S, y)
        EL += p[y] * L
        Eg += p[y] * g
    assert EL == pytest.approx(scipy.stats.entropy(p, np.exp(lpt)), rel=1e-12)
    assert np.allclose(Eg, _full_rkl_grad(zs, zt), rtol=1e-6, atol=1e-9)


def test_support_part_gradient_by_central_differences():
    """With y in S there is no tail: g_hat is the derivative of L_hat."""
    zs, zt, lps, lpt = _row(40)
    S = np.array([4, 0, 7])
    y = 0

    def val(z):
        lp = scipy.special.log_softmax(z)
        return K.estimator(lp, lpt[S], 123.0, S, y)[0]   # lpt_y unused: y in S
    _, g = K.estimator(lps, lpt[S], 123.0, S, y)
    fd = np.array([(val(zs + e) - val(zs - e)) / 2e-6 for e in np.eye(zs.size) * 1e-6])
    assert np.allclose(g, fd, rtol=1e-6, atol=1e-9)
    # and the gradient sums to zero over the vocabulary (softmax invariance)
    assert abs(np.sum(g)) < 1e-13


def test_two_token_closed_form():
    """V = 2, S = {0}, y = 1 (outside the support): L_hat = p0 f0 + f1,
    dL_hat/dz1 = -p1 p0 (f0 + 1) + (f1 + 1) p0, by hand."""
    zs, zt = np.array([0.3, -0.4]), np.array([-1.0, 0.5])
    lps, lpt = scipy.special.log_softmax(zs), scipy.special.log_softmax(zt)
    p0, p1 = np.exp(lps)
    f0, f1 = lps - lpt
    L, g = K.estimator(lps, lpt[[0]], lpt[1], np.array([0]), 1)
    assert L == pytest.approx(p0 * f0 + f1, rel=1e-14)
    assert g[1] == pytest.approx(-p1 * p0 * (f0 + 1) + (f1 + 1) * (1 - p1), rel=1e-13)
    assert g[0] == pytest.approx(p0 * (1 - p0) * (f0 + 1) - (f1 + 1) * p0, rel=1e-13)


def test_chain_rule_and_mask():
    r = _rng(50)
    N, V, H, Kk = 6, 11, 5, 3
    h, W = r.normal(0, 1, (N, H)), r.normal(0, 0.5, (V, H))
    lpt = scipy.special.log_softmax(r.normal(0, 1, (N, V)), axis=1)
    S = np.stack([r.choice(V, Kk, replace=False) for _ in range(N)])
    y = np.array([S[0, 1], 2, 3, S[3, 0], 9, 10])
    g = r.uniform(0.5, 1.5, N)
    mask = np.array([1, 1, 0, 1, 1, 1])
    out = K.forward_backward(h, W, y, S, np.take_along_axis(lpt, S, 1), lpt[np.arange(N), y], g, mask)
    assert out["L"][2] == 0.0 and np.all(out["dz"][2] == 0.0)
    lp = scipy.special.log_softmax(h @ W.T, axis=1)
    for i in range(N):
        if mask[i]:
            L, gz = K.estimator(lp[i], lpt[i, S[i]], lpt[i, y[i]], S[i], y[i])
            assert out["L"][i] == pytest.approx(L, rel=1e-13)
            assert np.allclose(out["dz"][i], g[i] * gz, rtol=1e-13, atol=1e-16)
    # dh = dz W and dW = dz^T h: central differences of the rows whose
    # sampled token lies in their support (no tail, so the value's derivative)
    live = [i for i in range(N) if mask[i] and y[i] in S[i]]

    def surrogate(hh, WW):
        lpp = scipy.special.log_softmax(hh @ WW.T, axis=1)
        return sum(g[i] * K.estimator(lpp[i], lpt[i, S[i]], 0.0, S[i], y[i])[0] for i in live)
    sub = K.forward_backward(h[live], W, y[live], S[live], np.take_along_axis(lpt[live], S[live], 1),
                             lpt[live, y[live]], g[live])
    eps = 1e-6
    fd_h = np.zeros((len(live), H))
    for a, i in enumerate(live):
        for k in range(H):
            e = np.zeros_like(h)
            e[i, k] = eps
            fd_h[a, k] = (surrogate(h + e, W) - surrogate(h - e, W)) / (2 * eps)
    assert np.allclose(sub["dh"], fd_h, rtol=1e-6, atol=1e-9)
    fd_W = np.zeros_like(W)
    for v in range(V):
        for k in range(H):
            e = np.zeros_like(W)
            e[v, k] = eps
            fd_W[v, k] = (surrogate(h, W + e) - surrogate(h, W - e)) / (2 * eps)
    assert np.allclose(sub["dW"], fd_W, rtol=1e-6, atol=1e-9)


def test_planted_mistakes_fail_the_pins():
    """A dropped '+1', a wrong tail sign, or a tail kept when y is in S each
    change the result of a pin above."""
    zs, zt, lps, lpt = _row(60)
    p = np.exp(lps)
    S = np.array([1, 2])
    y = 5

    def wrong_grad_no_plus_one(lp):
        pp = np.exp(lp)
        g = np.zeros_like(pp)
        for v in S:
            fv = lp[v] - lpt[v]
            g[v] += pp[v] * fv
            g -= pp[v] * fv * pp
        return g
    _, good = K.estimator(lps, lpt[S], lpt[y], S, y)
    assert not np.allclose(good, wrong_grad_no_plus_one(lps) + (lps[y] - lpt[y] + 1) * (np.eye(zs.size)[y] - p))
    # expectation over y with the tail's sign flipped is biased
    EL = sum(p[yy] * (K.estimator(lps, lpt[S], lpt[yy], S, yy)[0]
                      - 2 * (0 if yy in S else lps[yy] - lpt[yy])) for yy in range(zs.size))
    assert abs(EL - scipy.stats.entropy(p, np.exp(lpt))) > 1e-3
