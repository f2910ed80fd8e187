"""Pins for the vocabulary-shard oracle (CPU only).

The shard partials and their log-sum-exp merge are tied to the unsharded
definitions of oracle/rkl_oracle.py (full-row log-softmax and reverse KL), to
scipy's logsumexp for each shard, and to the shard order; the shard backward
is tied to the unsharded backward (dz columns, dW rows, dh as a sum over
shards).  A merge that forgot a rescaling factor, swapped the two sides, or
dropped a shard fails the first check: the shards' maxima differ.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import synth
from oracle import rkl_oracle as O
from oracle import vocab_shard_oracle as S


def _problem(seed, n=24, V=61, Hs=16, Ht=24, spread=3.0):
    rng = np.random.default_rng(seed)

    def bits(shape, sigma):
        return synth.f32_to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))

    b = dict(h_s=bits((n, Hs), 1.0), W_s=bits((V, Hs), 0.5), h_t=bits((n, Ht), 1.0), W_t=bits((V, Ht), 0.5))
    # give the shards different maxima: scale some vocabulary rows up
    w = {k: O.widen_bf16(v) for k, v in b.items()}
    w["W_s"][: V // 3] *= spread
    w["W_t"][V // 2:] *= spread
    return b, w


def _full(w):
    inp = O.Inputs.__new__(O.Inputs)
    inp.h_s, inp.W_s, inp.h_t, inp.W_t, inp.z_s, inp.z_t = w["h_s"], w["W_s"], w["h_t"], w["W_t"], None, None
    return inp


@pytest.mark.parametrize("bounds", [
    [(0, 61)],                                   # one shard
    [(0, 20), (20, 21), (21, 61)],               # uneven, with a one-column shard
    S.shard_bounds(61, 8),
    [(v, v + 1) for v in range(61)],             # every column its own shard
])
def test_merged_shards_equal_the_unsharded_definition(bounds):
    _, w = _problem(1)
    parts = [S.shard_partials(w["h_s"], w["W_s"], w["h_t"], w["W_t"], a, b) for a, b in bounds]
    L, ls, lt, lpmax = S.merge(parts)
    rows = np.arange(w["h_s"].shape[0])
    L0, ls0, lt0 = O.forward(_full(w), rows)
    assert np.allclose(ls, ls0, rtol=1e-14, atol=1e-13)
    assert np.allclose(lt, lt0, rtol=1e-14, atol=1e-13)
    assert np.allclose(L, L0, rtol=1e-11, atol=1e-13)
    lp = O.log_softmax(O.project(w["h_s"], w["W_s"]))
    assert np.allclose(lpmax, lp.max(axis=1), rtol=0, atol=1e-13)


def test_each_shard_partial_against_scipy():
    _, w = _problem(2)
    a, b = 10, 37
    P = S.shard_partials(w["h_s"], w["W_s"], w["h_t"], w["W_t"], a, b)
    zs = O.project(w["h_s"], w["W_s"][a:b])
    zt = O.project(w["h_t"], w["W_t"][a:b])
    assert np.allclose(P[0] + np.log(P[1]), scipy.special.logsumexp(zs, axis=1), rtol=1e-15, atol=1e-13)
    assert np.allclose(P[3] + np.log(P[4]), scipy.special.logsumexp(zt, axis=1), rtol=1e-15, atol=1e-13)
    assert np.array_equal(P[0], zs.max(axis=1)) and np.array_equal(P[3], zt.max(axis=1))
    # A / S_s is the shard-local softmax's expectation of z_s - z_t
    p = scipy.special.softmax(zs, axis=1)
    assert np.allclose(P[2] / P[1], np.sum(p * (zs - zt), axis=1), rtol=1e-12, atol=1e-13)


def test_shard_order_does_not_matter():
    _, w = _problem(3)
    bounds = S.shard_bounds(61, 5)
    parts = [S.shard_partials(w["h_s"], w["W_s"], w["h_t"], w["W_t"], a, b) for a, b in bounds]
    x = S.merge(parts)
    y = S.merge(parts[::-1])
    for a, b in zip(x, y):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


def test_shard_bounds_cover_the_vocabulary():
    for V, G in ((61, 8), (151936, 8), (7, 7), (5, 1)):
        b = S.shard_bounds(V, G)
        assert b[0][0] == 0 and b[-1][1] == V and len(b) == G
        assert all(b[i][1] == b[i + 1][0] for i in range(G - 1))
        assert max(e - s for s, e in b) - min(e - s for s, e in b) <= 1
    assert S.shard_bounds(151936, 8)[0] == (0, 18992)


def test_shard_backward_adds_up_to_the_unsharded_backward():
    _, w = _problem(4)
    rows = np.arange(w["h_s"].shape[0])
    g = np.random.default_rng(5).uniform(0.5, 1.5, rows.shape[0])
    bounds = [(0, 20), (20, 21), (21, 61)]
    parts = [S.shard_partials(w["h_s"], w["W_s"], w["h_t"], w["W_t"], a, b) for a, b in bounds]
    L, ls, lt, _ = S.merge(parts)
    full = O.backward(_full(w), rows, g, want_dz=True)
    dh = np.zeros_like(full["dh"])
    for a, b in bounds:
        r = S.shard_backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], a, b, (L, ls, lt), g)
        assert np.allclose(r["dz"], full["dz"][:, a:b], rtol=1e-10, atol=1e-14)
        assert np.allclose(r["dW"], full["dW"][a:b], rtol=1e-10, atol=1e-13)
        dh += r["dh"]
    assert np.allclose(dh, full["dh"], rtol=1e-10, atol=1e-13)


def test_logit_shards_equal_the_unsharded_definition():
    """Either side given as logits: shard partials of column slices merge to
    the full-row log-sum-exps and reverse KL of the same logits."""
    rng = np.random.default_rng(6)
    zs = rng.standard_normal((20, 97)) * 2.0
    zt = rng.standard_normal((20, 97)) * 2.0
    zs[:, 50:] += 4.0                       # different maxima per shard
    bounds = [(0, 13), (13, 50), (50, 51), (51, 97)]
    L, ls, lt, lpmax = S.merge([S.partials_of_logits(zs[:, a:b], zt[:, a:b]) for a, b in bounds])
    assert np.allclose(ls, scipy.special.logsumexp(zs, axis=1), rtol=1e-15, atol=1e-13)
    assert np.allclose(lt, scipy.special.logsumexp(zt, axis=1), rtol=1e-15, atol=1e-13)
    assert np.allclose(L, O.reverse_kl(zs, zt), rtol=1e-11, atol=1e-13)
    assert np.allclose(lpmax, O.log_softmax(zs).max(axis=1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("bounds", [
    [(0, 61)],
    [(0, 20), (20, 21), (21, 61)],
    S.shard_bounds(61, 8),
    [(v, v + 1) for v in range(61)],
])
def test_logprob_entropy_shards_equal_the_unsharded_definition(bounds):
    from oracle import logprob_entropy_oracle as E
    _, w = _problem(7)
    n = w["h_s"].shape[0]
    y = np.random.default_rng(8).integers(0, 61, n)
    y[:4] = (0, 19, 20, 60)                       # shard edges
    lp, H, lse, lpmax = S.lpe_merge([S.lpe_shard_partials(w["h_s"], w["W_s"], y, a, b) for a, b in bounds])
    z = O.project(w["h_s"], w["W_s"])
    lp0, H0, lse0 = E.logprob_entropy(z, y)
    assert np.allclose(lse, lse0, rtol=1e-14, atol=1e-13)
    assert np.allclose(lp, lp0, rtol=1e-12, atol=1e-12)
    assert np.allclose(H, H0, rtol=1e-11, atol=1e-12)
    assert np.allclose(H, scipy.stats.entropy(scipy.special.softmax(z, axis=1), axis=1), rtol=1e-10, atol=1e-12)
    assert np.allclose(lpmax, O.log_softmax(z).max(axis=1), rtol=0, atol=1e-13)


def test_logprob_entropy_shard_partial_pieces():
    _, w = _problem(9)
    y = np.arange(w["h_s"].shape[0]) * 3 % 61
    a, b = 10, 37
    P = S.lpe_shard_partials(w["h_s"], w["W_s"], y, a, b)
    z = O.project(w["h_s"], w["W_s"][a:b])
    assert np.allclose(P[0] + np.log(P[1]), scipy.special.logsumexp(z, axis=1), rtol=1e-15, atol=1e-13)
    p = scipy.special.softmax(z, axis=1)
    assert np.allclose(P[2] / P[1], np.sum(p * z, axis=1), rtol=1e-12, atol=1e-13)
    inside = (y >= a) & (y < b)
    assert np.all(np.isneginf(P[3][~inside]))
    assert np.array_equal(P[3][inside], z[np.nonzero(inside)[0], y[inside] - a])
