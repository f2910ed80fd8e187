"""Pins for the per-row-teacher reverse-KL oracle (CPU only).

The multi-teacher oracle selects W_t per row and otherwise reuses the
single-teacher definitions; these checks tie it to independent single-teacher
computations: one teacher equals the single-teacher oracle, each teacher's
rows equal a single-teacher run over that group alone (dW adds up over the
groups), a row permutation permutes every per-row result, and a teacher that
is the student gives exactly zero on its rows.
"""
import numpy as np

import synth
from oracle import multi_teacher_oracle as M
from oracle import rkl_oracle as O


def _bits(rng, shape, sigma):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def _problem(seed, n=40, V=53, Hs=16, Ht=24, K=3):
    rng = np.random.default_rng(seed)
    b = dict(h_s=_bits(rng, (n, Hs), 1.0), W_s=_bits(rng, (V, Hs), 0.5),
             h_t=_bits(rng, (n, Ht), 1.0), W_t=_bits(rng, (K, V, Ht), 0.5))
    teacher = rng.integers(0, K, n)
    g = rng.uniform(0.5, 1.5, n)
    return b, teacher, g


def _w(b):
    return {k: O.widen_bf16(v) for k, v in b.items()}


def test_one_teacher_is_the_single_teacher_oracle():
    b, _, g = _problem(1, K=1)
    w = _w(b)
    teacher = np.zeros(w["h_s"].shape[0], np.int64)
    got = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    inp = O.Inputs(h_s=b["h_s"], W_s=b["W_s"], h_t=b["h_t"], W_t=b["W_t"][0])
    rows = np.arange(w["h_s"].shape[0])
    want = O.forward(inp, rows)
    for x, y in zip(got, want):
        assert np.array_equal(x, y)
    gb = M.backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, g)
    wb = O.backward(inp, rows, g)
    assert np.allclose(gb["dh"], wb["dh"], rtol=0, atol=1e-14)
    assert np.allclose(gb["dW"], wb["dW"], rtol=0, atol=1e-13)


def test_each_group_is_a_single_teacher_run():
    """Rows of teacher k alone through the single-teacher oracle with W_t[k]
    give the same L, lse and dh; dW is the sum of the groups' dW."""
    b, teacher, g = _problem(2)
    w = _w(b)
    L, ls, lt = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    gb = M.backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, g)
    dW_sum = np.zeros_like(gb["dW"])
    for k in range(b["W_t"].shape[0]):
        rows = np.nonzero(teacher == k)[0]
        inp = O.Inputs(h_s=b["h_s"][rows], W_s=b["W_s"], h_t=b["h_t"][rows], W_t=b["W_t"][k])
        r = np.arange(rows.shape[0])
        Lk, lsk, ltk = O.forward(inp, r)
        assert np.allclose(L[rows], Lk, rtol=1e-13, atol=1e-15)
        assert np.allclose(lt[rows], ltk, rtol=1e-13, atol=1e-15)
        bk = O.backward(inp, r, g[rows])
        assert np.allclose(gb["dh"][rows], bk["dh"], rtol=1e-12, atol=1e-15)
        dW_sum += bk["dW"]
    assert np.allclose(gb["dW"], dW_sum, rtol=1e-12, atol=1e-14)


def test_row_permutation_equivariance():
    b, teacher, g = _problem(3)
    w = _w(b)
    perm = np.random.default_rng(9).permutation(w["h_s"].shape[0])
    L, _, _ = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    Lp, _, _ = M.forward(w["h_s"][perm], w["W_s"], w["h_t"][perm], w["W_t"], teacher[perm])
    assert np.allclose(Lp, L[perm], rtol=1e-13, atol=1e-15)
    gb = M.backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, g)
    gp = M.backward(w["h_s"][perm], w["W_s"], w["h_t"][perm], w["W_t"], teacher[perm], g[perm])
    assert np.allclose(gp["dh"], gb["dh"][perm], rtol=1e-12, atol=1e-15)
    assert np.allclose(gp["dW"], gb["dW"], rtol=1e-12, atol=1e-14)


def test_teacher_equal_to_student_gives_zero_on_its_rows():
    b, teacher, _ = _problem(4, Hs=16, Ht=16)
    b["W_t"][1] = b["W_s"]
    b["h_t"] = b["h_s"].copy()
    w = _w(b)
    L, _, _ = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    assert np.all(L[teacher == 1] == 0.0)
    assert np.all(L[teacher != 1] > 0.0)


def test_dW_rows_matches_backward():
    b, teacher, g = _problem(5)
    w = _w(b)
    stats = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    gb = M.backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, g, row_chunk=7)
    vocab = np.array([0, 7, 52])
    got = M.dW_rows(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, vocab, stats, g)
    assert np.allclose(got, gb["dW"][vocab], rtol=1e-12, atol=1e-14)
