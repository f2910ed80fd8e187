"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: a closed form, an
invariant of the mathematics, a library routine that computes the same
textbook quantity, brute force on tiny inputs, or central finite differences.
They are chosen so that a plausible slip (a dropped term, a wrong sign, a
swapped operand, a transposed weight) fails at least one of them.
"""
import inspect
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import rkl_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- data handling

def test_widen_bf16_known_bits():
    bits = np.array([0x0000, 0x3F80, 0xC000, 0x3F81, 0x7F7F, 0x0001, 0x8000], dtype=np.uint16)
    want = [0.0, 1.0, -2.0, 1.0078125, 3.3895313892515355e38, 2.0 ** -133, -0.0]
    got = O.widen_bf16(bits)
    assert got.dtype == np.float64
    assert list(got) == want


def test_bf16_rounding_of_inputs_is_nearest_even():
    # halfway cases go to the even mantissa; others to nearest
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert list(b) == [0x3F80, 0x3F82, 0x3F81, 0xC020]
    # every bf16 value survives the round trip exactly
    allb = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(O.widen_bf16(allb).astype(np.float32)), allb)


@pytest.mark.parametrize("T,p", [(0, 0.5), (1, 1.0), (1, 0.0), (17, 0.0), (17, 1.0), (257, 0.3), (1000, 0.9)])
def test_compact_rows_brute_force(T, p):
    mask = (_rng(T).random(T) < p).astype(np.uint8)
    mask[mask == 1] = _rng(T + 1).integers(1, 256, size=int(mask.sum())).astype(np.uint8)  # any nonzero byte counts
    idx = O.compact_rows(mask)
    assert idx.dtype == np.int32
    assert np.array_equal(idx, np.flatnonzero(mask))
    assert idx.shape[0] == int(np.count_nonzero(mask))
    assert np.all(np.diff(idx) > 0)


def test_gather_scatter_roundtrip_and_zero_fill():
    T, W = 50, 7
    src = _rng(3).standard_normal((T, W)).astype(np.float32)
    mask = (_rng(4).random(T) < 0.4).astype(np.uint8)
    idx = O.compact_rows(mask)
    g = O.gather_rows(src, idx)
    assert g.shape == (idx.shape[0], W)
    back = O.scatter_rows(g, idx, T)
    assert np.array_equal(back[idx], src[idx])
    assert np.all(back[mask == 0] == 0.0)
    assert not np.any(np.signbit(back[mask == 0]))   # literal +0.0
    # empty selection
    e = O.scatter_rows(O.gather_rows(src, O.compact_rows(np.zeros(T, np.uint8))), np.zeros(0, np.int32), T)
    assert np.array_equal(e, np.zeros_like(src))


# ---------------------------------------------------------------- log-softmax

def test_log_softmax_textbook_and_library():
    z = _rng(5).standard_normal((6, 9)) * 3
    direct = np.log(np.exp(z) / np.exp(z).sum(1, keepdims=True))
    assert np.allclose(O.log_softmax(z), direct, rtol=0, atol=1e-13)
    assert np.allclose(O.log_softmax(z), scipy.special.log_softmax(z, axis=1), rtol=0, atol=1e-13)
    assert np.allclose(O.logsumexp(z), scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-13)
    assert np.allclose(np.exp(O.log_softmax(z)).sum(1), 1.0, atol=1e-14)
    # single-entry vocabulary: probability one
    assert np.all(O.log_softmax(np.array([[3.7], [-1e3]])) == 0.0)


def test_log_softmax_shift_invariance_far_from_zero():
    z = _rng(6).standard_normal((4, 33))
    for c in (1000.0, -1000.0, 88.0):
        assert np.allclose(O.log_softmax(z + c), O.log_softmax(z), rtol=0, atol=1e-11)
        assert np.allclose(O.logsumexp(z + c), O.logsumexp(z) + c, rtol=1e-15, atol=1e-11)


# ---------------------------------------------------------------- reverse KL

def _kl_v2(a0, a1, b0, b1):
    p = 1.0 / (1.0 + math.exp(-(a1 - a0)))
    q = 1.0 / (1.0 + math.exp(-(b1 - b0)))
    return p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q)), p


def test_reverse_kl_two_token_closed_form():
    for a0, a1, b0, b1 in itertools.product([-1.3, 0.0, 2.1], [0.4, -3.0], [0.0, 1.7], [-0.6, 2.2]):
        want, p = _kl_v2(a0, a1, b0, b1)
        got = O.reverse_kl(np.array([[a0, a1]]), np.array([[b0, b1]]))[0]
        assert abs(got - want) <= 1e-14 * max(1.0, abs(want))


def test_reverse_kl_hand_value():
    # p = (1/4, 3/4), q = (1/2, 1/2): L = 1/4 ln(1/2) + 3/4 ln(3/2)
    got = O.reverse_kl(np.array([[0.0, math.log(3.0)]]), np.zeros((1, 2)))[0]
    assert abs(got - (0.25 * math.log(0.5) + 0.75 * math.log(1.5))) < 1e-15


def test_reverse_kl_matches_scipy_relative_entropy():
    zs = _rng(7).standard_normal((5, 101)) * 2
    zt = _rng(8).standard_normal((5, 101)) * 2
    ps = scipy.special.softmax(zs, axis=1)
    pt = scipy.special.softmax(zt, axis=1)
    want = np.array([scipy.stats.entropy(ps[i], pt[i]) for i in range(5)])   # sum p log(p/q)
    assert np.allclose(O.reverse_kl(zs, zt), want, rtol=1e-12, atol=1e-14)
    # the direction matters: KL(p_s || p_t) is not KL(p_t || p_s)
    other = np.array([scipy.stats.entropy(pt[i], ps[i]) for i in range(5)])
    assert np.max(np.abs(O.reverse_kl(zs, zt) - other)) > 1e-2


def test_reverse_kl_gibbs_and_self_distillation():
    rng = _rng(9)
    for V in (2, 3, 17, 1000):
        zs = rng.standard_normal((8, V)) * 3
        zt = rng.standard_normal((8, V)) * 3
        assert np.all(O.reverse_kl(zs, zt) >= 0.0)
        assert np.all(O.reverse_kl(zs, zs) == 0.0)          # identical inputs: exactly zero
        assert np.all(np.abs(O.reverse_kl(zs, zs + 5.0)) < 1e-12)   # same distribution


def test_reverse_kl_uniform_student_and_uniform_teacher():
    rng = _rng(10)
    V = 257
    zt = rng.standard_normal((4, V)) * 2
    zs = rng.standard_normal((4, V)) * 2
    # uniform student: L = -log V - mean_v log p_t
    want_u_s = -math.log(V) - O.log_softmax(zt).mean(1)
    assert np.allclose(O.reverse_kl(np.full((4, V), 0.3), zt), want_u_s, rtol=1e-12, atol=1e-13)
    # uniform teacher: L = log V - H(p_s)
    ps = scipy.special.softmax(zs, axis=1)
    ent = np.array([scipy.stats.entropy(ps[i]) for i in range(4)])
    assert np.allclose(O.reverse_kl(zs, np.full((4, V), -2.0)), math.log(V) - ent, rtol=1e-12, atol=1e-13)


def test_reverse_kl_shift_invariance():
    zs = _rng(11).standard_normal((3, 50))
    zt = _rng(12).standard_normal((3, 50))
    base = O.reverse_kl(zs, zt)
    for cs, ct in ((1000.0, -1000.0), (-700.0, 3.0)):
        assert np.allclose(O.reverse_kl(zs + cs, zt + ct), base, rtol=0, atol=1e-11)


def test_row_stats_consistent():
    zs = _rng(13).standard_normal((3, 40))
    zt = _rng(14).standard_normal((3, 40))
    ls, lt, L = O.row_stats(zs, zt)
    assert np.allclose(ls, scipy.special.logsumexp(zs, axis=1), atol=1e-13)
    assert np.allclose(lt, scipy.special.logsumexp(zt, axis=1), atol=1e-13)
    assert np.allclose(L, O.reverse_kl(zs, zt), atol=0)


# ---------------------------------------------------------------- dz

def test_dz_two_token_closed_form():
    for a0, a1, b0, b1 in itertools.product([-1.3, 0.0, 2.1], [0.4, -3.0], [0.0, 1.7], [-0.6, 2.2]):
        _, p = _kl_v2(a0, a1, b0, b1)
        d1 = p * (1 - p) * ((a1 - a0) - (b1 - b0))
        zs = np.array([[a0, a1]])
        zt = np.array([[b0, b1]])
        dz = O.reverse_kl_dz(zs, zt, *O.row_stats(zs, zt))
        assert abs(dz[0, 1] - d1) < 1e-14 and abs(dz[0, 0] + d1) < 1e-14


def _central_diff(f, x, eps):
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp = x.copy(); xp[i] += eps
        xm = x.copy(); xm[i] -= eps
        g[i] = (f(xp) - f(xm)) / (2 * eps)
    return g


def test_dz_finite_differences_and_row_sum():
    rng = _rng(15)
    for V in (2, 3, 7):
        zs = rng.standard_normal((4, V)) * 2
        zt = rng.standard_normal((4, V)) * 2
        g = rng.uniform(0.3, 2.0, 4)
        dz = O.reverse_kl_dz(zs, zt, *O.row_stats(zs, zt), g)
        fd = _central_diff(lambda z: float(np.dot(g, O.reverse_kl(z, zt))), zs, 1e-6)
        assert np.allclose(dz, fd, rtol=1e-7, atol=1e-9)
        assert np.all(np.abs(dz.sum(1)) <= 1e-14 * np.abs(dz).max())
        # linear in the upstream gradient
        dz1 = O.reverse_kl_dz(zs, zt, *O.row_stats(zs, zt))
        assert np.allclose(dz, dz1 * g[:, None], rtol=1e-15, atol=0)


def test_dz_on_column_subset_equals_full_columns():
    zs = _rng(16).standard_normal((3, 30))
    zt = _rng(17).standard_normal((3, 30))
    st = O.row_stats(zs, zt)
    cols = np.array([0, 4, 29, 11])
    full = O.reverse_kl_dz(zs, zt, *st)
    part = O.reverse_kl_dz(zs[:, cols], zt[:, cols], *st)
    assert np.array_equal(full[:, cols], part)


def test_dz_zero_for_self_distillation():
    zs = _rng(18).standard_normal((3, 30))
    assert np.all(O.reverse_kl_dz(zs, zs, *O.row_stats(zs, zs)) == 0.0)


# ---------------------------------------------------------------- whole path

def _tiny_hidden(seed, N=4, V=7, Hs=5, Ht=6):
    rng = _rng(seed)
    bits = lambda a: synth.f32_to_bf16_bits(a.astype(np.float32))
    return O.Inputs(h_s=bits(rng.standard_normal((N, Hs))), W_s=bits(rng.standard_normal((V, Hs)) * 0.7),
                    h_t=bits(rng.standard_normal((N, Ht))), W_t=bits(rng.standard_normal((V, Ht)) * 0.7))


def test_dh_dW_finite_differences():
    inp = _tiny_hidden(19)
    N = inp.h_s.shape[0]
    rows = np.arange(N)
    g = _rng(20).uniform(0.5, 1.5, N)
    out = O.backward(inp, rows, g)

    def loss_h(h):
        return float(np.dot(g, O.reverse_kl(O.project(h, inp.W_s), inp.zt(rows))))

    def loss_W(W):
        return float(np.dot(g, O.reverse_kl(O.project(inp.h_s, W), inp.zt(rows))))

    assert np.allclose(out["dh"], _central_diff(loss_h, inp.h_s.copy(), 1e-6), rtol=1e-6, atol=1e-9)
    assert np.allclose(out["dW"], _central_diff(loss_W, inp.W_s.copy(), 1e-6), rtol=1e-6, atol=1e-9)
    # the teacher side gets no gradient: L moves with W_t but backward reports
    # student grads only (beside the row statistics it rebuilt)
    assert set(out) == {"dh", "dW", "L", "lse_s", "lse_t"}


def test_forward_matches_definition_and_chunking():
    inp = _tiny_hidden(21, N=9, V=11, Hs=8, Ht=4)
    rows = np.arange(9)
    L, ls, lt = O.forward(inp, rows, row_chunk=2)
    zs = O.project(inp.h_s, inp.W_s)
    zt = O.project(inp.h_t, inp.W_t)
    ps = scipy.special.softmax(zs, axis=1)
    pt = scipy.special.softmax(zt, axis=1)
    want = np.array([scipy.stats.entropy(ps[i], pt[i]) for i in range(9)])
    assert np.allclose(L, want, rtol=1e-12, atol=1e-15)
    assert np.allclose(ls, scipy.special.logsumexp(zs, axis=1), atol=1e-13)
    b1 = O.backward(inp, rows, row_chunk=2)
    b2 = O.backward(inp, rows, row_chunk=100)
    assert np.allclose(b1["dW"], b2["dW"], rtol=0, atol=1e-15) and np.allclose(b1["dh"], b2["dh"], rtol=0, atol=1e-15)
    # the backward's row statistics are the scipy values too
    assert np.allclose(b1["L"], want, rtol=1e-12, atol=1e-15)
    assert np.allclose(b1["lse_s"], scipy.special.logsumexp(zs, axis=1), atol=1e-13)
    assert np.allclose(b1["lse_t"], scipy.special.logsumexp(zt, axis=1), atol=1e-13)


def test_projection_orientation():
    # z[i, v] = <h_i, W_v>: a one-hot hidden row picks out a column of W
    W = np.arange(12, dtype=np.float64).reshape(4, 3)   # [V=4, H=3]
    h = np.array([[0.0, 1.0, 0.0]])
    assert np.array_equal(O.project(h, W)[0], W[:, 1])


def test_logits_path_equals_hidden_path():
    case = synth.random_case(22, T=40, V=300, Hs=64, Ht=128)
    hid = O.Inputs.from_case(case)
    lg = O.Inputs(h_s=case.h_s, W_s=case.W_s, z_t=O.project_f32(case.h_t, case.W_t))
    rows = O.compact_rows(case.mask)
    Lh, _, _ = O.forward(hid, rows)
    Ll, _, _ = O.forward(lg, rows)
    assert np.allclose(Lh, Ll, rtol=1e-5, atol=1e-7)      # fp32 rounding of the payload only
    bh = O.backward(hid, rows)
    bl = O.backward(lg, rows)
    assert np.max(np.abs(bh["dW"] - bl["dW"])) <= 1e-5 * np.max(np.abs(bh["dW"]))
    # exact when the payload is the fp64 projection itself
    lg64 = O.Inputs(h_s=case.h_s, W_s=case.W_s, z_t=O.project(hid.h_t, hid.W_t))
    assert np.array_equal(O.forward(lg64, rows)[0], Lh)


def test_compact_equals_full_and_masked_rows_are_zero():
    case = synth.random_case(23, T=60, V=130, Hs=64, Ht=64, p_mask=0.4)
    inp = O.Inputs.from_case(case)
    per_pos = O.per_position_loss(inp, case.mask)
    L_all, _, _ = O.forward(inp, np.arange(60))
    m = case.mask != 0
    assert np.array_equal(per_pos[m], L_all[m])
    assert np.all(per_pos[~m] == 0.0)
    # gradients of the compact sum equal those of the full sum with g = mask
    idx = O.compact_rows(case.mask)
    bc = O.backward(inp, idx)
    bf = O.backward(inp, np.arange(60), g=m.astype(np.float64))
    assert np.allclose(bc["dW"], bf["dW"], rtol=0, atol=1e-15)
    assert np.allclose(O.scatter_rows(bc["dh"], idx, 60), bf["dh"], rtol=0, atol=1e-15)


def test_empty_mask():
    case = synth.random_case(24, T=12, V=50, Hs=64, Ht=64, p_mask=0.0)
    assert case.mask.sum() == 0
    inp = O.Inputs.from_case(case)
    assert np.array_equal(O.per_position_loss(inp, case.mask), np.zeros(12))
    b = O.backward(inp, O.compact_rows(case.mask))
    assert b["dh"].shape == (0, 64) and np.all(b["dW"] == 0.0)


def test_dW_rows_matches_full_backward():
    case = synth.random_case(25, T=30, V=90, Hs=64, Ht=128, p_mask=0.6, with_grad=True)
    inp = O.Inputs.from_case(case)
    idx = O.compact_rows(case.mask)
    g = case.grad[idx]
    full = O.backward(inp, idx, g)
    st = O.forward(inp, idx)
    vs = np.array([0, 7, 89, 45])
    assert np.allclose(O.dW_rows(inp, idx, vs, st, g), full["dW"][vs], rtol=1e-13, atol=1e-16)


def test_student_logits_backward_is_dz():
    case = synth.random_case(26, T=10, V=40, Hs=0, Ht=0, student_logits=True, teacher_logits=True)
    inp = O.Inputs.from_case(case)
    rows = np.arange(10)
    b = O.backward(inp, rows)
    assert set(b) == {"dz", "L", "lse_s", "lse_t"}
    fd = _central_diff(lambda z: float(O.reverse_kl(z, inp.zt(rows)).sum()),
                       case.z_s.astype(np.float64), 1e-5)
    assert np.allclose(b["dz"], fd, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- the pages' one number

def test_payload_ratio_claim():
    with open(os.path.join(GOLDEN, "payload_ratio.json")) as f:
        claim = json.load(f)
    # one token's teacher payload: V logits vs H hidden values, same element type
    ratio = claim["vocab"] / claim["hidden"]
    assert round(ratio) == claim["claimed_ratio"]
    # the Qwen3-1.7B-shaped synthetic workload has exactly these widths
    sig = inspect.signature(synth.qwen_shaped).parameters
    assert sig["V"].default == claim["vocab"] and sig["Ht"].default == claim["hidden"]
