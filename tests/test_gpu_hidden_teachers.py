"""GPU parity of reverse KL with a teacher chosen per row (through the C ABI)
against the fp64 oracle (oracle/multi_teacher_oracle.py).

A 128-row tile holding rows of several teachers runs one teacher pass per
teacher, each with the other teachers' token columns zeroed; these tests
cover tiles of one teacher (rows grouped by teacher) and of several (rows
interleaved), and check that a row's results do not depend on which rows
share its tile.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev, u8
from oracle import multi_teacher_oracle as M
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _problem(seed, T, V, Hs, Ht, K, p_mask=0.8):
    rng = np.random.default_rng(seed)
    case = synth.random_case(seed, T=T, V=V, Hs=Hs, Ht=Ht, p_mask=p_mask, with_grad=True)
    W_t = np.stack([synth.f32_to_bf16_bits((rng.standard_normal((V, Ht)) / np.sqrt(Ht)).astype(np.float32))
                    for _ in range(K)])
    teacher = rng.integers(0, K, T).astype(np.int32)
    return case, W_t, teacher


def _run(case, W_t, teacher, dev, full_row=False):
    torch = __import__("torch")
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    if full_row:
        idx = torch.arange(case.T, dtype=torch.int32, device=dev)
    hs = R.gather_rows(bf16(case.h_s, dev), idx)
    ht = R.gather_rows(bf16(case.h_t, dev), idx)
    tk = R.gather_rows(torch.from_numpy(teacher).to(dev), idx)
    g = R.gather_rows(f32(case.grad, dev), idx)
    Ws, Wt = bf16(case.W_s, dev), bf16(W_t, dev)
    rm = mask if full_row else None
    loss, stats = R.forward_hidden_teachers(hs, Ws, ht, Wt, tk, row_mask=rm)
    dh, dW = R.backward_hidden_teachers(hs, Ws, ht, Wt, tk, stats, grad_loss=g, row_mask=rm)
    torch.cuda.synchronize()
    return host(idx), host(loss), host(stats), host(dh), host(dW)


def _check(case, W_t, teacher, out):
    idx, loss, stats, dh, dW = out
    rows = O.compact_rows(case.mask)
    assert np.array_equal(idx, rows)
    w = {k: O.widen_bf16(v) for k, v in dict(h_s=case.h_s[rows], W_s=case.W_s, h_t=case.h_t[rows], W_t=W_t).items()}
    L, ls, lt = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher[rows])
    assert_loss_close(loss, L, "loss")
    assert_loss_close(stats[:, 0], ls, "lse_s")
    assert_loss_close(stats[:, 1], lt, "lse_t")
    b = M.backward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher[rows], case.grad[rows].astype(np.float64))
    assert_grad_close(dh, b["dh"], "dh")
    assert_grad_close(dW, b["dW"], "dW")


@pytest.mark.parametrize("order", ["interleaved", "grouped"])
def test_against_oracle(tdev, order):
    """K = 3 teachers, Ht != Hs, ragged token and vocabulary tails; rows
    interleaved (every tile holds all three teachers) or grouped by teacher."""
    torch, dev = tdev
    case, W_t, teacher = _problem(500, T=300, V=3001, Hs=128, Ht=192, K=3)
    if order == "grouped":
        teacher = np.sort(teacher)
    say("teachers", order)
    _check(case, W_t, teacher, _run(case, W_t, teacher, dev))


def test_splits_per_workgroup_do_not_change_results(tdev, monkeypatch):
    """With several teachers per row the forward takes one vocabulary split
    per workgroup; a workgroup that streams several splits (V = 3001: all
    twelve one-tile splits, or two) flushes each split's statistics the same
    way: bit for bit."""
    torch, dev = tdev
    case, W_t, teacher = _problem(505, T=300, V=3001, Hs=128, Ht=192, K=3)
    say("teachers splits per workgroup")
    ref = _run(case, W_t, teacher, dev)
    for spw in ("1000", "2"):
        monkeypatch.setenv("RKL_FWD_SPLITS_PER_WG", spw)
        got = _run(case, W_t, teacher, dev)
        for a, b, what in zip(got[1:], ref[1:], ("loss", "stats", "dh", "dW")):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (spw, what)


def test_one_teacher_equals_single_teacher_path(tdev):
    torch, dev = tdev
    case, W_t, teacher = _problem(501, T=200, V=1500, Hs=128, Ht=64, K=1)
    say("teachers K=1 vs single")
    got = _run(case, W_t, teacher, dev)
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    hs, ht = R.gather_rows(bf16(case.h_s, dev), idx), R.gather_rows(bf16(case.h_t, dev), idx)
    g = R.gather_rows(f32(case.grad, dev), idx)
    Ws, Wt = bf16(case.W_s, dev), bf16(W_t[0], dev)
    loss, stats = R.forward_hidden(hs, Ws, ht, Wt)
    dh, dW = R.backward_hidden(hs, Ws, ht, Wt, stats, grad_loss=g)
    for a, b, what in zip(got[1:], (host(loss), host(stats), host(dh), host(dW)), ("loss", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


def test_row_results_do_not_depend_on_tile_neighbours(tdev):
    """The same rows in a different order (other teachers sharing each tile):
    loss, stats and dh of every row are bit-identical; dW sums the rows in
    another order, so it agrees to the tolerance."""
    torch, dev = tdev
    case, W_t, teacher = _problem(502, T=256, V=2000, Hs=64, Ht=64, K=4, p_mask=1.0)
    say("teachers permuted rows")
    a = _run(case, W_t, teacher, dev)
    perm = np.random.default_rng(7).permutation(case.T)
    case.h_s, case.h_t, case.grad = case.h_s[perm], case.h_t[perm], case.grad[perm]
    b = _run(case, W_t, teacher[perm], dev)
    for i, what in ((1, "loss"), (2, "stats"), (3, "dh")):
        assert np.array_equal(b[i].view(np.uint32), a[i][perm].view(np.uint32)), what
    assert_grad_close(b[4], a[4], "dW")


def test_teacher_equal_to_student_is_exactly_zero(tdev):
    """Teacher 1 is the student (same weight, same hidden states): its rows
    give L = 0 exactly and contribute nothing to the gradients, also in tiles
    shared with the other teachers."""
    torch, dev = tdev
    case, W_t, teacher = _problem(503, T=300, V=2500, Hs=128, Ht=128, K=3, p_mask=1.0)
    W_t[1] = case.W_s
    case.h_t = case.h_s.copy()
    say("teachers self-distillation rows")
    idx, loss, stats, dh, dW = _run(case, W_t, teacher, dev)
    own = teacher == 1
    assert np.all(loss[own] == 0.0) and np.all(dh[own] == 0.0)
    assert np.all(loss[~own] > 0.0)


def test_out_of_range_ids_act_as_a_zero_teacher(tdev):
    """Ids outside [0, K) select no teacher: those rows see teacher logits 0,
    the same as a teacher whose weight is all zeros."""
    torch, dev = tdev
    case, W_t, teacher = _problem(504, T=200, V=1000, Hs=64, Ht=64, K=2, p_mask=1.0)
    bad = np.zeros(case.T, bool)
    bad[::5] = True
    teacher[bad] = np.where(np.arange(case.T)[bad] % 2 == 0, 7, -3)
    say("teachers out-of-range ids")
    out = _run(case, W_t, teacher, dev)
    W_z = np.concatenate([W_t, np.zeros_like(W_t[:1])])
    t_ref = teacher.copy()
    t_ref[bad] = 2
    _check(case, W_z, t_ref, out)


def test_full_row_equals_compact(tdev):
    torch, dev = tdev
    case, W_t, teacher = _problem(505, T=333, V=2100, Hs=128, Ht=64, K=3, p_mask=0.5)
    say("teachers full-row vs compact")
    c = _run(case, W_t, teacher, dev)
    f = _run(case, W_t, teacher, dev, full_row=True)
    rows, m = c[0], case.mask != 0
    for i, what in ((1, "loss"), (2, "stats"), (3, "dh")):
        assert np.array_equal(f[i][rows], c[i]), what
        assert np.all(f[i][~m] == 0.0), what
    assert_grad_close(f[4], c[4], "dW full-row vs compact")


def test_the_most_teachers_with_out_of_range_ids(tdev):
    """K = 31, the largest: tile sets use bits 0..30, and ids 31 and -1 (no
    teacher) set the out-of-range bit.  Every 128-row tile holds many
    teachers before grouping; rows are compared with a zero teacher for the
    out-of-range ids, in full-row mode with a partial mask."""
    torch, dev = tdev
    K = 31
    case, W_t, teacher = _problem(506, T=700, V=1300, Hs=64, Ht=64, K=K, p_mask=0.7)
    teacher[::7] = K
    teacher[3::11] = -1
    say("teachers K=31 with out-of-range ids")
    out = _run(case, W_t, teacher, dev)
    W_z = np.concatenate([W_t, np.zeros_like(W_t[:1])])
    t_ref = np.where((teacher >= 0) & (teacher < K), teacher, K)
    _check(case, W_z, t_ref, out)
    f = _run(case, W_t, teacher, dev, full_row=True)
    rows = out[0]
    for i, what in ((1, "loss"), (2, "stats"), (3, "dh")):
        assert np.array_equal(f[i][rows], out[i]), what


def test_tiles_of_only_out_of_range_ids(tdev):
    """260 of 400 rows name no teacher: grouped last, they fill whole 128-row
    tiles that run no teacher pass at all (their teacher logits are 0)."""
    torch, dev = tdev
    case, W_t, teacher = _problem(507, T=400, V=900, Hs=64, Ht=128, K=2, p_mask=1.0)
    teacher[:260] = -5
    say("teachers: whole tiles of out-of-range ids")
    out = _run(case, W_t, teacher, dev)
    W_z = np.concatenate([W_t, np.zeros_like(W_t[:1])])
    _check(case, W_z, np.where(teacher < 0, 2, teacher), out)
