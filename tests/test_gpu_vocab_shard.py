"""GPU parity of the vocabulary-shard path (through the C ABI) against the
plain unsharded fp64 definitions (oracle/rkl_oracle.py,
oracle/logprob_entropy_oracle.py): each shard's log-sum-exps over its own
columns, the merged loss and statistics over the whole vocabulary, the
summed dh and the shards' dW rows.

Every shard of a vocabulary runs on this one GPU in turn, as the ranks of a
vocabulary-parallel group would run theirs; the shards' partials are stacked
as an all-gather would leave them and merged by rkl_combine_shards.  Each
shard's backward is rkl_backward_hidden on the shard's weight rows (or
rkl_backward_logits on its logit columns) with the merged stats.  Bars as in
test_gpu_parity; the summed dh uses the same bar.
"""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev, u8
from oracle import rkl_oracle as O
from oracle import vocab_shard_oracle as S
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _run_shards(torch, hs, Ws, ht, Wt, bounds, g=None, row_mask=None):
    parts = [R.forward_hidden_shard(hs, Ws[a:b], ht, Wt[a:b]) for a, b in bounds]
    partials = torch.stack(parts).contiguous()
    loss, stats = R.combine_shards(partials, row_mask=row_mask)
    dh_terms, dW_rows = [], []
    for a, b in bounds:
        dh, dW = R.backward_hidden(hs, Ws[a:b], ht, Wt[a:b], stats, grad_loss=g, row_mask=row_mask)
        dh_terms.append(host(dh).astype(np.float64))
        dW_rows.append(host(dW))
    torch.cuda.synchronize()
    return host(partials), host(loss), host(stats), sum(dh_terms), np.concatenate(dW_rows)


@pytest.mark.parametrize("bounds", [
    [(0, 1000), (1000, 1001), (1001, 3001)],     # uneven, with a one-column shard
    S.shard_bounds(3001, 8),
])
def test_shards_against_oracle(tdev, bounds):
    torch, dev = tdev
    case = synth.random_case(600, T=300, V=3001, Hs=128, Ht=192, p_mask=1.0, with_grad=True)
    say("vocab shards", len(bounds))
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    g = f32(case.grad, dev)
    partials, loss, stats, dh, dW = _run_shards(torch, hs, Ws, ht, Wt, bounds, g)
    inp = O.Inputs.from_case(case)
    rows = np.arange(case.T)
    for (a, b), P in zip(bounds, partials):
        # each shard's m + log S is the log-sum-exp over its own columns
        cols = np.arange(a, b)
        assert_loss_close(P[0] + np.log(P[1]), O.logsumexp(inp.zs(rows, cols)), f"shard [{a},{b}) lse_s")
        assert_loss_close(P[3] + np.log(P[4]), O.logsumexp(inp.zt(rows, cols)), f"shard [{a},{b}) lse_t")
    # the merged statistics against the plain unsharded definitions
    full = O.backward(inp, rows, case.grad.astype(np.float64))
    lpmax = np.max(inp.zs(rows), axis=1) - full["lse_s"]   # log of the largest p_s
    assert_loss_close(loss, full["L"], "loss")
    assert_loss_close(stats[:, 0], full["lse_s"], "lse_s")
    assert_loss_close(stats[:, 1], full["lse_t"], "lse_t")
    assert np.array_equal(stats[:, 2], loss)
    assert_loss_close(stats[:, 3], lpmax, "log p_max")
    assert_grad_close(dh, full["dh"], "dh (sum over shards)")
    assert_grad_close(dW, full["dW"], "dW (shard rows)")


def test_sharded_equals_unsharded_within_tolerance(tdev):
    torch, dev = tdev
    case = synth.random_case(601, T=256, V=5000, Hs=64, Ht=64, p_mask=1.0)
    say("vocab shards vs single device")
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    _, loss, stats, dh, dW = _run_shards(torch, hs, Ws, ht, Wt, S.shard_bounds(5000, 4))
    loss1, stats1 = R.forward_hidden(hs, Ws, ht, Wt)
    dh1, dW1 = R.backward_hidden(hs, Ws, ht, Wt, stats1)
    assert_loss_close(loss, host(loss1).astype(np.float64), "loss")
    assert_loss_close(stats[:, :2], host(stats1)[:, :2].astype(np.float64), "lse")
    assert_grad_close(dh, host(dh1).astype(np.float64), "dh")
    assert_grad_close(dW, host(dW1).astype(np.float64), "dW")


def test_one_shard_partial_finalises_like_the_forward(tdev):
    """G = 1: merging one partial is the single-device forward's own combine
    over the same split plan, bit for bit."""
    torch, dev = tdev
    case = synth.random_case(602, T=200, V=2100, Hs=128, Ht=64, p_mask=1.0)
    say("vocab one shard")
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    P = R.forward_hidden_shard(hs, Ws, ht, Wt)
    loss, stats = R.combine_shards(P.unsqueeze(0).contiguous())
    loss1, stats1 = R.forward_hidden(hs, Ws, ht, Wt)
    assert np.array_equal(host(loss), host(loss1))
    assert np.array_equal(host(stats), host(stats1))


def test_full_row_mask_in_the_combine(tdev):
    """Full-row mode: the shards run over all T rows and the combine zeroes
    the rows whose mask is 0; the live rows equal the compacted rows' results
    bit for bit (a row's partial depends on the shard's vocabulary only)."""
    torch, dev = tdev
    case = synth.random_case(603, T=333, V=2500, Hs=64, Ht=128, p_mask=0.6)
    say("vocab shards full-row")
    bounds = S.shard_bounds(2500, 3)
    mask = u8(case.mask, dev)
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    _, loss_f, stats_f, dh_f, _ = _run_shards(torch, hs, Ws, ht, Wt, bounds, row_mask=mask)
    idx, N = R.compact_rows(mask)
    _, loss_c, stats_c, dh_c, _ = _run_shards(torch, R.gather_rows(hs, idx), Ws, R.gather_rows(ht, idx), Wt, bounds)
    rows, live = host(idx), case.mask != 0
    assert np.array_equal(loss_f[rows], loss_c) and np.array_equal(stats_f[rows], stats_c)
    assert np.all(loss_f[~live] == 0.0) and np.all(stats_f[~live] == 0.0)
    assert np.array_equal(dh_f[rows], dh_c) and np.all(dh_f[~live] == 0.0)


def test_empty_rows(tdev):
    torch, dev = tdev
    say("vocab shards N=0")
    z = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device=dev)
    P = R.forward_hidden_shard(z, W, z, W)
    loss, stats = R.combine_shards(torch.stack([P, P]).contiguous())
    assert loss.shape == (0,) and stats.shape == (0, 4)


@pytest.mark.parametrize("student_logits", [False, True])
def test_logit_shards_against_oracle(tdev, student_logits):
    """Teacher-logits payload: each shard gets its own columns of z_t (and of
    z_s when the student is given as logits) as a dense [N, V_shard] block."""
    torch, dev = tdev
    case = synth.random_case(604 + int(student_logits), T=200, V=2600, Hs=128, Ht=0, p_mask=1.0,
                             student_logits=student_logits, teacher_logits=True, with_grad=True)
    say("vocab shards, teacher logits, student logits" if student_logits else "vocab shards, teacher logits")
    bounds = [(0, 1300), (1300, 1301), (1301, 2600)]
    zt, g = f32(case.z_t, dev), f32(case.grad, dev)
    if student_logits:
        zs = f32(case.z_s, dev)
        side = [dict(z_s=zs[:, a:b].contiguous()) for a, b in bounds]
    else:
        hs, Ws = bf16(case.h_s, dev), bf16(case.W_s, dev)
        side = [dict(h_s=hs, W_s=Ws[a:b]) for a, b in bounds]
    zt_k = [zt[:, a:b].contiguous() for a, b in bounds]
    parts = [R.forward_logits_shard(z, **kw) for z, kw in zip(zt_k, side)]
    loss, stats = R.combine_shards(torch.stack(parts).contiguous())
    grads = [R.backward_logits(z, stats, grad_loss=g, **kw) for z, kw in zip(zt_k, side)]
    torch.cuda.synchronize()

    zs_ref = case.z_s.astype(np.float64) if student_logits else O.project(O.widen_bf16(case.h_s),
                                                                          O.widen_bf16(case.W_s))
    zt_ref = case.z_t.astype(np.float64)
    # the merged statistics against the plain unsharded definitions
    L, (ls, lt) = O.reverse_kl(zs_ref, zt_ref), (O.logsumexp(zs_ref), O.logsumexp(zt_ref))
    lpmax = np.max(zs_ref, axis=1) - ls
    assert_loss_close(host(loss), L, "loss")
    assert_loss_close(host(stats)[:, 0], ls, "lse_s")
    assert_loss_close(host(stats)[:, 1], lt, "lse_t")
    assert_loss_close(host(stats)[:, 3], lpmax, "log p_max")
    gg = case.grad.astype(np.float64)
    if student_logits:
        dz = np.concatenate([host(d) for d in grads], axis=1)
        assert_grad_close(dz, O.reverse_kl_dz(zs_ref, zt_ref, ls, lt, L, gg), "dz (shard columns)")
    else:
        full = O.backward(O.Inputs.from_case(case), np.arange(case.T), gg)
        assert_grad_close(sum(host(d).astype(np.float64) for d, _ in grads), full["dh"], "dh (sum over shards)")
        assert_grad_close(np.concatenate([host(w) for _, w in grads]), full["dW"], "dW (shard rows)")


def test_logprob_entropy_shards_against_oracle(tdev):
    """Log-probability / entropy over G = 3 uneven shards (one of a single
    column): each shard sees its own rows of W and the sampled tokens in its
    own coordinates (-1 when the token is in another shard)."""
    from oracle import logprob_entropy_oracle as E
    torch, dev = tdev
    case = synth.random_case(610, T=300, V=3001, Hs=128, Ht=64, p_mask=1.0, with_grad=True)
    rng = np.random.default_rng(611)
    y = rng.integers(0, 3001, case.T).astype(np.int32)
    y[:5] = (0, 999, 1000, 1001, 3000)                # both sides of every shard edge
    g_lp = case.grad
    g_H = rng.uniform(-0.5, 0.5, case.T).astype(np.float32)
    bounds = [(0, 1000), (1000, 1001), (1001, 3001)]
    say("log-probability / entropy shards")
    h, W = bf16(case.h_s, dev), bf16(case.W_s, dev)
    y_loc = [torch.from_numpy(np.where((y >= a) & (y < b), y - a, -1).astype(np.int32)).to(dev) for a, b in bounds]
    parts = [R.forward_logprob_entropy_shard(h, W[a:b], yl) for (a, b), yl in zip(bounds, y_loc)]
    logp, ent, stats = R.combine_shards_logprob_entropy(torch.stack(parts).contiguous())
    grads = [R.backward_logprob_entropy(h, W[a:b], yl, stats, grad_logp=f32(g_lp, dev), grad_entropy=f32(g_H, dev))
             for (a, b), yl in zip(bounds, y_loc)]
    logp1, ent1, _ = R.forward_logprob_entropy(h, W, torch.from_numpy(y).to(dev))
    torch.cuda.synchronize()

    wh, wW = O.widen_bf16(case.h_s), O.widen_bf16(case.W_s)
    # the merged statistics against the plain unsharded definitions
    lp, H, lse = E.forward(wh, wW, y)
    lpmax = np.max(O.project(wh, wW), axis=1) - lse
    assert_loss_close(host(logp), lp, "logp")
    assert_loss_close(host(ent), H, "entropy")
    assert_loss_close(host(stats)[:, 0], lse, "lse")
    assert_loss_close(host(stats)[:, 3], lpmax, "log p_max")
    assert_loss_close(host(logp), host(logp1).astype(np.float64), "logp sharded vs single device")
    assert_loss_close(host(ent), host(ent1).astype(np.float64), "entropy sharded vs single device")
    full = E.backward(wh, wW, y, g_lp.astype(np.float64), g_H.astype(np.float64))
    assert_grad_close(sum(host(d).astype(np.float64) for d, _ in grads), full["dh"], "dh (sum over shards)")
    assert_grad_close(np.concatenate([host(w) for _, w in grads]), full["dW"], "dW (shard rows)")
