"""GPU parity of the top-k estimator of the reverse KL (rkl_forward_topk /
rkl_backward_topk through the C ABI) against its fp64 oracle
(oracle/topk_oracle.py): per-row loss, whole dh and dW, at ragged shapes,
with supports holding and missing the sampled token; the K = V limit against
the full reverse KL of the library's own teacher-logits path; K = 0 (the
sampled token's log-probability gap); full-row mode; a many-chunk backward;
out-of-range support ids skipped.

Inputs: the student as seeded bf16 hidden states and weights; the teacher
as fp32 log-probabilities log_softmax(z_t) of seeded logits z_t, on a
support of the teacher's top-K ids (argsort of z_t) and at the sampled
token.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest
import scipy.special

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev, u8
from oracle import rkl_oracle as O
from oracle import topk_oracle as TK
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _problem(seed, T, V, H, K, p_mask=1.0):
    case = synth.random_case(seed, T=T, V=V, Hs=H, Ht=0, p_mask=p_mask, teacher_logits=True, with_grad=True)
    lpt = scipy.special.log_softmax(case.z_t.astype(np.float64), axis=1).astype(np.float32)
    S = np.argsort(-case.z_t, axis=1, kind="stable")[:, :K].astype(np.int32)
    y = synth.sampled_tokens(seed, T, V)
    # half of the rows sample a token of their support (when it has one)
    if K > 0:
        y[::2] = S[::2, min(1, K - 1)]
    lpt_S = np.take_along_axis(lpt, S.astype(np.int64), 1).astype(np.float32)
    lpt_y = lpt[np.arange(T), y].astype(np.float32)
    return case, y, S, lpt_S, lpt_y


def _run(dev, case, y, S, lpt_S, lpt_y, rows=None, row_mask=None):
    torch = __import__("torch")
    sel = np.arange(case.T) if rows is None else rows
    h = bf16(case.h_s[sel], dev)
    W = bf16(case.W_s, dev)
    yy = torch.from_numpy(y[sel].astype(np.int32)).to(dev)
    Sd = None if S.shape[1] == 0 else torch.from_numpy(np.ascontiguousarray(S[sel])).to(dev)
    lS = None if S.shape[1] == 0 else f32(lpt_S[sel], dev)
    g = f32(case.grad[sel], dev)
    rm = None if row_mask is None else u8(row_mask, dev)
    loss, stats = R.forward_topk(h, W, yy, Sd, lS, f32(lpt_y[sel], dev), row_mask=rm)
    dh, dW = R.backward_topk(h, W, yy, Sd, lS, stats, grad_loss=g, row_mask=rm)
    torch.cuda.synchronize()
    return host(loss), host(stats), host(dh), host(dW)


def _oracle(case, y, S, lpt_S, lpt_y, mask=None):
    return TK.forward_backward(O.widen_bf16(case.h_s), O.widen_bf16(case.W_s), y, S.astype(np.int64),
                               lpt_S.astype(np.float64), lpt_y.astype(np.float64), case.grad.astype(np.float64), mask)


@pytest.mark.parametrize("T,V,H,K", [(300, 3001, 128, 16), (129, 257, 64, 5), (517, 2053, 192, 64), (40, 700, 64, 1)])
def test_against_oracle(tdev, T, V, H, K):
    torch, dev = tdev
    case, y, S, lpt_S, lpt_y = _problem(900 + T, T, V, H, K)
    say("top-k", T, V, H, K)
    loss, stats, dh, dW = _run(dev, case, y, S, lpt_S, lpt_y)
    want = _oracle(case, y, S, lpt_S, lpt_y)
    assert_loss_close(loss, want["L"], "loss")
    assert_grad_close(dh, want["dh"], "dh")
    assert_grad_close(dW, want["dW"], "dW")
    # the tail coefficient is zero exactly on the rows that sampled a support token
    inS = np.array([y[i] in set(S[i].tolist()) for i in range(T)])
    assert np.all(stats[inS, 2] == 0.0) and np.all(stats[~inS, 2] != 0.0)


def test_whole_vocabulary_support_is_the_reverse_kl(tdev):
    """K = V: the loss and gradients equal the full reverse KL that the
    teacher-logits path computes from the teacher's log-probabilities."""
    torch, dev = tdev
    T, V, H = 96, 300, 64
    case, y, S, lpt_S, lpt_y = _problem(950, T, V, H, V)
    say("top-k K=V")
    loss, _, dh, dW = _run(dev, case, y, S, lpt_S, lpt_y)
    lpt = np.zeros((T, V), np.float32)
    np.put_along_axis(lpt, S.astype(np.int64), lpt_S, 1)
    hs, Ws, g = bf16(case.h_s, dev), bf16(case.W_s, dev), f32(case.grad, dev)
    Lf, st = R.forward_logits(f32(lpt, dev), h_s=hs, W_s=Ws)
    dhf, dWf = R.backward_logits(f32(lpt, dev), st, h_s=hs, W_s=Ws, grad_loss=g)
    assert_loss_close(loss, host(Lf).astype(np.float64), "loss vs full reverse KL")
    assert_grad_close(dh, host(dhf).astype(np.float64), "dh vs full reverse KL")
    assert_grad_close(dW, host(dWf).astype(np.float64), "dW vs full reverse KL")
    want = _oracle(case, y, S, lpt_S, lpt_y)
    assert_loss_close(loss, want["L"], "loss vs oracle")


def test_empty_support_is_the_sampled_token_gap(tdev):
    torch, dev = tdev
    T, V, H = 200, 1500, 128
    case, y, S, lpt_S, lpt_y = _problem(960, T, V, H, 0)
    say("top-k K=0")
    loss, _, dh, dW = _run(dev, case, y, S, lpt_S, lpt_y)
    lp = O.log_softmax(O.project(O.widen_bf16(case.h_s), O.widen_bf16(case.W_s)))
    assert_loss_close(loss, lp[np.arange(T), y] - lpt_y, "log-probability gap")
    want = _oracle(case, y, S, lpt_S, lpt_y)
    assert_grad_close(dh, want["dh"], "dh")
    assert_grad_close(dW, want["dW"], "dW")


def test_full_row_mode_and_skipped_ids(tdev):
    """Rows with mask 0 give exactly 0; live rows equal the compacted run bit
    for bit; support ids outside [0, V) contribute nothing."""
    torch, dev = tdev
    T, V, H, K = 250, 2100, 64, 12
    case, y, S, lpt_S, lpt_y = _problem(970, T, V, H, K, p_mask=0.6)
    S = S.copy()
    S[5, 3], S[6, 0], S[7, 11] = -1, V, V + 1000
    say("top-k full-row")
    lf, sf, dhf, dWf = _run(dev, case, y, S, lpt_S, lpt_y, row_mask=case.mask)
    rows = O.compact_rows(case.mask)
    lc, sc, dhc, dWc = _run(dev, case, y, S, lpt_S, lpt_y, rows=rows)
    m = case.mask != 0
    assert np.array_equal(lf[rows], lc) and np.array_equal(sf[rows], sc) and np.array_equal(dhf[rows], dhc)
    assert np.all(lf[~m] == 0.0) and np.all(sf[~m] == 0.0) and np.all(dhf[~m] == 0.0)
    # the oracle with the out-of-range ids removed
    keep = [(S[i] >= 0) & (S[i] < V) for i in range(T)]
    want_L = np.zeros(T)
    for i in rows:
        lp = O.log_softmax(O.project(O.widen_bf16(case.h_s[i:i + 1]), O.widen_bf16(case.W_s)))[0]
        want_L[i] = TK.estimator(lp, lpt_S[i][keep[i]], lpt_y[i], S[i][keep[i]], int(y[i]))[0]
    assert_loss_close(lf[rows], want_L[rows], "loss (ids outside the vocabulary skipped)")


@pytest.mark.parametrize("chunk", [256, 1024])
def test_many_backward_chunks(tdev, monkeypatch, chunk):
    """The support corrections land in the right vocabulary chunk."""
    torch, dev = tdev
    monkeypatch.setenv("RKL_VOCAB_CHUNK", str(chunk))
    T, V, H, K = 180, 3001, 64, 40
    case, y, S, lpt_S, lpt_y = _problem(980 + chunk, T, V, H, K)
    say("top-k chunks", chunk)
    loss, _, dh, dW = _run(dev, case, y, S, lpt_S, lpt_y)
    want = _oracle(case, y, S, lpt_S, lpt_y)
    assert_loss_close(loss, want["L"], "loss")
    assert_grad_close(dh, want["dh"], "dh")
    assert_grad_close(dW, want["dW"], "dW")


def test_empty_rows(tdev):
    torch, dev = tdev
    say("top-k N=0")
    h = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int32, device=dev)
    S = torch.empty((0, 4), dtype=torch.int32, device=dev)
    lS = torch.empty((0, 4), dtype=torch.float32, device=dev)
    loss, stats = R.forward_topk(h, W, y, S, lS, torch.empty(0, dtype=torch.float32, device=dev))
    dh, dW = R.backward_topk(h, W, y, S, lS, stats)
    assert loss.shape == (0,) and dh.shape == (0, 64) and int(torch.count_nonzero(dW)) == 0


@pytest.mark.parametrize("T,V,H,K", [(300, 3001, 128, 16), (129, 257, 64, 13)])
def test_support_logprobs_from_the_forward(tdev, T, V, H, K):
    """The forward's optional output, the student's log-probabilities on the
    support, matches the fp64 log-softmax there (0 for ids outside [0, V)
    and on masked rows), and handing it to the backward gives dh and dW bit
    for bit as forming the support's dot products again (several batches of
    eight ids per row, and a ragged last batch at K = 13)."""
    torch, dev = tdev
    case, y, S, lpt_S, lpt_y = _problem(950 + T, T, V, H, K, p_mask=0.8)
    S = S.copy()
    S[::5, 0] = -1
    S[1::7, K - 1] = V + 3
    say("top-k support log-probabilities", T, V, H, K)
    h, W = bf16(case.h_s, dev), bf16(case.W_s, dev)
    yy = torch.from_numpy(y.astype(np.int32)).to(dev)
    Sd, lS = torch.from_numpy(np.ascontiguousarray(S)).to(dev), f32(lpt_S, dev)
    g, rm = f32(case.grad, dev), u8(case.mask, dev)
    lps = torch.full((T, K), 7.0, dtype=torch.float32, device=dev)
    loss, stats = R.forward_topk(h, W, yy, Sd, lS, f32(lpt_y, dev), row_mask=rm, logps_support=lps)
    dh0, dW0 = R.backward_topk(h, W, yy, Sd, lS, stats, grad_loss=g, row_mask=rm)
    dh1, dW1 = R.backward_topk(h, W, yy, Sd, lS, stats, grad_loss=g, row_mask=rm, logps_support=lps)
    torch.cuda.synchronize()
    assert np.array_equal(host(dh0).view(np.uint32), host(dh1).view(np.uint32))
    assert np.array_equal(host(dW0).view(np.uint32), host(dW1).view(np.uint32))
    lp = scipy.special.log_softmax(O.widen_bf16(case.h_s) @ O.widen_bf16(case.W_s).T, axis=1)
    valid = (S >= 0) & (S < V) & (case.mask[:, None] != 0)
    want = np.where(valid, np.take_along_axis(lp, np.clip(S, 0, V - 1).astype(np.int64), 1), 0.0)
    got = host(lps)
    assert np.all(got[~valid] == 0.0)
    assert_loss_close(got[valid], want[valid], "log p_s on the support")
