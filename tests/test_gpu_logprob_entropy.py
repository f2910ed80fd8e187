"""GPU parity of the log-probability / entropy path (through the C ABI)
against the fp64 oracle (oracle/logprob_entropy_oracle.py).

Per row: log p(sampled token) and the entropy of softmax(h W^T), and the
gradients dh, dW of sum_i (g_lp,i logp_i + g_H,i H_i).  Bars as for the
reverse KL: per-row |d| <= 1e-4 + 1e-3 |ref| for logp and the entropy,
max|d| <= 2e-3 max|ref| for dh and dW; compaction bit-exact; exact zeros on
rows the mask drops.
"""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev, u8
from oracle import logprob_entropy_oracle as E
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _inputs(seed, T, V, H, p_mask):
    case = synth.random_case(seed, T=T, V=V, Hs=H, Ht=64, p_mask=p_mask)
    y = synth.sampled_tokens(seed, T, V)
    g_lp, g_h = synth.upstream_grads(seed, T)
    return case, y, g_lp, g_h


def _run(case, y, dev, g_lp=None, g_h=None, full_row=False):
    """Compaction -> gather -> forward -> backward through the binding."""
    torch = __import__("torch")
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    if full_row:
        idx = torch.arange(case.T, dtype=torch.int32, device=dev)
    h = R.gather_rows(bf16(case.h_s, dev), idx)
    W = bf16(case.W_s, dev)
    yy = R.gather_rows(torch.from_numpy(y).to(dev), idx)
    gl = None if g_lp is None else R.gather_rows(f32(g_lp, dev), idx)
    gh = None if g_h is None else R.gather_rows(f32(g_h, dev), idx)
    rm = mask if full_row else None
    logp, ent, stats = R.forward_logprob_entropy(h, W, yy, row_mask=rm)
    dh, dW = R.backward_logprob_entropy(h, W, yy, stats, grad_logp=gl, grad_entropy=gh, row_mask=rm)
    torch.cuda.synchronize()
    return host(idx), host(logp), host(ent), host(stats), host(dh), host(dW)


def _check(case, y, out, g_lp=None, g_h=None):
    idx, logp, ent, stats, dh, dW = out
    rows = O.compact_rows(case.mask)
    assert np.array_equal(idx, rows)
    h, W = O.widen_bf16(case.h_s[rows]), O.widen_bf16(case.W_s)
    lp_ref, H_ref, lse_ref = E.forward(h, W, y[rows])
    assert_loss_close(logp, lp_ref, "logp")
    assert_loss_close(ent, H_ref, "entropy")
    assert_loss_close(stats[:, 0], lse_ref, "lse")
    b = E.backward(h, W, y[rows], None if g_lp is None else g_lp[rows], None if g_h is None else g_h[rows])
    assert_grad_close(dh, b["dh"], "dh")
    assert_grad_close(dW, b["dW"], "dW")


@pytest.mark.parametrize("T,V,H", [(300, 1000, 128), (517, 5003, 192), (129, 257, 64), (40, 1, 64)])
def test_against_oracle_with_gradients(tdev, T, V, H):
    """Several token and vocabulary tiles with ragged tails (V = 1 included),
    random upstream gradients for both outputs."""
    torch, dev = tdev
    case, y, g_lp, g_h = _inputs(300 + T, T, V, H, 0.7)
    say("logprob/entropy", T, V, H)
    out = _run(case, y, dev, g_lp, g_h)
    if V == 1:
        # point mass: logp and the entropy are 0, and so is every gradient, up
        # to fp32 rounding of the log-sum-exp
        assert np.all(np.abs(out[1]) <= 1e-6) and np.all(np.abs(out[2]) <= 1e-6)
        assert np.max(np.abs(out[4]), initial=0) <= 1e-6 and np.max(np.abs(out[5])) <= 1e-6
        return
    _check(case, y, out, g_lp, g_h)


def test_default_gradients(tdev):
    """grad_logp NULL = ones, grad_entropy NULL = zeros."""
    torch, dev = tdev
    case, y, _, _ = _inputs(401, 200, 3000, 128, 0.8)
    say("logprob/entropy default grads")
    _check(case, y, _run(case, y, dev))


def test_sampled_tokens_at_the_vocabulary_edges(tdev):
    """Sampled ids 0, V-1 (inside the ragged last tile) and a tile boundary."""
    torch, dev = tdev
    V = 1000
    case, y, g_lp, g_h = _inputs(402, 96, V, 64, 1.0)
    y[0::3], y[1::3], y[2::3] = 0, V - 1, 256
    say("logprob/entropy edge tokens")
    _check(case, y, _run(case, y, dev, g_lp, g_h), g_lp, g_h)


def test_full_row_equals_compact(tdev):
    """Full-row mode gives bit-identical results on the masked rows and exact
    zeros (outputs and dh) on the others."""
    torch, dev = tdev
    case, y, g_lp, g_h = _inputs(403, 333, 2100, 128, 0.5)
    say("logprob/entropy full-row vs compact")
    c = _run(case, y, dev, g_lp, g_h)
    f = _run(case, y, dev, g_lp, g_h, full_row=True)
    rows, m = c[0], case.mask != 0
    for i, what in ((1, "logp"), (2, "entropy"), (3, "stats"), (4, "dh")):
        assert np.array_equal(f[i][rows], c[i]), what
        assert np.all(f[i][~m] == 0.0), what
    assert_grad_close(f[5], c[5], "dW full-row vs compact")


def test_chunk_plan_does_not_change_results(tdev, monkeypatch):
    """V = 140000 in one backward chunk (default at this N) or in three
    65536-column chunks: bit-identical results."""
    torch, dev = tdev
    case, y, g_lp, g_h = _inputs(404, 150, 140000, 64, 0.6)
    say("logprob/entropy chunk plans")
    one = _run(case, y, dev, g_lp, g_h)
    _check(case, y, one, g_lp, g_h)
    monkeypatch.setenv("RKL_VOCAB_CHUNK", "65536")
    three = _run(case, y, dev, g_lp, g_h)
    for a, b, what in zip(three[1:], one[1:], ("logp", "entropy", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


def test_bitwise_deterministic(tdev):
    torch, dev = tdev
    case, y, g_lp, g_h = _inputs(405, 300, 5000, 128, 0.5)
    say("logprob/entropy determinism")
    a = _run(case, y, dev, g_lp, g_h)
    b = _run(case, y, dev, g_lp, g_h)
    for x, z in zip(a, b):
        assert np.array_equal(x.view(np.uint8), z.view(np.uint8))


def test_empty_selection(tdev):
    torch, dev = tdev
    case, y, _, _ = _inputs(406, 40, 600, 64, 0.0)
    say("logprob/entropy empty mask")
    idx, logp, ent, stats, dh, dW = _run(case, y, dev)
    assert logp.shape == (0,) and ent.shape == (0,) and dh.shape == (0, 64)
    assert np.all(dW == 0.0)
