"""GPU parity over bf16's range: hidden states and weights whose magnitudes
lie far outside fp16's (the backward's dz, dW and dh GEMMs run on fp16
operands scaled by powers of two).

* planted hidden-state entries of magnitude 1e5 (beyond fp16's largest
  finite value), 3e4 and 1e-7 (an fp16 subnormal) in a few rows;
* a student weight row with an entry of 1e5 in a hidden column that every
  token holds at 0 (the logits stay moderate, dh's column carries it);
* weights around 1e-11 with hidden states around 1e9 (both far outside fp16,
  the logits moderate);
* student weights around 1e4 (the largest near 5e4: within fp16, above the
  band in which the unscaled copy is used) with hidden states around 1e-4.

Each must match the fp64 oracle: loss, the whole dh and the whole dW, all
finite.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, oracle_full, say, torch_dev, u8
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _widen(bits):
    return O.widen_bf16(bits).astype(np.float32)


def _run_and_check(case, dev, what):
    torch = __import__("torch")
    say("range", what)
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    hs, ht = R.gather_rows(bf16(case.h_s, dev), idx), R.gather_rows(bf16(case.h_t, dev), idx)
    Ws, Wt = bf16(case.W_s, dev), bf16(case.W_t, dev)
    g = R.gather_rows(f32(case.grad, dev), idx)
    loss, stats = R.forward_hidden(hs, Ws, ht, Wt)
    dh, dW = R.backward_hidden(hs, Ws, ht, Wt, stats, grad_loss=g)
    torch.cuda.synchronize()
    loss, dh, dW = host(loss), host(dh), host(dW)
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(dh)) and np.all(np.isfinite(dW))
    rows = O.compact_rows(case.mask)
    _, (L, _, _), b = oracle_full(case, rows, case.grad[rows].astype(np.float64))
    assert_loss_close(loss, L, f"{what}: loss")
    assert_grad_close(dh, b["dh"], f"{what}: dh")
    assert_grad_close(dW, b["dW"], f"{what}: dW")


def test_planted_large_and_tiny_hidden_states(tdev):
    torch, dev = tdev
    case = synth.random_case(700, T=300, V=3001, Hs=128, Ht=64, p_mask=0.8, with_grad=True)
    h = _widen(case.h_s)
    h[3, 5], h[3, 77] = 1e5, -1e5
    h[150, 0] = 3e4
    h[151, 100] = -3e4
    h[200, :8] = 1e-7
    h[201, 64] = -1e-7
    case.h_s = _bits(h)
    _run_and_check(case, dev, "planted hidden states")


def test_planted_large_weight_in_a_zero_column(tdev):
    torch, dev = tdev
    case = synth.random_case(701, T=260, V=2000, Hs=192, Ht=128, p_mask=0.9, with_grad=True)
    h = _widen(case.h_s)
    h[:, 40] = 0.0          # every token: hidden unit 40 is 0, so W[:, 40] never reaches a logit
    case.h_s = _bits(h)
    W = _widen(case.W_s)
    W[1234, 40] = 1e5
    W[7, 40] = -5e4
    case.W_s = _bits(W)
    _run_and_check(case, dev, "large weight, zero hidden column")


def test_tiny_weights_huge_hidden_states(tdev):
    torch, dev = tdev
    case = synth.random_case(702, T=200, V=1500, Hs=128, Ht=64, p_mask=0.7, with_grad=True)
    case.h_s = _bits(_widen(case.h_s) * np.float32(1e9))
    case.W_s = _bits(_widen(case.W_s) * np.float32(1e-9))
    _run_and_check(case, dev, "weights ~1e-11, hidden states ~1e9")


def test_weights_above_the_unscaled_band(tdev):
    torch, dev = tdev
    case = synth.random_case(703, T=200, V=1800, Hs=64, Ht=64, p_mask=0.7, with_grad=True)
    case.h_s = _bits(_widen(case.h_s) * np.float32(1e-4))
    case.W_s = _bits(_widen(case.W_s) * np.float32(8e4))
    assert 2.0 ** 15 <= np.max(np.abs(_widen(case.W_s))) < 65504
    _run_and_check(case, dev, "weights ~1e4, hidden states ~1e-4")
