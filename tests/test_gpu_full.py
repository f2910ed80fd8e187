"""Full-size workloads on the GPU, in the configuration bench.py times, with
every output compared element by element against the fp64 oracle.

* Qwen3-1.7B-shaped hidden-state path (B=4, S=1025, Hs=Ht=2048, V=151936):
  every position trainable (N=4096, the benchmark shape, token-mean upstream
  gradient) and the response-span mask (last 512 of each 1024 -> N=2048).
  Loss and log-sum-exps of every row, the whole dh [N, 2048] and the whole
  dW [151936, 2048].
* Self-distillation (B=8, S=1025 -> N=8192): a bit-identical teacher gives
  exactly zero loss and gradients; a perturbed teacher fed as hidden states
  and as fp32 logits gives the same answer, and both match the oracle on
  every row's loss, the whole dh and the whole dW.
* Long masked prompts (B=2, S=16385 -> T=32768, N=4096, Ht=4096): compacted
  and full-row results are identical on masked rows and zero elsewhere, and
  the compacted loss, dh and dW (Ht = 4096, a 4096-token dW reduction)
  match the oracle whole.

Bars as in test_gpu_parity (per-token loss |dL| <= 1e-4 + 1e-3|L|, gradient
max|d| <= 2e-3 max|ref| over the whole tensor).  The oracle runs in 256-row
chunks over all rows (about 10^13 fp64 FLOP per case on the host cores);
results it shares between tests (the headline shape with g = 1/T) are kept
for the process.
"""
import time

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, headline_oracle, host, oracle_whole, say, torch_dev, u8
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

V = 151936


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


@pytest.fixture(scope="module")
def qwen(tdev):
    """Seed-3 Qwen-shaped tensors (the mask is set per test)."""
    torch, dev = tdev
    say("qwen: generating inputs")
    case = synth.qwen_shaped(response=None)
    dev_t = dict(h_s=bf16(case.h_s, dev), h_t=bf16(case.h_t, dev), W_s=bf16(case.W_s, dev), W_t=bf16(case.W_t, dev))
    return case, dev_t


def _compact_run(torch, dev, mask_np, d, g_pos=None):
    mask = u8(mask_np, dev)
    idx, N = R.compact_rows(mask)
    hs, ht = R.gather_rows(d["h_s"], idx), R.gather_rows(d["h_t"], idx)
    g = None if g_pos is None else R.gather_rows(f32(g_pos, dev), idx)
    torch.cuda.synchronize()
    t0 = time.time()
    loss, stats = R.forward_hidden(hs, d["W_s"], ht, d["W_t"])
    dh, dW = R.backward_hidden(hs, d["W_s"], ht, d["W_t"], stats, grad_loss=g)
    torch.cuda.synchronize()
    el = time.time() - t0
    return host(idx), host(loss), host(stats), host(dh), host(dW), el


def _check_whole(b, loss, st, dh, dW, teacher_hidden=True):
    assert_loss_close(loss, b["L"], "loss")
    assert_loss_close(st[:, 2], b["L"], "stats L")
    assert_loss_close(st[:, 0], b["lse_s"], "lse_s")
    if teacher_hidden:
        assert_loss_close(st[:, 1], b["lse_t"], "lse_t")
    assert_grad_close(dh, b["dh"], "dh (every row)")
    assert_grad_close(dW, b["dW"], "dW (every vocabulary row)")


def test_qwen_headline_every_position(tdev, qwen):
    """N = 4096 (all positions trainable), token-mean upstream gradient."""
    torch, dev = tdev
    case, d = qwen
    mask = np.ones(case.T, np.uint8)
    g = np.full(case.T, 1.0 / case.T, np.float32)
    say("qwen headline N=4096")
    idx, loss, st, dh, dW, el = _compact_run(torch, dev, mask, d, g)
    say(f"qwen headline fwd+bwd {el * 1e3:.1f} ms (first call)")
    assert np.array_equal(idx, np.arange(case.T))
    _check_whole(headline_oracle(case), loss, st, dh, dW)


def test_qwen_response_mask(tdev, qwen):
    """Mask = last 512 positions of each 1024 (N = 2048), unit upstream gradient."""
    torch, dev = tdev
    case, d = qwen
    mask = np.zeros((case.B, case.S - 1), np.uint8)
    mask[:, -512:] = 1
    mask = mask.reshape(-1)
    say("qwen response mask N=2048")
    idx, loss, st, dh, dW, el = _compact_run(torch, dev, mask, d)
    assert np.array_equal(idx, O.compact_rows(mask))
    assert idx.shape[0] == 2048
    b = oracle_whole(case, idx.astype(np.int64), None, "qwen response mask")
    _check_whole(b, loss, st, dh, dW)


def test_self_distillation_exact_zero_full_size(tdev):
    """B=8, S=1025, bit-identical teacher: loss, dh and dW are exactly zero."""
    torch, dev = tdev
    say("self-distillation: generating inputs")
    case = synth.self_distill()
    h, W = bf16(case.h_s, dev), bf16(case.W_s, dev)
    say("self-distillation N=8192")
    loss, stats = R.forward_hidden(h, W, h, W)
    dh, dW = R.backward_hidden(h, W, h, W, stats)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(loss)) == 0
    assert int(torch.count_nonzero(dh)) == 0
    assert int(torch.count_nonzero(dW)) == 0
    # lse_s == lse_t bit for bit
    assert torch.equal(stats[:, 0], stats[:, 1])


def test_self_distillation_perturbed_logits_vs_hidden(tdev):
    """Teacher W' = bf16(W + N(0, 1e-3^2)) fed as hidden states and as fp32
    logits [8192, 151936] (an fp32 matmul of the same bf16 values): the two
    payload paths agree with each other and both match the oracle whole."""
    torch, dev = tdev
    say("perturbed self-distillation: generating inputs")
    case = synth.self_distill(perturb=1e-3)
    h, Ws, Wt = bf16(case.h_s, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    say("perturbed: hidden path")
    Lh, sh = R.forward_hidden(h, Ws, h, Wt)
    dh_h, dW_h = R.backward_hidden(h, Ws, h, Wt, sh)
    Lh, sh, dh_h, dW_h = host(Lh), host(sh), host(dh_h), host(dW_h)
    say("perturbed: logits path")
    z_t = h.float() @ Wt.float().t().contiguous()
    Ll, sl = R.forward_logits(z_t, h_s=h, W_s=Ws)
    dh_l, dW_l = R.backward_logits(z_t, sl, h_s=h, W_s=Ws)
    torch.cuda.synchronize()
    Ll, sl, dh_l, dW_l = host(Ll), host(sl), host(dh_l), host(dW_l)
    say("perturbed: logits path through an identity row index")
    ident = torch.arange(case.T, dtype=torch.int32, device=dev)
    Li, si = R.forward_logits(z_t, h_s=h, W_s=Ws, z_rows=ident)
    dh_i, dW_i = R.backward_logits(z_t, si, h_s=h, W_s=Ws, z_rows=ident)
    for a, b2, what in ((Li, Ll, "loss"), (si, sl, "stats"), (dh_i, dh_l, "dh"), (dW_i, dW_l, "dW")):
        assert np.array_equal(host(a).view(np.uint32), b2.view(np.uint32)), what
    del z_t, Li, si, dh_i, dW_i
    assert_loss_close(Ll, Lh, "logits vs hidden loss")
    assert_grad_close(dh_l, dh_h, "logits vs hidden dh")
    assert_grad_close(dW_l, dW_h, "logits vs hidden dW")
    assert np.all(Lh > -1e-5) and np.median(Lh) < 1e-2
    b = oracle_whole(case, np.arange(case.T), None, "perturbed self-distillation")
    say("perturbed: hidden path vs oracle")
    _check_whole(b, Lh, sh, dh_h, dW_h)
    say("perturbed: logits path vs oracle")
    # the logits path's lse_t comes from the fp32-rounded teacher logits: the
    # same bar applies
    _check_whole(b, Ll, sl, dh_l, dW_l)


def test_long_prompts_compact_vs_full_row(tdev):
    """B=2, S=16385 (T=32768), last 2048 positions of each sequence trainable
    (N=4096), Hs=2048, Ht=4096: compact and full-row agree on masked rows,
    and the compacted results match the oracle whole."""
    torch, dev = tdev
    say("long prompts: generating inputs")
    case = synth.config("c5")
    assert case.T == 32768 and int(case.mask.sum()) == 4096
    d = dict(h_s=bf16(case.h_s, dev), h_t=bf16(case.h_t, dev), W_s=bf16(case.W_s, dev), W_t=bf16(case.W_t, dev))
    mask = u8(case.mask, dev)
    rows = O.compact_rows(case.mask)

    say("long prompts: compact")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    t0 = time.time()
    idx, N = R.compact_rows(mask)
    hs, ht = R.gather_rows(d["h_s"], idx), R.gather_rows(d["h_t"], idx)
    lc, sc = R.forward_hidden(hs, d["W_s"], ht, d["W_t"])
    dhc, dWc = R.backward_hidden(hs, d["W_s"], ht, d["W_t"], sc)
    loss_c = R.scatter_rows(lc, idx, case.T)
    dh_c = R.scatter_rows(dhc, idx, case.T)
    torch.cuda.synchronize()
    t_c = time.time() - t0
    mem_c = torch.cuda.max_memory_allocated() - base
    del hs, ht

    say("long prompts: full-row")
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    t0 = time.time()
    lf, sf = R.forward_hidden(d["h_s"], d["W_s"], d["h_t"], d["W_t"], row_mask=mask)
    dh_f, dWf = R.backward_hidden(d["h_s"], d["W_s"], d["h_t"], d["W_t"], sf, row_mask=mask)
    torch.cuda.synchronize()
    t_f = time.time() - t0
    mem_f = torch.cuda.max_memory_allocated() - base
    say(f"long prompts: compact {t_c * 1e3:.0f} ms, {mem_c / 2**30:.2f} GiB extra; "
        f"full-row {t_f * 1e3:.0f} ms, {mem_f / 2**30:.2f} GiB extra (first calls)")

    m = case.mask != 0
    loss_c, lf, sc, sf = host(loss_c), host(lf), host(sc), host(sf)
    assert np.array_equal(loss_c[m], lf[m])
    assert np.all(lf[~m] == 0.0) and np.all(loss_c[~m] == 0.0)
    assert np.array_equal(sc, sf[m])
    dh_c, dh_f = host(dh_c), host(dh_f)
    assert np.array_equal(dh_c[m], dh_f[m])
    assert np.all(dh_f[~m] == 0.0)
    dWc, dWf = host(dWc), host(dWf)
    assert_grad_close(dWf, dWc, "dW full-row vs compact")

    b = oracle_whole(case, rows.astype(np.int64), None, "long prompts")
    _check_whole(b, loss_c[rows], sc, dh_c[rows], dWc)
    assert_grad_close(dWf, b["dW"], "full-row dW vs oracle")
