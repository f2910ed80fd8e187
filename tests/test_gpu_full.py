"""Full-size workloads on the GPU, in the configuration bench.py times.

* Qwen3-1.7B-shaped hidden-state path (B=4, S=1025, Hs=Ht=2048, V=151936):
  every position trainable (N=4096, the benchmark shape) and the
  response-span mask (last 512 of each 1024 -> N=2048).  Loss of every row,
  dh of sampled rows and sampled rows of dW against the fp64 oracle.
* Self-distillation (B=8, S=1025 -> N=8192): bit-identical teacher gives
  exactly zero loss and gradients; a perturbed teacher fed as hidden states
  and as fp32 logits gives the same answer, checked against the oracle on
  sampled rows.
* Long masked prompts (B=2, S=16385 -> T=32768, N=4096, Ht=4096): compacted
  and full-row results are identical on masked rows, zero elsewhere, and match
  the oracle on sampled rows.

Bars as in test_gpu_parity.  For dW and dh only sampled rows are compared;
their tolerance uses the largest reference value among the sampled rows,
which is never looser than the whole-gradient maximum.
"""
import time

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev, u8
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

V = 151936


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(x) for x in must if 0 <= x < n)
    s.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(s), dtype=np.int64)


@pytest.fixture(scope="module")
def qwen(tdev):
    """Seed-3 Qwen-shaped tensors (the mask is set per test) with the oracle's
    row statistics for all 4096 positions."""
    torch, dev = tdev
    say("qwen: generating inputs")
    case = synth.qwen_shaped(response=None)
    t0 = time.time()
    inp = O.Inputs.from_case(case)
    stats = O.forward(inp, np.arange(case.T))
    say(f"qwen: oracle forward over {case.T} rows took {time.time() - t0:.1f}s")
    dev_t = dict(h_s=bf16(case.h_s, dev), h_t=bf16(case.h_t, dev), W_s=bf16(case.W_s, dev), W_t=bf16(case.W_t, dev))
    return case, inp, stats, dev_t


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
    return host(idx), host(loss), host(stats), dh, dW, el


def _check_qwen(case, inp, stats, rows, loss, st, dh, dW, g_rows, seed):
    L_all, ls_all, lt_all = stats
    assert_loss_close(loss, L_all[rows], "loss")
    assert_loss_close(st[:, 0], ls_all[rows], "lse_s")
    assert_loss_close(st[:, 1], lt_all[rows], "lse_t")
    # dh on sampled rows (first, last, tile edges, random)
    n = rows.shape[0]
    pick = _sample(n, 12, seed, must=(0, 127, 128, n - 1))
    b = O.backward(inp, rows[pick], g_rows[pick])
    assert_grad_close(host(dh[pick.tolist()]), b["dh"], "dh (sampled rows)")
    # dW on sampled vocabulary rows (incl. the ragged last tile)
    vs = _sample(V, 40, seed + 1, must=(0, 255, 256, V - 129, V - 1))
    want = O.dW_rows(inp, rows, vs, (L_all[rows], ls_all[rows], lt_all[rows]), g_rows)
    assert_grad_close(host(dW[vs.tolist()]), want, "dW (sampled rows)")


def test_qwen_headline_every_position(tdev, qwen):
    """N = 4096 (all positions trainable), token-mean upstream gradient."""
    torch, dev = tdev
    case, inp, stats, d = qwen
    mask = np.ones(case.T, np.uint8)
    g = np.full(case.T, 1.0 / case.T, np.float32)
    say("qwen headline N=4096")
    idx, loss, st, dh, dW, el = _compact_run(torch, dev, mask, d, g)
    say(f"qwen headline fwd+bwd {el * 1e3:.1f} ms (first call)")
    assert np.array_equal(idx, np.arange(case.T))
    _check_qwen(case, inp, stats, idx, loss, st, dh, dW, g[idx].astype(np.float64), seed=11)


def test_qwen_response_mask(tdev, qwen):
    """Mask = last 512 positions of each 1024 (N = 2048)."""
    torch, dev = tdev
    case, inp, stats, d = qwen
    mask = np.zeros((case.B, case.S - 1), np.uint8)
    mask[:, -512:] = 1
    mask = mask.reshape(-1)
    say("qwen response mask N=2048")
    idx, loss, st, dh, dW, el = _compact_run(torch, dev, mask, d)
    assert np.array_equal(idx, O.compact_rows(mask))
    assert idx.shape[0] == 2048
    _check_qwen(case, inp, stats, idx, loss, st, dh, dW, np.ones(2048), seed=12)


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
    logits [8192, 151936] (an fp32 matmul of the same bf16 values)."""
    torch, dev = tdev
    say("perturbed self-distillation: generating inputs")
    case = synth.self_distill(perturb=1e-3)
    h, Ws, Wt = bf16(case.h_s, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    say("perturbed: hidden path")
    Lh, sh = R.forward_hidden(h, Ws, h, Wt)
    dh_h, dW_h = R.backward_hidden(h, Ws, h, Wt, sh)
    Lh, dh_h, dW_h = host(Lh), host(dh_h), host(dW_h)
    say("perturbed: logits path")
    z_t = h.float() @ Wt.float().t().contiguous()
    Ll, sl = R.forward_logits(z_t, h_s=h, W_s=Ws)
    dh_l, dW_l = R.backward_logits(z_t, sl, h_s=h, W_s=Ws)
    torch.cuda.synchronize()
    del z_t
    Ll = host(Ll)
    assert_loss_close(Ll, Lh, "logits vs hidden loss")
    assert_grad_close(host(dh_l), dh_h, "logits vs hidden dh")
    assert_grad_close(host(dW_l), dW_h, "logits vs hidden dW")
    assert np.all(Lh > -1e-5) and np.median(Lh) < 1e-2
    # oracle on sampled rows
    rows = _sample(case.T, 24, 13, must=(0, case.T - 1))
    inp = O.Inputs(h_s=case.h_s[rows], W_s=case.W_s, h_t=case.h_t[rows], W_t=case.W_t)
    L, _, _ = O.forward(inp, np.arange(rows.shape[0]))
    assert_loss_close(Lh[rows], L, "hidden loss vs oracle")
    b = O.backward(inp, np.arange(rows.shape[0]))
    assert_grad_close(dh_h[rows], b["dh"], "hidden dh vs oracle (sampled rows)")


def test_long_prompts_compact_vs_full_row(tdev):
    """B=2, S=16385 (T=32768), last 2048 positions of each sequence trainable
    (N=4096), Hs=2048, Ht=4096: compact and full-row agree on masked rows."""
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
    assert_grad_close(host(dWf), host(dWc), "dW full-row vs compact")

    # oracle on sampled masked rows
    pick = rows[_sample(rows.shape[0], 8, 14, must=(0, rows.shape[0] - 1))]
    inp = O.Inputs(h_s=case.h_s[pick], W_s=case.W_s, h_t=case.h_t[pick], W_t=case.W_t)
    L, _, _ = O.forward(inp, np.arange(pick.shape[0]))
    assert_loss_close(loss_c[pick], L, "loss vs oracle")
    b = O.backward(inp, np.arange(pick.shape[0]))
    assert_grad_close(dh_c[pick], b["dh"], "dh vs oracle (sampled rows)")
