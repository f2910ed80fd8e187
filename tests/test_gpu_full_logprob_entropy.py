"""Full-size log-probability / entropy on the GPU, in the configuration
bench.py --workload logprob_entropy times: Qwen3-1.7B-shaped student
(B=4, S=1025 -> N=4096 trainable rows, H=2048, V=151936), uniform sampled
tokens, token-mean upstream gradients for both outputs.

logp and the entropy of sampled rows, dh of sampled rows and sampled rows
of dW against the fp64 oracle (whose row statistics cover every row, since
each dW row sums over all of them).  Bars as in test_gpu_parity; for dh and
dW the tolerance uses the largest reference value among the sampled rows.
"""
import time

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev
from oracle import logprob_entropy_oracle as E
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(x) for x in must if 0 <= x < n)
    s.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(s), dtype=np.int64)


def test_headline_shape_sampled_rows():
    torch, dev = torch_dev()
    R.lib()
    say("logprob/entropy full size: generating inputs")
    case = synth.config("headline")
    T, V, H = case.T, case.V, case.Hs
    y = synth.sampled_tokens(3, T, V)
    y[:3] = (0, V - 1, 256)
    g_lp = np.full(T, 1.0 / T, np.float32)
    g_h = np.full(T, -0.01 / T, np.float32)

    h_d, W_d = bf16(case.h_s, dev), bf16(case.W_s, dev)
    say("logprob/entropy full size: GPU forward + backward")
    logp, ent, stats = R.forward_logprob_entropy(h_d, W_d, torch.from_numpy(y).to(dev))
    dh, dW = R.backward_logprob_entropy(h_d, W_d, torch.from_numpy(y).to(dev), stats,
                                        grad_logp=f32(g_lp, dev), grad_entropy=f32(g_h, dev))
    torch.cuda.synchronize()
    logp, ent, stats = host(logp), host(ent), host(stats)

    t0 = time.time()
    h, W = O.widen_bf16(case.h_s), O.widen_bf16(case.W_s)
    lp_ref, H_ref, lse_ref = E.forward(h, W, y)
    say(f"logprob/entropy full size: oracle forward over {T} rows took {time.time() - t0:.1f}s")
    assert_loss_close(logp, lp_ref, "logp")
    assert_loss_close(ent, H_ref, "entropy")
    assert_loss_close(stats[:, 0], lse_ref, "lse")

    pick = _sample(T, 12, 21, must=(0, 1, 2, 127, 128, T - 1))
    b = E.backward(h[pick], W, y[pick], g_lp[pick].astype(np.float64), g_h[pick].astype(np.float64))
    assert_grad_close(host(dh[pick.tolist()]), b["dh"], "dh (sampled rows)")
    vs = _sample(V, 40, 22, must=(0, 255, 256, V - 129, V - 1, int(y[5])))
    want = E.dW_rows(h, W, y, vs, lse_ref, H_ref, g_lp.astype(np.float64), g_h.astype(np.float64))
    assert_grad_close(host(dW[vs.tolist()]), want, "dW (sampled rows)")
