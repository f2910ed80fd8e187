"""Full-size reverse KL with a teacher chosen per row on the GPU, in the
configuration bench.py --workload teachers --teacher-order interleaved times
(with three teachers here): Qwen3-1.7B-shaped student and teachers
(B=4, S=1025 -> N=4096, Hs=Ht=2048, V=151936), i.i.d. teacher ids, so every
128-row tile holds several teachers.

Loss of every row, dh of sampled rows and sampled rows of dW against the fp64
oracle.  Bars as in test_gpu_parity; for dh and dW the tolerance uses the
largest reference value among the sampled rows.
"""
import time

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev
from oracle import multi_teacher_oracle as M
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(x) for x in must if 0 <= x < n)
    s.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(s), dtype=np.int64)


def test_headline_shape_interleaved_teachers():
    torch, dev = torch_dev()
    R.lib()
    K = 3
    say("teachers full size: generating inputs")
    case = synth.config("headline")
    T, V = case.T, case.V
    W_t_bits = synth.teacher_weights(3, K, V, case.Ht)
    teacher = synth.teacher_ids(3, T, K, "interleaved")
    g = np.full(T, 1.0 / T, np.float32)

    say("teachers full size: GPU forward + backward")
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(W_t_bits, dev)
    tk = torch.from_numpy(teacher).to(dev)
    loss, stats = R.forward_hidden_teachers(hs, Ws, ht, Wt, tk)
    dh, dW = R.backward_hidden_teachers(hs, Ws, ht, Wt, tk, stats, grad_loss=f32(g, dev))
    torch.cuda.synchronize()
    loss, stats = host(loss), host(stats)
    del Wt

    t0 = time.time()
    w = dict(h_s=O.widen_bf16(case.h_s), W_s=O.widen_bf16(case.W_s), h_t=O.widen_bf16(case.h_t),
             W_t=O.widen_bf16(W_t_bits))
    L, ls, lt = M.forward(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher)
    say(f"teachers full size: oracle forward over {T} rows took {time.time() - t0:.1f}s")
    assert_loss_close(loss, L, "loss")
    assert_loss_close(stats[:, 0], ls, "lse_s")
    assert_loss_close(stats[:, 1], lt, "lse_t")

    pick = _sample(T, 12, 31, must=(0, 127, 128, T - 1))
    b = M.backward(w["h_s"][pick], w["W_s"], w["h_t"][pick], w["W_t"], teacher[pick], g[pick].astype(np.float64))
    assert_grad_close(host(dh[pick.tolist()]), b["dh"], "dh (sampled rows)")
    vs = _sample(V, 40, 32, must=(0, 255, 256, V - 129, V - 1))
    want = M.dW_rows(w["h_s"], w["W_s"], w["h_t"], w["W_t"], teacher, vs, (L, ls, lt), g.astype(np.float64))
    assert_grad_close(host(dW[vs.tolist()]), want, "dW (sampled rows)")
