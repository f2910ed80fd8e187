"""Full-size vocabulary shards on the GPU, in the configuration bench.py
--workload vocab_shard times: the Qwen3-1.7B-shaped problem (B=4, S=1025 ->
N=4096 rows, Hs=Ht=2048, V=151936) split into 8 shards of 18992 vocabulary
rows -- one rank's share of an 8-way vocabulary-parallel group -- run one
after another on this GPU, partials merged by rkl_combine_shards, each
shard's backward with the merged stats.

Loss and lse of every row, the summed dh of sampled rows and sampled rows of
dW (including both sides of every shard boundary) against the fp64 oracle.
Bars as in test_gpu_parity; for dh and dW the tolerance uses the largest
reference value among the sampled rows.
"""
import time

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, say, torch_dev
from oracle import rkl_oracle as O
from oracle import vocab_shard_oracle as S
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(x) for x in must if 0 <= x < n)
    s.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(s), dtype=np.int64)


def test_headline_shape_eight_shards():
    torch, dev = torch_dev()
    R.lib()
    say("vocab shards full size: generating inputs")
    case = synth.config("headline")
    T, V = case.T, case.V
    bounds = S.shard_bounds(V, 8)
    g = np.full(T, 1.0 / T, np.float32)

    say("vocab shards full size: GPU shard forwards, combine, shard backwards")
    hs, ht, Ws, Wt = bf16(case.h_s, dev), bf16(case.h_t, dev), bf16(case.W_s, dev), bf16(case.W_t, dev)
    partials = torch.stack([R.forward_hidden_shard(hs, Ws[a:b], ht, Wt[a:b]) for a, b in bounds]).contiguous()
    loss, stats = R.combine_shards(partials)
    dh = np.zeros((T, case.Hs))
    dW = []
    for a, b in bounds:
        d, w = R.backward_hidden(hs, Ws[a:b], ht, Wt[a:b], stats, grad_loss=f32(g, dev))
        dh += host(d)
        dW.append(w)
    dW = torch.cat(dW)
    torch.cuda.synchronize()
    loss, stats = host(loss), host(stats)

    t0 = time.time()
    inp = O.Inputs.from_case(case)
    rows = np.arange(T)
    L, ls, lt = O.forward(inp, rows)
    say(f"vocab shards full size: oracle forward over {T} rows took {time.time() - t0:.1f}s")
    assert_loss_close(loss, L, "loss")
    assert_loss_close(stats[:, 0], ls, "lse_s")
    assert_loss_close(stats[:, 1], lt, "lse_t")

    pick = _sample(T, 12, 41, must=(0, 127, 128, T - 1))
    b = O.backward(inp, pick, g[pick].astype(np.float64))
    assert_grad_close(dh[pick], b["dh"], "dh (sampled rows, sum over shards)")
    edges = [e for a, b_ in bounds for e in (a, b_ - 1)]
    vs = _sample(V, 24, 42, must=edges)
    want = O.dW_rows(inp, rows, vs, (L, ls, lt), g.astype(np.float64))
    assert_grad_close(host(dW[vs.tolist()]), want, "dW (sampled rows)")
