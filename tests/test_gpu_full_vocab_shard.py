"""Full-size vocabulary shards on the GPU, in the configuration bench.py
--workload vocab_shard times: the Qwen3-1.7B-shaped problem (B=4, S=1025 ->
N=4096 rows, Hs=Ht=2048, V=151936) split into 8 shards of 18992 vocabulary
rows -- one rank's share of an 8-way vocabulary-parallel group -- run one
after another on this GPU, partials merged by rkl_combine_shards, each
shard's backward with the merged stats.

Loss and lse of every row, the whole summed dh and the whole dW (the
shards' rows concatenated) against the fp64 oracle of the unsharded
problem.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, headline_oracle, host, say, torch_dev
from oracle import vocab_shard_oracle as S
from tolerances import assert_grad_close, assert_loss_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


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

    b = headline_oracle(case)
    assert_loss_close(loss, b["L"], "loss")
    assert_loss_close(stats[:, 0], b["lse_s"], "lse_s")
    assert_loss_close(stats[:, 1], b["lse_t"], "lse_t")
    assert_grad_close(dh, b["dh"], "dh (every row, sum over shards)")
    assert_grad_close(host(dW), b["dW"], "dW (every vocabulary row, shards concatenated)")
