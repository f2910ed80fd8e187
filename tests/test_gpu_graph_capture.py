"""The forward that allocates nothing (rkl_forward_hidden_noalloc) under HIP
graph capture, the use it exists for: captured once, the graph is replayed
several times with eager work and synchronisation between the replays, and
every replay gives the eager rkl_forward_hidden results bit for bit."""
import ctypes

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, host, say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


def _noalloc():
    f = R.lib().rkl_forward_hidden_noalloc
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P]
    f.restype = ctypes.c_int
    return f


def test_noalloc_forward_replays_in_a_graph(tdev):
    torch, dev = tdev
    f = _noalloc()
    case = synth.random_case(91, T=300, V=3001, Hs=128, Ht=192, p_mask=1.0)
    hs, Ws, ht, Wt = bf16(case.h_s, dev), bf16(case.W_s, dev), bf16(case.h_t, dev), bf16(case.W_t, dev)
    N, Hs = hs.shape
    V, Ht = Wt.shape
    ref_loss, ref_stats = R.forward_hidden(hs, Ws, ht, Wt)
    ref_loss, ref_stats = host(ref_loss), host(ref_stats)
    loss = torch.empty((N,), dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)

    def call():
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        return f(N, V, Hs, Ht, hs.data_ptr(), Ws.data_ptr(), ht.data_ptr(), Wt.data_ptr(), None,
                 loss.data_ptr(), stats.data_ptr(), stream)

    say("graph capture of the no-allocation forward")
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):   # first call outside the capture: the scratch address is looked up
        assert call() == 0, R.lib().rkl_last_error().decode()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert call() == 0, R.lib().rkl_last_error().decode()
    for rep in range(3):
        loss.fill_(7.0)
        stats.fill_(7.0)
        R.forward_hidden(hs, Ws, ht, Wt)   # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(loss).view(np.uint32), ref_loss.view(np.uint32)), rep
        assert np.array_equal(host(stats).view(np.uint32), ref_stats.view(np.uint32)), rep
