"""rkl_forward_hidden_noalloc (include/rkl_noalloc.h) through the C ABI: the
forward without a workspace argument gives the results of
rkl_forward_hidden bit for bit, on two calls in a row with the second
smaller (the scratch keeps the first call's contents), in full-row mode,
and rejects sizes beyond its scratch with a message, launching nothing."""
import ctypes

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, host, say, torch_dev, u8

pytestmark = pytest.mark.gpu


def _noalloc():
    L = R.lib()
    f = L.rkl_forward_hidden_noalloc
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P]
    f.restype = ctypes.c_int
    return f


def _call(f, torch, dev, case, row_mask=None):
    hs, Ws, ht, Wt = bf16(case.h_s, dev), bf16(case.W_s, dev), bf16(case.h_t, dev), bf16(case.W_t, dev)
    N, Hs = hs.shape
    V, Ht = Wt.shape
    loss = torch.full((N,), 7.0, dtype=torch.float32, device=dev)
    stats = torch.full((N, 4), 7.0, dtype=torch.float32, device=dev)
    rm = None if row_mask is None else u8(row_mask, dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = f(N, V, Hs, Ht, hs.data_ptr(), Ws.data_ptr(), ht.data_ptr(), Wt.data_ptr(),
           None if rm is None else rm.data_ptr(), loss.data_ptr(), stats.data_ptr(), stream)
    assert rc == 0, R.lib().rkl_last_error().decode()
    ref_loss, ref_stats = R.forward_hidden(hs, Ws, ht, Wt, row_mask=rm)
    torch.cuda.synchronize()
    return host(loss), host(stats), host(ref_loss), host(ref_stats)


def test_noalloc_forward_equals_forward_on_two_calls():
    torch, dev = torch_dev()
    f = _noalloc()
    big = synth.random_case(1101, T=1500, V=9001, Hs=192, Ht=128, p_mask=1.0)
    small = synth.random_case(1102, T=130, V=2500, Hs=64, Ht=256, p_mask=0.6)
    for name, case, rm in (("first, larger", big, None), ("second, smaller", small, None),
                           ("third, full-row mode", small, small.mask)):
        say("no-alloc forward", name, case.T, case.V)
        loss, stats, ref_loss, ref_stats = _call(f, torch, dev, case, rm)
        assert np.array_equal(loss.view(np.uint32), ref_loss.view(np.uint32)), name
        assert np.array_equal(stats.view(np.uint32), ref_stats.view(np.uint32)), name
        assert np.all(np.isfinite(loss))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    torch, dev = torch_dev()
    f = _noalloc()
    # V = 3001: 12 vocabulary splits, 240 bytes per row; 150000 rows need
    # 36 MB > 32 MiB
    N, V, H = 150000, 3001, 64
    say("no-alloc size limit", N, V)
    h = torch.zeros((N, H), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=dev)
    loss = torch.full((N,), 7.0, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = f(N, V, H, H, h.data_ptr(), W.data_ptr(), h.data_ptr(), W.data_ptr(), None, loss.data_ptr(),
           stats.data_ptr(), stream)
    torch.cuda.synchronize()
    assert rc == R.RKL_UNSUPPORTED
    assert "scratch" in R.lib().rkl_last_error().decode()
    assert bool(torch.all(loss == 7.0))   # nothing launched
