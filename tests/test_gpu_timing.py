"""Per-kernel timing (rkl_kernel_timing / rkl_kernel_times) on the GPU: every
launch of a timed call is one entry under its kernel's name with a positive
device time, a call that launches nothing leaves no entry and no events
behind for the next launch, and timing never changes a result bit."""
import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, host, say, torch_dev, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    R.kernel_timing(False)
    R.kernel_times()
    return torch, dev


def _case(dev):
    c = synth.random_case(41, 300, 1500, 128, 192, p_mask=1.0)
    return (bf16(c.h_s, dev), bf16(c.W_s, dev), bf16(c.h_t, dev), bf16(c.W_t, dev))


def test_each_launch_is_one_entry(tdev):
    torch, dev = tdev
    h_s, W_s, h_t, W_t = _case(dev)
    say("timing: forward + backward, N=300 V=1500")
    R.kernel_timing(True)
    try:
        loss, stats = R.forward_hidden(h_s, W_s, h_t, W_t)
        R.backward_hidden(h_s, W_s, h_t, W_t, stats)
        t = R.kernel_times()
    finally:
        R.kernel_timing(False)
    for k in ("fwd_tiles", "fwd_combine", "bwd_dz_tiles", "dw_gemm", "dh_gemm", "grad_scale", "convert_h"):
        assert k in t, (k, sorted(t))
        ms, n = t[k]
        assert n >= 1 and ms > 0.0, (k, ms, n)
    assert t["fwd_tiles"][1] == 1 and t["fwd_combine"][1] == 1
    # the records were consumed, and nothing is recorded with timing off
    assert R.kernel_times() == {}
    R.forward_hidden(h_s, W_s, h_t, W_t)
    torch.cuda.synchronize()
    assert R.kernel_times() == {}


def test_a_call_that_launches_nothing_leaves_no_entry(tdev):
    torch, dev = tdev
    empty = torch.empty(0, dtype=torch.int32, device=dev)
    src = torch.arange(12, dtype=torch.float32, device=dev).reshape(3, 4)
    idx = torch.tensor([2, 0, 1], dtype=torch.int32, device=dev)
    R.kernel_timing(True)
    try:
        out0 = R.scatter_rows(torch.empty((0, 4), dtype=torch.float32, device=dev), empty, 0)   # no kernel
        t0 = R.kernel_times()
        got = R.gather_rows(src, idx)   # the next launch takes fresh events
        t1 = R.kernel_times()
    finally:
        R.kernel_timing(False)
    assert out0.shape == (0, 4)
    assert t0 == {}, t0
    assert set(t1) == {"gather"} and t1["gather"][1] == 1 and t1["gather"][0] > 0.0
    assert np.array_equal(host(got), host(src)[[2, 0, 1]])


def test_timing_changes_no_result_bit(tdev):
    torch, dev = tdev
    h_s, W_s, h_t, W_t = _case(dev)
    mask = u8((np.arange(300) % 3 != 1).astype(np.uint8), dev)

    def run():
        loss, stats = R.forward_hidden(h_s, W_s, h_t, W_t, row_mask=mask)
        dh, dW = R.backward_hidden(h_s, W_s, h_t, W_t, stats, row_mask=mask)
        return [host(x).copy() for x in (loss, stats, dh, dW)]

    plain = run()
    R.kernel_timing(True)
    try:
        timed = run()
        R.kernel_times()
    finally:
        R.kernel_timing(False)
    for a, b in zip(plain, timed):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
