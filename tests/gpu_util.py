"""Shared helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""
import sys

import numpy as np

from oracle import rkl_oracle as O


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch, torch.device("cuda:0")


def bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def f32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def u8(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def oracle_full(case, rows, g=None, want_dz=False):
    """Oracle loss/stats and gradients over the given positions."""
    inp = O.Inputs.from_case(case)
    L, ls, lt = O.forward(inp, rows)
    b = O.backward(inp, rows, g, want_dz=want_dz)
    return inp, (L, ls, lt), b


_oracle_cache = {}


def oracle_cached(key, compute):
    """Oracle results shared by several tests of one process (full-size
    cases cost tens of seconds of host time each)."""
    if key not in _oracle_cache:
        _oracle_cache[key] = compute()
    return _oracle_cache[key]


def oracle_whole(case, rows, g_rows, what):
    """Oracle loss, stats, dh and dW over the given rows, timed."""
    import time
    t0 = time.time()
    b = O.backward(O.Inputs.from_case(case), rows, g_rows)
    say(f"{what}: oracle forward+backward over {len(rows)} rows took {time.time() - t0:.1f}s")
    return b


def headline_oracle(case):
    """Oracle results of the headline shape (all T = 4096 rows trainable,
    upstream gradient g = 1/T), computed once per process."""
    T = case.T
    g = np.full(T, 1.0 / T, np.float64)
    return oracle_cached("headline_g_mean", lambda: oracle_whole(case, np.arange(T), g, "headline shape"))
