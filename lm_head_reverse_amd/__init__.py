"""lm_head_reverse_amd -- Python binding of librkl.so.

Argument marshalling only: every step of the path (compaction, gather,
projection, log-sum-exp / reverse-KL epilogue, dz, dh and dW GEMMs, scatter)
runs in the HIP kernels of librkl.so.  PyTorch provides device memory and the
current stream.  There is no fallback: if librkl.so is missing or the device
is not a HIP device, calls raise.

Function names mirror the C ABI in include/rkl.h (without the ``rkl_``
prefix).  bf16 tensors are torch.bfloat16; every tensor must be contiguous
and on the same CUDA (HIP) device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "RKLError", "lib", "LIB_PATH", "version", "kernel_timing", "kernel_times", "workspace_bytes", "workspace_bytes_teachers", "compact_rows",
    "gather_rows", "scatter_rows", "forward_hidden", "forward_logits", "backward_hidden", "backward_logits",
    "forward_hidden_teachers", "backward_hidden_teachers", "forward_logprob_entropy", "backward_logprob_entropy",
    "forward_hidden_shard", "forward_logits_shard", "combine_shards", "forward_logprob_entropy_shard",
    "combine_shards_logprob_entropy", "forward_topk", "backward_topk", "ReverseKL",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librkl.so")

RKL_OK, RKL_INVALID_ARG, RKL_UNSUPPORTED, RKL_WORKSPACE_TOO_SMALL, RKL_DEVICE_ERROR = range(5)


class RKLError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rkl status {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded librkl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RKLError(-1, f"{LIB_PATH} not found; build it with `python -m lm_head_reverse_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "rkl_last_error": ([], ctypes.c_char_p),
        "rkl_version": ([], ctypes.c_char_p),
        "rkl_kernel_timing": ([I32], I32),
        "rkl_kernel_times": ([I32, P, P, P, P], I32),
        "rkl_workspace_bytes": ([I64, I64, I64, I64], SZ),
        "rkl_workspace_bytes_teachers": ([I64, I64, I64, I64], SZ),
        "rkl_compact_rows": ([P, I64, P, P, P, P], I32),
        "rkl_gather_rows": ([P, I64, I64, P, I64, P, P], I32),
        "rkl_scatter_rows": ([P, I64, I64, P, I64, P, P], I32),
        "rkl_forward_hidden": ([I64, I64, I64, I64, P, P, P, P, P, P, P, P, SZ, P], I32),
        "rkl_forward_logits": ([I64, I64, I64, P, P, P, P, P, I64, P, P, P, P, SZ, P], I32),
        "rkl_backward_hidden": ([I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, I32, P, SZ, P], I32),
        "rkl_backward_logits": ([I64, I64, I64, P, P, P, P, P, I64, P, P, P, P, P, I32, P, P, SZ, P], I32),
        "rkl_forward_hidden_shard": ([I64, I64, I64, I64, P, P, P, P, P, P, SZ, P], I32),
        "rkl_forward_logits_shard": ([I64, I64, I64, P, P, P, P, P, P, SZ, P], I32),
        "rkl_combine_shards": ([I64, I64, P, P, P, P, P], I32),
        "rkl_forward_logprob_entropy_shard": ([I64, I64, I64, P, P, P, P, P, SZ, P], I32),
        "rkl_combine_shards_logprob_entropy": ([I64, I64, P, P, P, P, P, P], I32),
        "rkl_forward_hidden_teachers": ([I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "rkl_backward_hidden_teachers": ([I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, I32, P, SZ, P],
                                         I32),
        "rkl_forward_logprob_entropy": ([I64, I64, I64, P, P, P, P, P, P, P, P, SZ, P], I32),
        "rkl_forward_topk": ([I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "rkl_backward_topk": ([I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, P, I32, P, SZ, P], I32),
        "rkl_backward_logprob_entropy": ([I64, I64, I64, P, P, P, P, P, P, P, P, P, I32, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(rc: int):
    if rc != RKL_OK:
        raise RKLError(rc, lib().rkl_last_error().decode())


def version() -> str:
    return lib().rkl_version().decode()


def kernel_timing(enable: bool) -> None:
    """Turn per-kernel event timing on or off for this host thread."""
    _check(lib().rkl_kernel_timing(int(bool(enable))))


def kernel_times() -> dict:
    """{kernel name: (total ms, launches)} recorded since the last call (waits
    for the recorded events)."""
    cap = 64
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    launches = (ctypes.c_int * cap)()
    count = ctypes.c_int(0)
    _check(lib().rkl_kernel_times(cap, names, ms, launches, ctypes.byref(count)))
    return {names[k].decode(): (ms[k], launches[k]) for k in range(min(count.value, cap))}


def workspace_bytes(N: int, V: int, Hs: int, Ht: int) -> int:
    return int(lib().rkl_workspace_bytes(N, V, Hs, Ht))


def workspace_bytes_teachers(N: int, V: int, Hs: int, Ht: int) -> int:
    return int(lib().rkl_workspace_bytes_teachers(N, V, Hs, Ht))


# ---------------------------------------------------------------- torch plumbing

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, dev=None, shape=None):
    torch = _torch()
    if t is None:
        raise RKLError(RKL_INVALID_ARG, f"{name} is required")
    if not t.is_cuda:
        raise RKLError(RKL_INVALID_ARG, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise RKLError(RKL_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise RKLError(RKL_INVALID_ARG, f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise RKLError(RKL_INVALID_ARG, f"{name} is on {t.device}, expected {dev}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise RKLError(RKL_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


_ws_cache = {}


def _workspace(dev, nbytes: int):
    """A cached device byte buffer of at least nbytes (grown on demand), one
    per (device, current stream): calls queued on one stream run in order and
    may share it; calls on different streams may overlap, so they do not."""
    torch = _torch()
    key = (str(dev), torch.cuda.current_stream(dev).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


# ---------------------------------------------------------------- entry points

def compact_rows(mask):
    """mask uint8 [T] -> (row_idx int32 [N] ascending, N).  Synchronises the stream."""
    torch = _torch()
    _need(mask, "mask", torch.uint8)
    T = mask.numel()
    row_idx = torch.empty(max(T, 1), dtype=torch.int32, device=mask.device)
    n_dev = torch.empty(1, dtype=torch.int32, device=mask.device)
    n_host = ctypes.c_int64(0)
    _check(lib().rkl_compact_rows(_ptr(mask), T, _ptr(row_idx), _ptr(n_dev), ctypes.byref(n_host),
                                  _stream(mask.device)))
    return row_idx[: n_host.value], int(n_host.value)


def gather_rows(src, row_idx):
    """dst[i] = src[row_idx[i]] for a contiguous [T, ...] tensor (bit copy)."""
    torch = _torch()
    _need(row_idx, "row_idx", torch.int32, src.device)
    T = src.shape[0]
    N = row_idx.numel()
    dst = torch.empty((N,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    row_bytes = src[0].numel() * src.element_size() if T > 0 else 4
    _check(lib().rkl_gather_rows(_ptr(src), T, row_bytes, _ptr(row_idx), N, _ptr(dst), _stream(src.device)))
    return dst


def scatter_rows(src, row_idx, T: int):
    """[T, ...] tensor with dst[row_idx[i]] = src[i] and +0 in every other row."""
    torch = _torch()
    _need(row_idx, "row_idx", torch.int32, src.device)
    N = row_idx.numel()
    dst = torch.empty((T,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    inner = 1
    for d in src.shape[1:]:
        inner *= d
    row_bytes = inner * src.element_size()
    _check(lib().rkl_scatter_rows(_ptr(src), N, row_bytes, _ptr(row_idx), T, _ptr(dst), _stream(src.device)))
    return dst


def forward_hidden(h_s, W_s, h_t, W_t, row_mask=None):
    """Per-row reverse KL with the teacher given as hidden states.
    Returns (loss fp32 [N], stats fp32 [N, 4] = (lse_s, lse_t, L, lpmax))."""
    torch = _torch()
    dev = h_s.device
    N, Hs = h_s.shape
    V, Ht = W_t.shape
    _need(h_s, "h_s", torch.bfloat16, dev)
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    _need(h_t, "h_t", torch.bfloat16, dev, (N, Ht))
    _need(W_t, "W_t", torch.bfloat16, dev)
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    nb = workspace_bytes(N, V, Hs, Ht)
    ws = _workspace(dev, nb)
    _check(lib().rkl_forward_hidden(N, V, Hs, Ht, _ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), _ptr(row_mask),
                                    _ptr(loss), _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, stats


def _logit_rows(z_t, z_rows, dev):
    """(N, V, T) of a logits call: z_t holds T rows; without z_rows N = T."""
    torch = _torch()
    T, V = z_t.shape
    if z_rows is None:
        return T, V, 0
    _need(z_rows, "z_rows", torch.int32, dev)
    if z_rows.dim() != 1:
        raise RKLError(RKL_INVALID_ARG, "z_rows must be one-dimensional")
    return z_rows.shape[0], V, T


def forward_logits(z_t, h_s=None, W_s=None, z_s=None, row_mask=None, z_rows=None):
    """Per-row reverse KL with the teacher given as fp32 logits z_t [N, V]; the
    student as (h_s, W_s) bf16 or as fp32 logits z_s.  With z_rows (int32
    [N]), z_t and z_s hold [T, V] and row i reads their row z_rows[i]."""
    torch = _torch()
    dev = z_t.device
    _need(z_t, "z_t", torch.float32, dev)
    N, V, T = _logit_rows(z_t, z_rows, dev)
    Hs = 0
    if z_s is None:
        Hs = h_s.shape[1]
        _need(h_s, "h_s", torch.bfloat16, dev, (N, Hs))
        _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    else:
        _need(z_s, "z_s", torch.float32, dev, tuple(z_t.shape))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, Hs, 0))
    _check(lib().rkl_forward_logits(N, V, Hs, _ptr(h_s), _ptr(W_s), _ptr(z_s), _ptr(z_t), _ptr(z_rows), T,
                                    _ptr(row_mask), _ptr(loss), _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, stats


def backward_hidden(h_s, W_s, h_t, W_t, stats, grad_loss=None, row_mask=None, dW=None, accumulate_dW=False):
    """Gradients of sum_i g_i L_i: returns (dh_s fp32 [N, Hs], dW_s fp32 [V, Hs])."""
    torch = _torch()
    dev = h_s.device
    N, Hs = h_s.shape
    V, Ht = W_t.shape
    _need(h_s, "h_s", torch.bfloat16, dev)
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    _need(h_t, "h_t", torch.bfloat16, dev, (N, Ht))
    _need(W_t, "W_t", torch.bfloat16, dev)
    _need(stats, "stats", torch.float32, dev, (N, 4))
    if grad_loss is not None:
        _need(grad_loss, "grad_loss", torch.float32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    if dW is None:
        if accumulate_dW:
            raise RKLError(RKL_INVALID_ARG, "accumulate_dW needs a dW tensor")
        dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    else:
        _need(dW, "dW", torch.float32, dev, (V, Hs))
    dh = torch.empty((N, Hs), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, Hs, Ht))
    _check(lib().rkl_backward_hidden(N, V, Hs, Ht, _ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), _ptr(row_mask),
                                     _ptr(grad_loss), _ptr(stats), _ptr(dh), _ptr(dW), int(bool(accumulate_dW)),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return dh, dW


def backward_logits(z_t, stats, h_s=None, W_s=None, z_s=None, grad_loss=None, row_mask=None, dW=None,
                    accumulate_dW=False, z_rows=None):
    """Teacher as logits.  Student as (h_s, W_s): returns (dh_s, dW_s).
    Student as logits z_s: returns dz_s fp32 [N, V].  z_rows as
    forward_logits."""
    torch = _torch()
    dev = z_t.device
    _need(z_t, "z_t", torch.float32, dev)
    N, V, T = _logit_rows(z_t, z_rows, dev)
    _need(stats, "stats", torch.float32, dev, (N, 4))
    if grad_loss is not None:
        _need(grad_loss, "grad_loss", torch.float32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    if z_s is not None:
        _need(z_s, "z_s", torch.float32, dev, tuple(z_t.shape))
        dz = torch.empty((N, V), dtype=torch.float32, device=dev)
        _check(lib().rkl_backward_logits(N, V, 0, None, None, _ptr(z_s), _ptr(z_t), _ptr(z_rows), T, _ptr(row_mask),
                                         _ptr(grad_loss), _ptr(stats), None, None, 0, _ptr(dz), None, 0,
                                         _stream(dev)))
        return dz
    Hs = h_s.shape[1]
    _need(h_s, "h_s", torch.bfloat16, dev, (N, Hs))
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    if dW is None:
        if accumulate_dW:
            raise RKLError(RKL_INVALID_ARG, "accumulate_dW needs a dW tensor")
        dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    else:
        _need(dW, "dW", torch.float32, dev, (V, Hs))
    dh = torch.empty((N, Hs), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, Hs, 0))
    _check(lib().rkl_backward_logits(N, V, Hs, _ptr(h_s), _ptr(W_s), None, _ptr(z_t), _ptr(z_rows), T,
                                     _ptr(row_mask), _ptr(grad_loss), _ptr(stats), _ptr(dh), _ptr(dW),
                                     int(bool(accumulate_dW)), None, _ptr(ws), ws.numel(), _stream(dev)))
    return dh, dW


class ReverseKL:
    """Per-position reverse KL over a [B, S-1] loss mask with compaction:
    compact -> gather -> fused forward -> scatter, and the matching backward.

        rk = ReverseKL(W_s, W_t)                     # hidden-state teacher
        loss_pos = rk.forward(h_s, mask, h_t=h_t)    # fp32 [T], zeros where mask == 0
        dh_pos, dW = rk.backward(grad_pos)           # fp32 [T, Hs] and [V, Hs]

    With the teacher as fp32 logits: ReverseKL(W_s) and rk.forward(h_s, mask,
    z_t=z_t), z_t [T, V].
    """

    def __init__(self, W_s, W_t=None):
        self.W_s, self.W_t = W_s, W_t

    def forward(self, h_s, mask, h_t=None, z_t=None):
        T = h_s.shape[0]
        self.T = T
        self.row_idx, self.N = compact_rows(mask)
        self.h_s = gather_rows(h_s, self.row_idx)
        if z_t is None:
            self.h_t, self.z_t = gather_rows(h_t, self.row_idx), None
            loss, self.stats = forward_hidden(self.h_s, self.W_s, self.h_t, self.W_t)
        else:
            # the logits rows are read through row_idx, not copied
            self.h_t, self.z_t = None, z_t
            loss, self.stats = forward_logits(z_t, h_s=self.h_s, W_s=self.W_s, z_rows=self.row_idx)
        return scatter_rows(loss, self.row_idx, T)

    def backward(self, grad_pos=None, dW=None, accumulate_dW=False):
        g = None if grad_pos is None else gather_rows(grad_pos.contiguous(), self.row_idx)
        if self.z_t is None:
            dh, dW = backward_hidden(self.h_s, self.W_s, self.h_t, self.W_t, self.stats, g, dW=dW,
                                     accumulate_dW=accumulate_dW)
        else:
            dh, dW = backward_logits(self.z_t, self.stats, h_s=self.h_s, W_s=self.W_s, grad_loss=g, dW=dW,
                                     accumulate_dW=accumulate_dW, z_rows=self.row_idx)
        return scatter_rows(dh, self.row_idx, self.T), dW


def forward_logprob_entropy(h, W, y, row_mask=None):
    """Log-probability of the sampled token and entropy per row of the
    projection h W^T.  Returns (logp fp32 [N], entropy fp32 [N], stats fp32
    [N, 4] = (lse, entropy, logp, lpmax))."""
    torch = _torch()
    dev = h.device
    N, H = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, dev)
    _need(W, "W", torch.bfloat16, dev, (V, H))
    _need(y, "y", torch.int32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, H, 0))
    _check(lib().rkl_forward_logprob_entropy(N, V, H, _ptr(h), _ptr(W), _ptr(y), _ptr(row_mask), _ptr(logp),
                                             _ptr(ent), _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    return logp, ent, stats


def backward_logprob_entropy(h, W, y, stats, grad_logp=None, grad_entropy=None, row_mask=None, dW=None,
                             accumulate_dW=False):
    """Gradients of sum_i (g_lp,i logp_i + g_H,i entropy_i) (grad_logp
    defaults to ones, grad_entropy to zeros): returns (dh fp32 [N, H], dW fp32
    [V, H])."""
    torch = _torch()
    dev = h.device
    N, H = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, dev)
    _need(W, "W", torch.bfloat16, dev, (V, H))
    _need(y, "y", torch.int32, dev, (N,))
    _need(stats, "stats", torch.float32, dev, (N, 4))
    for g, name in ((grad_logp, "grad_logp"), (grad_entropy, "grad_entropy")):
        if g is not None:
            _need(g, name, torch.float32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    if dW is None:
        if accumulate_dW:
            raise RKLError(RKL_INVALID_ARG, "accumulate_dW needs a dW tensor")
        dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    else:
        _need(dW, "dW", torch.float32, dev, (V, H))
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, H, 0))
    _check(lib().rkl_backward_logprob_entropy(N, V, H, _ptr(h), _ptr(W), _ptr(y), _ptr(row_mask), _ptr(grad_logp),
                                              _ptr(grad_entropy), _ptr(stats), _ptr(dh), _ptr(dW),
                                              int(bool(accumulate_dW)), _ptr(ws), ws.numel(), _stream(dev)))
    return dh, dW


def forward_hidden_shard(h_s, W_s, h_t, W_t):
    """One vocabulary shard's per-row statistics: W_s [V, Hs] and W_t [V, Ht]
    are the shard's vocabulary rows.  Returns partial fp32 [5, N] = (m_s, S_s,
    A, m_t, S_t) planes; merge the shards' with combine_shards."""
    torch = _torch()
    dev = h_s.device
    N, Hs = h_s.shape
    V = W_s.shape[0]
    Ht = h_t.shape[1]
    _need(h_s, "h_s", torch.bfloat16, dev)
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    _need(h_t, "h_t", torch.bfloat16, dev, (N, Ht))
    _need(W_t, "W_t", torch.bfloat16, dev, (V, Ht))
    partial = torch.empty((5, N), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, Hs, Ht))
    _check(lib().rkl_forward_hidden_shard(N, V, Hs, Ht, _ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), _ptr(partial),
                                          _ptr(ws), ws.numel(), _stream(dev)))
    return partial


def forward_logits_shard(z_t, h_s=None, W_s=None, z_s=None):
    """One vocabulary shard with the teacher given as the shard's fp32 logits
    z_t [N, V]; the student as the shard's (h_s, W_s) rows or as its fp32
    logits z_s [N, V].  Returns partial fp32 [5, N] as forward_hidden_shard."""
    torch = _torch()
    dev = z_t.device
    N, V = z_t.shape
    _need(z_t, "z_t", torch.float32, dev)
    Hs = 0
    if z_s is None:
        Hs = h_s.shape[1]
        _need(h_s, "h_s", torch.bfloat16, dev, (N, Hs))
        _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    else:
        _need(z_s, "z_s", torch.float32, dev, (N, V))
    partial = torch.empty((5, N), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, Hs, 0))
    _check(lib().rkl_forward_logits_shard(N, V, Hs, _ptr(h_s), _ptr(W_s), _ptr(z_s), _ptr(z_t), _ptr(partial),
                                          _ptr(ws), ws.numel(), _stream(dev)))
    return partial


def combine_shards(partials, row_mask=None):
    """Merge [G, 5, N] shard partials into (loss [N], stats [N, 4]) over the
    whole vocabulary, as forward_hidden returns them."""
    torch = _torch()
    dev = partials.device
    G, five, N = partials.shape
    if five != 5:
        raise RKLError(RKL_INVALID_ARG, "partials must be [G, 5, N]")
    _need(partials, "partials", torch.float32, dev)
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    _check(lib().rkl_combine_shards(G, N, _ptr(partials), _ptr(row_mask), _ptr(loss), _ptr(stats), _stream(dev)))
    return loss, stats


def forward_logprob_entropy_shard(h, W, y):
    """One vocabulary shard of the log-probability / entropy forward: W [V,
    H] holds the shard's vocabulary rows, y int32 [N] the sampled tokens in
    the shard's coordinates (outside [0, V) when in another shard).  Returns
    partial fp32 [5, N] = (m, S, B, z_y, 0) planes; merge the shards' with
    combine_shards_logprob_entropy."""
    torch = _torch()
    dev = h.device
    N, H = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, dev)
    _need(W, "W", torch.bfloat16, dev, (V, H))
    _need(y, "y", torch.int32, dev, (N,))
    partial = torch.empty((5, N), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, H, 0))
    _check(lib().rkl_forward_logprob_entropy_shard(N, V, H, _ptr(h), _ptr(W), _ptr(y), _ptr(partial), _ptr(ws),
                                                   ws.numel(), _stream(dev)))
    return partial


def combine_shards_logprob_entropy(partials, row_mask=None):
    """Merge [G, 5, N] log-probability / entropy shard partials into (logp
    [N], entropy [N], stats [N, 4]) over the whole vocabulary."""
    torch = _torch()
    dev = partials.device
    G, five, N = partials.shape
    if five != 5:
        raise RKLError(RKL_INVALID_ARG, "partials must be [G, 5, N]")
    _need(partials, "partials", torch.float32, dev)
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    _check(lib().rkl_combine_shards_logprob_entropy(G, N, _ptr(partials), _ptr(row_mask), _ptr(logp), _ptr(ent),
                                                    _ptr(stats), _stream(dev)))
    return logp, ent, stats


def forward_hidden_teachers(h_s, W_s, h_t, W_t, teacher, row_mask=None):
    """Per-row reverse KL with row i's teacher logits h_t[i] W_t[teacher[i]]^T
    (W_t bf16 [K, V, Ht], teacher int32 [N]).  Returns (loss, stats) as
    forward_hidden."""
    torch = _torch()
    dev = h_s.device
    N, Hs = h_s.shape
    K, V, Ht = W_t.shape
    _need(h_s, "h_s", torch.bfloat16, dev)
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    _need(h_t, "h_t", torch.bfloat16, dev, (N, Ht))
    _need(W_t, "W_t", torch.bfloat16, dev)
    _need(teacher, "teacher", torch.int32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes_teachers(N, V, Hs, Ht))
    _check(lib().rkl_forward_hidden_teachers(N, V, Hs, Ht, K, _ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t),
                                             _ptr(teacher), _ptr(row_mask), _ptr(loss), _ptr(stats), _ptr(ws),
                                             ws.numel(), _stream(dev)))
    return loss, stats


def backward_hidden_teachers(h_s, W_s, h_t, W_t, teacher, stats, grad_loss=None, row_mask=None, dW=None,
                             accumulate_dW=False):
    """Backward of forward_hidden_teachers: returns (dh_s, dW_s)."""
    torch = _torch()
    dev = h_s.device
    N, Hs = h_s.shape
    K, V, Ht = W_t.shape
    _need(h_s, "h_s", torch.bfloat16, dev)
    _need(W_s, "W_s", torch.bfloat16, dev, (V, Hs))
    _need(h_t, "h_t", torch.bfloat16, dev, (N, Ht))
    _need(W_t, "W_t", torch.bfloat16, dev)
    _need(teacher, "teacher", torch.int32, dev, (N,))
    _need(stats, "stats", torch.float32, dev, (N, 4))
    if grad_loss is not None:
        _need(grad_loss, "grad_loss", torch.float32, dev, (N,))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    if dW is None:
        if accumulate_dW:
            raise RKLError(RKL_INVALID_ARG, "accumulate_dW needs a dW tensor")
        dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    else:
        _need(dW, "dW", torch.float32, dev, (V, Hs))
    dh = torch.empty((N, Hs), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes_teachers(N, V, Hs, Ht))
    _check(lib().rkl_backward_hidden_teachers(N, V, Hs, Ht, K, _ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t),
                                              _ptr(teacher), _ptr(row_mask), _ptr(grad_loss), _ptr(stats), _ptr(dh),
                                              _ptr(dW), int(bool(accumulate_dW)), _ptr(ws), ws.numel(),
                                              _stream(dev)))
    return dh, dW


def _topk_args(h, W, y, support, logpt_support, row_mask):
    torch = _torch()
    dev = h.device
    N, H = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, dev)
    _need(W, "W", torch.bfloat16, dev, (V, H))
    _need(y, "y", torch.int32, dev, (N,))
    if support is None:
        K = 0
    else:
        K = support.shape[1]
        _need(support, "support", torch.int32, dev, (N, K))
        _need(logpt_support, "logpt_support", torch.float32, dev, (N, K))
    if row_mask is not None:
        _need(row_mask, "row_mask", torch.uint8, dev, (N,))
    return dev, N, V, H, K


def forward_topk(h, W, y, support, logpt_support, logpt_y, row_mask=None, logps_support=None):
    """Top-k estimator of the reverse KL per row: the student projected (h
    [N, H], W [V, H] bf16), y int32 [N] the sampled tokens, support int32
    [N, K] the support ids (None for K = 0), logpt_support fp32 [N, K] and
    logpt_y fp32 [N] the teacher's log-probabilities there.  Returns (loss
    fp32 [N], stats fp32 [N, 4] = (lse, c, sp, bound)).  logps_support: an
    optional fp32 [N, K] tensor that receives the student's
    log-probabilities on the support (hand it to backward_topk)."""
    torch = _torch()
    dev, N, V, H, K = _topk_args(h, W, y, support, logpt_support, row_mask)
    _need(logpt_y, "logpt_y", torch.float32, dev, (N,))
    if logps_support is not None:
        _need(logps_support, "logps_support", torch.float32, dev, (N, K))
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, H, 0))
    _check(lib().rkl_forward_topk(N, V, H, K, _ptr(h), _ptr(W), _ptr(y), _ptr(support), _ptr(logpt_support),
                                  _ptr(logpt_y), _ptr(row_mask), _ptr(loss), _ptr(stats), _ptr(logps_support),
                                  _ptr(ws), ws.numel(), _stream(dev)))
    return loss, stats


def backward_topk(h, W, y, support, logpt_support, stats, grad_loss=None, row_mask=None, dW=None,
                  accumulate_dW=False, logps_support=None):
    """Backward of sum_i g_i L_i for forward_topk: returns (dh fp32 [N, H], dW
    fp32 [V, H]).  logps_support: the forward's optional output on the same
    inputs (spares the support's dot products; same results)."""
    torch = _torch()
    dev, N, V, H, K = _topk_args(h, W, y, support, logpt_support, row_mask)
    _need(stats, "stats", torch.float32, dev, (N, 4))
    if logps_support is not None:
        _need(logps_support, "logps_support", torch.float32, dev, (N, K))
    if grad_loss is not None:
        _need(grad_loss, "grad_loss", torch.float32, dev, (N,))
    if dW is None:
        if accumulate_dW:
            raise RKLError(RKL_INVALID_ARG, "accumulate_dW needs a dW tensor")
        dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    else:
        _need(dW, "dW", torch.float32, dev, (V, H))
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    ws = _workspace(dev, workspace_bytes(N, V, H, 0))
    _check(lib().rkl_backward_topk(N, V, H, K, _ptr(h), _ptr(W), _ptr(y), _ptr(support), _ptr(logpt_support),
                                   _ptr(row_mask), _ptr(grad_loss), _ptr(stats), _ptr(logps_support), _ptr(dh),
                                   _ptr(dW), int(bool(accumulate_dW)), _ptr(ws), ws.numel(), _stream(dev)))
    return dh, dW
