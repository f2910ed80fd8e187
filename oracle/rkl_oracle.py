"""fp64 CPU oracle for the fused LM-head projection + full-vocabulary reverse KL.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library under ``lm_head_reverse_amd/`` never does, and this module imports
nothing from it: the two share no code.

Everything here is the plain definition, evaluated in float64 (numpy).  A
matrix product (``@``) and numpy's elementwise exp/log/max/sum are the only
library primitives used.  Processing rows in groups (``row_chunk``) changes
nothing because every quantity below is defined per row.

Sources (three pull-request pages):

* NeMo-RL "add full-vocabulary on-policy distillation to SingleController",
  summary: the per-token objective L_t = sum_v p_s(v) (log p_s(v) - log p_t(v))
  over the whole vocabulary; the two teacher payloads (hidden states projected
  through the teacher's output-layer weight, or full-vocabulary logits).
* same page, implementation notes: the shared backward
  dL/dz = p_s * (w - L) with w = log p_s - log p_t; log-softmaxes are
  recomputed rather than cached; the per-token output is a [B, S-1] tensor.
* slime "compact actor logits before projection", summary: only the N
  loss-masked rows are projected; scalar results are scattered back to the
  original layout; an empty mask still gives a (zero) gradient.
* Fast-LLM "distill with loss_mask", description: reverse KL restricted by a
  loss mask.

Readings where the pages are silent:
natural log; no temperature; logits kept at full precision (never rounded to
bf16); the teacher receives no gradient; the library does not reduce L over
tokens -- the caller does and hands back the per-token upstream gradient g;
compacted rows keep ascending position order; a row whose mask is 0 has L = 0
and contributes nothing to any gradient.

Pins: tests/test_oracle.py checks every function here against closed forms,
invariants, central finite differences and brute force (no function is left
unpinned).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# data handling
# --------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def compact_rows(mask: np.ndarray) -> np.ndarray:
    """Positions whose mask is nonzero, ascending (slime page, summary: project
    only the loss-masked rows).  int32 [N]."""
    m = np.asarray(mask).reshape(-1)
    return np.array([i for i in range(m.shape[0]) if m[i] != 0], dtype=np.int32)


def gather_rows(src: np.ndarray, row_idx: np.ndarray) -> np.ndarray:
    """dst[i] = src[row_idx[i]] (bit copy)."""
    return src[np.asarray(row_idx, dtype=np.int64)]


def scatter_rows(src: np.ndarray, row_idx: np.ndarray, T: int) -> np.ndarray:
    """Inverse of gather over all T positions: dst[row_idx[i]] = src[i], every
    other row literally zero (slime page, summary: scatter scalar results back
    to the original layout)."""
    out = np.zeros((T,) + src.shape[1:], dtype=src.dtype)
    out[np.asarray(row_idx, dtype=np.int64)] = src
    return out


# --------------------------------------------------------------------------
# the method, per row
# --------------------------------------------------------------------------

def project(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Logits z = h W^T in float64 (NeMo-RL page, summary: hidden states
    projected with an output-layer weight, W stored [V, H])."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def log_softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise log p = z - (m + log sum_v exp(z - m)), m = max_v z."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return z - (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))


def logsumexp(z: np.ndarray) -> np.ndarray:
    """Row-wise log sum_v exp(z)."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1)
    return m + np.log(np.sum(np.exp(z - m[..., None]), axis=-1))


def reverse_kl(z_s: np.ndarray, z_t: np.ndarray) -> np.ndarray:
    """Per-row L = sum_v p_s(v) (log p_s(v) - log p_t(v))  (NeMo-RL page,
    summary equation), over the full vocabulary."""
    lp_s = log_softmax(z_s)
    lp_t = log_softmax(z_t)
    return np.sum(np.exp(lp_s) * (lp_s - lp_t), axis=-1)


def row_stats(z_s: np.ndarray, z_t: np.ndarray):
    """(lse_s, lse_t, L) per row -- what a backward needs to rebuild the
    log-softmaxes without caching them (NeMo-RL page, implementation notes)."""
    return logsumexp(z_s), logsumexp(z_t), reverse_kl(z_s, z_t)


def reverse_kl_dz(z_s: np.ndarray, z_t: np.ndarray, lse_s: np.ndarray, lse_t: np.ndarray,
                  L: np.ndarray, g: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/dz_s = g * p_s * (w - L), w = log p_s - log p_t  (NeMo-RL page,
    implementation notes).  The columns of z may be any subset of the
    vocabulary: the row statistics carry the full-vocabulary normalisation."""
    lp_s = np.asarray(z_s, dtype=np.float64) - np.asarray(lse_s)[..., None]
    lp_t = np.asarray(z_t, dtype=np.float64) - np.asarray(lse_t)[..., None]
    dz = np.exp(lp_s) * (lp_s - lp_t - np.asarray(L)[..., None])
    if g is not None:
        dz = dz * np.asarray(g, dtype=np.float64)[..., None]
    return dz


# --------------------------------------------------------------------------
# whole path over a set of rows (row-chunked only to bound memory)
# --------------------------------------------------------------------------

class Inputs:
    """fp64 views of one problem.  Either side may be given as hidden states +
    weight (bf16 bits) or as fp32 logits [rows, V]."""

    def __init__(self, h_s=None, W_s=None, h_t=None, W_t=None, z_s=None, z_t=None):
        self.h_s = None if h_s is None else widen_bf16(h_s)
        self.W_s = None if W_s is None else widen_bf16(W_s)
        self.h_t = None if h_t is None else widen_bf16(h_t)
        self.W_t = None if W_t is None else widen_bf16(W_t)
        self.z_s = z_s
        self.z_t = z_t
        if (self.h_s is None) == (self.z_s is None):
            raise ValueError("student: give exactly one of (h_s, W_s) or z_s")
        if (self.h_t is None) == (self.z_t is None):
            raise ValueError("teacher: give exactly one of (h_t, W_t) or z_t")

    @classmethod
    def from_case(cls, case) -> "Inputs":
        return cls(case.h_s, case.W_s, case.h_t, case.W_t, case.z_s, case.z_t)

    def zs(self, rows, cols=None) -> np.ndarray:
        if self.z_s is not None:
            z = np.asarray(self.z_s[rows], dtype=np.float64)
            return z if cols is None else z[:, cols]
        W = self.W_s if cols is None else self.W_s[cols]
        return project(self.h_s[rows], W)

    def zt(self, rows, cols=None) -> np.ndarray:
        if self.z_t is not None:
            z = np.asarray(self.z_t[rows], dtype=np.float64)
            return z if cols is None else z[:, cols]
        W = self.W_t if cols is None else self.W_t[cols]
        return project(self.h_t[rows], W)


def forward(inp: Inputs, rows: np.ndarray, row_chunk: int = 256):
    """(L, lse_s, lse_t) for the given positions (float64 [len(rows)] each)."""
    rows = np.asarray(rows, dtype=np.int64)
    L = np.zeros(rows.shape[0])
    ls = np.zeros(rows.shape[0])
    lt = np.zeros(rows.shape[0])
    for r0 in range(0, rows.shape[0], row_chunk):
        rr = rows[r0:r0 + row_chunk]
        ls[r0:r0 + len(rr)], lt[r0:r0 + len(rr)], L[r0:r0 + len(rr)] = row_stats(inp.zs(rr), inp.zt(rr))
    return L, ls, lt


def backward(inp: Inputs, rows: np.ndarray, g: Optional[np.ndarray] = None,
             row_chunk: int = 256, want_dz: bool = False):
    """Gradients of sum_i g_i L_i over the given positions.

    Returns dict with ``dh`` [len(rows), Hs] = dz W_s and ``dW`` [V, Hs] =
    sum_i dz_i^T h_s,i when the student is given as hidden states, and ``dz``
    [len(rows), V] when asked for (or when the student is given as logits).
    The per-row statistics the backward rebuilt its log-softmaxes from are
    returned too: ``L``, ``lse_s``, ``lse_t`` (the same values ``forward``
    gives, from the same projection).
    """
    rows = np.asarray(rows, dtype=np.int64)
    hidden = inp.h_s is not None
    out = {"L": np.zeros(rows.shape[0]), "lse_s": np.zeros(rows.shape[0]), "lse_t": np.zeros(rows.shape[0])}
    if hidden:
        out["dh"] = np.zeros((rows.shape[0], inp.h_s.shape[1]))
        out["dW"] = np.zeros(inp.W_s.shape)
    if want_dz or not hidden:
        V = inp.W_s.shape[0] if hidden else inp.z_s.shape[1]
        out["dz"] = np.zeros((rows.shape[0], V))
    for r0 in range(0, rows.shape[0], row_chunk):
        rr = rows[r0:r0 + row_chunk]
        zs, zt = inp.zs(rr), inp.zt(rr)
        ls, lt, L = row_stats(zs, zt)
        out["L"][r0:r0 + len(rr)], out["lse_s"][r0:r0 + len(rr)], out["lse_t"][r0:r0 + len(rr)] = L, ls, lt
        gg = None if g is None else np.asarray(g, dtype=np.float64)[r0:r0 + len(rr)]
        dz = reverse_kl_dz(zs, zt, ls, lt, L, gg)
        if "dz" in out:
            out["dz"][r0:r0 + len(rr)] = dz
        if hidden:
            out["dh"][r0:r0 + len(rr)] = dz @ inp.W_s
            out["dW"] += dz.T @ inp.h_s[rr]
    return out


def dW_rows(inp: Inputs, rows: np.ndarray, vocab: np.ndarray, stats,
            g: Optional[np.ndarray] = None) -> np.ndarray:
    """Selected rows of dW_s: dW[v] = sum_i dz[i, v] h_s[i] for v in ``vocab``,
    given the per-row (L, lse_s, lse_t) of every contributing position."""
    rows = np.asarray(rows, dtype=np.int64)
    vocab = np.asarray(vocab, dtype=np.int64)
    L, ls, lt = stats
    zs, zt = inp.zs(rows, vocab), inp.zt(rows, vocab)
    dz = reverse_kl_dz(zs, zt, ls, lt, L, g)
    return dz.T @ inp.h_s[rows]


def per_position_loss(inp: Inputs, mask: np.ndarray) -> np.ndarray:
    """Compaction -> per-row L -> scatter back to all T positions ([B, S-1]
    flattened); positions with mask 0 are exactly 0."""
    idx = compact_rows(mask)
    L, _, _ = forward(inp, idx)
    return scatter_rows(L, idx, np.asarray(mask).reshape(-1).shape[0])


def project_f32(h_bits: np.ndarray, W_bits: np.ndarray, row_chunk: int = 512) -> np.ndarray:
    """Teacher logits payload: fp32 rounding of the exact projection h W^T."""
    h = widen_bf16(h_bits)
    W = widen_bf16(W_bits)
    out = np.empty((h.shape[0], W.shape[0]), dtype=np.float32)
    for r0 in range(0, h.shape[0], row_chunk):
        out[r0:r0 + row_chunk] = project(h[r0:r0 + row_chunk], W)
    return out
