"""fp64 CPU oracle for the compact actor log-probability / entropy workload.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library under ``lm_head_reverse_amd/`` never does, and this module imports
nothing from it.

What is computed (slime pull request "compact actor logits before
projection", summary: the log-probability / entropy computation takes the
[N, V] logits of the N loss-masked rows and its scalar results are scattered
back; NeMo-RL pull request "add full-vocabulary on-policy distillation",
implementation notes: the neighbouring entropy kernel recomputes its
log-softmax in the backward).  Per row i with logits z_i = h_i W^T and
sampled token y_i:

    log p(y_i)  = z_i[y_i] - lse(z_i)
    H_i         = -sum_v p_i(v) log p_i(v)              (natural log)

and the gradient of sum_i (g_lp,i log p(y_i) + g_H,i H_i) with respect to z_i:

    dz_i[v] = g_lp,i (1[v = y_i] - p_i(v)) - g_H,i p_i(v) (log p_i(v) + H_i)

(d log p(y)/dz_v = 1[v = y] - p_v; dH/dz_v = -p_v (log p_v + H)), then
dh = dz W and dW = sum_i dz_i^T h_i.  The top-p masks the slime page also
mentions are not part of this (their rule is not given there).

Everything is the plain definition in float64 (numpy); a matrix product and
numpy's elementwise exp/log/max/sum are the only library primitives used.
Pins: tests/test_oracle_logprob_entropy.py.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.rkl_oracle import log_softmax, logsumexp, project


def logprob_entropy(z: np.ndarray, y: np.ndarray):
    """(log p(y), H, lse) per row of the logits z [rows, V] for the sampled
    token indices y [rows]."""
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    lp = log_softmax(z)
    logp = lp[np.arange(z.shape[0]), y]
    H = -np.sum(np.exp(lp) * lp, axis=-1)
    return logp, H, logsumexp(z)


def logprob_entropy_dz(z: np.ndarray, y: np.ndarray, lse: np.ndarray, H: np.ndarray,
                       g_lp: Optional[np.ndarray] = None, g_H: Optional[np.ndarray] = None,
                       cols: Optional[np.ndarray] = None) -> np.ndarray:
    """Gradient of sum_i (g_lp,i log p(y_i) + g_H,i H_i) with respect to the
    logits.  z holds the columns ``cols`` of the vocabulary (all when None);
    lse and H are the full-vocabulary row values.  g_lp defaults to ones,
    g_H to zeros."""
    z = np.asarray(z, dtype=np.float64)
    rows = z.shape[0]
    g_lp = np.ones(rows) if g_lp is None else np.asarray(g_lp, dtype=np.float64)
    g_H = np.zeros(rows) if g_H is None else np.asarray(g_H, dtype=np.float64)
    lp = z - np.asarray(lse, dtype=np.float64)[:, None]
    p = np.exp(lp)
    dz = -g_lp[:, None] * p - g_H[:, None] * p * (lp + np.asarray(H, dtype=np.float64)[:, None])
    vocab = np.arange(z.shape[1]) if cols is None else np.asarray(cols, dtype=np.int64)
    hit = vocab[None, :] == np.asarray(y, dtype=np.int64)[:, None]
    dz += np.where(hit, g_lp[:, None], 0.0)
    return dz


def forward(h: np.ndarray, W: np.ndarray, y: np.ndarray, row_chunk: int = 256):
    """(log p(y), H, lse) for every row of h [rows, H] (float64 values) with the
    output-layer weight W [V, H] (float64 values)."""
    n = h.shape[0]
    out = [np.zeros(n), np.zeros(n), np.zeros(n)]
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        res = logprob_entropy(project(h[r0:r1], W), y[r0:r1])
        for o, v in zip(out, res):
            o[r0:r1] = v
    return tuple(out)


def backward(h: np.ndarray, W: np.ndarray, y: np.ndarray, g_lp: Optional[np.ndarray] = None,
             g_H: Optional[np.ndarray] = None, row_chunk: int = 256, want_dz: bool = False):
    """dict with dh [rows, H] = dz W and dW [V, H] = sum_i dz_i^T h_i (and dz
    [rows, V] when asked for)."""
    n = h.shape[0]
    out = {"dh": np.zeros(h.shape), "dW": np.zeros(W.shape)}
    if want_dz:
        out["dz"] = np.zeros((n, W.shape[0]))
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        z = project(h[r0:r1], W)
        _, H, lse = logprob_entropy(z, y[r0:r1])
        dz = logprob_entropy_dz(z, y[r0:r1], lse, H,
                                None if g_lp is None else g_lp[r0:r1], None if g_H is None else g_H[r0:r1])
        if want_dz:
            out["dz"][r0:r1] = dz
        out["dh"][r0:r1] = dz @ W
        out["dW"] += dz.T @ h[r0:r1]
    return out


def dW_rows(h: np.ndarray, W: np.ndarray, y: np.ndarray, vocab: np.ndarray, lse: np.ndarray, H: np.ndarray,
            g_lp: Optional[np.ndarray] = None, g_H: Optional[np.ndarray] = None) -> np.ndarray:
    """Selected rows of dW: dW[v] = sum_i dz[i, v] h_i for v in ``vocab``,
    given every row's full-vocabulary lse and H."""
    vocab = np.asarray(vocab, dtype=np.int64)
    z = project(h, W[vocab])
    dz = logprob_entropy_dz(z, y, lse, H, g_lp, g_H, cols=vocab)
    return dz.T @ h
