"""fp64 CPU oracle for reverse KL with a teacher chosen per row.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library under ``lm_head_reverse_amd/`` never does, and this module imports
nothing from it.

What is computed (NeMo-RL pull request "add full-vocabulary on-policy
distillation to SingleController": the summary defines the per-token reverse
KL with the teacher's hidden states projected through that teacher's
output-layer weight; its first-version limits allow exactly one teacher
checkpoint and note that the payload column is shaped so that a per-row
teacher index can be added).  Reading: with K teachers, row i names its
teacher k_i, and

    z_t,i = h_t,i W_t[k_i]^T,    L_i = sum_v p_s,i(v) (log p_s,i(v) - log p_t,i(v)),

with the student side, the backward dL/dz_s = p_s (w - L) and the gradients
dh, dW exactly as for one teacher (the teachers receive no gradient).

Everything reuses the single-teacher definitions of oracle/rkl_oracle.py row
by row; only the choice of W_t per row is new.  Pins:
tests/test_oracle_multi_teacher.py.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.rkl_oracle import project, reverse_kl_dz, row_stats


def teacher_logits(h_t: np.ndarray, W_t: np.ndarray, teacher: np.ndarray) -> np.ndarray:
    """z_t [rows, V]: row i projected through W_t[teacher[i]] (float64 values;
    W_t is [K, V, Ht])."""
    teacher = np.asarray(teacher, dtype=np.int64)
    out = np.empty((h_t.shape[0], W_t.shape[1]))
    for k in np.unique(teacher):
        sel = teacher == k
        out[sel] = project(h_t[sel], W_t[k])
    return out


def forward(h_s, W_s, h_t, W_t, teacher, row_chunk: int = 256):
    """(L, lse_s, lse_t) per row (float64 inputs: h_s [rows, Hs], W_s [V, Hs],
    h_t [rows, Ht], W_t [K, V, Ht], teacher [rows])."""
    n = h_s.shape[0]
    L, ls, lt = np.zeros(n), np.zeros(n), np.zeros(n)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        zs = project(h_s[r0:r1], W_s)
        zt = teacher_logits(h_t[r0:r1], W_t, teacher[r0:r1])
        ls[r0:r1], lt[r0:r1], L[r0:r1] = row_stats(zs, zt)
    return L, ls, lt


def backward(h_s, W_s, h_t, W_t, teacher, g: Optional[np.ndarray] = None, row_chunk: int = 256):
    """dict with dh [rows, Hs] and dW [V, Hs] of sum_i g_i L_i."""
    n = h_s.shape[0]
    out = {"dh": np.zeros(h_s.shape), "dW": np.zeros(W_s.shape)}
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        zs = project(h_s[r0:r1], W_s)
        zt = teacher_logits(h_t[r0:r1], W_t, teacher[r0:r1])
        ls, lt, L = row_stats(zs, zt)
        dz = reverse_kl_dz(zs, zt, ls, lt, L, None if g is None else g[r0:r1])
        out["dh"][r0:r1] = dz @ W_s
        out["dW"] += dz.T @ h_s[r0:r1]
    return out


def dW_rows(h_s, W_s, h_t, W_t, teacher, vocab, stats, g: Optional[np.ndarray] = None) -> np.ndarray:
    """Selected rows of dW_s given every row's (L, lse_s, lse_t)."""
    vocab = np.asarray(vocab, dtype=np.int64)
    L, ls, lt = stats
    zs = project(h_s, W_s[vocab])
    zt = teacher_logits(h_t, W_t[:, vocab], teacher)
    dz = reverse_kl_dz(zs, zt, ls, lt, L, g)
    return dz.T @ h_s
