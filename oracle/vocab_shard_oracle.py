"""fp64 CPU oracle for reverse KL over a vocabulary split into shards.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library under ``lm_head_reverse_amd/`` never does, and this module imports
nothing from it.

What is computed (NeMo-RL pull request "add full-vocabulary on-policy
distillation to SingleController", implementation notes: the two reverse-KL
autograd functions are chunked and tensor-parallel, next to the distributed
entropy function, and the divergence is formed where the vocabulary-parallel
group is held).  Reading: a rank owns a contiguous range [v0, v1) of the
vocabulary (those rows of W_s and W_t) and reduces it to five numbers per
row,

    m_s = max_v z_s,   S_s = sum_v exp(z_s - m_s),
    A   = sum_v exp(z_s - m_s) (z_s - z_t),
    m_t = max_v z_t,   S_t = sum_v exp(z_t - m_t),

the ranks exchange these, and every rank merges them with the log-sum-exp
rule: M = max_g m_g, S = sum_g S_g exp(m_g - M), A = sum_g A_g exp(m_s,g -
M_s).  Then lse = M + log S for each side, L = A / S_s - lse_s + lse_t, and
log max_v p_s(v) = -log S_s.  The backward of a shard is the single-device
backward restricted to the shard's columns, with the merged statistics: its
dz columns and dW rows are the shard's part of the full ones, and its dh is
one term of a sum over the shards.

The same split applies to the log-probability of a sampled token and the
entropy (the same notes put these functions beside the distributed entropy
function): a shard reduces its columns to

    m = max_v z,   S = sum_v exp(z - m),   B = sum_v exp(z - m) z,
    z_y = z[y] when the sampled token y lies in the shard, else -inf,

and the merge gives lse = M + log S, H = lse - B / S, log p(y) = z_y - lse
(z_y from the one shard that holds y).

Pins: tests/test_oracle_vocab_shard.py (merged shards against the
unsharded definitions in oracle/rkl_oracle.py and
oracle/logprob_entropy_oracle.py for uneven shards, one-column shards and a
single shard; each shard's m + log S against scipy's logsumexp; shard
order; the backward's dh adding up over shards and its dW rows matching the
full dW).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from oracle.rkl_oracle import project, reverse_kl_dz


def shard_partials(h_s, W_s, h_t, W_t, v0: int, v1: int) -> np.ndarray:
    """[5, rows] float64: (m_s, S_s, A, m_t, S_t) of vocabulary columns
    [v0, v1) (float64 inputs: h [rows, H], W [V, H])."""
    return partials_of_logits(project(h_s, W_s[v0:v1]), project(h_t, W_t[v0:v1]))


def partials_of_logits(zs, zt) -> np.ndarray:
    """[5, rows] float64: (m_s, S_s, A, m_t, S_t) of one shard's logits
    z_s, z_t [rows, shard columns] (the teacher-logits payload, or either
    side given as logits)."""
    zs = np.asarray(zs, dtype=np.float64)
    zt = np.asarray(zt, dtype=np.float64)
    m_s = np.max(zs, axis=1)
    e_s = np.exp(zs - m_s[:, None])
    m_t = np.max(zt, axis=1)
    return np.stack([m_s, np.sum(e_s, axis=1), np.sum(e_s * (zs - zt), axis=1),
                     m_t, np.sum(np.exp(zt - m_t[:, None]), axis=1)])


def merge(partials: Sequence[np.ndarray]):
    """Merge shard partials ([G] of [5, rows]) into per-row (L, lse_s, lse_t,
    lpmax), lpmax = log of the row's largest student probability."""
    P = np.stack([np.asarray(p, dtype=np.float64) for p in partials])   # [G, 5, rows]
    M_s = np.max(P[:, 0], axis=0)
    f_s = np.exp(P[:, 0] - M_s)
    S_s = np.sum(P[:, 1] * f_s, axis=0)
    A = np.sum(P[:, 2] * f_s, axis=0)
    M_t = np.max(P[:, 3], axis=0)
    S_t = np.sum(P[:, 4] * np.exp(P[:, 3] - M_t), axis=0)
    lse_s = M_s + np.log(S_s)
    lse_t = M_t + np.log(S_t)
    return A / S_s - lse_s + lse_t, lse_s, lse_t, -np.log(S_s)


def shard_bounds(V: int, G: int) -> list:
    """Contiguous shards of sizes differing by at most one (the first V % G
    shards one column longer)."""
    q, r = divmod(V, G)
    b = [0]
    for g in range(G):
        b.append(b[-1] + q + (1 if g < r else 0))
    return list(zip(b[:-1], b[1:]))


def shard_backward(h_s, W_s, h_t, W_t, v0: int, v1: int, stats, g: Optional[np.ndarray] = None) -> dict:
    """One shard's backward with the merged per-row stats (L, lse_s, lse_t):
    dz [rows, v1 - v0], its dh term dz W_s[v0:v1] and dW rows v0..v1-1."""
    L, lse_s, lse_t = stats
    zs = project(h_s, W_s[v0:v1])
    zt = project(h_t, W_t[v0:v1])
    dz = reverse_kl_dz(zs, zt, lse_s, lse_t, L, g)
    return {"dz": dz, "dh": dz @ W_s[v0:v1], "dW": dz.T @ h_s}


def lpe_shard_partials(h, W, y, v0: int, v1: int) -> np.ndarray:
    """[4, rows] float64: (m, S, B, z_y) of vocabulary columns [v0, v1) for
    the projection h W^T and sampled tokens y (global vocabulary indices)."""
    z = project(h, W[v0:v1])
    m = np.max(z, axis=1)
    e = np.exp(z - m[:, None])
    y = np.asarray(y, dtype=np.int64)
    inside = (y >= v0) & (y < v1)
    zy = np.full(z.shape[0], -np.inf)
    zy[inside] = z[np.nonzero(inside)[0], y[inside] - v0]
    return np.stack([m, np.sum(e, axis=1), np.sum(e * z, axis=1), zy])


def lpe_merge(partials: Sequence[np.ndarray]):
    """Merge shard partials ([G] of [4, rows]) into per-row (log p(y),
    entropy, lse, lpmax)."""
    P = np.stack([np.asarray(p, dtype=np.float64) for p in partials])   # [G, 4, rows]
    M = np.max(P[:, 0], axis=0)
    f = np.exp(P[:, 0] - M)
    S = np.sum(P[:, 1] * f, axis=0)
    B = np.sum(P[:, 2] * f, axis=0)
    lse = M + np.log(S)
    return np.max(P[:, 3], axis=0) - lse, lse - B / S, lse, -np.log(S)
