"""fp64 CPU oracle for the top-k estimator of the reverse KL (support plus a
score-function tail).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library under ``lm_head_reverse_amd/`` never does, and this module imports
nothing from it.

Source: NeMo-RL pull request "add full-vocabulary on-policy distillation to
SingleController", summary.  The page gives the full reverse KL
L = sum_v p_s(v) (log p_s(v) - log p_t(v)) and says it is the K = V limit of
the top-k estimator it replaces: once the support spans the whole
vocabulary, the estimator's score-function tail term vanishes and the
objective is exact; the estimator it replaces is the log-probability gap
of the sampled token.  The page prints no formula for K < V.

Reading (the plainest one the page supports; every statement below is
fixed by the two limits the page names plus the estimator being unbiased):
per row, with f(v) = log p_s(v) - log p_t(v), a support S of K distinct
vocabulary entries (chosen without looking at y; e.g. the teacher's top K),
and a token y sampled from the student p_s,

    L_hat = sum_{v in S} p_s(v) f(v)  +  [y not in S] f(y).

The first term is the reverse KL restricted to S, exact; the second is a
one-sample estimate of the rest of the sum (the tail), unbiased because y
is drawn from p_s: E_y[ [y not in S] f(y) ] = sum_{v not in S} p_s(v) f(v).
Its gradient with respect to the student logits z (S and the sample y held
fixed):

    g_hat_j = sum_{v in S} p_v (delta_vj - p_j)(f_v + 1)
              + [y not in S] (f_y + 1)(delta_yj - p_j),

the exact gradient of the first term plus the score-function estimate of
the tail's gradient, E_y[[y not in S] (f(y) grad log p_s(y) + grad f(y))] with
grad f(y) = grad log p_s(y) = e_y - p.  With S = the whole vocabulary the
tail term is absent and L_hat, g_hat are the reverse KL and its gradient
(the page's K = V limit); with S empty, L_hat = f(y) is the sampled token's
log-probability gap.  The teacher enters only through log p_t on S and at
y: a payload of K + 1 values per row instead of V.

The chain rule gives dh = g_hat W and dW = sum_rows g_hat^T h, as for the
full reverse KL.  Rows whose mask is 0 contribute nothing.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def log_softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return z - (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))


def estimator(lp_s: np.ndarray, lpt_S: np.ndarray, lpt_y: float, S: np.ndarray, y: int):
    """L_hat and g_hat (over the whole vocabulary) of one row, from the
    student's log-probabilities lp_s [V], the teacher's log-probabilities on
    the support lpt_S [K] and at the sampled token lpt_y, the support S [K]
    (distinct ids) and the sampled token y."""
    lp_s = np.asarray(lp_s, dtype=np.float64)
    S = np.asarray(S, dtype=np.int64)
    p = np.exp(lp_s)
    f_S = lp_s[S] - np.asarray(lpt_S, dtype=np.float64)
    L = float(np.sum(p[S] * f_S))
    g = np.zeros_like(p)
    # exact part: sum over the support of p_v (delta_vj - p_j)(f_v + 1)
    for v, fv in zip(S, f_S):
        w = p[v] * (fv + 1.0)
        g[v] += w
        g -= w * p
    # tail: one sample, score function
    if y not in set(S.tolist()):
        f_y = lp_s[y] - float(lpt_y)
        L += f_y
        g[y] += f_y + 1.0
        g -= (f_y + 1.0) * p
    return L, g


def forward_backward(h: np.ndarray, W: np.ndarray, y: np.ndarray, S: np.ndarray, lpt_S: np.ndarray,
                     lpt_y: np.ndarray, g: Optional[np.ndarray] = None, mask: Optional[np.ndarray] = None):
    """All rows of one problem: h [N, H], W [V, H] (float64 values), y [N],
    S [N, K], teacher log-probabilities lpt_S [N, K] and lpt_y [N], upstream
    gradients g [N] (default ones), row mask [N] (default all live).
    Returns dict L [N], dz [N, V], dh [N, H], dW [V, H]."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    N = h.shape[0]
    lp = log_softmax(h @ W.T)
    out = {"L": np.zeros(N), "dz": np.zeros(lp.shape)}
    for i in range(N):
        if mask is not None and mask[i] == 0:
            continue
        L, gz = estimator(lp[i], lpt_S[i], lpt_y[i], S[i], int(y[i]))
        out["L"][i] = L
        out["dz"][i] = gz * (1.0 if g is None else float(g[i]))
    out["dh"] = out["dz"] @ W
    out["dW"] = out["dz"].T @ h
    return out
