"""Seeded synthetic inputs for the fused LM-head reverse-KL path.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no projection, softmax, divergence or gradient), so
that both the fp64 oracle and the HIP library can be fed from it without
sharing any computation.

Recipe (shapes and distributions follow the workloads described on the
NeMo-RL full-vocabulary on-policy distillation page -- a 2k-hidden / 152k-vocab
Qwen3-1.7B-shaped model -- and on the slime compact-actor-logits page -- long
masked prompts where only the response rows are trainable):

* every tensor is drawn from its own PCG64 stream, keyed by (seed, tensor id),
  in fp32, then rounded to bf16 with round-to-nearest-even; bf16 tensors are
  returned as raw uint16 bit patterns, fp32 tensors as float32 arrays;
* hidden states: i.i.d. N(0, 1) per element, optionally rescaled so that each
  row has root-mean-square 1 (the output of an RMS norm);
* LM-head weights: i.i.d. N(0, sigma^2), row-major [V, H];
* logits (when a side is handed over as logits): i.i.d. N(0, sigma^2) fp32;
* loss masks: uint8 [T], 1 = trainable position, laid out as [B, S-1].

No public dataset or checkpoint is used: these arrays stand in for the
Qwen3-1.7B checkpoint and the SFT data named on the pages.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids for the sub-streams
_HS, _HT, _WS, _WT, _ZS, _ZT, _MASK, _PERT, _G, _Y, _GH = range(11)

_ROW_CHUNK = 4096


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(seed: int, tid: int, rows: int, cols: int, sigma: float,
                 rms_rows: bool = False) -> np.ndarray:
    """[rows, cols] bf16 bits of N(0, sigma^2); optionally each row set to RMS 1."""
    g = _rng(seed, tid)
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _ROW_CHUNK):
        r1 = min(rows, r0 + _ROW_CHUNK)
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if rms_rows:
            x /= np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)).astype(np.float32)
        elif sigma != 1.0:
            x *= np.float32(sigma)
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def _normal_f32(seed: int, tid: int, rows: int, cols: int, sigma: float) -> np.ndarray:
    g = _rng(seed, tid)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(sigma)
    return x


@dataclass
class Case:
    """One workload: inputs over all T = B*(S-1) positions plus the loss mask.

    bf16 tensors are uint16 bit arrays.  ``Ht == 0`` means the teacher is
    handed over as fp32 logits ``z_t``; ``Hs == 0`` means the student is handed
    over as fp32 logits ``z_s`` as well.
    """
    name: str
    B: int
    S: int
    V: int
    Hs: int
    Ht: int
    mask: np.ndarray                      # uint8 [T]
    h_s: Optional[np.ndarray] = None      # bf16 [T, Hs]
    W_s: Optional[np.ndarray] = None      # bf16 [V, Hs]
    h_t: Optional[np.ndarray] = None      # bf16 [T, Ht]
    W_t: Optional[np.ndarray] = None      # bf16 [V, Ht]
    z_s: Optional[np.ndarray] = None      # fp32 [T, V]
    z_t: Optional[np.ndarray] = None      # fp32 [T, V]
    grad: Optional[np.ndarray] = None     # fp32 [T] upstream dL (None = ones)
    notes: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.B * (self.S - 1)


def _span_mask(B: int, Sm1: int, starts) -> np.ndarray:
    m = np.zeros((B, Sm1), dtype=np.uint8)
    for b, s in enumerate(starts):
        m[b, s:] = 1
    return m.reshape(-1)


def logits_tiny(seed: int = 1, T: int = 64, V: int = 1024, sigma: float = 2.0,
                p_mask: float = 0.7) -> Case:
    """Both sides handed over as fp32 logits, N(0, sigma^2); Bernoulli(p) mask."""
    mask = (_rng(seed, _MASK).random(T) < p_mask).astype(np.uint8)
    return Case("logits_tiny", 1, T + 1, V, 0, 0, mask,
                z_s=_normal_f32(seed, _ZS, T, V, sigma),
                z_t=_normal_f32(seed, _ZT, T, V, sigma))


def hidden_small(seed: int = 2, B: int = 2, S: int = 129, H: int = 256, V: int = 8192) -> Case:
    """Hidden-state path; each sequence's response span starts at a random offset."""
    Sm1 = S - 1
    starts = _rng(seed, _MASK).integers(0, Sm1, size=B)
    T = B * Sm1
    return Case("hidden_small", B, S, V, H, H, _span_mask(B, Sm1, starts),
                h_s=_normal_bf16(seed, _HS, T, H, 1.0),
                W_s=_normal_bf16(seed, _WS, V, H, 1.0 / np.sqrt(H)),
                h_t=_normal_bf16(seed, _HT, T, H, 1.0),
                W_t=_normal_bf16(seed, _WT, V, H, 1.0 / np.sqrt(H)))


def qwen_shaped(seed: int = 3, B: int = 4, S: int = 1025, Hs: int = 2048, Ht: int = 2048,
                V: int = 151936, response: Optional[int] = 512, wsigma: float = 0.02) -> Case:
    """Qwen3-1.7B-shaped hidden-state path: RMS-1 hidden rows, N(0, 0.02^2) weights.

    ``response`` = number of trailing loss-masked positions per sequence
    (None = every position is trainable).
    """
    Sm1 = S - 1
    T = B * Sm1
    starts = [0 if response is None else Sm1 - response] * B
    return Case(f"qwen_B{B}_S{S}_Hs{Hs}_Ht{Ht}_V{V}", B, S, V, Hs, Ht, _span_mask(B, Sm1, starts),
                h_s=_normal_bf16(seed, _HS, T, Hs, 1.0, rms_rows=True),
                W_s=_normal_bf16(seed, _WS, V, Hs, wsigma),
                h_t=_normal_bf16(seed, _HT, T, Ht, 1.0, rms_rows=True),
                W_t=_normal_bf16(seed, _WT, V, Ht, wsigma))


def self_distill(seed: int = 4, B: int = 8, S: int = 1025, H: int = 2048, V: int = 151936,
                 perturb: float = 0.0) -> Case:
    """Teacher hidden states and weights bit-identical to the student's.

    With ``perturb > 0`` the teacher weight is bf16(W + N(0, perturb^2)) instead
    (the fp32 sum of the student's bf16 value and the noise, rounded once).
    """
    Sm1 = S - 1
    T = B * Sm1
    h = _normal_bf16(seed, _HS, T, H, 1.0, rms_rows=True)
    W = _normal_bf16(seed, _WS, V, H, 0.02)
    if perturb > 0.0:
        g = _rng(seed, _PERT)
        Wt = np.empty_like(W)
        for r0 in range(0, V, _ROW_CHUNK):
            r1 = min(V, r0 + _ROW_CHUNK)
            w32 = (W[r0:r1].astype(np.uint32) << np.uint32(16)).view(np.float32)
            w32 = w32 + np.float32(perturb) * g.standard_normal((r1 - r0, H), dtype=np.float32)
            Wt[r0:r1] = f32_to_bf16_bits(w32)
    else:
        Wt = W
    return Case(f"selfdistill_p{perturb:g}", B, S, V, H, H, np.ones(T, dtype=np.uint8),
                h_s=h, W_s=W, h_t=h, W_t=Wt)


def random_case(seed: int, T: int, V: int, Hs: int, Ht: int, p_mask: float = 0.5,
                student_logits: bool = False, teacher_logits: bool = False,
                logit_sigma: float = 2.0, with_grad: bool = False) -> Case:
    """Ragged small case for parity: Bernoulli mask, N(0, 1/H) weights, N(0,1) hidden."""
    mask = (_rng(seed, _MASK).random(T) < p_mask).astype(np.uint8)
    c = Case(f"random_T{T}_V{V}_Hs{Hs}_Ht{Ht}", 1, T + 1, V,
             0 if student_logits else Hs, 0 if teacher_logits else Ht, mask)
    if student_logits:
        c.z_s = _normal_f32(seed, _ZS, T, V, logit_sigma)
    else:
        c.h_s = _normal_bf16(seed, _HS, T, Hs, 1.0)
        c.W_s = _normal_bf16(seed, _WS, V, Hs, 1.0 / np.sqrt(Hs))
    if teacher_logits:
        c.z_t = _normal_f32(seed, _ZT, T, V, logit_sigma)
    else:
        c.h_t = _normal_bf16(seed, _HT, T, Ht, 1.0)
        c.W_t = _normal_bf16(seed, _WT, V, Ht, 1.0 / np.sqrt(Ht))
    if with_grad:
        c.grad = _rng(seed, _G).uniform(0.5, 1.5, size=T).astype(np.float32)
    return c


# The five workloads (and the headline shape) by name.
def config(name: str) -> Case:
    if name == "c1":
        return logits_tiny()
    if name == "c2":
        return hidden_small()
    if name == "c3":
        return qwen_shaped()
    if name == "headline":           # the c3 tensors, every position trainable
        return qwen_shaped(response=None)
    if name == "c4a":
        return self_distill()
    if name == "c4b":
        return self_distill(perturb=1e-3)
    if name == "c5":
        return qwen_shaped(seed=5, B=2, S=16385, Hs=2048, Ht=4096, response=2048)
    raise KeyError(name)


# ------------------------------------------------- log-probability / entropy

def sampled_tokens(seed: int, T: int, V: int) -> np.ndarray:
    """int32 [T] token ids, uniform on [0, V): stands in for the tokens a
    policy sampled (any id is a valid input; uniform ids reach every
    vocabulary tile, the ragged last one included)."""
    return _rng(seed, _Y).integers(0, V, size=T, dtype=np.int64).astype(np.int32)


def upstream_grads(seed: int, T: int):
    """(g_logp, g_entropy) fp32 [T] each: per-token upstream gradients of the
    log-probability and of the entropy, N(0, 1) and U(-0.1, 0.1) (an entropy
    bonus is a small coefficient)."""
    g = _rng(seed, _G).standard_normal(T).astype(np.float32)
    gh = _rng(seed, _GH).uniform(-0.1, 0.1, size=T).astype(np.float32)
    return g, gh


# ------------------------------------------------- teacher chosen per row

def teacher_weights(seed: int, K: int, V: int, Ht: int, sigma: float = 0.02) -> np.ndarray:
    """[K, V, Ht] bf16 bits: K independent output-layer weights N(0, sigma^2)."""
    return np.stack([_normal_bf16(seed, 16 + k, V, Ht, sigma) for k in range(K)])


def teacher_ids(seed: int, T: int, K: int, order: str = "grouped") -> np.ndarray:
    """int32 [T] teacher id per row: `grouped` gives K contiguous runs of about
    T/K rows (a batch assembled per teacher), `interleaved` i.i.d. uniform ids
    (every 128-row tile then holds several teachers)."""
    if order == "grouped":
        return (np.arange(T, dtype=np.int64) * K // max(T, 1)).astype(np.int32)
    return _rng(seed, 15).integers(0, K, size=T, dtype=np.int64).astype(np.int32)
