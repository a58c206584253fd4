"""Initial window scores from the prefill attention (oracle, test infrastructure).

The RDKV summary ("Technische Samenvatting: RDKV", 2.1 Theoretische
Formulering) weighs each cached token by the attention it receives from all
query positions, w_t = sum over tau of a_{tau,t}, and (2.2, phase 1) computes
these weights once after the prefill with the full, uncompressed cache.  Here
they seed QEvict's cumulative window scores ("Technische Samenvatting:
QEvict", Kernmechanismen, cumulative scoring) in place of a random prior:

    S[w] = sum over query heads h, over tokens t of window w, of w_t^(h),
    w_t^(h) = sum over tau >= t of a^(h)_{tau,t},

with a^(h) the causal softmax attention of the prefill: query tau attends to
keys 0..tau, logits q_tau . k_t / sqrt(D), query head h reading kv head
h // G.  Readings: the prefill is causal (a decoder's prefill); the heads of a
layer add up as the decode-time scores do.  Float64 throughout.
"""
from __future__ import annotations

import math

import numpy as np


def token_weights(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """w [Hq][T]: column sums of each query head's causal attention.

    q  [Hq][T][D] prefill queries, k [Hkv][T][D] keys (float64 values).
    """
    hq, t, d = q.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    g = hq // hkv
    scale = 1.0 / math.sqrt(d)
    causal = np.tril(np.ones((t, t), dtype=bool))        # [tau][t]: t <= tau
    w = np.zeros((hq, t))
    for h in range(hq):
        z = (q[h] @ k[h // g].T) * scale                 # [tau][t]
        z = np.where(causal, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        w[h] = p.sum(axis=0)
    return w


def window_scores(w: np.ndarray, window: int) -> np.ndarray:
    """S [n]: the token weights of every head summed over each window's tokens."""
    hq, t = w.shape
    n = -(-t // window)
    per_token = w.sum(axis=0)
    return np.array([per_token[i * window: (i + 1) * window].sum() for i in range(n)])


def head_token_weights(q: np.ndarray, k: np.ndarray, block: int = 1024) -> np.ndarray:
    """w [T] of one query head: q [T][D] its prefill queries, k [T][D] the keys
    of its kv head (float64 values).

    The same column sums as token_weights, w_t = sum over tau >= t of a_{tau,t},
    taken over blocks of `block` query rows: every row's causal softmax lies
    wholly inside its block, and the blocks' column sums are added, so a long
    prefill (32K tokens: a 32K x 32K attention matrix per head) fits in memory.
    """
    t, d = q.shape
    scale = 1.0 / math.sqrt(d)
    w = np.zeros(t)
    for r0 in range(0, t, block):
        r1 = min(t, r0 + block)
        z = (q[r0:r1] @ k[:r1].T) * scale                 # rows tau in [r0, r1), keys 0..r1-1
        causal = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]
        z = np.where(causal, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        w[:r1] += p.sum(axis=0)
    return w
