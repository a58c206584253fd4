"""Tiered decode attention with per-window mass (oracle, test infrastructure).

What one decode step computes for one sequence (QEvict summary,
"Methodologie: QEvict" and "Kernmechanismen"):

* windows in the full-precision tier attend with their bf16 K/V values;
* windows in the recoverable INT2 tier stay visible to attention, with K/V
  taken from their ledger entry (dequantised exactly: c*s + m);
* evicted windows take no part: the softmax normaliser runs over the tokens
  that remain (the LogQuant summary, "Kwantisatie versus Verwijdering", notes
  that eviction changes the softmax normalisation, which is what this does);
* grouped-query attention: query head h reads kv head h // G
  ("Implementatie" bullet: GQA support);
* the mass of window w for head h is the softmax probability summed over the
  window's tokens: the per-step attention a window receives, which the
  cumulative scoring of "Kernmechanismen" adds up over time.

The order of tokens does not matter (A.V = A_P.V_P, LogQuant summary,
"Positie-agnostische optimalisatie").  Everything here is float64.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

from .codec import bf16_to_f64


def attend(q: np.ndarray,
           windows: List[Optional[Tuple[np.ndarray, np.ndarray]]]):
    """One decode step for one sequence.

    q        float64 [Hq][D] (the bf16 query, converted exactly)
    windows  per window either None (evicted) or (K, V), float64 arrays of
             shape [Hkv][ntok][D] holding the window's valid tokens.
    Returns (out float64 [Hq][D], mass float64 [Hq][n_windows]).
    """
    hq, d = q.shape
    live = [(w, kv) for w, kv in enumerate(windows) if kv is not None]
    n = len(windows)
    if not live:
        raise ValueError("no attendable window")
    hkv = live[0][1][0].shape[0]
    if hq % hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    g = hq // hkv
    k_all = np.concatenate([kv[0] for _, kv in live], axis=1)        # [Hkv][T][D]
    v_all = np.concatenate([kv[1] for _, kv in live], axis=1)
    owner = np.concatenate([np.full(kv[0].shape[1], w) for w, kv in live])
    out = np.zeros((hq, d))
    mass = np.zeros((hq, n))
    scale = 1.0 / math.sqrt(d)
    for h in range(hq):
        kvh = h // g
        z = (k_all[kvh] @ q[h]) * scale
        p = np.exp(z - z.max())
        p /= p.sum()
        out[h] = p @ v_all[kvh]
        mass[h] = np.bincount(owner, weights=p, minlength=n)
    return out, mass


def query_f64(q_bits: np.ndarray) -> np.ndarray:
    return bf16_to_f64(q_bits)
