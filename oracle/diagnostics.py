"""Routing diagnostics of the window cache (oracle, test infrastructure).

The QEvict summary ("Kernbijdragen", item 1) introduces instruments that
characterise cache dynamics during decoding: Future Missed Mass, Global LIR
(latent importance reactivation) and selection churn.  The page describes each
in one sentence; the definitions below are the plainest readings of them for
the three-tier cache built here:

* selection churn of one routing event: the share of the windows that were
  live (not evicted) before the event whose tier the event changes
  (demotions, promotions and evictions over the live windows);
* Global LIR: how often windows that left the full-precision (active) set
  come back to it.  A window leaves it by a demotion and can only return by a
  promotion (an evicted window never returns), so over a run it is the number
  of promotions divided by the number of demotions (0 before any demotion);
* Future Missed Mass of one decode step: the attention that a cache keeping
  every window in full precision (a shadow cache) gives to windows the policy
  has already evicted, averaged over the query heads.

All three are functions of tier vectors and window masses; nothing here
touches K/V.  Ratios are returned as float32 quotients of exact integers (the
precision the device reports them in), the missed mass in float64.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .router import E, F, Q


def selection_churn(before: Sequence[int], after: Sequence[int]) -> np.float32:
    """Share of the windows live before a routing event whose tier changed.

    ``before`` and ``after`` are the tiers (E=0, Q=1, F=2) of the same windows
    just before and just after the event (windows opened since the previous
    event are live full-precision windows in ``before``).
    """
    if len(before) != len(after):
        raise ValueError("tier vectors of different lengths")
    live = [w for w, t in enumerate(before) if t != E]
    for w, t in enumerate(before):
        if t == E and after[w] != E:
            raise ValueError(f"window {w} came back from eviction")
    changed = sum(1 for w in live if after[w] != before[w])
    if not live:
        return np.float32(0.0)
    return np.float32(changed) / np.float32(len(live))


class ReactivationCounter:
    """Global LIR over a run of routing events of one segment."""

    def __init__(self):
        self.departures = 0      # full precision -> INT2
        self.reactivations = 0   # INT2 -> full precision

    def event(self, before: Sequence[int], after: Sequence[int]) -> None:
        for a, b in zip(before, after):
            if a == F and b == Q:
                self.departures += 1
            elif a == Q and b == F:
                self.reactivations += 1

    @property
    def lir(self) -> np.float32:
        if self.departures == 0:
            return np.float32(0.0)
        return np.float32(self.reactivations) / np.float32(self.departures)


def future_missed_mass(shadow_mass: np.ndarray, tier: Sequence[int]) -> float:
    """Mean over query heads of the shadow cache's mass on evicted windows.

    shadow_mass  [Hq][>= n] window masses of one decode step from a cache that
                 holds every window in full precision
    tier         the policy's tiers of the n windows at that step
    """
    m = np.asarray(shadow_mass, dtype=np.float64)
    ev = np.array([t == E for t in tier], dtype=bool)
    n = len(tier)
    return float(m[:, :n][:, ev].sum(axis=1).mean()) if ev.any() else 0.0
