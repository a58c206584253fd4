"""Byte-budget tier counts and the score-ranked window router (oracle).

QEvict routes whole windows between three states within a fixed memory
budget: high-confidence windows stay full precision, intermediate ones go to
the recoverable INT2 tier, only the lowest are evicted, for good
("Methodologie: QEvict"; "Kernbijdragen" item 2: a byte-constrained
hierarchy).  Window confidence is the cumulative attention score
("Kernmechanismen").

Readings where the pages are silent:

* the most recent R windows always stay full precision;
* counts from the byte budget beta (fraction of the full bf16 KV) and the
  full-precision fraction phi, with n windows and a b-bit ledger:
      n_hi = min(n, max(R, floor(phi * n)))
      n_lo = max(0, min(n - n_hi, floor((beta * n - n_hi) * 16 / (b + 1))))
  16/(b + 1) is bf16 bytes over ledger bytes of one window: 16 bits per
  value against b-bit codes plus an fp16 scale and min per 32 values (one
  more bit per value); 16/3 for INT2.  The expression is evaluated in IEEE
  double in exactly this order;
* ranking key: score descending, ties to the lower (older) window index;
* an evicted window is never eligible again.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

E, Q, F = 0, 1, 2


def tier_counts(n: int, n_recent: int, budget_frac: float, hi_frac: float,
                bits: int = 2) -> Tuple[int, int]:
    """(n_hi, n_lo) for a segment of n windows and a ledger of `bits`-bit codes."""
    if bits not in (2, 4, 8):
        raise ValueError(f"ledger bit width {bits} is not one of 2, 4, 8")
    n_hi = min(n, max(n_recent, math.floor(hi_frac * n)))
    lo = math.floor((budget_frac * n - n_hi) * 16.0 / float(bits + 1))
    n_lo = max(0, min(n - n_hi, lo))
    return n_hi, n_lo


def route(tier: Sequence[int], scores: Sequence[float], n_recent: int,
          n_hi: int, n_lo: int) -> List[int]:
    """New tier of every window of one segment.

    tier    current tiers (E=0, Q=1, F=2) of the n windows
    scores  cumulative scores, compared exactly as given
    """
    n = len(tier)
    new = list(tier)
    first_recent = max(0, n - n_recent)
    for w in range(first_recent, n):
        if tier[w] != E:
            new[w] = F
    elig = [w for w in range(first_recent) if tier[w] != E]
    ranked = sorted(elig, key=lambda w: (-float(scores[w]), w))
    n_f = max(0, n_hi - (n - first_recent))
    for r, w in enumerate(ranked):
        new[w] = F if r < n_f else (Q if r < n_f + n_lo else E)
    return new


def transitions(old: Sequence[int], new: Sequence[int]) -> Dict[str, List[int]]:
    """Window lists per transition kind, ascending window order."""
    out = {"demote": [], "promote": [], "evict": []}
    for w, (a, b) in enumerate(zip(old, new)):
        if a == F and b == Q:
            out["demote"].append(w)
        elif a == Q and b == F:
            out["promote"].append(w)
        elif a != E and b == E:
            out["evict"].append(w)
    return out
