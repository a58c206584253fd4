"""Per-segment state machine of the three-tier window cache (oracle).

A segment is one (sequence, layer) pair: the unit the router ranks.  Each
window spans all kv heads of the layer.  The transitions follow the QEvict
summary ("Kernmechanismen", recoverable hierarchy):

* demote (full precision -> INT2, or the ledger's b bits): quantise the
  window's current bf16 values
  only if it has no ledger entry yet; the ledger entry is written once and
  kept ("Write-Once Quantization Ledger");
* promote (INT2 -> full precision): dequantise the ledger entry back into
  bf16; the ledger entry stays, so a later demotion reuses it and
  approximation error does not compound;
* evict: permanent; an evicted window never returns ("Methodologie: QEvict",
  evicted tier).

Scores are cumulative: S[w] += sum over the layer's query heads of the mass
window w receives at a step ("Kernmechanismen", cumulative scoring); they
start from a prior and are never reset.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import attention, codec, router
from .router import E, F, Q


class Segment:
    def __init__(self, kv_heads: int, window: int, head_dim: int, n_recent: int = 4,
                 bits: int = 2):
        codec.levels(bits)
        self.bits = bits                         # ledger code width (2, 4, 8)
        self.hkv = kv_heads
        self.W = window
        self.D = head_dim
        self.R = n_recent
        self.tokens = 0
        self.tier: List[int] = []
        self.k: Dict[int, np.ndarray] = {}       # bf16 bits [Hkv][W][D] of F windows
        self.v: Dict[int, np.ndarray] = {}
        self.ledger: Dict[int, List[dict]] = {}  # per kv head ledger entries
        self.quantized: List[int] = []           # quantisations per window
        self.S = np.zeros(0)

    # ------------------------------------------------------------ shape ---
    @property
    def n(self) -> int:
        return -(-self.tokens // self.W)

    def valid(self, w: int) -> int:
        return min(self.W, self.tokens - w * self.W)

    def _grow(self):
        while len(self.tier) < self.n:
            w = len(self.tier)
            self.tier.append(F)
            self.quantized.append(0)
            self.k[w] = np.zeros((self.hkv, self.W, self.D), np.uint16)
            self.v[w] = np.zeros((self.hkv, self.W, self.D), np.uint16)
        if self.S.size < self.n:
            self.S = np.concatenate([self.S, np.zeros(self.n - self.S.size)])

    # ------------------------------------------------------- populating ---
    def prefill(self, k_bits: np.ndarray, v_bits: np.ndarray, prior=None):
        """Cache a context: K, V bf16 bits [Hkv][T][D]; every window starts bf16."""
        assert self.tokens == 0
        t = k_bits.shape[1]
        self.tokens = t
        self._grow()
        for w in range(self.n):
            a, b = w * self.W, min(t, (w + 1) * self.W)
            self.k[w][:, : b - a] = k_bits[:, a:b]
            self.v[w][:, : b - a] = v_bits[:, a:b]
        if prior is not None:
            self.S[: len(prior)] = np.asarray(prior, dtype=np.float64)

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray):
        """Append one token (bf16 bits [Hkv][D]) to the newest window."""
        pos = self.tokens
        w = pos // self.W
        if w < len(self.tier) and self.tier[w] != F:
            raise ValueError("appending into a window that is not full precision")
        self.tokens += 1
        self._grow()
        self.k[w][:, pos % self.W] = k_bits
        self.v[w][:, pos % self.W] = v_bits

    # ------------------------------------------------------ transitions ---
    def demote(self, w: int):
        if self.tier[w] != F:
            raise ValueError(f"demote of window {w} in tier {self.tier[w]}")
        if self.valid(w) != self.W:
            raise ValueError("a partial window cannot be quantised")
        if w not in self.ledger:
            self.ledger[w] = [codec.quantize_window(self.k[w][h], self.v[w][h], self.bits)
                              for h in range(self.hkv)]
            self.quantized[w] += 1
        del self.k[w], self.v[w]
        self.tier[w] = Q

    def promote(self, w: int):
        if self.tier[w] != Q or w not in self.ledger:
            raise ValueError(f"promote of window {w} in tier {self.tier[w]}")
        ks, vs = zip(*[codec.promote_bits(e) for e in self.ledger[w]])
        self.k[w] = np.stack(ks)
        self.v[w] = np.stack(vs)
        self.tier[w] = F

    def evict(self, w: int):
        if self.tier[w] == E:
            return
        self.k.pop(w, None)
        self.v.pop(w, None)
        self.ledger.pop(w, None)
        self.tier[w] = E

    # -------------------------------------------------------- attention ---
    def window_kv(self, w: int) -> Optional[tuple]:
        """float64 K, V [Hkv][ntok][D] of window w, or None when evicted."""
        t = self.tier[w]
        nt = self.valid(w)
        if t == E:
            return None
        if t == F:
            return (codec.bf16_to_f64(self.k[w][:, :nt]), codec.bf16_to_f64(self.v[w][:, :nt]))
        kv = [codec.dequant_window_f64(e) for e in self.ledger[w]]
        return (np.stack([a for a, _ in kv])[:, :nt], np.stack([b for _, b in kv])[:, :nt])

    def attend(self, q_bits: np.ndarray):
        """out [Hq][D], mass [Hq][n] (float64) for query bf16 bits [Hq][D]."""
        return attention.attend(codec.bf16_to_f64(q_bits),
                                [self.window_kv(w) for w in range(self.n)])

    def add_scores(self, mass: np.ndarray):
        """S[w] += sum_h mass[h][w] over the windows that are not evicted."""
        m = np.asarray(mass, dtype=np.float64).sum(axis=0)[: self.n]
        live = np.array([t != E for t in self.tier])
        self.S[: self.n] += np.where(live, m, 0.0)

    # ---------------------------------------------------------- routing ---
    def counts(self, budget_frac: float, hi_frac: float):
        return router.tier_counts(self.n, self.R, budget_frac, hi_frac, self.bits)

    def route(self, budget_frac: float, hi_frac: float, scores=None) -> dict:
        """Route every window; apply demotions, promotions and evictions.

        ``scores`` overrides the segment's own S (e.g. an S array kept in
        float32 elsewhere) so the decision can be taken on identical values.
        """
        s = self.S if scores is None else scores
        n_hi, n_lo = self.counts(budget_frac, hi_frac)
        new = router.route(self.tier, s, self.R, n_hi, n_lo)
        tr = router.transitions(self.tier, new)
        tr["first_quant"] = [w for w in tr["demote"] if w not in self.ledger]
        for w in tr["demote"]:
            self.demote(w)
        for w in tr["promote"]:
            self.promote(w)
        for w in tr["evict"]:
            self.evict(w)
        assert self.tier == new
        return tr

    # ------------------------------------------------------------ views ---
    def bytes_used(self) -> int:
        """Tier bytes of the segment (bf16 windows + ledger windows), all heads."""
        f = sum(1 for t in self.tier if t == F)
        q = sum(1 for t in self.tier if t == Q)
        return self.hkv * (f * 4 * self.W * self.D + q * codec.entry_nbytes(self.W, self.D, self.bits))
