"""Pins of the oracle's routing diagnostics (selection churn, Global LIR,
future missed mass) against a hand-worked example, the router's own
transition lists, a repeated-routing fixed point and a token-level softmax
computed here by brute force (CPU)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, codec, router
from oracle.diagnostics import ReactivationCounter, future_missed_mass, selection_churn
from oracle.pool import Segment
from oracle.router import E, F, Q


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "routing_diagnostics.json")))
    lir = ReactivationCounter()
    for ev in g["events"]:
        c = selection_churn(ev["before"], ev["after"])
        if "churn" in ev:
            assert c == np.float32(ev["churn"])
        else:
            assert c == np.float32(ev["churn_num"]) / np.float32(ev["churn_den"])
        lir.event(ev["before"], ev["after"])
        assert (lir.departures, lir.reactivations) == (ev["departures"], ev["reactivations"])
        assert lir.lir == np.float32(ev["lir"])
    mm = g["missed_mass"]
    assert future_missed_mass(np.array(mm["shadow_mass"]), mm["tier"]) == pytest.approx(mm["fmm"], abs=1e-15)


def test_churn_counts_the_routers_transition_lists():
    """Churn from tier vectors equals (demote + promote + evict) / live from the
    router's own transition lists, over random routing events."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        before = [int(x) for x in rng.choice([E, Q, F], size=n, p=[0.3, 0.4, 0.3])]
        scores = rng.lognormal(size=n)
        n_hi, n_lo = router.tier_counts(n, 4, float(rng.uniform(0, 1)), float(rng.uniform(0, 0.5)))
        after = router.route(before, scores, 4, n_hi, n_lo)
        tr = router.transitions(before, after)
        live = sum(1 for t in before if t != E)
        want = np.float32(len(tr["demote"]) + len(tr["promote"]) + len(tr["evict"])) / np.float32(live) \
            if live else np.float32(0)
        assert selection_churn(before, after) == want


def test_churn_is_zero_when_scores_do_not_move():
    """Routing twice on the same scores reaches a fixed point: the second event
    changes nothing (the top ranks stay, the rest was evicted by the first)."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(5, 60))
        s = rng.lognormal(size=n)
        n_hi, n_lo = router.tier_counts(n, 4, 0.3, 0.1)
        t1 = router.route([F] * n, s, 4, n_hi, n_lo)
        t2 = router.route(t1, s, 4, n_hi, n_lo)
        assert t2 == t1
        assert selection_churn(t1, t2) == 0


def test_lir_follows_a_window_out_and_back():
    """12 windows, 4 recent: 2 of the 8 older ones stay bf16, 5 go INT2, 1 is
    evicted.  Scores 12..1 by index; then window 0's score drops to the bottom,
    rises to the top, drops again.  Worked by hand: event 1 demotes 2..6 (5
    departures) and evicts 7; each later event swaps windows 0 and 2 between
    the tiers (one departure and one reactivation each): 8 departures, 3
    reactivations."""
    n, R = 12, 4
    n_hi, n_lo = router.tier_counts(n, R, 0.59, 0.5)
    assert (n_hi, n_lo) == (6, 5)
    s = np.arange(n, 0, -1, dtype=np.float64)
    lir = ReactivationCounter()
    tier = [F] * n
    seq = []
    for bump in (None, -100.0, +200.0, -300.0):
        if bump is not None:
            s[0] += bump
        new = router.route(tier, s, R, n_hi, n_lo)
        lir.event(tier, new)
        seq.append((new[0], new[2]))
        tier = new
    assert seq == [(F, Q), (Q, F), (F, Q), (Q, F)]
    assert tier[7] == E
    assert (lir.departures, lir.reactivations) == (8, 3)
    assert lir.lir == np.float32(3) / np.float32(8)


def _brute_missed_mass(q, ks, tier, g):
    """Mean over heads of the softmax probability of tokens in evicted windows,
    computed over all tokens at once (no windowed bookkeeping)."""
    hq, d = q.shape
    toks = np.concatenate(ks, axis=1)                 # [Hkv][T][D]
    owner = np.concatenate([np.full(k.shape[1], w) for w, k in enumerate(ks)])
    ev = np.array([tier[w] == E for w in owner])
    tot = 0.0
    for h in range(hq):
        z = toks[h // g] @ q[h] / math.sqrt(d)
        p = np.exp(z - z.max())
        p /= p.sum()
        tot += p[ev].sum()
    return tot / hq


def test_missed_mass_matches_a_token_softmax():
    rng = np.random.default_rng(11)
    hq, hkv, d, wsz = 4, 2, 16, 8
    n = 9
    q = rng.standard_normal((hq, d))
    ks = [rng.standard_normal((hkv, wsz if w < n - 1 else 3, d)) * 1.5 for w in range(n)]
    vs = [rng.standard_normal(k.shape) for k in ks]
    _, shadow = attention.attend(q, list(zip(ks, vs)))
    for tier in ([F] * n, [E, Q, E, F, Q, E, E, F, F], [E] * (n - 1) + [F]):
        fmm = future_missed_mass(shadow, tier)
        assert fmm == pytest.approx(_brute_missed_mass(q, ks, tier, hq // hkv), abs=1e-12)
        live = [w for w in range(n) if tier[w] != E]
        assert fmm == pytest.approx(1.0 - shadow[:, live].sum(axis=1).mean(), abs=1e-12)
    assert future_missed_mass(shadow, [F] * n) == 0.0
