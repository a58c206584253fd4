"""Pins of the oracle's tier counts, router and ledger state machine (CPU)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import codec, router
from oracle.pool import Segment
from oracle.router import E, F, Q


def test_counts_match_workload_descriptions(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tier_counts.json")))
    for c in g["cases"]:
        n_hi, n_lo = router.tier_counts(c["n"], 4, c["budget"], c["hi"])
        assert (n_hi, n_lo, c["n"] - n_hi - n_lo) == (c["n_hi"], c["n_lo"], c["n_ev"]), c["name"]
        frac = (n_hi + n_lo * 3 / 16) / c["n"]
        assert frac <= c["budget"] + 1e-12
        if "percent_bytes" in c:
            assert round(100 * frac, 2) == pytest.approx(c["percent_bytes"], abs=0.006)
        if "percent_int2" in c:
            assert round(100 * n_lo / c["n"], 1) == c["percent_int2"]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_counts_fill_the_byte_budget(bits):
    """The counts spend the budget: bf16 windows cost 16 bits per value,
    ledger windows b + 1 (codes plus fp16 scale and min per 32 values); the
    tiers fit the budget and one more ledger window would not, unless every
    window is already kept."""
    rng = np.random.default_rng(12)
    for _ in range(3000):
        n = int(rng.integers(1, 1200))
        beta = float(rng.uniform(0.01, 0.6))
        phi = float(rng.uniform(0.0, beta))
        n_hi, n_lo = router.tier_counts(n, 4, beta, phi, bits)
        assert n_hi == min(n, max(4, int(np.floor(phi * n))))
        cost = lambda f, q: 16 * f + (bits + 1) * q
        if n_lo > 0:
            assert cost(n_hi, n_lo) <= 16 * beta * n * (1 + 1e-12)
        if n_hi + n_lo < n and cost(n_hi, 0) <= 16 * beta * n:
            assert cost(n_hi, n_lo + 1) > 16 * beta * n * (1 - 1e-12)


def test_counts_wider_ledgers_on_the_llama_32k_shape():
    # 256 windows, 20 % budget, 10 % bf16: 25 bf16 windows, then what the
    # remaining 26.2 window-budgets buy at 3, 5 and 9 bits per value
    assert router.tier_counts(256, 4, 0.2, 0.1, 2) == (25, 139)   # floor(26.2 * 16 / 3)
    assert router.tier_counts(256, 4, 0.2, 0.1, 4) == (25, 83)    # floor(26.2 * 16 / 5)
    assert router.tier_counts(256, 4, 0.2, 0.1, 8) == (25, 46)    # floor(26.2 * 16 / 9)
    with pytest.raises(ValueError):
        router.tier_counts(256, 4, 0.2, 0.1, 3)


def test_counts_edge_cases():
    assert router.tier_counts(3, 4, 0.2, 0.1) == (3, 0)          # fewer windows than R
    assert router.tier_counts(10, 4, 0.1, 0.1) == (4, 0)          # budget below the recent tail
    assert router.tier_counts(100, 4, 1.0, 1.0) == (100, 0)       # everything bf16
    assert router.tier_counts(100, 4, 1.0, 0.0) == (4, 96)        # rest fits as INT2


def _brute(tier, s, R, n_hi, n_lo):
    """Best assignment by exhaustive search: maximise the score mass kept in
    bf16, then the mass kept in INT2, then prefer older windows."""
    n = len(tier)
    fr = max(0, n - R)
    elig = [w for w in range(fr) if tier[w] != E]
    nf = max(0, n_hi - (n - fr))
    nf_e = min(nf, len(elig))
    nq_e = min(n_lo, len(elig) - nf_e)
    best = None
    for fset in itertools.combinations(elig, nf_e):
        rest = [w for w in elig if w not in fset]
        for qset in itertools.combinations(rest, nq_e):
            key = (sum(s[w] for w in fset), sum(s[w] for w in qset),
                   [-w for w in sorted(fset)], [-w for w in sorted(qset)])
            if best is None or key > best[0]:
                best = (key, fset, qset)
    new = list(tier)
    for w in range(fr, n):
        if tier[w] != E:
            new[w] = F
    for w in elig:
        new[w] = F if w in best[1] else (Q if w in best[2] else E)
    return new


@pytest.mark.parametrize("seed", range(40))
def test_router_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(5, 13))
    tier = [int(t) for t in rng.choice([E, Q, F, F], n)]
    s = list(rng.permutation(n).astype(float) + rng.random(n))   # distinct scores
    n_hi = int(rng.integers(4, n + 1))
    n_lo = int(rng.integers(0, n - n_hi + 1))
    assert router.route(tier, s, 4, n_hi, n_lo) == _brute(tier, s, 4, n_hi, n_lo)


def test_tie_break_prefers_older_window():
    tier = [F] * 10
    s = [1.0] * 10
    new = router.route(tier, s, 4, 6, 2)        # 2 bf16 + 2 INT2 among windows 0..5
    assert new == [F, F, Q, Q, E, E, F, F, F, F]


def test_evicted_never_return_and_recent_stay_bf16():
    tier = [E, F, Q, E, F, Q, F, F, Q, F]
    s = [100.0, 1, 2, 50.0, 3, 4, 0, 0, 0, 0]
    new = router.route(tier, s, 4, 6, 3)
    assert new[0] == E and new[3] == E
    assert new[6:] == [F] * 4
    tr = router.transitions(tier, new)
    assert 8 in tr["promote"]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_route_respects_budget_and_counts(bits):
    rng = np.random.default_rng(200)
    seg = Segment(1, 64, 64, 4, bits=bits)
    k = (rng.standard_normal((1, 64 * 40, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    seg.prefill(k, k, prior=rng.lognormal(0, 1, 40))
    tr = seg.route(0.2, 0.1)
    n_hi, n_lo = router.tier_counts(40, 4, 0.2, 0.1, bits)
    assert seg.tier.count(F) == n_hi and seg.tier.count(Q) == n_lo
    assert len(tr["first_quant"]) == n_lo and tr["evict"]
    full = 40 * 4 * 64 * 64
    assert seg.bytes_used() <= 0.2 * full


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_write_once_ledger(bits):
    """demote -> promote -> demote: the ledger bytes stay identical and the
    window is quantised exactly once; the promoted bf16 is the ledger's
    dequantisation, not the original."""
    rng = np.random.default_rng(201)
    seg = Segment(2, 64, 64, 4, bits=bits)
    k = (rng.standard_normal((2, 64 * 8, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    v = (rng.standard_normal((2, 64 * 8, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    seg.prefill(k, v)
    seg.demote(1)
    first = [codec.entry_bytes(e, bits) for e in seg.ledger[1]]
    assert len(first[0]) == codec.entry_nbytes(64, 64, bits)
    seg.promote(1)
    assert seg.tier[1] == F
    pk, pv = codec.promote_bits(seg.ledger[1][0])
    assert np.array_equal(seg.k[1][0], pk) and np.array_equal(seg.v[1][0], pv)
    assert not np.array_equal(seg.k[1][0], k[0, 64:128])
    seg.demote(1)
    assert [codec.entry_bytes(e, bits) for e in seg.ledger[1]] == first
    assert seg.quantized[1] == 1
    seg.evict(1)
    assert 1 not in seg.ledger and seg.tier[1] == E


def test_invalid_transitions_raise():
    rng = np.random.default_rng(202)
    seg = Segment(1, 64, 64, 4)
    k = (rng.standard_normal((1, 64 * 3 + 10, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    seg.prefill(k, k)
    with pytest.raises(ValueError):
        seg.promote(0)                 # no ledger entry
    with pytest.raises(ValueError):
        seg.demote(3)                  # partial window
    seg.demote(0)
    with pytest.raises(ValueError):
        seg.demote(0)                  # already INT2


def test_scores_accumulate_only_live_windows():
    seg = Segment(1, 64, 64, 4)
    seg.prefill(np.zeros((1, 64 * 5, 64), np.uint16), np.zeros((1, 64 * 5, 64), np.uint16),
                prior=[1, 2, 3, 4, 5])
    seg.evict(0)
    seg.add_scores(np.array([[0.5, 0.1, 0.1, 0.2, 0.1], [0.5, 0.2, 0.2, 0.0, 0.1]]))
    assert np.allclose(seg.S, [1, 2.3, 3.3, 4.2, 5.2])
