"""GPU parity of the routing diagnostics (kv_route_diagnostics) on a decode
loop: two sequences of the tiny shape, 120 steps appending a token each,
routing every 16 steps, beside a shadow pool that keeps every window in bf16
(never routed, fed the same tokens).

* Selection churn, cumulative promotions and demotions and Global LIR of each
  routing event: bit-exact against the oracle's diagnostics on the oracle's
  tier vectors before and after the event.
* Future missed mass of each step: against the oracle's reduction of the
  library's own shadow masses (1e-5: only the summation order differs) and
  against the oracle's shadow attention (the mass bar, summed over the
  evicted windows).
"""
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle.diagnostics import ReactivationCounter, future_missed_mass, selection_churn  # noqa: E402
from oracle.router import E  # noqa: E402
from tests.gpu_harness import MASS_TOL, Pair, log  # noqa: E402


def test_route_diagnostics_on_a_decode_loop():
    c = dataclasses.replace(CONFIGS["tiny"], name="diag", batch=2, steps=120, route_every=16, append=True)
    p, shadow = Pair(c), Pair(c)
    p.load(0)
    shadow.load(0)
    diag = torch.zeros(c.batch, 5, dtype=torch.float32, device="cuda")
    lir = {b: ReactivationCounter() for b in p.seqs}

    def routing_event():
        before = {b: list(p.oracle[(0, b)].tier) for b in p.seqs}
        p.route(0, c.budget_frac, c.hi_frac)
        p.check_state(0)
        p.pool.diagnostics(0, diag, counts=p.last_counts)
        d = diag.cpu().numpy()
        for b in p.seqs:
            after = p.oracle[(0, b)].tier
            lir[b].event(before[b], after)
            assert d[b][0] == selection_churn(before[b], after), (b, d[b][0])
            assert (d[b][1], d[b][2]) == (lir[b].reactivations, lir[b].departures), (b, d[b])
            assert d[b][3] == lir[b].lir, (b, d[b][3])
        return d

    d = routing_event()
    assert (d[:, 0] > 0).all() and (d[:, 2] > 0).all()
    worst = 0.0
    for s in range(c.steps):
        _, mass, o_mass, _ = p.step(0, s, append=True)
        _, smass, so_mass, _ = shadow.step(0, s, append=True)
        p.add_scores(0, mass, o_mass)
        p.pool.diagnostics(0, diag, shadow_mass=smass)
        d = diag.cpu().numpy()
        sm = smass.cpu().numpy()
        for b in p.seqs:
            tier = p.oracle[(0, b)].tier
            n_ev = sum(1 for t in tier if t == E)
            assert n_ev > 0
            assert abs(d[b][4] - future_missed_mass(sm[b], tier)) <= 1e-5, (s, b)
            want = future_missed_mass(so_mass[b], tier)
            assert abs(d[b][4] - want) <= MASS_TOL * n_ev, (s, b, d[b][4], want)
            worst = max(worst, abs(d[b][4] - want))
        if (s + 1) % c.route_every == 0:
            d = routing_event()
    log("diagnostics: churn %s, LIR %s, last missed mass %s, worst missed-mass error %.2e"
        % (d[:, 0].tolist(), d[:, 3].tolist(), d[:, 4].tolist(), worst))
    assert p.pool.check() == 0


def test_route_diagnostics_rejects_missing_inputs():
    from tiered_int2_fp16_amd.binding import KvError
    c = CONFIGS["tiny"]
    p = Pair(c)
    p.load(0)
    diag = torch.zeros(c.batch, 5, dtype=torch.float32, device="cuda")
    with pytest.raises(KvError):
        p.pool.diagnostics(0, diag)
