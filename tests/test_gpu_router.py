"""The device router's tier counts where a fused multiply-add would change
them.

The counts are n_hi = min(n, max(R, floor(phi n))) and
n_lo = max(0, min(n - n_hi, floor((beta n - n_hi) 16 / (b + 1)))) with every
double operation rounded on its own.  If beta n - n_hi were one fused
multiply-add, beta n would not be rounded first, and for decimal fractions
such as 0.15 or 0.3 the result can land just below an integer that the
rounded product reaches exactly: n_lo one smaller.  The cases below are found
on the host by comparing both evaluations in exact rational arithmetic; each
becomes a layer of a pool (one layer per case, every window bf16 after the
prefill), and one routing event per layer must produce the oracle's counts.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle.router import tier_counts

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_harness import dev, log  # noqa: E402

R = 4


def _fused_counts(n, beta, phi, bits):
    hi = min(n, max(R, math.floor(phi * n)))
    x = float(Fraction(beta) * n - hi)          # beta * n - hi rounded once
    return hi, max(0, min(n - hi, math.floor(x * 16.0 / (bits + 1))))


def _boundary_cases(bits, limit):
    out = []
    for beta in (0.15, 0.2, 0.3, 0.35, 0.45, 0.6, 0.7, 0.9):
        for phi in (0.02, 0.1, 0.2, 0.0625):
            for n in range(5, 700):
                if tier_counts(n, R, beta, phi, bits) != _fused_counts(n, beta, phi, bits):
                    out.append((n, beta, phi))
                    break
    return out[:limit]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_router_counts_where_contraction_would_differ(bits):
    from tiered_int2_fp16_amd import binding as B
    cases = _boundary_cases(bits, 12)
    assert cases, "no boundary case in the search range"
    maxw = max(n for n, _, _ in cases)
    W, D = 32, 64
    cfg = B.make_config(1, len(cases), 1, 1, D, W, maxw, R, maxw, maxw, bits)
    pool = B.Pool(cfg)
    rng = np.random.default_rng(bits)
    for layer, (n, beta, phi) in enumerate(cases):
        kv = torch.zeros(1, 1, n * W, D, dtype=torch.int16, device="cuda")
        prior = dev(rng.lognormal(0.0, 1.0, (1, n)).astype(np.float32))
        pool.prefill(layer, kv, kv, n * W, prior)
        _, cnt = pool.score_route(layer, None, 1, beta, phi)
        hi, lo = tier_counts(n, R, beta, phi, bits)
        got = cnt.cpu().numpy()[:, 0].tolist()
        assert got == [lo, 0, n - hi - lo, lo], (n, beta, phi, bits, got, (hi, lo),
                                                 _fused_counts(n, beta, phi, bits))
        assert B.kv_tier_counts(n, R, beta, phi, bits) == (hi, lo)
    assert pool.check() == 0
    log(f"{bits}-bit ledger: {len(cases)} routing events at counts a fused multiply-add would change")
