"""Plain CPU oracle of window-tiered decode attention (TEST INFRASTRUCTURE).

This package is the reference the HIP library is checked against.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the product path never does and shares no code with it.

It follows the QEvict technical summary ("Technische Samenvatting: QEvict",
gist.science paper 2608.05326; the Chinese page of the same paper says the
same): windows of consecutive tokens are routed between a full-precision tier,
a recoverable INT2 tier backed by a write-once quantisation ledger, and an
evicted tier, under a byte budget, by cumulative attention scores.

Precision: the codec decides integers (codes) and fp16 scale/min values, so it
runs in IEEE float32 with round-half-even, the precision the codec reading
fixes; attention, masses and scores run in float64.

Modules
  codec     rounding helpers, b-bit (2, 4, 8) group quantiser, ledger layout,
            promote rule
  attention tiered attention with per-window mass
  router    tier counts from the byte budget and the score-ranked router
  pool      the per-segment ledger/tier state machine (demote, promote, evict,
            append, score update, routing)
  diagnostics  selection churn, Global LIR and future missed mass of a run
  prefill_scores  token weights of the causal prefill attention, window sums

Every function is pinned by tests under tests/ (marked "not gpu") against
closed forms, library routines, brute force and hand-derived examples; none is
"parity unpinned".
"""
from . import attention, codec, diagnostics, pool, prefill_scores, router  # noqa: F401
