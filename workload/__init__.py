"""Seeded synthetic inputs for the tiered decode-attention path.

This package draws random numbers only: query vectors, key/value histories,
new tokens, prior window scores and the outlier-channel choices.  It holds
none of the method's arithmetic (no quantisation, rounding rule, attention,
scoring or routing), so the oracle and the HIP path can both consume it.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    Config,
    kv_history,
    kv_history_device,
    new_kv,
    prefill_queries,
    query,
    score_prior,
)
