"""Groups of 32 bf16 values at the edge cases of the min/max codec, shared by
the oracle's pins (test_oracle_codec.py) and the GPU demote test
(test_gpu_codec.py).  Test infrastructure: no arithmetic of the method here,
only inputs and, where the value is fixed by the codec's definition alone, the
expected codes.

The codec (QEvict technical summary, "Kernmechanismen" and its quantisation
formula): s = fp16((max - min) / L), m = fp16(min), code = clamp(rint_even(
(x - m) / s), 0, L), 0 where s == 0.
"""
from __future__ import annotations

import numpy as np


def _bf16(x):
    """float32 values that are exactly bf16 (asserted), as bf16 bits."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "not a bf16 value"
    return (b >> 16).astype(np.uint16)


def _trunc(x):
    """bf16 bits of float32 values by dropping the low 16 bits."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _value(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def edge_groups(bits: int, rng) -> list:
    """[(name, bf16 bits [32], expected codes [32] or None)].

    Expected codes are given where the definition fixes them by inspection:
      * ties: min m0, max m0 + L s (s a power of two, so s and m are exact) and
        values exactly (k + 1/2) s + m0: code k for even k, k + 1 for odd k
        (round half to even);
      * the bf16 neighbours of those values: k + 1 above the half-way point, k
        below it;
      * s == 0: all 0; min below -65504 (m = -inf) with a finite s: all L; min
        above 65504 (m = +inf): all 0; s = inf with a finite m: all 0.
    """
    L = (1 << bits) - 1
    s = 1.0 if bits == 8 else 0.125            # (k + 1/2) s + m0 stays bf16-exact
    top = min(L, 128)                          # 8 bits: k + 1/2 needs 9 bits from k = 128 on
    out = []
    for m0 in (0.0, 1.0, -2.0):
        if bits == 8 and m0 != 0.0:
            continue
        ks = np.arange(30) % top
        ties = ((ks + 0.5) * s + m0).astype(np.float32)
        ends = _bf16([m0, m0 + L * s])
        tie_codes = np.where(ks % 2 == 0, ks, ks + 1)
        out.append((f"ties m0={m0}", np.concatenate([ends, _bf16(ties)]),
                    np.concatenate([[0, L], tie_codes]).astype(np.uint8)))
        tb = _bf16(ties)
        for d in (+1, -1):
            nb = (tb.astype(np.int32) + d).astype(np.uint16)      # next bf16 away from / towards zero
            above = _value(nb) > ties
            out.append((f"tie neighbours {d:+d} m0={m0}", np.concatenate([ends, nb]),
                        np.concatenate([[0, L], ks + above]).astype(np.uint8)))
    zeros = np.zeros(32, np.uint8)
    out.append(("s = 0", _bf16(np.full(32, 3.0)), zeros))
    out.append(("s = 0, m = +inf", _bf16(np.full(32, 70144.0)), zeros))
    out.append(("s = 0, m = -inf", _bf16(np.full(32, -70144.0)), zeros))
    g = np.round(np.linspace(-70656.0, -69632.0, 32) / 512) * 512     # (bf16 spacing 512 there)
    out.append(("m = -inf", _bf16(g), np.full(32, L, np.uint8)))
    g = np.round(np.linspace(70144.0, 71168.0, 32) / 512) * 512
    out.append(("m = +inf", _bf16(g), zeros))
    g = np.concatenate([[0.0, 2.0 ** 25], rng.uniform(0, 1000, 30)])    # (max - min) / L > 65504
    out.append(("s = inf, m = 0", _trunc(g), zeros))
    g = np.concatenate([[0.0, 2.0 ** -16], rng.choice([0.0, 2.0 ** -17, 2.0 ** -18, 2.0 ** -16], 30)])
    out.append(("fp16-subnormal s", _bf16(g), None))
    out.append(("signed zeros", _trunc(np.array([0.0, -0.0, 0.5, -0.25] * 8)), None))
    out.append(("only zeros", _trunc(np.array([-0.0] * 16 + [0.0] * 16)), zeros))
    for i in range(8):
        g = rng.standard_normal(32) * rng.choice([1e-3, 1.0, 40.0])
        out.append((f"normal {i}", _trunc(g), None))
    return out
