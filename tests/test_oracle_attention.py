"""Pins of the oracle's tiered attention and mass (CPU only).

Library reference: torch's scaled_dot_product_attention on the CPU in
float64, on explicitly assembled token sets; plus brute-force scalar loops.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, codec
from oracle.pool import Segment
from oracle.router import E, F, Q


def _bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _sdpa(q, k, v):
    """q [Hq][D]; k, v [Hkv][T][D] float64 -> [Hq][D] via torch SDPA (GQA by repeat)."""
    hq, hkv = q.shape[0], k.shape[0]
    kt = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=0)
    qt = torch.from_numpy(q)[:, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()


def _segment(rng, hkv=2, w=64, d=64, tokens=640, outlier=False, bits=2):
    seg = Segment(hkv, w, d, 4, bits=bits)
    k = _bits(rng, (hkv, tokens, d))
    if outlier:
        k = _bits(rng, (hkv, tokens, d), 1.0)
        kk = codec.bf16_to_f32(k)
        kk[:, :, 3] *= 8
        k = (kk.view(np.uint32) >> 16).astype(np.uint16)
    v = _bits(rng, (hkv, tokens, d))
    seg.prefill(k, v)
    return seg, k, v


def test_all_full_precision_equals_sdpa():
    """Every window bf16 (100 % budget): plain softmax attention."""
    rng = np.random.default_rng(10)
    seg, k, v = _segment(rng, hkv=2, tokens=640)
    q = _bits(rng, (8, 64))
    out, mass = seg.attend(q)
    ref = _sdpa(codec.bf16_to_f64(q), codec.bf16_to_f64(k), codec.bf16_to_f64(v))
    assert np.abs(out - ref).max() < 1e-12
    assert np.allclose(mass.sum(1), 1.0, atol=1e-12)


def test_eviction_renormalises_over_remaining_tokens():
    rng = np.random.default_rng(11)
    seg, k, v = _segment(rng, hkv=2, tokens=640)
    for w in (0, 3, 4, 7):
        seg.evict(w)
    q = _bits(rng, (4, 64))
    out, mass = seg.attend(q)
    keep = np.concatenate([np.arange(w * 64, (w + 1) * 64) for w in range(10) if w not in (0, 3, 4, 7)])
    ref = _sdpa(codec.bf16_to_f64(q), codec.bf16_to_f64(k[:, keep]), codec.bf16_to_f64(v[:, keep]))
    assert np.abs(out - ref).max() < 1e-12
    assert (mass[:, [0, 3, 4, 7]] == 0).all()
    assert np.allclose(mass.sum(1), 1.0, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_int2_windows_attend_with_dequantised_values(bits):
    rng = np.random.default_rng(12)
    seg, k, v = _segment(rng, hkv=1, tokens=640, outlier=True, bits=bits)
    for w in (1, 2, 5):
        seg.demote(w)
    seg.evict(6)
    q = _bits(rng, (4, 64))
    out, mass = seg.attend(q)
    kf, vf = codec.bf16_to_f64(k).copy(), codec.bf16_to_f64(v).copy()
    for w in (1, 2, 5):
        dk, dv = codec.dequant_window_f64(seg.ledger[w][0])
        kf[0, w * 64:(w + 1) * 64] = dk
        vf[0, w * 64:(w + 1) * 64] = dv
    keep = np.concatenate([np.arange(w * 64, (w + 1) * 64) for w in range(10) if w != 6])
    ref = _sdpa(codec.bf16_to_f64(q), kf[:, keep], vf[:, keep])
    assert np.abs(out - ref).max() < 1e-12
    # ledger windows still receive mass; the evicted one gets none
    assert (mass[:, [1, 2, 5]] > 0).all() and (mass[:, 6] == 0).all()


def test_window_mass_is_probability_sum():
    rng = np.random.default_rng(13)
    seg, k, v = _segment(rng, hkv=1, w=64, d=64, tokens=300)    # ragged last window
    q = _bits(rng, (4, 64))
    _, mass = seg.attend(q)
    qf = codec.bf16_to_f64(q)
    kf = codec.bf16_to_f64(k)[0]
    for h in range(4):
        z = kf @ qf[h] / 8.0
        p = np.exp(z - z.max())
        p /= p.sum()
        for w in range(5):
            assert abs(mass[h, w] - p[w * 64:(w + 1) * 64].sum()) < 1e-12


def test_permutation_invariance():
    """Reordering windows (and the tokens inside them) leaves out unchanged."""
    rng = np.random.default_rng(14)
    hkv, d, n, w = 2, 32, 6, 32
    wins = [(rng.standard_normal((hkv, w, d)), rng.standard_normal((hkv, w, d))) for _ in range(n)]
    wins[2] = None
    q = rng.standard_normal((4, d))
    out, mass = attention.attend(q, wins)
    perm = rng.permutation(n)
    tok = rng.permutation(w)
    wins_p = [None if wins[i] is None else (wins[i][0][:, tok], wins[i][1][:, tok]) for i in perm]
    out_p, mass_p = attention.attend(q, wins_p)
    assert np.abs(out - out_p).max() < 1e-12
    assert np.abs(mass[:, perm] - mass_p).max() < 1e-12


def test_gqa_mapping():
    """Query head h reads kv head h // G (changing kv head 1 moves only heads 2, 3)."""
    rng = np.random.default_rng(15)
    hkv, d = 2, 16
    wins = [(rng.standard_normal((hkv, 8, d)), rng.standard_normal((hkv, 8, d))) for _ in range(3)]
    q = rng.standard_normal((4, d))
    out, _ = attention.attend(q, wins)
    wins2 = [(a.copy(), b.copy()) for a, b in wins]
    for a, b in wins2:
        a[1] += 1.0
        b[1] -= 2.0
    out2, _ = attention.attend(q, wins2)
    assert np.abs(out[:2] - out2[:2]).max() == 0
    assert np.abs(out[2:] - out2[2:]).min() > 0


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(16)
    hkv, g, d, w, n = 1, 3, 4, 2, 4
    wins = [(rng.standard_normal((hkv, w, d)), rng.standard_normal((hkv, w, d))) for _ in range(n)]
    wins[1] = None
    q = rng.standard_normal((g, d))
    out, mass = attention.attend(q, wins)
    for h in range(g):
        logits = []
        for wi, kv in enumerate(wins):
            if kv is None:
                continue
            for t in range(w):
                s = 0.0
                for c in range(d):
                    s += q[h][c] * kv[0][0][t][c]
                logits.append((wi, t, s / math.sqrt(d)))
        mx = max(x[2] for x in logits)
        den = sum(math.exp(x[2] - mx) for x in logits)
        o = [0.0] * d
        ms = [0.0] * n
        for wi, t, s in logits:
            p = math.exp(s - mx) / den
            ms[wi] += p
            for c in range(d):
                o[c] += p * wins[wi][1][0][t][c]
        assert max(abs(o[c] - out[h][c]) for c in range(d)) < 1e-12
        assert max(abs(ms[i] - mass[h][i]) for i in range(n)) < 1e-12


def test_append_attends_new_token():
    rng = np.random.default_rng(17)
    seg, k, v = _segment(rng, hkv=1, w=64, d=64, tokens=128)
    kn, vn = _bits(rng, (1, 64)), _bits(rng, (1, 64))
    seg.append(kn, vn)
    assert seg.n == 3 and seg.valid(2) == 1 and seg.tier[2] == F
    q = _bits(rng, (4, 64))
    out, mass = seg.attend(q)
    kk = np.concatenate([k, kn[:, None]], axis=1)
    vv = np.concatenate([v, vn[:, None]], axis=1)
    ref = _sdpa(codec.bf16_to_f64(q), codec.bf16_to_f64(kk), codec.bf16_to_f64(vv))
    assert np.abs(out - ref).max() < 1e-12
    assert mass.shape == (4, 3) and np.allclose(mass.sum(1), 1)


def test_tiers_constants():
    assert (E, Q, F) == (0, 1, 2)
