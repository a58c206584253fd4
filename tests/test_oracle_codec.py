"""Pins of the oracle's low-bit codec (INT2, INT4, INT8) and rounding helpers (CPU only).

Each test ties the oracle to something outside itself: a library conversion,
a hand-derived example, exact rational arithmetic, brute force over the four
codes, or a property any correct min/max quantiser has.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec


def _bf16(x):
    return codec.bf16_to_f32((np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16))


# ------------------------------------------------------------- rounding ----
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(100)
    # force exact ties (low half 0x8000) on both even and odd kept patterns
    u = x.view(np.uint32).copy()
    u[:5000] = (u[:5000] & 0xFFFF0000) | 0x8000
    x = u.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codec.f32_to_bf16_rne(x), ref)


def test_bf16_rne_known_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even pattern is 1.0 (0x3F80)
    assert codec.f32_to_bf16_rne(np.float32(1 + 2 ** -8))[()] == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even): 0x3F82
    assert codec.f32_to_bf16_rne(np.float32(1 + 3 * 2 ** -8))[()] == 0x3F82
    assert codec.f32_to_bf16_rne(np.float32(-2.0))[()] == 0xC000


def test_fp16_matches_torch_and_known_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 10,
                        rng.standard_normal(20000) * 1e-6,        # subnormal range
                        rng.uniform(-60000, 60000, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).half().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codec.f32_to_f16(x).view(np.uint16), ref)
    known = {1.0 / 3.0: 0x3555, 2.0 ** -24: 0x0001, 65504.0: 0x7BFF, -1.5: 0xBE00, 0.0: 0x0000}
    for v, bits in known.items():
        assert codec.f32_to_f16(np.float32(v)).view(np.uint16)[()] == bits


# ------------------------------------------------------------ quantiser ----
def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int2_worked_example.json")))
    x = np.array(g["values"], np.float32)
    c, s16, m16 = codec.quantize_groups(x)
    assert s16.view(np.uint16)[()] == g["scale_fp16_bits"]
    assert m16.view(np.uint16)[()] == g["min_fp16_bits"]
    assert c.tolist() == g["codes"]
    assert c.tolist() != g["codes_if_ties_round_away_from_zero"]


def test_worked_examples_int4_int8(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int4_int8_worked_examples.json")))
    for case in g["cases"]:
        x = np.array(case["values"], np.float32)
        assert np.array_equal(_bf16(x), x)                  # bf16 inputs, as in the cache
        c, s16, m16 = codec.quantize_groups(x, case["bits"])
        assert s16.view(np.uint16)[()] == case["scale_fp16_bits"]
        assert m16.view(np.uint16)[()] == case["min_fp16_bits"]
        assert c.tolist() == case["codes"]
        assert c.tolist() != case["codes_if_ties_round_away_from_zero"]


def test_unsupported_width_raises():
    with pytest.raises(ValueError):
        codec.quantize_groups(np.zeros(32, np.float32), 3)
    with pytest.raises(ValueError):
        codec.entry_nbytes(128, 128, 16)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_lattice_groups_are_recovered_exactly(bits):
    """Values on a grid m + k*s (s a power of two, k covering 0..L) give the
    grid back: scale s, min m, codes k, and dequantisation returns x."""
    rng = np.random.default_rng(10)
    top = (1 << bits) - 1
    for _ in range(200):
        e = int(rng.integers(-12, 4))
        s = np.float32(2.0 ** e)
        k = rng.integers(0, top + 1, 32)
        k[rng.integers(0, 32)] = 0
        k[(rng.integers(1, 32) + 0) % 32] = top
        if k.min() != 0 or k.max() != top:
            continue
        m = np.float32(-float(rng.integers(0, 128)) * s)
        x = (m + k.astype(np.float32) * s).astype(np.float32)
        assert np.array_equal(_bf16(x), x)
        c, s16, m16 = codec.quantize_groups(x, bits)
        assert np.float32(s16) == s and np.float32(m16) == m
        assert np.array_equal(c, k)


def test_constant_group():
    x = np.full(32, _bf16(0.7)[()], np.float32)
    c, s16, m16 = codec.quantize_groups(x)
    assert s16.astype(np.float32) == 0 and s16.view(np.uint16) == 0
    assert m16 == np.float16(x[0])
    assert not c.any()


def test_signed_zero_is_canonical():
    x = np.zeros(32, np.float32)
    x[::2] = -0.0
    c, s16, m16 = codec.quantize_groups(x)
    assert s16.view(np.uint16) == 0 and m16.view(np.uint16) == 0 and not c.any()
    x = np.full(32, -0.0, np.float32)
    c, s16, m16 = codec.quantize_groups(x)
    assert s16.view(np.uint16) == 0 and m16.view(np.uint16) == 0


def _groups(rng, n, scale=1.0, offset=0.0):
    return _bf16(rng.standard_normal((n, 32)) * scale + offset)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("scale,offset", [(1.0, 0.0), (10.0, 0.0), (1e-3, 5.0), (300.0, -1e3)])
def test_extremes_and_range(scale, offset, bits):
    rng = np.random.default_rng(2)
    top = (1 << bits) - 1
    x = _groups(rng, 20000, scale, offset)
    c, s16, m16 = codec.quantize_groups(x, bits)
    assert c.max() <= top
    # fp16 rounding of the scale can move the largest value by a code when
    # the group is nearly flat relative to its offset; these groups are not
    ok = s16.astype(np.float32) > 0
    rows = np.arange(len(x))
    assert (c[rows, x.argmin(1)][ok] == 0).all()
    hi = c[rows, x.argmax(1)][ok]
    assert (hi >= top - 1).all() and (hi == top).mean() > 0.9


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("scale,offset", [(1.0, 0.0), (8.0, 0.0), (0.01, 3.0), (50.0, 200.0)])
def test_error_bound(scale, offset, bits):
    """|x - (c*s + m)| <= s/2 plus the fp16 rounding of s and m (exact arithmetic)."""
    rng = np.random.default_rng(3)
    top = (1 << bits) - 1
    x = _groups(rng, 20000, scale, offset).astype(np.float64)
    c, s16, m16 = codec.quantize_groups(x.astype(np.float32), bits)
    s = s16.astype(np.float64)
    m = m16.astype(np.float64)
    s_exact = (x.max(1) - x.min(1)) / top
    deq = c * s[:, None] + m[:, None]
    slack = top * np.abs(s - s_exact) + np.abs(m - x.min(1)) + 1e-6 * np.abs(x).max(1)
    assert (np.abs(x - deq).max(1) <= s / 2 + slack).all()


@pytest.mark.parametrize("bits,groups", [(2, 3000), (4, 1000), (8, 150)])
def test_codes_are_nearest_grid_point(bits, groups):
    """Away from ties, each code is the argmin over 0..L of |x - (m + c*s)|
    on the stored fp16 grid (exact rational distances, every code tried)."""
    rng = np.random.default_rng(4)
    top = (1 << bits) - 1
    x = _groups(rng, groups, 2.0, 0.3)
    c, s16, m16 = codec.quantize_groups(x, bits)
    checked = 0
    for g in range(len(x)):
        s = Fraction(float(s16[g]))
        m = Fraction(float(m16[g]))
        if s == 0:
            continue
        for i in range(32):
            xi = Fraction(float(x[g, i]))
            d = [abs(xi - (m + k * s)) for k in range(top + 1)]
            best = min(range(top + 1), key=lambda k: d[k])
            second = sorted(d)[1]
            if second - d[best] > s / 1000:
                assert c[g, i] == best
                checked += 1
    assert checked > 0.9 * 32 * groups


def test_grouping_orientation():
    """K groups run over tokens of one channel, V groups over channels of one token."""
    w, d = 64, 64
    t = np.arange(w)[:, None]
    ch = np.arange(d)[None, :]
    # channel d of K spans [0, 31*(d+1)/64] inside every 32-token group
    k = _bf16(((t % 32) * (ch + 1) / 64.0).astype(np.float32))
    # token t of V spans [0, 31*(t+1)/64] inside every 32-channel group
    v = _bf16(((ch % 32) * (t + 1) / 64.0).astype(np.float32))
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    e = codec.quantize_window(to_bits(k), to_bits(v))
    assert e["Ks"].shape == (w // 32, d) and e["Vs"].shape == (w, d // 32)
    for j in range(w // 32):
        for dd in range(d):
            top = float(k[32 * j + 31, dd])
            assert e["Ks"][j, dd] == np.float16(np.float32(top) / np.float32(3))
            assert e["Km"][j, dd] == 0
    for tt in range(w):
        for j in range(d // 32):
            top = float(v[tt, 32 * j + 31])
            assert e["Vs"][tt, j] == np.float16(np.float32(top) / np.float32(3))
    # codes of the ramp: position i of a group maps to round(3*i/31)
    expect = np.rint(np.arange(32) * 3 / 31.0)
    assert np.array_equal(e["Kc"][:32, 5], expect)
    assert np.array_equal(e["Vc"][7, 32:64], expect)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(5)
    c = rng.integers(0, 1 << bits, (128, 128)).astype(np.uint8)
    p = codec.pack_codes(c, bits)
    assert p.shape == (128, 128 * bits // 8)
    assert np.array_equal(codec.unpack_codes(p, bits), c)


def test_pack_bit_order():
    one = np.zeros((1, 4), np.uint8)
    one[0] = [1, 2, 3, 0]
    assert codec.pack_codes(one)[0, 0] == 0b00111001
    two = np.array([[0x3, 0xA, 0xF, 0x1]], np.uint8)
    assert codec.pack_codes(two, 4).tolist() == [[0xA3, 0x1F]]
    three = np.array([[7, 200, 0, 255]], np.uint8)
    assert codec.pack_codes(three, 8).tolist() == [[7, 200, 0, 255]]


@pytest.mark.parametrize("bits,nbytes", [(2, 12288), (4, 20480), (8, 36864)])
def test_entry_bytes_roundtrip_and_size(bits, nbytes):
    rng = np.random.default_rng(6)
    kb = (rng.standard_normal((128, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (rng.standard_normal((128, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e = codec.quantize_window(kb, vb, bits)
    raw = codec.entry_bytes(e, bits)
    assert len(raw) == codec.entry_nbytes(128, 128, bits) == nbytes
    # b + 1 bits per element: the code plus the fp16 scale and min per 32 values
    assert len(raw) * 8 == (bits + 1) * 2 * 128 * 128
    e2 = codec.entry_from_bytes(raw, 128, 128, bits)
    for key in e:
        assert np.array_equal(np.asarray(e[key]).view(np.uint8), np.asarray(e2[key]).view(np.uint8))


def test_promote_sum_is_exact_in_float64():
    """c*s + m with fp16 s, m and c <= 255 is exact in float64, so one cast to
    float32 is a single rounding (what a fused multiply-add gives)."""
    rng = np.random.default_rng(7)
    s = rng.choice(np.concatenate([rng.standard_normal(5000) * 1e-5, rng.standard_normal(5000) * 1e3]),
                   20000).astype(np.float16)
    m = rng.choice(np.concatenate([rng.standard_normal(5000) * 1e4, rng.standard_normal(5000) * 1e-6]),
                   20000).astype(np.float16)
    c = rng.integers(0, 256, 20000)
    got = c * s.astype(np.float64) + m.astype(np.float64)
    for i in range(0, 20000, 7):
        assert Fraction(float(got[i])) == c[i] * Fraction(float(s[i])) + Fraction(float(m[i]))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_promote_bits_match_torch_rounding(bits):
    rng = np.random.default_rng(8)
    kb = (rng.standard_normal((64, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (rng.standard_normal((64, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e = codec.quantize_window(kb, vb, bits)
    pk, pv = codec.promote_bits(e)
    k, v = codec.dequant_window_f64(e)
    ref = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pk, ref(k)) and np.array_equal(pv, ref(v))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("scale,offset", [(1.0, 0.0), (8.0, 0.0), (1e-3, 0.0), (100.0, 5e3)])
def test_requantize_idempotent(scale, offset, bits):
    """Requantising a promoted window returns the ledger's codes, scales, mins
    (INT2 and INT4, on these distributions)."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        kf = (rng.standard_normal((128, 128)) * scale + offset).astype(np.float32)
        vf = (rng.standard_normal((128, 128)) * scale + offset).astype(np.float32)
        kb = (kf.view(np.uint32) >> 16).astype(np.uint16)
        vb = (vf.view(np.uint32) >> 16).astype(np.uint16)
        e = codec.quantize_window(kb, vb, bits)
        e2 = codec.quantize_window(*codec.promote_bits(e), bits)
        assert codec.entry_bytes(e, bits) == codec.entry_bytes(e2, bits)


def test_int8_requantize_can_drift():
    """With 8-bit codes the bf16 rounding of a promoted value can reach half a
    code step (and a small scale rounded to an fp16 subnormal moves the grid
    further), so quantising a promoted window again may change codes: the
    drift a write-once ledger avoids by never quantising a window twice."""
    rng = np.random.default_rng(11)
    moved = 0
    for _ in range(10):
        kf = (rng.standard_normal((128, 128)) * 1e-3).astype(np.float32)
        vf = (rng.standard_normal((128, 128)) * 1e-3).astype(np.float32)
        kb = (kf.view(np.uint32) >> 16).astype(np.uint16)
        vb = (vf.view(np.uint32) >> 16).astype(np.uint16)
        e = codec.quantize_window(kb, vb, 8)
        e2 = codec.quantize_window(*codec.promote_bits(e), 8)
        moved += int((e["Kc"] != e2["Kc"]).sum() + (e["Vc"] != e2["Vc"]).sum())
    assert moved > 0


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_edge_case_groups_have_their_defined_codes(bits):
    """Ties exactly on the half-way points (round half to even), their bf16
    neighbours, s == 0, fp16 overflow of the min (m = +-inf) and of the scale:
    codes fixed by the definition alone (tests/codec_cases.py), the same groups
    the GPU demote test feeds the kernel."""
    from tests.codec_cases import edge_groups
    pinned = 0
    with np.errstate(over="ignore"):
        for name, g, want in edge_groups(bits, np.random.default_rng(bits)):
            got, _, _ = codec.quantize_groups(codec.bf16_to_f32(g)[None], bits)
            if want is not None:
                assert np.array_equal(got[0], want), name
                pinned += 1
            else:
                assert got.max() <= (1 << bits) - 1, name
    assert pinned >= 10
