"""Low-bit window codec of the oracle (test infrastructure).

The QEvict summary fixes only that the recoverable tier is a compact low-bit
format, INT2 in its experiments ("Methodologie: QEvict", tier 2), and that a
window is quantised once, at its first demotion, into a persistent ledger that
every later promotion and demotion reuses ("Kernmechanismen", Write-Once
Quantization Ledger).  The RDKV summary lists 2, 4 and 8 as the hardware
bit widths of its packed stream, grouped by width so that each group has one
dequantisation path ("2.3 Efficiente Gepakte Decode (TriZone)", Zone A); the
ledger width b is therefore a parameter, one of 2, 4, 8, with 2 the default.
The codec reading adopted here:

* asymmetric min/max per group of 32 values, b-bit codes 0..2^b - 1;
* K grouped per channel over 32 consecutive tokens (the key-per-channel
  strategy the LogQuant summary names in its "Implementatie" section);
* V grouped per token over 32 consecutive channels;
* scale and min stored as fp16; encoding uses the stored (fp16) values;
* the code decision is float32 arithmetic with round-half-even.

All codec arithmetic here is numpy float32 (IEEE single, correctly rounded),
so every decision is taken in the precision the reading fixes.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


# ---------------------------------------------------------------- rounding ---
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs).

    Adding 0x7FFF plus the lowest kept bit and truncating rounds the dropped
    16 bits to nearest with ties going to the even kept pattern.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """IEEE binary16, round to nearest even, subnormals kept (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------- quantiser ---
BITS = (2, 4, 8)


def levels(bits: int) -> int:
    """Largest code of a b-bit group: 2^b - 1."""
    if bits not in BITS:
        raise ValueError(f"ledger bit width {bits} is not one of {BITS}")
    return (1 << bits) - 1


def quantize_groups(x: np.ndarray, bits: int = 2):
    """Quantise groups along the last axis (length 32) of float32 values.

    Returns (codes uint8 [..., 32], scale fp16 [...], min fp16 [...]).
    Steps, all in float32, with L = 2^bits - 1:
      1. signed zeros are made +0 so min/max are unique values;
      2. mn, mx = min, max of the group;
      3. s32 = (mx - mn) / L   (a true IEEE divide);
      4. stored s16 = fp16(s32), m16 = fp16(mn); s, m = their float32 values;
      5. s == 0: all codes 0; otherwise c = clamp(rint((x - m) / s), 0, L),
         rint = round half to even.
    """
    top = levels(bits)
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == GROUP
    x = np.where(x == 0, np.float32(0.0), x).astype(np.float32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s32 = ((mx - mn) / np.float32(top)).astype(np.float32)
    s16 = f32_to_f16(s32)
    m16 = f32_to_f16(mn)
    s = s16.astype(np.float32)[..., None]
    m = m16.astype(np.float32)[..., None]
    u = (x - m).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (u / np.where(s == 0, np.float32(1.0), s)).astype(np.float32)
    c = np.clip(np.rint(t), 0, top)
    c = np.where(s == 0, 0, c).astype(np.uint8)
    return c, s16, m16


def quantize_window(k_bits: np.ndarray, v_bits: np.ndarray, bits: int = 2) -> dict:
    """Quantise one window of one kv head to b-bit codes.

    k_bits, v_bits: bf16 bits [W][D] (W, D multiples of 32).
    Returns the ledger entry in unpacked form:
      Kc, Vc uint8 [W][D]; Ks, Km fp16 [W/32][D]; Vs, Vm fp16 [W][D/32].
    K groups run over 32 consecutive tokens of one channel, V groups over 32
    consecutive channels of one token, so no group crosses a window.
    """
    k = bf16_to_f32(k_bits)
    v = bf16_to_f32(v_bits)
    w, d = k.shape
    assert w % GROUP == 0 and d % GROUP == 0
    kg = k.reshape(w // GROUP, GROUP, d).transpose(0, 2, 1)          # [W/32][D][32]
    kc, ks, km = quantize_groups(kg, bits)
    vg = v.reshape(w, d // GROUP, GROUP)                              # [W][D/32][32]
    vc, vs, vm = quantize_groups(vg, bits)
    return {
        "Kc": np.ascontiguousarray(kc.transpose(0, 2, 1).reshape(w, d)),
        "Ks": ks, "Km": km,
        "Vc": np.ascontiguousarray(vc.reshape(w, d)),
        "Vs": vs, "Vm": vm,
    }


def dequant_window_f64(e: dict):
    """Exact dequantised K, V (float64 [W][D]) of a ledger entry: c*s + m."""
    w, d = e["Kc"].shape
    ks = np.repeat(e["Ks"].astype(np.float64), GROUP, axis=0)        # [W][D]
    km = np.repeat(e["Km"].astype(np.float64), GROUP, axis=0)
    vs = np.repeat(e["Vs"].astype(np.float64), GROUP, axis=1)        # [W][D]
    vm = np.repeat(e["Vm"].astype(np.float64), GROUP, axis=1)
    k = e["Kc"].astype(np.float64) * ks + km
    v = e["Vc"].astype(np.float64) * vs + vm
    return k, v


def promote_bits(e: dict):
    """bf16 bits a promotion writes back: bf16_rne(float32(c*s + m)).

    c*s + m is exact in float64 (fp16 operands are multiples of 2^-24 below
    2^16 and c <= 255, so the sum needs at most 48 significant bits), so one
    cast to float32 is the single rounding of a fused multiply-add, then one
    rounding to bf16.
    """
    k, v = dequant_window_f64(e)
    return f32_to_bf16_rne(k.astype(np.float32)), f32_to_bf16_rne(v.astype(np.float32))


# ------------------------------------------------------- canonical layout ---
def pack_codes(c: np.ndarray, bits: int = 2) -> np.ndarray:
    """[W][D] b-bit codes -> [W][D*b/8] bytes, LSB first: code (t, d) sits in
    byte (d*b)//8 at bits (d*b) % 8 .. +b-1."""
    levels(bits)
    c = np.asarray(c, dtype=np.uint8)
    w, d = c.shape
    per = 8 // bits
    q = c.reshape(w, d // per, per).astype(np.uint16)
    out = np.zeros((w, d // per), np.uint16)
    for i in range(per):
        out |= q[..., i] << (bits * i)
    return out.astype(np.uint8)


def unpack_codes(p: np.ndarray, bits: int = 2) -> np.ndarray:
    levels(bits)
    p = np.asarray(p, dtype=np.uint8)
    w, nb = p.shape
    per = 8 // bits
    out = np.empty((w, nb, per), dtype=np.uint8)
    for i in range(per):
        out[..., i] = (p >> (bits * i)) & ((1 << bits) - 1)
    return out.reshape(w, nb * per)


def entry_bytes(e: dict, bits: int = 2) -> bytes:
    """Canonical ledger bytes of one (window, kv head): Kc, Vc, Ks, Km, Vs, Vm."""
    return b"".join([
        pack_codes(e["Kc"], bits).tobytes(), pack_codes(e["Vc"], bits).tobytes(),
        e["Ks"].astype("<f2").tobytes(), e["Km"].astype("<f2").tobytes(),
        e["Vs"].astype("<f2").tobytes(), e["Vm"].astype("<f2").tobytes(),
    ])


def entry_from_bytes(buf: bytes, w: int, d: int, bits: int = 2) -> dict:
    """Inverse of :func:`entry_bytes`."""
    a = np.frombuffer(buf, dtype=np.uint8)
    o = 0
    n = w * d * bits // 8
    kc = unpack_codes(a[o:o + n].reshape(w, d * bits // 8), bits); o += n
    vc = unpack_codes(a[o:o + n].reshape(w, d * bits // 8), bits); o += n
    g = (w // GROUP) * d * 2
    ks = a[o:o + g].view("<f2").reshape(w // GROUP, d); o += g
    km = a[o:o + g].view("<f2").reshape(w // GROUP, d); o += g
    g = w * (d // GROUP) * 2
    vs = a[o:o + g].view("<f2").reshape(w, d // GROUP); o += g
    vm = a[o:o + g].view("<f2").reshape(w, d // GROUP); o += g
    assert o == a.size
    return {"Kc": kc, "Vc": vc, "Ks": ks.astype(np.float16), "Km": km.astype(np.float16),
            "Vs": vs.astype(np.float16), "Vm": vm.astype(np.float16)}


def entry_nbytes(w: int, d: int, bits: int = 2) -> int:
    """Bytes of one (window, kv head) entry: 2*W*D*b/8 codes + 4*(W*D/32)*2."""
    levels(bits)
    return 2 * (w * d * bits // 8) + 4 * (w * d // GROUP) * 2
