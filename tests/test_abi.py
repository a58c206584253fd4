"""The C-ABI library loads, exports every symbol include/kvtier.h declares,
and its host-only logic (sizing, validation, tier counts) is right.  No GPU
work is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import router
from workload import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvtier.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def B():
    from tiered_int2_fp16_amd import binding
    return binding


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("kv_pool_create", "kv_demote_quantize", "kv_promote_dequantize",
              "kv_tiered_decode_attn", "kv_score_route"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(B.EXPORTS) == _declared()


def _cfg(B, c, maxw=None, nb=None, nl=None):
    m = maxw or c.max_windows()
    return B.make_config(c.batch, c.layers, c.q_heads, c.kv_heads, c.head_dim, c.window, m,
                         c.n_recent, nb or m, nl or m)


def test_arena_size_matches_layout(B):
    c = CONFIGS["llama8b_32k"]
    cfg = _cfg(B, c, nb=40, nl=200)
    n = B.kv_pool_arena_bytes(cfg)
    bf16 = 1 * 40 * 8 * (2 * 128 * 128 * 2)
    ledger = 1 * 200 * 8 * 12288
    assert bf16 + ledger < n < bf16 + ledger + 64 * 1024
    assert B.kv_ledger_entry_bytes(128, 128) == 12288
    assert B.kv_ledger_entry_bytes(64, 64) == 3072
    # b + 1 bits per value: b-bit code + (16 + 16) bits per 32 values
    for bits in (2, 4, 8):
        assert B.kv_ledger_entry_bytes(128, 128, bits) * 8 == (bits + 1) * 2 * 128 * 128
    assert B.kv_ledger_entry_bytes(128, 128, 0) == 12288
    assert B.kv_ledger_entry_bytes(128, 128, 3) == 0
    cfg.ledger_bits = 8
    assert B.kv_pool_arena_bytes(cfg) - n == 200 * 8 * (36864 - 12288)


@pytest.mark.parametrize("field,value", [
    ("q_heads", 30), ("head_dim", 96), ("window", 48), ("max_windows", 0),
    ("max_windows", 5000), ("bf16_slots", 0), ("bf16_slots", 20000), ("kv_heads", 0),
    ("ledger_bits", 3), ("ledger_bits", 16), ("ledger_bits", -2), ("n_recent", 0)])
def test_invalid_configs_are_rejected(B, field, value):
    cfg = _cfg(B, CONFIGS["tiny"])
    setattr(cfg, field, value)
    with pytest.raises(B.KvError):
        B.kv_pool_arena_bytes(cfg)
    assert B.LIB.kv_last_error().decode()


def test_host_tier_counts_match_oracle(B):
    rng = np.random.default_rng(0)
    for _ in range(3000):
        n = int(rng.integers(0, 5000))
        r = int(rng.integers(0, 8))
        beta = float(rng.choice([rng.random(), 0.2, 0.05, 0.1, 0.125, 0.325]))
        phi = float(rng.choice([rng.random() * beta, 0.1, 0.02, 0.0625, 0.09375, 0.25]))
        bits = int(rng.choice([2, 4, 8]))
        assert B.kv_tier_counts(n, r, beta, phi) == router.tier_counts(n, r, beta, phi)
        assert B.kv_tier_counts(n, r, beta, phi, bits) == router.tier_counts(n, r, beta, phi, bits)
    with pytest.raises(B.KvError):
        B.kv_tier_counts(10, 4, 0.2, 0.1, 5)


def test_null_arguments_fail_without_a_gpu(B):
    assert B.LIB.kv_pool_create(None, None, 0, None, None) == B.KV_EINVAL
    assert B.LIB.kv_tiered_decode_attn(None, 0, None, None, None, None, None, None, 0, None) == B.KV_EINVAL
    assert B.LIB.kv_score_route(None, 0, None, 0, 0.0, 0.0, None, None, None) == B.KV_EINVAL
    assert B.LIB.kv_pool_destroy(None) == B.KV_OK
