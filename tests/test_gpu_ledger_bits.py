"""GPU parity of pools whose ledger holds 4-bit or 8-bit codes.

The QEvict summary quantises its recoverable tier to INT2 in its experiments
("Methodologie: QEvict", tier 2); the RDKV summary packs 2-, 4- and 8-bit rows
("2.3 Efficiente Gepakte Decode (TriZone)", Zone A).  A pool's ledger width is
one of 2, 4, 8; the INT2 pools are covered by the other GPU tests.  Each case
here runs the library through the C ABI beside the oracle at the same width:
codes, scales, mins, tiers, transitions and promoted bf16 bit-exact; outputs
within 2e-3 and window masses within 1e-4 (the harness's bars).
"""
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS, query

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_harness import Pair, dev, log  # noqa: E402


@pytest.mark.parametrize("bits", [4, 8])
def test_tiny_loop(bits):
    """Route, then 120 decode steps appending a token each (two new windows),
    scores every step, routing every 16 steps with demote/promote traffic."""
    c = dataclasses.replace(CONFIGS["tiny"], steps=120, route_every=16, append=True)
    p = Pair(c, bits=bits)
    p.load(0)
    p.route(0, c.budget_frac, c.hi_frac)
    p.check_state(0)
    moved, worst = 0, (0.0, 0.0)
    for s in range(c.steps):
        _, mass, o_mass, errs = p.step(0, s, append=True)
        worst = (max(worst[0], errs[0]), max(worst[1], errs[1]))
        p.add_scores(0, mass, o_mass)
        if (s + 1) % c.route_every == 0:
            _, cnt = p.route(0, c.budget_frac, c.hi_frac)
            moved += int(cnt[0].sum() + cnt[1].sum())
            p.check_state(0)
    log("tiny loop, %d-bit ledger: %d moves, out err %.2e mass err %.2e" % (bits, moved, *worst))
    assert moved > 0


@pytest.mark.parametrize("bits", [4, 8])
def test_write_once_ledger(bits):
    c = CONFIGS["tiny"]
    p = Pair(c, bits=bits)
    p.load(0)
    seg = p.oracle[(0, 0)]
    one = dev(np.array([1], np.int32))
    p.pool.demote(0, dev(np.array([[3, 5]], np.int32)), dev(np.array([2], np.int32)))
    seg.demote(3)
    seg.demote(5)
    first = p.pool.read_ledger(0, 0, 3).cpu().numpy().copy()
    assert first.shape[1] == (bits + 1) * c.window * c.head_dim // 4
    p.pool.promote(0, dev(np.array([[3]], np.int32)), one)
    seg.promote(3)
    p.check_state(0)
    p.pool.demote(0, dev(np.array([[3]], np.int32)), one)
    seg.demote(3)
    assert p.pool.read_ledger(0, 0, 3).cpu().numpy().tobytes() == first.tobytes()
    p.check_state(0)
    p.step(0, 0)


@pytest.mark.parametrize("bits,n_lo", [(4, 83), (8, 46)])
def test_llama_32k(bits, n_lo):
    """The 32K Llama-3.1-8B shape at a 20 % budget: 25 bf16 windows, and as
    many ledger windows as the rest of the budget buys at b + 1 bits per
    value; one decode step, every output."""
    c = CONFIGS["llama8b_32k"]
    p = Pair(c, bits=bits)
    p.load(0)
    _, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert cnt[0][0] == n_lo and cnt[2][0] == c.n_windows - 25 - n_lo
    p.check_state(0, ledger_sample=20, window_sample=6, rng=np.random.default_rng(bits))
    out, mass, _, errs = p.step(0, 0)
    log("llama 32K, %d-bit ledger: out err %.2e mass err %.2e" % (bits, *errs))
    # the same step again gives the same bits (no run-to-run variation), also
    # without the mass emission
    q = dev(query(c, 0, 0))
    out2, mass2 = p.pool.attn(0, q)
    assert torch.equal(out, out2) and torch.equal(mass, mass2)
    out3, _ = p.pool.attn(0, q, want_mass=False)
    assert torch.equal(out, out3)


SHAPES = [
    ("g1_d64", 31, 2, 2, 64, 64),
    ("g7_d128", 32, 14, 2, 128, 64),
    ("g8_d64", 33, 8, 1, 64, 128),
]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name,seed,hq,hkv,d,w", SHAPES, ids=[s[0] for s in SHAPES])
def test_head_group_shapes(name, seed, hq, hkv, d, w, bits):
    """Group sizes 1, 7, 8 at head_dim 64 and 128 (both operand layouts of the
    attention kernel): route, 33 decode steps with appends, routing every 16."""
    c = dataclasses.replace(CONFIGS["tiny"], name=name, seed=seed, batch=2, q_heads=hq, kv_heads=hkv,
                            head_dim=d, window=w, context=40 * w - 17, budget_frac=0.3, hi_frac=0.2,
                            steps=33, route_every=16, append=True)
    p = Pair(c, bits=bits)
    p.load(0)
    p.route(0, c.budget_frac, c.hi_frac)
    p.check_state(0)
    worst = (0.0, 0.0)
    for s in range(c.steps):
        _, mass, o_mass, errs = p.step(0, s, append=True)
        worst = (max(worst[0], errs[0]), max(worst[1], errs[1]))
        p.add_scores(0, mass, o_mass)
        if (s + 1) % c.route_every == 0:
            p.route(0, c.budget_frac, c.hi_frac)
            p.check_state(0)
    log("%s, %d-bit ledger: out err %.2e mass err %.2e" % (name, bits, *worst))


@pytest.mark.parametrize("bits,n_lo", [(4, 24), (8, 13)])
def test_qwen_32k(bits, n_lo):
    """The Qwen2.5-7B shape (batch 8, groups of 7 query heads, 4 K outlier
    channels x10) at a 5 % budget: 5 bf16 windows per sequence and the ledger
    windows the rest buys at b + 1 bits per value; one step, every output."""
    c = CONFIGS["qwen7b_32k"]
    p = Pair(c, bits=bits)
    p.load(0)
    _, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert (cnt[0] == n_lo).all() and (cnt[2] == c.n_windows - 5 - n_lo).all()
    p.check_state(0, ledger_sample=6, window_sample=3, rng=np.random.default_rng(10 + bits))
    out, mass, _, errs = p.step(0, 0)
    log("qwen 32K, %d-bit ledger: out err %.2e mass err %.2e" % (bits, *errs))
    out2, mass2 = p.pool.attn(0, dev(query(c, 0, 0)))
    assert torch.equal(out, out2) and torch.equal(mass, mass2)


@pytest.mark.timeout(900)
def test_llama_128k_loop_4bit_sampled():
    """The 128K loop shape with a 4-bit ledger (102 bf16 / 328 ledger windows
    per sequence): 17 decode steps appending a token each (the first opens
    window 1024), scores every step, routing after step 16; two of the four
    sequences compared in full against the oracle."""
    c = CONFIGS["llama8b_128k_loop"]
    p = Pair(c, seqs=[1, 2], bits=4)
    p.load(0)
    _, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert (cnt[0] == 328).all()
    p.check_state(0, ledger_sample=8, window_sample=4, rng=np.random.default_rng(14))
    for s in range(17):
        _, mass, o_mass, errs = p.step(0, s, append=True)
        p.add_scores(0, mass, o_mass)
        log("128K 4-bit step %d: out err %.2e mass err %.2e" % (s, *errs))
        if (s + 1) % c.route_every == 0:
            p.route(0, c.budget_frac, c.hi_frac)
            p.check_state(0, ledger_sample=8, window_sample=4, rng=np.random.default_rng(15))
