"""GPU parity for shapes the benchmark configurations do not reach.

* Query-head group sizes 1, 2, 7 and 8 at head_dim 64 and 128: the attention
  kernel lays the group's heads out differently for G <= 4 and G > 4 (column
  groups of the MFMA operands), and head_dim 64 halves the channel groups.
* Windows of 32, 96, 160 and 256 tokens (one, three, five and eight 32-token
  tiles), with INT2 and 4-bit ledgers.
* More than 64 tiles of one tier per wave: at 64 sequences x 8 kv heads the
  kernel runs one split per (sequence, kv head), so a wave walks its tile list
  in chunks of 64 - first for INT2 tiles, then (after promotions) for bf16.

Every case compares outputs and window masses with the oracle (tolerances of
the harness) and the routed state bit for bit.
"""
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS, score_prior

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_harness import CachedSegment, Pair, dev, log  # noqa: E402


# (name, seed, q_heads, kv_heads, head_dim, window)
SHAPES = [
    ("g1_d64", 11, 2, 2, 64, 64),
    ("g2_d128", 12, 4, 2, 128, 64),
    ("g7_d64", 13, 7, 1, 64, 64),
    ("g8_d64", 14, 8, 1, 64, 128),
    ("g8_d128", 15, 16, 2, 128, 64),
]


@pytest.mark.parametrize("name,seed,hq,hkv,d,w", SHAPES, ids=[s[0] for s in SHAPES])
def test_head_group_shapes(name, seed, hq, hkv, d, w):
    """Route, then 40 decode steps with appends, routing every 16 steps."""
    c = dataclasses.replace(CONFIGS["tiny"], name=name, seed=seed, batch=2, q_heads=hq, kv_heads=hkv,
                            head_dim=d, window=w, context=40 * w - 17, budget_frac=0.3, hi_frac=0.2,
                            steps=40, route_every=16, append=True)
    p = Pair(c)
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
    log("%s: out err %.2e mass err %.2e" % (name, *worst))


# (name, seed, q_heads, kv_heads, head_dim, window): windows of one tile (32),
# of a tile count that is not a power of two (96, 160) and of eight tiles (256,
# the most a window may have: the tile field of the attention's tile lists and
# the combine's per-window loop)
WINDOWS = [
    ("w32_g4_d128", 16, 8, 2, 128, 32),
    ("w96_g4_d64", 17, 4, 1, 64, 96),
    ("w160_g8_d128", 18, 16, 2, 128, 160),
    ("w256_g4_d128", 19, 8, 2, 128, 256),
    ("w256_g7_d64", 20, 7, 1, 64, 256),
]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("name,seed,hq,hkv,d,w", WINDOWS, ids=[s[0] for s in WINDOWS])
def test_window_sizes(name, seed, hq, hkv, d, w, bits):
    """Route, then 40 decode steps with appends (new windows open at W = 32),
    routing every 16 steps, with an INT2 and a 4-bit ledger; the routed state
    (tiers, ledger bytes, bf16 windows) is compared bit for bit after every
    routing event."""
    c = dataclasses.replace(CONFIGS["tiny"], name=name, seed=seed, batch=2, q_heads=hq, kv_heads=hkv,
                            head_dim=d, window=w, context=24 * w - 17, budget_frac=0.3, hi_frac=0.2,
                            steps=40, route_every=16, append=True)
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


def test_many_tiles_per_wave():
    """64 sequences x 8 kv heads, 16K context (128 windows of 128): one split
    per (sequence, kv head), so 4 waves share each unit's tiles.  Route to 12
    bf16 / 116 INT2 windows (116 INT2 tiles per wave: two list chunks), check
    a step; route again to 76 bf16 / 52 INT2 (76 bf16 tiles per wave), check
    another.  Contexts are drawn on the device; sequences 0 and 63 are checked
    against the oracle."""
    from workload import kv_history_device
    c = dataclasses.replace(CONFIGS["llama8b_32k"], name="many_tiles", seed=21, batch=64, context=16384)
    n = c.n_windows
    p = Pair(c, seqs=[0, 63])
    K = torch.empty((c.batch, c.kv_heads, c.context, c.head_dim), dtype=torch.int16, device="cuda")
    V = torch.empty_like(K)
    for b in range(c.batch):
        K[b], V[b] = kv_history_device(c, 0, b, "cuda")
    prior = np.stack([score_prior(c, 0, b) for b in range(c.batch)])
    p.pool.prefill(0, K, V, c.context, dev(prior))
    for b in p.seqs:
        seg = CachedSegment(c.kv_heads, c.window, c.head_dim, c.n_recent)
        seg.prefill(K[b].cpu().numpy().view(np.uint16), V[b].cpu().numpy().view(np.uint16),
                    prior=prior[b].astype(np.float64))
        p.oracle[(0, b)] = seg
    del K, V
    rng = np.random.default_rng(5)
    for step, (beta, phi, n_f, n_q) in enumerate([(0.45, 0.1, 12, 116), (1.0, 0.6, 76, 52)]):
        p.route(0, beta, phi)
        pages = p.pool.pages(0).cpu().numpy().view(np.uint32)[:, :n] & 3
        assert (pages == 2).sum(axis=1).tolist() == [n_f] * c.batch
        assert (pages == 1).sum(axis=1).tolist() == [n_q] * c.batch
        p.check_state(0, ledger_sample=16, window_sample=8, rng=rng)
        _, _, _, errs = p.step(0, step)
        log("many tiles per wave (%d bf16 / %d INT2): out err %.2e mass err %.2e" % (n_f, n_q, *errs))
    assert p.pool.check() == 0
