"""Parity of the HIP path (through the C ABI) with the oracle, on MI355X.

Inputs are the seeded workloads; expected values come from the oracle run on
the same bf16 bits.  Sizes: the tiny shape in full (every tile, ragged tails,
appends that open new windows, routing with demote/promote traffic), and the
32K Llama / Qwen shapes and the 128K loop at their full sizes (all outputs of
the 32K shapes; all outputs of two of the four 128K sequences).
"""
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS
from workload.synth import small

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle.router import F, Q  # noqa: E402
from tests.gpu_harness import CachedSegment, Pair, dev, log  # noqa: E402
from workload import score_prior  # noqa: E402


def test_tiny_route_state_and_attention():
    c = CONFIGS["tiny"]
    p = Pair(c)
    p.load(0)
    tr, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert (cnt[0][0], cnt[2][0]) == (12, 12)  # 12 windows quantised, 12 evicted
    p.check_state(0)
    _, _, _, errs = p.step(0, 0)
    log("tiny: out err %.2e mass err %.2e" % errs)


def test_tiny_decode_loop_with_routing():
    """Append 200 tokens (3 new windows), accumulate mass every step, route
    every 16 steps with the resulting demote/promote/evict traffic."""
    c = dataclasses.replace(CONFIGS["tiny"], steps=200, route_every=16, append=True)
    p = Pair(c)
    p.load(0)
    p.route(0, c.budget_frac, c.hi_frac)
    p.check_state(0)
    moved = 0
    for s in range(c.steps):
        _, mass, o_mass, _ = p.step(0, s, append=True)
        p.add_scores(0, mass, o_mass)
        if (s + 1) % c.route_every == 0:
            _, cnt = p.route(0, c.budget_frac, c.hi_frac)
            moved += int(cnt[0].sum() + cnt[1].sum())
            p.check_state(0)
    log(f"tiny loop: {moved} demotions+promotions")
    assert moved > 0


def test_write_once_ledger_on_gpu():
    c = CONFIGS["tiny"]
    p = Pair(c)
    p.load(0)
    seg = p.oracle[(0, 0)]
    items = dev(np.array([[3, 5]], np.int32))
    one = dev(np.array([2], np.int32))
    p.pool.demote(0, items, one)
    seg.demote(3)
    seg.demote(5)
    first = p.pool.read_ledger(0, 0, 3).cpu().numpy().copy()
    p.pool.promote(0, items[:, :1], dev(np.array([1], np.int32)))
    seg.promote(3)
    p.check_state(0)
    p.pool.demote(0, items[:, :1], dev(np.array([1], np.int32)))
    seg.demote(3)
    again = p.pool.read_ledger(0, 0, 3).cpu().numpy()
    assert again.tobytes() == first.tobytes()
    assert seg.quantized[3] == 1
    p.check_state(0)
    p.step(0, 0)


def test_device_state_errors_are_reported():
    c = CONFIGS["tiny"]
    p = Pair(c, ledger_slots=2)
    p.load(0)
    one = dev(np.array([1], np.int32))
    p.pool.promote(0, dev(np.array([[4]], np.int32)), one)       # bf16 window: not INT2
    assert p.pool.check() & 2
    p.pool.demote(0, dev(np.array([[40]], np.int32)), one)       # out of range
    assert p.pool.check() & 32
    p.pool.demote(0, dev(np.array([[1, 2, 3]], np.int32)), dev(np.array([3], np.int32)))
    assert p.pool.check() & 8                                    # only 2 ledger slots
    p.pool.read_window(0, 0, 3)                                  # window 3 stayed bf16
    assert p.pool.check() == 0
    p.pool.read_ledger(0, 0, 9)
    assert p.pool.check() & 64


def test_device_state_errors_demote_slots_append_capacity():
    """The other four error bits, each forced through the C ABI (or, for an
    append into a window that is not bf16 - a state no call of the library
    produces, since the newest window always stays bf16 - by writing that
    page-table entry of the caller-owned arena from the host).  Each bit is
    read and cleared by kv_pool_check, and the offending item is skipped."""
    from workload import new_kv
    one = dev(np.array([1], np.int32))
    # 1 DEMOTE_STATE: a window already in the ledger tier, then the newest,
    # partial window
    c = dataclasses.replace(CONFIGS["tiny"], context=2048 - 17)
    p = Pair(c)
    p.load(0)
    w3 = dev(np.array([[3]], np.int32))
    p.pool.demote(0, w3, one)
    assert p.pool.check() == 0
    p.pool.demote(0, w3, one)
    assert p.pool.check() == 1
    p.pool.demote(0, dev(np.array([[31]], np.int32)), one)
    assert p.pool.check() == 1
    pages = p.pool.pages(0).cpu().numpy().view(np.uint32)[0]
    assert pages[31] & 3 == F and pages[3] & 3 == Q
    # 16 APPEND_STATE: the partial window 31 set to the ledger tier (window 3's
    # entry) from the host; the step's token is not stored
    p.pool.pages(0)[0, 31] = int((pages[3] & ~np.uint32(0x1FFF8)))   # tier Q, has-ledger, slot of window 3
    kn, vn = new_kv(c, 0, 0)
    p.pool.attn(0, dev(__import__("workload").query(c, 0, 0)), dev(kn), dev(vn))
    assert p.pool.check() == 16
    assert int(p.pool.tokens(0)[0]) == c.context
    # 4 NO_BF16_SLOT: a full context whose 32 windows take every bf16 slot;
    # the append that opens window 32 finds none
    ca = dataclasses.replace(CONFIGS["tiny"], steps=1, append=True)
    p = Pair(ca, bf16_slots=32)
    p.load(0)
    kn, vn = new_kv(ca, 0, 0)
    p.pool.attn(0, dev(__import__("workload").query(ca, 0, 0)), dev(kn), dev(vn))
    assert p.pool.check() == 4
    assert int(p.pool.tokens(0)[0]) == ca.context
    # 128 CAPACITY: the page table has no room for window 32
    p = Pair(CONFIGS["tiny"])
    assert p.maxw == 32
    p.load(0)
    p.pool.attn(0, dev(__import__("workload").query(ca, 0, 0)), dev(kn), dev(vn))
    assert p.pool.check() == 128
    assert int(p.pool.tokens(0)[0]) == ca.context
    assert p.pool.check() == 0


def test_llama_32k_full():
    c = CONFIGS["llama8b_32k"]
    p = Pair(c)
    p.load(0)
    _, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert cnt[0][0] == 139 and cnt[2][0] == 92
    p.check_state(0, ledger_sample=40, window_sample=10, rng=np.random.default_rng(0))
    out, mass, _, errs = p.step(0, 0)
    log("llama 32K: out err %.2e mass err %.2e" % errs)
    # determinism and the mass-free path
    out2, mass2 = p.pool.attn(0, dev(__import__("workload").query(c, 0, 0)))
    assert torch.equal(out, out2) and torch.equal(mass, mass2)
    out3, _ = p.pool.attn(0, dev(__import__("workload").query(c, 0, 0)), want_mass=False)
    assert torch.equal(out, out3)


def test_qwen_32k_full():
    c = CONFIGS["qwen7b_32k"]
    p = Pair(c)
    p.load(0)
    _, cnt = p.route(0, c.budget_frac, c.hi_frac)
    assert (cnt[0] == 41).all() and (cnt[2] == 210).all()
    p.check_state(0, ledger_sample=8, window_sample=3, rng=np.random.default_rng(1))
    _, _, _, errs = p.step(0, 0)
    log("qwen 32K: out err %.2e mass err %.2e" % errs)


@pytest.mark.timeout(900)
def test_llama_128k_loop_sampled():
    """The 128K loop shape: 17 decode steps appending a token each (the first
    opens window 1024), scores every step, routing after step 16; two of the
    four sequences compared in full against the oracle."""
    c = CONFIGS["llama8b_128k_loop"]
    p = Pair(c, seqs=[0, 3])
    p.load(0)
    log("128K: loaded")
    p.route(0, c.budget_frac, c.hi_frac)
    p.check_state(0, ledger_sample=12, window_sample=4, rng=np.random.default_rng(2))
    for s in range(17):
        _, mass, o_mass, errs = p.step(0, s, append=True)
        p.add_scores(0, mass, o_mass)
        log("128K step %d: out err %.2e mass err %.2e" % (s, *errs))
        if (s + 1) % c.route_every == 0:
            p.route(0, c.budget_frac, c.hi_frac)
            p.check_state(0, ledger_sample=12, window_sample=4, rng=np.random.default_rng(3))


def test_decode_step_fuses_the_score_update_bit_exactly():
    """kv_decode_step == kv_tiered_decode_attn + kv_score_route, bit for bit."""
    from workload import query
    c = CONFIGS["llama8b_32k"]
    a, b = Pair(c, seqs=[]), Pair(c, seqs=[])
    for p in (a, b):
        p.load(0)
        p.route(0, c.budget_frac, c.hi_frac)
    for s in range(3):
        q = dev(query(c, 0, s))
        oa, ma = a.pool.attn(0, q)
        a.pool.score_route(0, ma, 0)
        ob, mb = b.pool.attn(0, q, scores=True)
        assert torch.equal(oa, ob) and torch.equal(ma, mb)
        assert torch.equal(a.pool.scores(0), b.pool.scores(0))
    assert a.pool.check() == 0 and b.pool.check() == 0


@pytest.mark.gpu
def test_mistral_full_step_sampled():
    """The Mistral-7B full step at full size: 32 layers x 32 sequences, 16K
    context.  Per (layer, sequence): route to the pre-state (12 bf16 / 21 INT2 /
    95 evicted windows), demote the 8 non-recent bf16 windows (first
    quantisation into the ledger), promote the 4 highest-score windows of the
    pre-state INT2 tier (older ledger entries), then one attention step.  The
    contexts are drawn on the device (they are 34 G values); the oracle checks
    sampled (layer, sequence) pairs on copies of their inputs: routing
    bit-exact, ledger bytes, promoted bf16, output and window mass."""
    from workload import kv_history_device
    c = CONFIGS["mistral7b_step"]
    checked = {0: [0, 31], 13: [7], 31: [0, 20]}
    n, R = c.n_windows, c.n_recent
    p = Pair(c, seqs=[], bf16_slots=n, ledger_slots=40)
    rng = np.random.default_rng(4)
    for layer in range(c.layers):
        p.seqs = checked.get(layer, [])
        K = torch.empty((c.batch, c.kv_heads, c.context, c.head_dim), dtype=torch.int16, device="cuda")
        V = torch.empty_like(K)
        for b in range(c.batch):
            K[b], V[b] = kv_history_device(c, layer, b, "cuda")
        prior = np.stack([score_prior(c, layer, b) for b in range(c.batch)])
        p.pool.prefill(layer, K, V, c.context, dev(prior))
        for b in p.seqs:
            seg = CachedSegment(c.kv_heads, c.window, c.head_dim, c.n_recent)
            seg.prefill(K[b].cpu().numpy().view(np.uint16), V[b].cpu().numpy().view(np.uint16),
                        prior=prior[b].astype(np.float64))
            p.oracle[(layer, b)] = seg
        del K, V
        # the pre-state: 12 bf16 (4 recent + 8), 21 INT2, 95 evicted
        _, cnt = p.route(layer, c.pre_budget_frac, c.pre_hi_frac)
        pages = p.pool.pages(layer).cpu().numpy().view(np.uint32)[:, :n] & 3
        assert (pages == F).sum(axis=1).tolist() == [12] * c.batch
        assert (pages == Q).sum(axis=1).tolist() == [21] * c.batch
        # the move set: demote the 8 non-recent bf16 windows, then promote the
        # 4 highest-score windows of the pre-state INT2 tier (score descending,
        # lower index first), whose ledger entries were written by the
        # pre-state routing - not the windows demoted a moment earlier
        S = p.pool.scores(layer).cpu().numpy()[:, :n]
        dem = np.zeros((c.batch, n), np.int32)
        pro = np.zeros((c.batch, n), np.int32)
        for b in range(c.batch):
            d = [w for w in range(n - R) if pages[b][w] == F]
            assert len(d) == c.demote_per_seg
            dem[b, : len(d)] = d
            q_pre = [w for w in range(n) if pages[b][w] == Q]   # ledger entries from the pre-state routing
            top = sorted(q_pre, key=lambda w: (-float(S[b][w]), w))[: c.promote_per_seg]
            pro[b, : len(top)] = sorted(top)
        cnt_d = np.full(c.batch, c.demote_per_seg, np.int32)
        cnt_p = np.full(c.batch, c.promote_per_seg, np.int32)
        # both lists in one call, as the bench's step makes them (one plan launch)
        p.pool.transitions(layer, dev(dem), dev(cnt_d), dev(pro), dev(cnt_p))
        for b in p.seqs:
            seg = p.oracle[(layer, b)]
            for w in dem[b][: c.demote_per_seg]:
                seg.demote(int(w))
            for w in pro[b][: c.promote_per_seg]:
                seg.promote(int(w))
        pages = p.pool.pages(layer).cpu().numpy().view(np.uint32)[:, :n] & 3
        assert (pages == F).sum(axis=1).tolist() == [8] * c.batch
        assert (pages == Q).sum(axis=1).tolist() == [25] * c.batch
        if p.seqs:
            p.check_state(layer, ledger_sample=12, window_sample=8, rng=rng)
        _, _, _, errs = p.step(layer, 0, check=bool(p.seqs))
        if p.seqs:
            log("mistral layer %d: out err %.2e mass err %.2e" % (layer, *errs))
        if layer % 8 == 7:
            log(f"mistral: {layer + 1} layers done")
    assert p.pool.check() == 0
