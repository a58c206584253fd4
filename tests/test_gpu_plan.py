"""Transition plans with repeated items, bad items and too few slots.

The plan's outcome is defined as taking the items one by one in list order:
an item outside the window range is an error; a window in the wrong tier is a
state error; a valid item takes a free slot, and when none is left fails with
a no-slot error (kvtier.h, kv_demote_quantize / kv_promote_dequantize).  The
kernel computes all items at once; these lists mix every case, repeat
windows (a repeat after a success sees the moved window, after a failure
fails the same way), and run past 256 items (more than one round of the
workgroup).  The expected tiers and error bits come from walking the list in
order here; the moved windows' bytes are compared with the oracle bit for bit.
"""
import numpy as np
import pytest

from oracle import codec

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_harness import dev, log  # noqa: E402

F, Q = 2, 1
ITEM_RANGE, DEMOTE_STATE, PROMOTE_STATE, NO_BF16, NO_LEDGER = 32, 1, 2, 4, 8


def _walk(tier, has_ledger, items, n, promote, free_slots):
    """The list taken in order: new tiers, error bits, the moved windows."""
    tier = list(tier)
    errs, moved = 0, []
    for w in items:
        if w < 0 or w >= n:
            errs |= ITEM_RANGE
        elif not promote:
            if tier[w] != F:
                errs |= DEMOTE_STATE
            elif has_ledger[w]:
                tier[w] = Q
            elif free_slots > 0:
                free_slots -= 1
                tier[w] = Q
                moved.append(w)
            else:
                errs |= NO_LEDGER
        else:
            if tier[w] != Q or not has_ledger[w]:
                errs |= PROMOTE_STATE
            elif free_slots > 0:
                free_slots -= 1
                tier[w] = F
                moved.append(w)
            else:
                errs |= NO_BF16
    return tier, errs, moved


def _pool(n, ledger_slots, bf16_slots, rng, bits=2):
    from tiered_int2_fp16_amd import binding as B
    W, D = 32, 64
    cfg = B.make_config(1, 1, 1, 1, D, W, n, 1, bf16_slots, ledger_slots, bits)
    pool = B.Pool(cfg)
    kv = rng.standard_normal((2, n * W, D)).astype(np.float32)
    bits = (kv.view(np.uint32) >> 16).astype(np.uint16)
    pool.prefill(0, dev(bits[0].reshape(1, 1, n * W, D)), dev(bits[1].reshape(1, 1, n * W, D)), n * W,
                 dev(np.ones((1, n), np.float32)))
    return pool, bits.reshape(2, n, W, D)


def _state(pool, n):
    pages = pool.pages(0).cpu().numpy().view(np.uint32)[0][:n]
    return (pages & 3).tolist(), ((pages >> 2) & 1).astype(bool).tolist()


@pytest.mark.parametrize("n,ledger_slots,extra", [(16, 3, 0), (512, 280, 40)])
def test_plan_repeats_bad_items_and_exhaustion(n, ledger_slots, extra):
    rng = np.random.default_rng(n)
    pool, bits = _pool(n, ledger_slots, n, rng)
    if n == 16:
        dem = [2, 5, 2, 7, 100, 9, 5, 11, -1, 7]
    else:   # 300 distinct windows, 40 repeats and a few out of range, shuffled
        base = rng.permutation(n - 1)[:300].tolist()
        dem = base + rng.choice(base, extra).tolist() + [n + 3, -7, n - 1 + 100]
        dem = [dem[i] for i in rng.permutation(len(dem))]
    tier0, led0 = _state(pool, n)
    want_tier, want_err, moved = _walk(tier0, led0, dem, n, False, ledger_slots)
    pool.demote(0, dev(np.array([dem], np.int32)), dev(np.array([len(dem)], np.int32)))
    tier, led = _state(pool, n)
    assert tier == want_tier
    assert pool.check() == want_err
    for w in moved[:12] + moved[-4:]:
        got = pool.read_ledger(0, 0, w).cpu().numpy()[0]
        want = codec.entry_bytes(codec.quantize_window(bits[0, w], bits[1, w], 2), 2)
        assert got.tobytes() == want, w
    # promotions: repeats, windows in the wrong tier, and more than the free bf16 slots
    q = [w for w in range(n) if tier[w] == Q]
    free_bf16 = n - sum(1 for w in range(n) if tier[w] == F)
    pro = q[:3] + q[:2] + [0 if tier[0] == F else 1, n + 5] + q[3:]
    want_tier2, want_err2, moved2 = _walk(tier, led, pro, n, True, free_bf16)
    pool.promote(0, dev(np.array([pro], np.int32)), dev(np.array([len(pro)], np.int32)))
    tier2, _ = _state(pool, n)
    assert tier2 == want_tier2
    assert pool.check() == want_err2
    for w in moved2[:8]:
        got = pool.read_window(0, 0, w).cpu().numpy().view(np.uint16)[0]
        e = codec.quantize_window(bits[0, w], bits[1, w], 2)
        wk, wv = codec.promote_bits(e)
        assert np.array_equal(got[0], wk) and np.array_equal(got[1], wv), w
    log(f"{n} windows: {len(dem)} demote items ({len(moved)} moved, errors {want_err:#x}), "
        f"{len(pro)} promote items ({len(moved2)} moved, errors {want_err2:#x})")


@pytest.mark.parametrize("n,ledger_slots,bf16_slots,bits", [(16, 3, 12, 2), (512, 280, 400, 2), (64, 40, 48, 4)])
def test_one_launch_for_both_lists_matches_two_calls(n, ledger_slots, bf16_slots, bits):
    """kv_apply_transitions against kv_demote_quantize then kv_promote_dequantize
    on twin pools: the same rows, error bits, ledger entries and bf16 windows.
    The promote list names windows the demote list moves in the same call (so
    a promotion reads the entry the quantise kernel has just written and may
    take the bf16 slot a demotion has just freed), older ledger windows,
    repeats, wrong-tier and out-of-range items, and more windows than slots."""
    rng = np.random.default_rng(1000 + n)
    n_live = min(n, bf16_slots)          # prefill puts window w in bf16 slot w
    pools = []
    for _ in range(2):
        pool, bits_kv = _pool(n_live, ledger_slots, bf16_slots, np.random.default_rng(7 + n), bits)
        pools.append(pool)
    n = n_live
    # a first demotion so that some windows already have ledger entries
    first = rng.permutation(n - 1)[: n // 4].tolist()
    for pool in pools:
        pool.demote(0, dev(np.array([first], np.int32)), dev(np.array([len(first)], np.int32)))
    tier0, led0 = _state(pools[0], n)
    assert pools[0].check() == pools[1].check()
    f_now = [w for w in range(n - 1) if tier0[w] == F]
    q_now = [w for w in range(n) if tier0[w] == Q]
    dem = rng.permutation(f_now)[: max(1, 2 * len(f_now) // 3)].tolist()
    dem = dem + dem[:2] + [n + 1, -3] + q_now[:1]
    pro = dem[:3] + q_now[:5] + q_now[:1] + [n + 9] + rng.permutation(q_now)[5:].tolist() + dem[3:]
    d_items, d_cnt = dev(np.array([dem], np.int32)), dev(np.array([len(dem)], np.int32))
    p_items, p_cnt = dev(np.array([pro], np.int32)), dev(np.array([len(pro)], np.int32))
    pools[0].demote(0, d_items, d_cnt)
    pools[0].promote(0, p_items, p_cnt)
    pools[1].transitions(0, d_items, d_cnt, p_items, p_cnt)
    rows = [p.pages(0).cpu().numpy().copy() for p in pools]
    assert np.array_equal(rows[0], rows[1])
    errs = [p.check() for p in pools]
    assert errs[0] == errs[1]
    tier, led = _state(pools[0], n)
    # and both against the lists taken in order
    t1, e1, moved_d = _walk(tier0, led0, dem, n, False, ledger_slots - sum(led0))
    led1 = [led0[w] or w in moved_d for w in range(n)]
    t2, e2, moved_p = _walk(t1, led1, pro, n, True, bf16_slots - sum(1 for t in t1 if t == F))
    assert tier == t2 and errs[0] == e1 | e2
    if n > 16:   # windows demoted and promoted back in the same call
        assert set(moved_d) & set(moved_p)
    for w in range(n):
        if tier[w] != 0 and led[w]:
            a = pools[0].read_ledger(0, 0, w).cpu().numpy()
            b = pools[1].read_ledger(0, 0, w).cpu().numpy()
            assert a.tobytes() == b.tobytes(), ("ledger", w)
        if tier[w] == F:
            a = pools[0].read_window(0, 0, w).cpu().numpy()
            b = pools[1].read_window(0, 0, w).cpu().numpy()
            assert a.tobytes() == b.tobytes(), ("bf16", w)
    log(f"{n} windows, {bits}-bit ledger: {len(dem)} demote and {len(pro)} promote items in one call, "
        f"errors {errs[0]:#x}, {sum(1 for t in tier if t == F)} bf16 / {sum(1 for t in tier if t == Q)} ledger after")


def test_moves_planned_ahead_on_a_second_stream_match_one_call():
    """kv_plan_transitions for every layer on a second stream, then per layer
    kv_move_planned and a decode step on the first (waiting only for that
    layer's plan), against kv_apply_transitions and the same decode step per
    layer on one stream: pages, scores, ledger entries, bf16 windows, outputs
    and masses bit for bit (three layers, so that later plans run ahead of
    earlier layers' moves and each layer keeps its own work lists)."""
    from tiered_int2_fp16_amd import binding as B
    L, Bsz, Hq, Hkv, D, W, n = 3, 2, 8, 2, 64, 64, 24
    rng = np.random.default_rng(77)
    kv = [rng.standard_normal((2, Bsz, Hkv, n * W, D)).astype(np.float32) for _ in range(L)]
    kvb = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in kv]
    prior = [rng.lognormal(0.0, 1.0, (Bsz, n)).astype(np.float32) for _ in range(L)]
    q = [dev(((rng.standard_normal((Bsz, Hq, D)).astype(np.float32)).view(np.uint32) >> 16)
             .astype(np.uint16).view(np.int16)) for _ in range(L)]
    pools = []
    for _ in range(2):
        pool = B.Pool(B.make_config(Bsz, L, Hq, Hkv, D, W, n, 2, n, 20, 2))
        for l in range(L):
            pool.prefill(l, dev(kvb[l][0].view(np.int16)), dev(kvb[l][1].view(np.int16)), n * W, dev(prior[l]))
            tr, cn = pool.score_route(l, None, 1, 0.4, 0.25)
            pool.transitions(l, tr[0], cn[0], tr[1], cn[1])
        pools.append(pool)
    torch.cuda.synchronize()
    assert pools[0].check() == 0 and pools[1].check() == 0
    # per layer: demote half of the non-recent bf16 windows, promote the ledger
    # windows of highest prior (repeats and a wrong-tier item included)
    dems, pros = [], []
    for l in range(L):
        pg = pools[0].pages(l).cpu().numpy().view(np.uint32)[:, :n] & 3
        d = np.zeros((Bsz, n), np.int32)
        p = np.zeros((Bsz, n), np.int32)
        cd, cp = np.zeros(Bsz, np.int32), np.zeros(Bsz, np.int32)
        for b in range(Bsz):
            f = [w for w in range(n - 2) if pg[b][w] == F][::2]
            qq = sorted([w for w in range(n) if pg[b][w] == Q], key=lambda w: -prior[l][b][w])[:3]
            lst_d = f + f[:1]
            lst_p = qq + f[1:2] + qq[:1]
            d[b, :len(lst_d)], p[b, :len(lst_p)] = lst_d, lst_p
            cd[b], cp[b] = len(lst_d), len(lst_p)
        dems.append((dev(d), dev(cd)))
        pros.append((dev(p), dev(cp)))
    outs = [[torch.empty(Bsz, Hq, D, dtype=torch.float32, device="cuda") for _ in range(L)] for _ in range(2)]
    masses = [[torch.zeros(Bsz, Hq, n, dtype=torch.float32, device="cuda") for _ in range(L)] for _ in range(2)]
    for l in range(L):
        pools[0].transitions(l, dems[l][0], dems[l][1], pros[l][0], pros[l][1])
        pools[0].attn(l, q[l], out=outs[0][l], mass=masses[0][l], scores=True)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev0 = torch.cuda.Event()
    ev0.record(main)
    side.wait_event(ev0)
    evs = []
    for l in range(L):
        pools[1].plan_transitions(l, dems[l][0], dems[l][1], pros[l][0], pros[l][1], stream=side)
        evs.append(torch.cuda.Event())
        evs[-1].record(side)
    for l in range(L):
        main.wait_event(evs[l])
        pools[1].move_planned(l)
        pools[1].attn(l, q[l], out=outs[1][l], mass=masses[1][l], scores=True)
    main.wait_stream(side)
    torch.cuda.synchronize()
    errs = [p.check() for p in pools]
    assert errs[0] == errs[1] == DEMOTE_STATE | PROMOTE_STATE
    for l in range(L):
        assert torch.equal(outs[0][l], outs[1][l]) and torch.equal(masses[0][l], masses[1][l]), l
        assert torch.equal(pools[0].pages(l), pools[1].pages(l)), l
        assert torch.equal(pools[0].scores(l), pools[1].scores(l)), l
        pg = pools[0].pages(l).cpu().numpy().view(np.uint32)[:, :n]
        for b in range(Bsz):
            for w in range(n):
                if (pg[b][w] & 3) == F:
                    assert torch.equal(pools[0].read_window(l, b, w), pools[1].read_window(l, b, w)), (l, b, w)
                if (pg[b][w] & 3) != 0 and (pg[b][w] >> 2) & 1:
                    assert torch.equal(pools[0].read_ledger(l, b, w), pools[1].read_ledger(l, b, w)), (l, b, w)
    log(f"{L} layers planned ahead on a second stream: identical to one call per layer")
