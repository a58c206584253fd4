"""Benchmark of the tiered decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]

Headline workload (default): the Llama-3.1-8B attention shape at 32K context
(batch 1, 32 query / 8 kv heads, head_dim 128, windows of 128 tokens, 20 % byte
budget with 10 % of windows in bf16: 25 bf16 / 139 INT2 / 92 evicted windows),
synthetic seeded data.  One step = one decode step over the tiered cache
(kv_decode_step: the attention kernel and its combine kernel, which writes the
per-window mass and adds it to the cumulative scores), and every 16th step of a
pool a routing event (router, demotions into the write-once ledger,
promotions).  Steps rotate over enough pool replicas (each its own arena) that
every step reads its windows from HBM, not from the 256 MB Infinity Cache; the
replicas' routing phases are staggered, so about one step in 16 of any timed
region carries a routing event (the line reports how many did).

The timed region replays a HIP graph of exactly K steps between two device
synchronisations.  The attention kernel's own duration is then taken over the
same K steps run eagerly with dispatch timing events (hipExtLaunchKernel),
queued behind replays of the graph so that they run back to back.

Beside the headline the default run reports, each with its own roofline and
the oracle timed on a bounded sample of it:
  * `ceiling`: a plain streaming read (kv_stream_probe) of the step's bytes
    on the attention's grid, cold, timed by the same dispatch events;
  * `workloads.qwen7b_32k`: the Qwen2.5-7B shape (batch 8, 28 query / 4 kv
    heads, 5 bf16 / 41 INT2 / 210 evicted windows per sequence);
  * `workloads.llama8b_128k_loop`: 64 consecutive decode steps at 128K
    context (batch 4), each appending a token, routing after every 16;
  * `workloads.mistral7b_step`: the Mistral-7B full step, 32 layers x 32
    sequences at 16K, each (layer, sequence) demoting 8 windows (first
    quantisation into the ledger), promoting 4 and then attending.
`--workload NAME --only` runs one of them as the whole line (for profiling).

`--ledger-bits 4` or `8` gives the pools a 4-bit or 8-bit ledger instead of
INT2 (same budget: fewer ledger windows, b + 1 bits per value each).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from workload import CONFIGS, kv_history, kv_history_device, new_kv, query, score_prior  # noqa: E402

HBM_PEAK_GBS = 8000.0
ROUTE_EVERY = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_bytes(c, n_f, n_q, n_windows, bits=2):
    """Algorithmic bytes of one attention launch: every bf16 window's K and V
    (4*W*D per kv head), every ledger window's codes + fp16 scale/min
    ((b+1)*W*D/4: 3*W*D/4 for INT2), the query, the output, the window masses
    and the page table."""
    wd = c.window * c.head_dim
    kv = c.batch * c.kv_heads * (n_f * 4 * wd + n_q * (bits + 1) * wd // 4)
    io = c.batch * c.q_heads * c.head_dim * (2 + 4) + c.batch * c.q_heads * n_windows * 4
    return kv + io + c.batch * n_windows * 4


def score_bytes(c, n_windows):
    return c.batch * c.q_heads * n_windows * 4 + c.batch * n_windows * (8 + 4)


def move_bytes(c, windows, bits=2):
    """Algorithmic bytes of demoting (read the bf16 K and V, write the ledger
    entry) or promoting (the reverse) `windows` windows of all kv heads."""
    wd = c.window * c.head_dim
    return windows * c.kv_heads * (4 * wd + (bits + 1) * wd // 4)


def route_bytes(c, n_windows, first_quant, promotions, bits=2):
    return c.batch * n_windows * (4 + 4) + move_bytes(c, first_quant + promotions, bits)


# the sources the attention kernel is compiled from (the traffic counters of a
# launch depend on these alone), and its build flags
ATTN_SOURCES = ("attn.hip", "device_common.h", "layout.h", "launch.h")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "tiered_int2_fp16_amd", "csrc", f), "rb").read())
    h.update(open(os.path.join(ROOT, "tiered_int2_fp16_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash):
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "attn_kernel_llama8b_32k_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_hash:
        return None
    return d.get("bytes_per_launch")


def blas_cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


# ------------------------------------------------------------ oracle timing
def cpu_baseline(c, seconds):
    """The oracle (plain numpy float64) timed on the host on a sample of the
    workload: decode steps of one sequence (tiered attention + window mass +
    score update; with appends and routing every 16 steps for the decode loop)
    until about `seconds` of work.  Host-drawn inputs of the workload's shape
    and distributions (the GPU's larger workloads draw theirs on the device)."""
    from oracle.pool import Segment
    k, v = kv_history(c, 0, 0)
    prior = score_prior(c, 0, 0).astype(np.float64)
    seg = Segment(c.kv_heads, c.window, c.head_dim, c.n_recent)
    seg.prefill(k, v, prior=prior)
    seg.route(c.budget_frac, c.hi_frac)
    del k, v
    n_f, n_q = seg.tier.count(2), seg.tier.count(1)
    one = type("one", (), {})()
    for f in ("window", "head_dim", "kv_heads", "q_heads"):
        setattr(one, f, getattr(c, f))
    one.batch = 1
    steps, moved = 0, 0
    t0 = time.perf_counter()
    while True:
        q = query(c, 0, steps)
        if c.append:
            kn, vn = new_kv(c, 0, steps)
            seg.append(kn[0], vn[0])
        _, mass = seg.attend(q[0])
        seg.add_scores(mass)
        steps += 1
        if c.route_every and steps % c.route_every == 0:
            tr = seg.route(c.budget_frac, c.hi_frac)
            moved += len(tr["first_quant"]) + len(tr["promote"])
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_step = attn_bytes(one, n_f, n_q, seg.n) + score_bytes(one, seg.n)
    total = per_step * steps + move_bytes(one, moved)
    what = "appending a token, routing every 16 steps, " if c.append else ""
    return {"value": round(total / el / 1e9, 4), "unit": "GB/s", "cores": blas_cores(), "kind": "oracle",
            "sample": f"{steps} decode steps of one sequence of the {c.name} workload ({what}attention with "
                      f"window mass + score update, {c.kv_heads} kv heads, {c.context} cached tokens) in "
                      f"{el:.1f} s, {steps / el:.3f} sequence-steps/s; a full step has {c.batch} sequence(s)"}


def cpu_baseline_full_step(c, seconds):
    """The oracle on (layer, sequence) segments of the Mistral full step: route
    to the pre-state, then (timed) demote the 8 non-recent bf16 windows, promote
    the 4 highest-score ledger windows and attend, segment after segment until
    about `seconds` of timed work; extrapolated per step of 32 x 32 segments."""
    from oracle.pool import Segment
    from oracle.router import F, Q
    one = type("one", (), {})()
    for f in ("window", "head_dim", "kv_heads", "q_heads"):
        setattr(one, f, getattr(c, f))
    one.batch = 1
    done, el, nbytes = 0, 0.0, 0
    while el < seconds:
        layer, b = done // c.batch, done % c.batch
        k, v = kv_history(c, layer, b)
        seg = Segment(c.kv_heads, c.window, c.head_dim, c.n_recent)
        seg.prefill(k, v, prior=score_prior(c, layer, b).astype(np.float64))
        seg.route(c.pre_budget_frac, c.pre_hi_frac)
        n = seg.n
        dem = [w for w in range(n - c.n_recent) if seg.tier[w] == F]
        pro = sorted([w for w in range(n) if seg.tier[w] == Q], key=lambda w: (-seg.S[w], w))[: c.promote_per_seg]
        q = query(c, layer, 0)
        t0 = time.perf_counter()
        for w in dem:
            seg.demote(w)
        for w in pro:
            seg.promote(w)
        _, mass = seg.attend(q[b])
        seg.add_scores(mass)
        el += time.perf_counter() - t0
        nbytes += attn_bytes(one, seg.tier.count(F), seg.tier.count(Q), n) + score_bytes(one, n) + \
            move_bytes(one, len(dem) + len(pro))
        done += 1
    segs = c.layers * c.batch
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": blas_cores(), "kind": "oracle",
            "sample": f"{done} of the {segs} (layer, sequence) segments of one step (demote 8, promote 4, attend, "
                      f"score update) in {el:.1f} s of timed work, {el / done:.3f} s per segment: "
                      f"{el / done * segs:.1f} s per full step extrapolated"}


# ------------------------------------------------------------------ ceiling
def stream_ceiling(B, torch, dev, nbytes, workgroups, count=48):
    """Cold streaming reads of `nbytes` (kv_stream_probe) on `workgroups`
    workgroups, rotating over a buffer larger than the Infinity Cache; median
    of the dispatch-event durations."""
    stride = ((nbytes + 4095) // 4096) * 4096
    count = max(4, min(count, (3 << 30) // stride - 1))
    buf = torch.ones((count + 1) * stride, dtype=torch.uint8, device=dev)
    sink = torch.empty(workgroups * 4, dtype=torch.int32, device=dev)
    B.kv_stream_probe(buf, nbytes, stride, count, workgroups, sink)            # warm-up
    ms = sorted(B.kv_stream_probe(buf, nbytes, stride, count, workgroups, sink))
    del buf
    us = 1e3 * ms[len(ms) // 2]
    return {"bytes": nbytes, "workgroups": workgroups, "launches": count, "us": round(us, 3),
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


# ----------------------------------------------------------- decode workloads
def decode_workload(c, B, torch, dev, steps, warmup, replicas, bits=2, extras=False):
    """Graph-timed decode steps of workload `c` over `replicas` pools; returns
    the measurement dict (see the module docstring)."""
    loop = c.append
    n = c.n_windows
    R = replicas
    if c.batch > 1:
        # device-drawn contexts; with appends, room for the windows that every
        # pass below opens (warm-up, timed region, its six replays, event pass)
        K = torch.empty((c.batch, c.kv_heads, c.context, c.head_dim), dtype=torch.int16, device=dev)
        V = torch.empty_like(K)
        for b in range(c.batch):
            K[b], V[b] = kv_history_device(c, 0, b, dev)
        P = torch.from_numpy(np.stack([score_prior(c, 0, b) for b in range(c.batch)])).to(dev)
        appended = -(-(warmup + 8 * steps + 16) // R) if loop else 0
        maxw = -(-(c.context + appended) // c.window) + (1 if loop else 0)
    else:
        k, v = kv_history(c, 0, 0)
        K = torch.from_numpy(k.view(np.int16)[None]).to(dev)
        V = torch.from_numpy(v.view(np.int16)[None]).to(dev)
        P = torch.from_numpy(score_prior(c, 0, 0)[None]).to(dev)
        maxw = n
    nq = 16
    Q = [torch.from_numpy(query(c, 0, s).view(np.int16)).to(dev) for s in range(nq)]
    KN, VN = [], []
    if loop:
        for s in range(nq):
            kn, vn = new_kv(c, 0, s)
            KN.append(torch.from_numpy(kn.view(np.int16)).to(dev))
            VN.append(torch.from_numpy(vn.view(np.int16)).to(dev))
    cfg = B.make_config(c.batch, c.layers, c.q_heads, c.kv_heads, c.head_dim, c.window, maxw,
                        c.n_recent, maxw, maxw, bits)
    pools, outs, masses, trs, cnts = [], [], [], [], []
    for r in range(R):
        p = B.Pool(cfg, dev)
        p.prefill(0, K, V, c.context, P)
        tr = torch.zeros(3, c.batch, maxw, dtype=torch.int32, device=dev)
        cn = torch.zeros(4, c.batch, dtype=torch.int32, device=dev)
        p.score_route(0, None, 1, c.budget_frac, c.hi_frac, tr, cn)
        p.apply_route(0, tr, cn)
        pools.append(p)
        outs.append(torch.empty(c.batch, c.q_heads, c.head_dim, dtype=torch.float32, device=dev))
        masses.append(torch.zeros(c.batch, c.q_heads, maxw, dtype=torch.float32, device=dev))
        trs.append(tr)
        cnts.append(cn)
    K_keys = K if extras else None   # for the prefill-score pass below
    del K, V
    torch.cuda.synchronize()
    pages = pools[0].pages(0).cpu().numpy() & 3
    n_f, n_q = int((pages[0] == 2).sum()), int((pages[0] == 1).sum())
    assert all(int((pg == 2).sum()) == n_f and int((pg == 1).sum()) == n_q for pg in pages)
    assert all(p.check() == 0 for p in pools)
    log(f"{c.name}: {R} replica(s) ready: {n_f} bf16 / {n_q} {bits}-bit / {n - n_f - n_q} evicted windows")
    # routing phases staggered over the replicas: replica r routes after its
    # local steps 15 - (r mod 16), 31 - (r mod 16), ...
    local = [r % ROUTE_EVERY for r in range(R)]

    def step(i, record=None):
        r = i % R
        p = pools[r]
        if loop:   # kv_decode_step with the step's new token
            p.attn(0, Q[i % nq], KN[i % nq], VN[i % nq], out=outs[r], mass=masses[r], scores=True)
        else:      # kv_decode_step
            p.attn(0, Q[i % nq], out=outs[r], mass=masses[r], scores=True)
        if local[r] % ROUTE_EVERY == ROUTE_EVERY - 1:
            p.score_route(0, None, 1, c.budget_frac, c.hi_frac, trs[r], cnts[r])
            p.apply_route(0, trs[r], cnts[r])
            if record is not None:
                record.append(r)
        local[r] += 1

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    routed = []
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(warmup + i, routed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t_timed = time.perf_counter() - t0
    # demotions that quantised and promotions, from the counts each routing
    # event left (a replica routes at most once in a timed region of <= 16*R steps)
    fq = sum(int(cnts[r][3].sum()) for r in set(routed))
    pr = sum(int(cnts[r][1].sum()) for r in set(routed))
    assert all(p.check() == 0 for p in pools)

    # ---------------------------------------------- attention kernel duration
    # The same K steps again, eagerly, with dispatch events on every attention
    # launch.  Six replays of the timed graph are queued first: they keep the
    # GPU busy while the host issues the eager steps, so those steps run back
    # to back as in the timed region instead of each starting on an idle GPU.
    for p in pools:
        B.kv_attn_profile(p.h, steps // R + 2)
    for _ in range(6):
        g.replay()
    for i in range(steps):
        step(warmup + steps + i)
    durs = []
    for p in pools:
        durs += B.kv_attn_timings(p.h)
        B.kv_attn_profile(p.h, 0)
    attn_ms = float(np.mean(durs))
    del g

    per_attn = attn_bytes(c, n_f, n_q, n, bits)
    total_bytes = steps * (per_attn + score_bytes(c, n)) + \
        len(routed) * route_bytes(c, n, 0, 0, bits) + route_bytes(c, 0, fq, pr, bits)
    value = total_bytes / t_timed / 1e9
    achieved = per_attn / (attn_ms * 1e-3) / 1e9
    res = {
        "value": round(value, 2), "unit": "GB/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(1e3 * t_timed / steps, 5),
        "decode_steps_per_s": round(steps / t_timed, 1),
        "percent_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "attn_kernel_us": round(attn_ms * 1e3, 3),
        "attn_bytes": per_attn,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "routing_events_timed": len(routed),
        "tiers": {"bf16": n_f, "ledger": n_q, "evicted": n - n_f - n_q},
        "replicas": R,
    }
    if not extras:
        return res

    # -------------------------------------- cost of emitting the window mass
    def step_graph(with_mass, count):
        gr = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream(device=dev)
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(gr, stream=st):
                for i in range(count):
                    r = i % R
                    if with_mass:
                        pools[r].attn(0, Q[i % nq], out=outs[r], mass=masses[r], scores=True)
                    else:
                        pools[r].attn(0, Q[i % nq], out=outs[r], want_mass=False)
        torch.cuda.synchronize()
        return gr

    def replay_us(gr, count):
        gr.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        gr.replay()
        torch.cuda.synchronize()
        return 1e6 * (time.perf_counter() - t) / count

    n_me = max(R, min(steps, 256))
    g_with, g_without = step_graph(True, n_me), step_graph(False, n_me)
    mass_us = [replay_us(g_with, n_me), replay_us(g_without, n_me), replay_us(g_with, n_me),
               replay_us(g_without, n_me)]
    del g_with, g_without
    res["mass_emission"] = {"steps": n_me, "with_mass_us": round((mass_us[0] + mass_us[2]) / 2, 3),
                            "without_mass_us": round((mass_us[1] + mass_us[3]) / 2, 3)}
    res["mass_emission"]["overhead_us"] = round(res["mass_emission"]["with_mass_us"]
                                                - res["mass_emission"]["without_mass_us"], 3)

    # ------------------------------------------------ routing diagnostics
    diag = torch.zeros(c.batch, 5, dtype=torch.float32, device=dev)
    gd = torch.cuda.CUDAGraph()
    sd = torch.cuda.Stream(device=dev)
    sd.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sd):
        with torch.cuda.graph(gd, stream=sd):
            for i in range(n_me):
                pools[i % R].diagnostics(0, diag, counts=cnts[i % R], shadow_mass=masses[i % R])
    torch.cuda.synchronize()
    diag_us = replay_us(gd, n_me)
    del gd
    diag_bytes = c.batch * (maxw * 4 + c.q_heads * n * 4 + 5 * 4 + 3 * 4)
    res["route_diagnostics"] = {"calls": n_me, "us_per_call": round(diag_us, 3), "bytes_per_call": diag_bytes,
                                "gbs": round(diag_bytes / (diag_us * 1e-6) / 1e9, 2)}

    # ------------------------------------- initial scores from the prefill
    # kv_prefill_scores on the 32K context: causal attention of 32768 prefill
    # queries (drawn on the device) over the context's keys, twice (row
    # normalisers, then column sums), then window sums.  Algorithmic work:
    # 2 passes x q_heads x T (T + 1) / 2 query-key pairs x D multiply-adds.
    if K_keys is not None and c.batch == 1:
        gq = torch.Generator(device=dev)
        gq.manual_seed(int(np.random.SeedSequence([c.seed, 99]).generate_state(1, np.uint64)[0] >> 1))
        qf = torch.randn((c.batch, c.q_heads, c.context, c.head_dim), generator=gq, device=dev)
        qp = (qf.view(torch.int32) >> 16).to(torch.int16)
        del qf
        ws = pools[0].prefill_scores(0, qp, K_keys, c.context)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            pools[0].prefill_scores(0, qp, K_keys, c.context, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        pf_ms = e0.elapsed_time(e1) / reps
        flops = 2.0 * c.q_heads * c.context * (c.context + 1) / 2 * c.head_dim * 2 * c.batch
        res["prefill_scores"] = {"tokens": c.context, "ms": round(pf_ms, 3),
                                 "tflops": round(flops / (pf_ms * 1e-3) / 1e12, 1), "bound": "mfma",
                                 "peak_tflops": 2500.0, "frac": round(flops / (pf_ms * 1e-3) / 1e12 / 2500.0, 4)}
        del qp, ws
    del K_keys
    return res


def full_step_workload(c, B, torch, dev, steps, warmup, bits=2):
    """The Mistral-7B full step: 32 layers x 32 sequences at 16K context.  Each
    (layer, sequence) is routed to the pre-state (12 bf16 / 21 ledger / 95
    evicted windows); a step then demotes, per layer and sequence, the 8
    non-recent bf16 windows (first quantisation into the ledger), promotes the
    4 highest-score windows of the pre-state ledger tier, and runs the decode
    step (attention, window mass, score update).  Between timed steps the page
    tables go back to the pre-state (a 512 KB device copy inside the timed
    graph), so every step demotes into the ledger for the first time again."""
    F, Q = B.KV_TIER_F, B.KV_TIER_Q
    n, R = c.n_windows, c.n_recent
    cfg = B.make_config(c.batch, c.layers, c.q_heads, c.kv_heads, c.head_dim, c.window, n, R, n, 40, bits)
    pool = B.Pool(cfg, dev)
    for layer in range(c.layers):
        K = torch.empty((c.batch, c.kv_heads, c.context, c.head_dim), dtype=torch.int16, device=dev)
        V = torch.empty_like(K)
        for b in range(c.batch):
            K[b], V[b] = kv_history_device(c, layer, b, dev)
        prior = torch.from_numpy(np.stack([score_prior(c, layer, b) for b in range(c.batch)])).to(dev)
        pool.prefill(layer, K, V, c.context, prior)
        del K, V
        tr, cn = pool.score_route(layer, None, 1, c.pre_budget_frac, c.pre_hi_frac)
        pool.apply_route(layer, tr, cn)
    torch.cuda.synchronize()
    assert pool.check() == 0
    dem_l, pro_l = [], []
    for layer in range(c.layers):
        pages = pool.pages(layer).cpu().numpy().view(np.uint32)[:, :n] & 3
        S = pool.scores(layer).cpu().numpy()[:, :n]
        dem = np.zeros((c.batch, n), np.int32)
        pro = np.zeros((c.batch, n), np.int32)
        for b in range(c.batch):
            d = [w for w in range(n - R) if pages[b][w] == F]
            assert len(d) == c.demote_per_seg and int((pages[b] == Q).sum()) == 21
            dem[b, : len(d)] = d
            q_pre = [w for w in range(n) if pages[b][w] == Q]
            pro[b, : c.promote_per_seg] = sorted(sorted(q_pre, key=lambda w: (-float(S[b][w]), w))[: c.promote_per_seg])
        dem_l.append(torch.from_numpy(dem).to(dev))
        pro_l.append(torch.from_numpy(pro).to(dev))
    cnt_d = torch.full((c.batch,), c.demote_per_seg, dtype=torch.int32, device=dev)
    cnt_p = torch.full((c.batch,), c.promote_per_seg, dtype=torch.int32, device=dev)
    pages_all = pool.region(B.KV_REGION_PAGES, torch.int32)
    saved = pages_all.clone()
    Q_l = [torch.from_numpy(query(c, layer, 0).view(np.int16)).to(dev) for layer in range(c.layers)]
    out = torch.empty(c.batch, c.q_heads, c.head_dim, dtype=torch.float32, device=dev)
    mass = torch.zeros(c.batch, c.q_heads, n, dtype=torch.float32, device=dev)
    log(f"{c.name}: pool ready ({pool.arena.numel() / 2**30:.1f} GiB arena)")

    def restore():
        torch.add(saved, 0, out=pages_all)   # a copy kernel (no memset or memcpy node in the graph)

    # Every layer's moves are known at the start of the step, so their plans
    # (latency-bound single launches) run ahead on a second stream; each
    # layer's data kernels wait only for its own plan.
    side = torch.cuda.Stream(device=dev)
    ev_restored = torch.cuda.Event()
    ev_plan = [torch.cuda.Event() for _ in range(c.layers)]

    def step():
        restore()
        main = torch.cuda.current_stream()
        ev_restored.record(main)
        side.wait_event(ev_restored)
        for layer in range(c.layers):
            pool.plan_transitions(layer, dem_l[layer], cnt_d, pro_l[layer], cnt_p, stream=side)
            ev_plan[layer].record(side)
        for layer in range(c.layers):
            main.wait_event(ev_plan[layer])
            pool.move_planned(layer)
            pool.attn(layer, Q_l[layer], out=out, mass=mass, scores=True)
        main.wait_stream(side)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert pool.check() == 0
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t_timed = time.perf_counter() - t0
    assert pool.check() == 0
    # the parts of one layer's step, eagerly with stream events (two more
    # steps, on one stream: the moves as one call, then as a demote and a
    # promote call)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * c.layers)]
    restore()
    for layer in range(c.layers):
        ev[4 * layer].record()
        pool.transitions(layer, dem_l[layer], cnt_d, pro_l[layer], cnt_p)
        ev[4 * layer + 1].record()
        pool.attn(layer, Q_l[layer], out=out, mass=mass, scores=True)
        ev[4 * layer + 2].record()
    torch.cuda.synchronize()
    part = lambda k: float(np.mean([ev[4 * l + k].elapsed_time(ev[4 * l + k + 1]) for l in range(c.layers)])) * 1e3
    mov_us, att_us = part(0), part(1)
    restore()
    for layer in range(c.layers):
        ev[4 * layer].record()
        pool.demote(layer, dem_l[layer], cnt_d)
        ev[4 * layer + 1].record()
        pool.promote(layer, pro_l[layer], cnt_p)
        ev[4 * layer + 2].record()
        pool.attn(layer, Q_l[layer], out=out, mass=mass, scores=True)
        ev[4 * layer + 3].record()
    torch.cuda.synchronize()
    assert pool.check() == 0
    dem_us, pro_us = part(0), part(1)
    n_f, n_q = 12 - c.demote_per_seg + c.promote_per_seg, 21 + c.demote_per_seg - c.promote_per_seg
    lay = type("lay", (), {})()
    for f in ("window", "head_dim", "kv_heads", "q_heads", "batch"):
        setattr(lay, f, getattr(c, f))
    a_b = attn_bytes(lay, n_f, n_q, n, bits) + score_bytes(lay, n)
    d_b = c.batch * move_bytes(lay, c.demote_per_seg, bits)
    p_b = c.batch * move_bytes(lay, c.promote_per_seg, bits)
    per_step = c.layers * (a_b + d_b + p_b)
    value = per_step * steps / t_timed / 1e9
    pk = lambda nb, us: {"bound": "hbm", "achieved": round(nb / (us * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    res = {"value": round(value, 2), "unit": "GB/s", "steps": steps, "warmup": warmup,
           "ms_per_step": round(1e3 * t_timed / steps, 4), "full_steps_per_s": round(steps / t_timed, 2),
           "bytes_per_step": per_step, "percent_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
           "per_layer_us": {"transitions": round(mov_us, 2), "decode_step": round(att_us, 2),
                            "demote": round(dem_us, 2), "promote": round(pro_us, 2)},
           "per_layer_bytes": {"transitions": d_b + p_b, "decode_step": a_b, "demote": d_b, "promote": p_b},
           "roofline": pk(a_b, att_us), "roofline_transitions": pk(d_b + p_b, mov_us),
           "roofline_demote": pk(d_b, dem_us), "roofline_promote": pk(p_b, pro_us),
           "tiers_after_moves": {"bf16": n_f, "ledger": n_q, "evicted": n - n_f - n_q}}
    del g, pool
    return res


def workload_name(c, bits, n_f, n_q):
    n = c.n_windows
    lw = "INT2" if bits == 2 else f"{bits}-bit"
    if c.name == "llama8b_128k_loop":
        return (f"{c.name}: Llama-3.1-8B attention shape, 128K context, batch {c.batch}, 32 q / 8 kv heads, "
                f"head_dim 128, window 128, 64 consecutive decode steps each appending a token, 20% byte budget "
                f"({n_f} bf16 / {n_q} {lw} / {n - n_f - n_q} evicted windows per sequence at the start), route "
                f"after every 16 steps")
    if c.name == "qwen7b_32k":
        return (f"{c.name}: Qwen2.5-7B attention shape, 32K context, batch {c.batch}, 28 q / 4 kv heads, "
                f"head_dim 128, window 128, 4 K outlier channels x10, 5% byte budget ({n_f} bf16 / {n_q} {lw} / "
                f"{n - n_f - n_q} evicted windows per sequence), one decode step per pool, routing every 16 steps "
                f"of a pool")
    if c.name == "mistral7b_step":
        return (f"{c.name}: Mistral-7B shape full step, 32 layers x 32 sequences x (32 q / 8 kv heads, head_dim "
                f"128), 16K context, window 128, 10% budget; per (layer, sequence) demote 8 windows (first INT2 "
                f"quantisation into the write-once ledger), promote 4 from the ledger, then the decode step")
    return (f"{c.name}: Llama-3.1-8B attention shape, 32K context, one decode step per pool, batch 1, 32 q / 8 kv "
            f"heads, head_dim 128, window 128, 20% byte budget ({n_f} bf16 / {n_q} {lw} / {n - n_f - n_q} evicted "
            f"windows), each pool routing after every 16 of its steps")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool replicas the headline steps rotate over (default: 24)")
    ap.add_argument("--workload", choices=("llama8b_32k", "qwen7b_32k", "llama8b_128k_loop", "mistral7b_step"),
                    default="llama8b_32k")
    ap.add_argument("--only", action="store_true",
                    help="measure only --workload (no other workloads, no ceiling sweep)")
    ap.add_argument("--ledger-bits", type=int, choices=(2, 4, 8), default=2,
                    help="code width of the pools' ledger (default 2: INT2)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run 8 plain device copies of this many MiB (a known-size kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the tiered decode path here is single-GPU "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_mb > 0:
        nb = args.copy_mb << 20
        src = torch.ones(nb // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nb, "copies": 8}), flush=True)
        return
    from tiered_int2_fp16_amd import binding as B

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bits = args.ledger_bits
    cpu = not args.no_cpu_baseline
    khash = kernel_source_hash()
    c = CONFIGS[args.workload]

    if c.name == "mistral7b_step":
        r = full_step_workload(c, B, torch, dev, max(1, min(args.steps, 16)), max(1, min(args.warmup, 2)), bits)
        head = {"metric": "tiered full-step effective HBM GB/s (% of peak) + full steps/s (Mistral-7B, 32 layers)",
                "value": r["value"], "unit": "GB/s", "n_gpus": 1, "steps": r["steps"], "warmup": r["warmup"],
                "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": f"bf16+int{bits}", "data": "synthetic",
                "config": {"workload": workload_name(c, bits, 0, 0), "global_batch": c.batch, "seq_len": c.context,
                           "parallelism": "none (1 GPU)"},
                "roofline": r["roofline"], "kernel_source_hash": khash, "detail": r}
        if cpu:
            head["cpu_baseline"] = cpu_baseline_full_step(c, args.cpu_seconds)
        print(json.dumps(head), flush=True)
        return

    R = max(1, args.replicas or (1 if c.append else 24))
    r = decode_workload(c, B, torch, dev, args.steps, args.warmup, R, bits, extras=c.name == "llama8b_32k")
    n_f, n_q = r["tiers"]["bf16"], r["tiers"]["ledger"]
    if c.name == "llama8b_32k" and bits == 2:
        r["roofline"]["traffic"] = measured_traffic(khash)
    name = workload_name(c, bits, n_f, n_q)
    if bits != 2:
        name += f" ({bits}-bit ledger: {bits + 1} bits per ledger value)"
    result = {
        "metric": "tiered decode-attn effective HBM GB/s (% of peak) + decode steps/s at "
                  + ("128K ctx" if c.append else "32K ctx"),
        "value": r["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"bf16+int{bits}", "data": "synthetic",
        "config": {"workload": name, "global_batch": c.batch, "seq_len": c.context, "parallelism": "none (1 GPU)",
                   "replicas": R, "timed_region": "HIP graph replay of exactly K steps"},
        "decode_steps_per_s": r["decode_steps_per_s"], "percent_of_peak": r["percent_of_peak"],
        "attn_kernel_us": r["attn_kernel_us"], "roofline": r["roofline"],
        "routing_events_timed": r["routing_events_timed"], "kernel_source_hash": khash,
    }
    for k in ("mass_emission", "route_diagnostics", "prefill_scores"):
        if k in r:
            result[k] = r[k]
    if bits != 2:
        result["config"]["ledger_bits"] = bits
    if not args.only or c.name == "llama8b_32k":
        # the attainable rate of one cold read of the step's bytes on the
        # attention's grid (and the best grid of a small sweep)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        pairs = c.batch * c.kv_heads
        grid = pairs * max(1, min(64, -(-2 * cus // pairs)))
        ceil = stream_ceiling(B, torch, dev, r["attn_bytes"], grid)
        sweep = [stream_ceiling(B, torch, dev, r["attn_bytes"], wg) for wg in (256, 1024, 2048) if wg != grid]
        best = min([ceil] + sweep, key=lambda x: x["us"])
        result["ceiling"] = {"same_grid": ceil, "best_grid": best,
                             "attn_frac_of_ceiling": round(ceil["us"] / r["attn_kernel_us"], 4)}
    if cpu and bits == 2:
        result["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
    if not args.only and c.name == "llama8b_32k" and bits == 2:
        extra = {}
        for wn, steps, warm, reps in (("qwen7b_32k", 64, 8, 24), ("llama8b_128k_loop", 64, 8, 1)):
            cw = CONFIGS[wn]
            rw = decode_workload(cw, B, torch, dev, steps, warm, reps, bits)
            rw["workload"] = workload_name(cw, bits, rw["tiers"]["bf16"], rw["tiers"]["ledger"])
            ceil = stream_ceiling(B, torch, dev, rw["attn_bytes"], cw.batch * cw.kv_heads * max(
                1, min(64, -(-2 * torch.cuda.get_device_properties(dev).multi_processor_count // (cw.batch * cw.kv_heads)))))
            rw["ceiling"] = {"same_grid": ceil, "attn_frac_of_ceiling": round(ceil["us"] / rw["attn_kernel_us"], 4)}
            if cpu:
                rw["cpu_baseline"] = cpu_baseline(cw, args.cpu_seconds)
            extra[wn] = rw
            torch.cuda.empty_cache()
        cm = CONFIGS["mistral7b_step"]
        rm = full_step_workload(cm, B, torch, dev, 4, 1, bits)
        rm["workload"] = workload_name(cm, bits, 0, 0)
        if cpu:
            rm["cpu_baseline"] = cpu_baseline_full_step(cm, args.cpu_seconds)
        extra["mistral7b_step"] = rm
        torch.cuda.empty_cache()
        result["workloads"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
