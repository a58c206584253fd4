"""Benchmark of the tiered decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workload (default): the Llama-3.1-8B attention shape at 32K context (batch 1, 32 query /
8 kv heads, head_dim 128, windows of 128 tokens, 20 % byte budget with 10 % of
windows in bf16: 25 bf16 / 139 INT2 / 92 evicted windows), synthetic seeded
data.  One step = one decode step over the tiered cache (kv_decode_step: the
attention kernel and its combine kernel, which writes the per-window mass and
adds it to the cumulative scores), and every 16th step of a pool a routing
event (router, demotions into the write-once ledger, promotions).  Steps rotate over enough pool replicas (each its own arena) that
every step reads its windows from HBM, not from the 256 MB Infinity Cache.

`--ledger-bits 4` or `8` gives the pools a 4-bit or 8-bit ledger instead of
INT2 (same budget: fewer ledger windows, b + 1 bits per value each).

`--workload qwen7b_32k` runs it on the Qwen2.5-7B shape (batch 8, 28 query /
4 kv heads, 5 bf16 / 41 INT2 / 210 evicted windows per sequence; contexts drawn
on the device).  `--workload llama8b_128k_loop` runs the same measurement on
the 128K decode loop shape instead (batch 4, 131072 cached tokens, 102 bf16 / 548 INT2 / 374
evicted windows per sequence, every step appending a token, routing every 16
steps of a replica; contexts drawn on the device).  Its bytes per step are
counted at the starting tier counts; the windows that appends open only add to
them.  The oracle baseline is timed on the default workload only.

The timed region replays a HIP graph of exactly K steps between two device
synchronisations.  The attention kernel's own duration is then taken over the
same K steps run eagerly with dispatch timing events (hipExtLaunchKernel),
queued behind replays of the graph so that they run back to back.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from workload import CONFIGS, kv_history, kv_history_device, new_kv, query, score_prior  # noqa: E402

HBM_PEAK_GBS = 8000.0
ROUTE_EVERY = 16


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


def route_bytes(c, n_windows, first_quant, promotions, bits=2):
    wd = c.window * c.head_dim
    move = c.kv_heads * (4 * wd + (bits + 1) * wd // 4)
    return c.batch * n_windows * (4 + 4) + (first_quant + promotions) * move


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "tiered_int2_fp16_amd", "csrc"))):
        h.update(open(os.path.join(ROOT, "tiered_int2_fp16_amd", "csrc", f), "rb").read())
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


def cpu_baseline(c, seconds):
    """The oracle (plain numpy float64) timed on the host on the same workload:
    one sequence's decode steps (tiered attention + window mass + score update)
    until about `seconds` of work."""
    from oracle.pool import Segment
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    k, v = kv_history(c, 0, 0)
    prior = score_prior(c, 0, 0).astype(np.float64)
    seg = Segment(c.kv_heads, c.window, c.head_dim, c.n_recent)
    seg.prefill(k, v, prior=prior)
    seg.route(c.budget_frac, c.hi_frac)
    n_f, n_q = seg.tier.count(2), seg.tier.count(1)
    steps = 0
    t0 = time.perf_counter()
    while True:
        q = query(c, 0, steps)
        _, mass = seg.attend(q[0])
        seg.add_scores(mass)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_step = attn_bytes(c, n_f, n_q, seg.n) + score_bytes(c, seg.n)
    return {"value": round(per_step * steps / el / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{steps} decode steps of the same 32K Llama-3.1-8B-shaped workload "
                      f"(attention with window mass + score update, batch 1, 8 kv heads) in "
                      f"{el:.1f} s; {steps / el:.3f} steps/s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool replicas the steps rotate over (default: 24 at 32K, 2 at 128K)")
    ap.add_argument("--workload", choices=("llama8b_32k", "qwen7b_32k", "llama8b_128k_loop"),
                    default="llama8b_32k")
    ap.add_argument("--ledger-bits", type=int, choices=(2, 4, 8), default=2,
                    help="code width of the pools' ledger (default 2: INT2)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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
        n = args.copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 8}), flush=True)
        return
    from tiered_int2_fp16_amd import binding as B

    c = CONFIGS[args.workload]
    bits = args.ledger_bits
    loop = c.append
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n = c.n_windows
    R = max(1, args.replicas or (2 if loop else 24))
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    if c.batch > 1:
        # device-drawn contexts; with appends, room for the windows that every
        # pass below opens (warm-up, timed region, its six replays, event pass)
        K = torch.empty((c.batch, c.kv_heads, c.context, c.head_dim), dtype=torch.int16, device=dev)
        V = torch.empty_like(K)
        for b in range(c.batch):
            K[b], V[b] = kv_history_device(c, 0, b, dev)
        P = torch.from_numpy(np.stack([score_prior(c, 0, b) for b in range(c.batch)])).to(dev)
        appended = -(-(args.warmup + 8 * args.steps) // R) if loop else 0
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
    K_keys = K if c.name == "llama8b_32k" and bits == 2 else None   # for the prefill-score pass below
    del K, V
    torch.cuda.synchronize()
    pages = pools[0].pages(0).cpu().numpy() & 3
    n_f, n_q = int((pages[0] == 2).sum()), int((pages[0] == 1).sum())
    assert all(int((pg == 2).sum()) == n_f and int((pg == 1).sum()) == n_q for pg in pages)
    assert all(p.check() == 0 for p in pools)
    log(f"{R} replicas ready: {n_f} bf16 / {n_q} {bits}-bit / {n - n_f - n_q} evicted windows")
    local = [0] * R
    route_log = []  # (replica, counts tensor snapshot index)

    def step(i, record=None):
        r = i % R
        p = pools[r]
        if loop:   # kv_decode_step with the step's new token
            p.attn(0, Q[i % nq], KN[i % nq], VN[i % nq], out=outs[r], mass=masses[r], scores=True)
        else:      # kv_decode_step
            p.attn(0, Q[i % nq], out=outs[r], mass=masses[r], scores=True)
        do_route = (local[r] % ROUTE_EVERY) == ROUTE_EVERY - 1
        if do_route:
            p.score_route(0, None, 1, c.budget_frac, c.hi_frac, trs[r], cnts[r])
            p.apply_route(0, trs[r], cnts[r])
            if record is not None:
                record.append(r)
        local[r] += 1

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    K_steps = args.steps
    routed = []
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    local_before = list(local)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K_steps):
                step(args.warmup + i, routed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t_timed = time.perf_counter() - t0
    # demotions that quantised and promotions, from the counts each routing
    # event left (a replica routes at most once in a timed region of <= 16*R steps)
    fq = sum(int(cnts[r][3].sum()) for r in routed)
    pr = sum(int(cnts[r][1].sum()) for r in routed)
    assert all(p.check() == 0 for p in pools)

    # ---------------------------------------------- attention kernel duration
    # The same K steps again, eagerly, with dispatch events on every attention
    # launch.  Six replays of the timed graph are queued first: they keep the
    # GPU busy while the host issues the eager steps (about three times slower
    # to issue than to run), so those steps run back to back as in the timed
    # region instead of each starting on an idle GPU.
    for p in pools:
        B.kv_attn_profile(p.h, K_steps // R + 2)
    for _ in range(6):
        g.replay()
    for i in range(K_steps):
        step(args.warmup + K_steps + i)
    durs = []
    for p in pools:
        durs += B.kv_attn_timings(p.h)
        B.kv_attn_profile(p.h, 0)
    attn_ms = float(np.mean(durs))

    # -------------------------------------- cost of emitting the window mass
    # The same decode steps (attention + combine, no routing), each variant
    # captured in a HIP graph and replayed: with the mass emission and score
    # update, and with mass = NULL (what a step that does not feed the router
    # would save).
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

    n_me = max(R, min(K_steps, 256))
    g_with, g_without = step_graph(True, n_me), step_graph(False, n_me)
    mass_us = [replay_us(g_with, n_me), replay_us(g_without, n_me), replay_us(g_with, n_me),
               replay_us(g_without, n_me)]
    del g_with, g_without
    mass_emission = {"steps": n_me, "with_mass_us": round((mass_us[0] + mass_us[2]) / 2, 3),
                     "without_mass_us": round((mass_us[1] + mass_us[3]) / 2, 3)}
    mass_emission["overhead_us"] = round(mass_emission["with_mass_us"] - mass_emission["without_mass_us"], 3)

    # ------------------------------------------------ routing diagnostics
    # kv_route_diagnostics after a routing event (counts) with a step's window
    # masses standing in for the shadow cache's: churn, Global LIR and future
    # missed mass of every sequence, graph-replayed.
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
    diagnostics = {"calls": n_me, "us_per_call": round(diag_us, 3),
                   "bytes_per_call": diag_bytes, "gbs": round(diag_bytes / (diag_us * 1e-6) / 1e9, 2)}

    # ------------------------------------- initial scores from the prefill
    # kv_prefill_scores on the 32K context: causal attention of 32768 prefill
    # queries (drawn on the device) over the context's keys, twice (row
    # normalisers, then column sums), then window sums.  Algorithmic work:
    # 2 passes x q_heads x T (T + 1) / 2 query-key pairs x D multiply-adds.
    prefill = None
    if K_keys is not None:
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
        prefill = {"tokens": c.context, "ms": round(pf_ms, 3), "tflops": round(flops / (pf_ms * 1e-3) / 1e12, 1),
                   "bound": "mfma", "peak_tflops": 2500.0,
                   "frac": round(flops / (pf_ms * 1e-3) / 1e12 / 2500.0, 4)}
        del qp, ws, K_keys

    per_attn = attn_bytes(c, n_f, n_q, n, bits)
    total_bytes = K_steps * (per_attn + score_bytes(c, n)) + \
        len(routed) * route_bytes(c, n, 0, 0, bits) + route_bytes(c, 0, fq, pr, bits)
    ms_per_step = 1e3 * t_timed / K_steps
    value = total_bytes / t_timed / 1e9
    achieved = per_attn / (attn_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    if loop:
        workload_name = (f"{c.name}: Llama-3.1-8B attention shape, 128K context, batch {c.batch}, "
                         f"32 q / 8 kv heads, head_dim 128, window 128, every step appends a token, "
                         f"20% byte budget ({n_f} bf16 / {n_q} INT2 / {n - n_f - n_q} evicted windows "
                         f"per sequence at the start), route every 16 steps")
    elif c.name == "qwen7b_32k":
        workload_name = (f"{c.name}: Qwen2.5-7B attention shape, 32K context, batch {c.batch}, "
                         f"28 q / 4 kv heads, head_dim 128, window 128, 4 K outlier channels x10, "
                         f"5% byte budget ({n_f} bf16 / {n_q} INT2 / {n - n_f - n_q} evicted windows "
                         f"per sequence), route every 16 steps")
    else:
        workload_name = ("llama8b_32k: Llama-3.1-8B attention shape, 32K context, one decode "
                         "step per pool, batch 1, 32 q / 8 kv heads, head_dim 128, window 128, "
                         f"20% byte budget ({n_f} bf16 / {n_q} INT2 / {n - n_f - n_q} evicted windows), "
                         "route every 16 steps")
    result = {
        "metric": "tiered decode-attn effective HBM GB/s (% of peak) + decode steps/s at "
                  + ("128K ctx" if loop else "32K ctx"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16+int{bits}",
        "data": "synthetic",
        "config": {"workload": workload_name,
                   "global_batch": c.batch, "seq_len": c.context, "parallelism": "none (1 GPU)",
                   "replicas": R, "timed_region": "HIP graph replay of exactly K steps"},
        "decode_steps_per_s": round(K_steps / t_timed, 1),
        "percent_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "attn_kernel_us": round(attn_ms * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(khash) if c.name == "llama8b_32k" and bits == 2 else None},
        "kernel_source_hash": khash,
        "mass_emission": mass_emission,
        "route_diagnostics": diagnostics,
    }
    if prefill is not None:
        result["prefill_scores"] = prefill
    if bits != 2:
        result["config"]["workload"] = workload_name.replace("INT2", f"{bits}-bit") + \
            f" ({bits}-bit ledger: {bits + 1} bits per ledger value)"
        result["config"]["ledger_bits"] = bits
    if not args.no_cpu_baseline and c.name == "llama8b_32k" and bits == 2:
        result["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
