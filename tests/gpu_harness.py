"""Drive the HIP library and the oracle side by side on identical inputs.

Test infrastructure: the library runs through the C ABI (ctypes binding); the
oracle runs on the CPU from the same seeded bf16 bits.  Bars:
  codes, scales, mins, tiers, transitions, promoted bf16: bit-exact;
  attention output: max |err| <= 2e-3;  window mass: max |err| <= 1e-4.
Routing is compared on identical float32 scores (the library's own S), so the
integer decision is taken in the same precision on both sides.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import codec
from oracle.pool import Segment
from oracle.router import E, F, Q
from workload import kv_history, new_kv, query, score_prior

OUT_TOL = 2e-3
MASS_TOL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class CachedSegment(Segment):
    """Oracle segment that memoises the exact dequantisation of ledger entries
    (entries are write-once, so the cached values never go stale)."""

    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self._deq = {}

    def window_kv(self, w):
        if self.tier[w] != Q:
            return super().window_kv(w)
        ent = self.ledger[w]
        hit = self._deq.get(w)
        if hit is None or hit[0] is not ent:
            hit = (ent, super().window_kv(w))
            self._deq[w] = hit
        return hit[1]


class Pair:
    def __init__(self, cfg, layers=None, seqs=None, bf16_slots=None, ledger_slots=None, bits=2):
        from tiered_int2_fp16_amd import binding as B
        self.B = B
        self.cfg = cfg
        self.bits = bits          # ledger code width of the pool (and of the oracle's segments)
        self.maxw = cfg.max_windows()
        pc = B.make_config(cfg.batch, cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.window,
                           self.maxw, cfg.n_recent, bf16_slots or self.maxw, ledger_slots or self.maxw,
                           bits)
        self.pool = B.Pool(pc)
        self.seqs = list(range(cfg.batch)) if seqs is None else list(seqs)
        self.oracle = {}
        self.steps_done = 0

    # ------------------------------------------------------------ setup ---
    def load(self, layer=0):
        c = self.cfg
        ks, vs, prs = [], [], []
        for b in range(c.batch):
            k, v = kv_history(c, layer, b)
            pr = score_prior(c, layer, b)
            ks.append(k)
            vs.append(v)
            prs.append(pr)
            if b in self.seqs:
                seg = CachedSegment(c.kv_heads, c.window, c.head_dim, c.n_recent, bits=self.bits)
                seg.prefill(k, v, prior=pr.astype(np.float64))
                self.oracle[(layer, b)] = seg
        self.pool.prefill(layer, dev(np.stack(ks)), dev(np.stack(vs)), c.context, dev(np.stack(prs)))
        del ks, vs

    # ---------------------------------------------------------- routing ---
    def route(self, layer, beta, phi):
        tr, cnt = self.pool.score_route(layer, None, 1, beta, phi)
        self.last_counts = cnt   # device counts of this event
        s_gpu = self.pool.scores(layer).cpu().numpy().copy()
        self.pool.apply_route(layer, tr, cnt)
        tr_h, cnt_h = tr.cpu().numpy(), cnt.cpu().numpy()
        for b in self.seqs:
            seg = self.oracle[(layer, b)]
            otr = seg.route(beta, phi, scores=s_gpu[b][: seg.n].astype(np.float64))
            for k, name in enumerate(("demote", "promote", "evict")):
                assert cnt_h[k][b] == len(otr[name]), (b, name, cnt_h[k][b], len(otr[name]))
                assert tr_h[k][b][: cnt_h[k][b]].tolist() == otr[name], (b, name)
            assert cnt_h[3][b] == len(otr["first_quant"]), (b, "first_quant")
        return tr_h, cnt_h

    def add_scores(self, layer, mass_gpu, mass_oracle):
        self.pool.score_route(layer, mass_gpu, 0)
        for b in self.seqs:
            self.oracle[(layer, b)].add_scores(mass_oracle[b])

    # ------------------------------------------------------------ state ---
    def check_state(self, layer, ledger_sample=None, window_sample=None, rng=None):
        pages = self.pool.pages(layer).cpu().numpy().view(np.uint32)
        s_gpu = self.pool.scores(layer).cpu().numpy()
        tok = self.pool.tokens(layer).cpu().numpy()
        for b in self.seqs:
            seg = self.oracle[(layer, b)]
            n = seg.n
            assert tok[b] == seg.tokens
            tiers = (pages[b][:n] & 3).tolist()
            assert tiers == seg.tier, f"tiers differ for sequence {b}"
            hl = ((pages[b][:n] >> 2) & 1).astype(bool)
            for w in range(n):
                if seg.tier[w] != E:
                    assert hl[w] == (w in seg.ledger), (b, w)
            tol = 1e-4 * self.cfg.q_heads * max(1, self.steps_done) + 1e-5 * np.abs(seg.S[:n]).max()
            assert np.abs(s_gpu[b][:n] - seg.S[:n]).max() <= tol
            led = sorted(seg.ledger)
            fw = [w for w in range(n) if seg.tier[w] == F]
            if rng is not None and ledger_sample is not None and len(led) > ledger_sample:
                led = sorted(rng.choice(led, ledger_sample, replace=False).tolist())
            if rng is not None and window_sample is not None and len(fw) > window_sample:
                fw = sorted(rng.choice(fw, window_sample, replace=False).tolist())
            for w in led:
                got = self.pool.read_ledger(layer, b, w).cpu().numpy()
                for h in range(self.cfg.kv_heads):
                    assert got[h].tobytes() == codec.entry_bytes(seg.ledger[w][h], seg.bits), (b, w, h)
            for w in fw:
                got = self.pool.read_window(layer, b, w).cpu().numpy().view(np.uint16)
                nt = seg.valid(w)
                assert np.array_equal(got[:, 0, :nt], seg.k[w][:, :nt]), (b, w, "K")
                assert np.array_equal(got[:, 1, :nt], seg.v[w][:, :nt]), (b, w, "V")
        bits = self.pool.check()
        assert bits == 0, f"device error bits {bits:#x}"

    # --------------------------------------------------------- decoding ---
    def step(self, layer, step, append=False, check=True):
        c = self.cfg
        q = query(c, layer, step)
        kn = vn = None
        if append:
            kn, vn = new_kv(c, layer, step)
        out, mass = self.pool.attn(layer, dev(q), None if kn is None else dev(kn),
                                   None if vn is None else dev(vn))
        self.steps_done += 1
        o_mass_all = {}
        errs = (0.0, 0.0)
        if check:
            out_h = out.cpu().numpy()
            mass_h = mass.cpu().numpy()
            for b in self.seqs:
                seg = self.oracle[(layer, b)]
                if append:
                    seg.append(kn[b], vn[b])
                o_out, o_mass = seg.attend(q[b])
                o_mass_all[b] = o_mass
                eo = np.abs(out_h[b] - o_out).max()
                em = np.abs(mass_h[b][:, : seg.n] - o_mass).max()
                assert eo <= OUT_TOL, f"step {step} seq {b}: out error {eo:.3e}"
                assert em <= MASS_TOL, f"step {step} seq {b}: mass error {em:.3e}"
                errs = (max(errs[0], eo), max(errs[1], em))
        return out, mass, o_mass_all, errs
