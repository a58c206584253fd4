"""kv_decode_step_noalloc (static scratch, no device allocation) against
kv_decode_step with a caller workspace, through the C ABI.

Two calls in a row on one GPU share the library's static scratch: first the
Llama-3.1-8B 32K step, then the smaller tiny shape with an appended token, so
the second call runs on the first one's leftovers.  Each call is compared
with kv_decode_step on an identical pool: outputs, window masses and scores
bit for bit (the same kernels), and with the oracle to the parity bars.
"""
import ctypes
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS, new_kv, query

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_harness import MASS_TOL, OUT_TOL, Pair, dev, log  # noqa: E402


def _step_both(name, c, append):
    from tiered_int2_fp16_amd import binding as B
    ref, nal = Pair(c), Pair(c)
    for p in (ref, nal):
        p.load(0)
        p.route(0, c.budget_frac, c.hi_frac)
    q = dev(query(c, 0, 0))
    kn = vn = None
    if append:
        kn_h, vn_h = new_kv(c, 0, 0)
        kn, vn = dev(kn_h), dev(vn_h)
    outs = []
    for p, noalloc in ((ref, False), (nal, True)):
        cc = p.pool.cfg
        out = torch.empty(cc.batch, cc.q_heads, cc.head_dim, dtype=torch.float32, device="cuda")
        mass = torch.zeros(cc.batch, cc.q_heads, cc.max_windows, dtype=torch.float32, device="cuda")
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        if noalloc:
            st = B.LIB.kv_decode_step_noalloc(p.pool.h, 0, P(q), P(kn), P(vn), P(out), P(mass), s)
        else:
            ws = p.pool.workspace
            st = B.LIB.kv_decode_step(p.pool.h, 0, P(q), P(kn), P(vn), P(out), P(mass), P(ws), ws.numel(), s)
        assert st == B.KV_OK, B.LIB.kv_last_error().decode()
        torch.cuda.synchronize()
        assert p.pool.check() == 0
        outs.append((out, mass, p.pool.scores(0).clone(), p.pool.tokens(0).clone()))
    (o1, m1, s1, t1), (o2, m2, s2, t2) = outs
    assert torch.equal(o1, o2) and torch.equal(m1, m2) and torch.equal(s1, s2) and torch.equal(t1, t2)
    # and the oracle, to the parity bars
    qh = query(c, 0, 0)
    worst = (0.0, 0.0)
    for b in nal.seqs:
        seg = nal.oracle[(0, b)]
        if append:
            seg.append(kn_h[b], vn_h[b])
        o_out, o_mass = seg.attend(qh[b])
        eo = float(np.abs(o2[b].cpu().numpy() - o_out).max())
        em = float(np.abs(m2[b, :, : seg.n].cpu().numpy() - o_mass).max())
        assert eo <= OUT_TOL and em <= MASS_TOL, (name, b, eo, em)
        worst = (max(worst[0], eo), max(worst[1], em))
    log("%s: no-alloc step equals the workspace step; oracle out err %.2e mass err %.2e" % (name, *worst))


def test_noalloc_step_matches_workspace_step_twice():
    """The 32K Llama step, then the smaller tiny step with an append."""
    _step_both("llama8b_32k", CONFIGS["llama8b_32k"], append=False)
    c = dataclasses.replace(CONFIGS["tiny"], steps=1, append=True)
    _step_both("tiny+append", c, append=True)


def test_noalloc_step_rejects_a_workspace_beyond_the_scratch():
    from tiered_int2_fp16_amd import binding as B
    # 16 sequences x 32 query heads x 1024 windows x 4 tiles of tile masses
    # alone exceed 16 MiB; the call must fail before launching anything
    cfg = B.make_config(16, 1, 32, 8, 128, 128, 1024, 4, bf16_slots=1, ledger_slots=0)
    pool = B.Pool(cfg)
    assert B.kv_attn_workspace_bytes(pool.h) > B.KV_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(16, 32, 128, dtype=torch.int16, device="cuda")
    out = torch.empty(16, 32, 128, dtype=torch.float32, device="cuda")
    st = B.LIB.kv_decode_step_noalloc(pool.h, 0, ctypes.c_void_p(q.data_ptr()), None, None,
                                      ctypes.c_void_p(out.data_ptr()), None,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.KV_ENOMEM
    assert "scratch" in B.LIB.kv_last_error().decode()
    torch.cuda.synchronize()
    assert pool.check() == 0
    pool.close()
