"""GPU parity of the prefill token weights and initial window scores
(kv_prefill_scores) against the oracle, then routing on those scores.

Shapes span head groups of 1, 2, 4, 7 and 8, head_dim 64 and 128, windows of
64 and 128 and ragged token counts (last window partial, last query block
partial), a single token, token counts at and one past the kernels' 64-row
stages and 192-row workgroups; one case has the Llama-3.1-8B head layout at
2048 tokens, and the benchmark's 32768-token pass (two heads checked).  Token weights and
window scores are float sums of up to T probabilities per token: the bar is
relative 1e-5 plus T * 1e-6 absolute (float32 accumulation), checked against
the oracle in float64.  Routing on the library's scores is then bit-exact
against the oracle router, as everywhere.
"""
import dataclasses

import numpy as np
import pytest

from workload import CONFIGS, kv_history, prefill_queries

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle.codec import bf16_to_f64  # noqa: E402
from oracle.prefill_scores import head_token_weights, token_weights, window_scores  # noqa: E402
from tests.gpu_harness import Pair, dev, log  # noqa: E402

# (name, seed, batch, q_heads, kv_heads, head_dim, window, tokens)
CASES = [
    ("g4_d128_w128", 31, 2, 8, 2, 128, 128, 300),
    ("g7_d128_w64", 32, 1, 7, 1, 128, 64, 161),
    ("g4_d64_w64", 33, 2, 4, 1, 64, 64, 257),
    ("g1_d64_w64", 34, 1, 2, 2, 64, 64, 33),
    ("llama_2k", 35, 1, 32, 8, 128, 128, 2048),
    # edges of the kernels' 64-row LDS stages and 192-row workgroups (4 waves
    # of 48 rows): one token; exactly one workgroup; one row past two; whole
    # stages (256, 512) and one row past (513, head_dim 64)
    ("g4_d128_t1", 36, 1, 4, 1, 128, 64, 1),
    ("g4_d128_t192", 40, 1, 8, 2, 128, 64, 192),
    ("g4_d64_t385", 41, 2, 4, 1, 64, 64, 385),
    ("g8_d128_t256", 37, 1, 8, 1, 128, 64, 256),
    ("g4_d128_t512", 38, 1, 8, 2, 128, 128, 512),
    ("g2_d64_t513", 39, 2, 4, 2, 64, 64, 513),
]


@pytest.mark.parametrize("name,seed,batch,hq,hkv,d,w,T", CASES, ids=[c[0] for c in CASES])
def test_prefill_scores(name, seed, batch, hq, hkv, d, w, T):
    c = dataclasses.replace(CONFIGS["tiny"], name=name, seed=seed, batch=batch, q_heads=hq, kv_heads=hkv,
                            head_dim=d, window=w, context=T, budget_frac=0.3, hi_frac=0.2, k_outliers=0)
    p = Pair(c)
    p.load(0)
    q = np.stack([prefill_queries(c, 0, b) for b in range(batch)])
    k = np.stack([kv_history(c, 0, b)[0] for b in range(batch)])
    ws = p.pool.prefill_scores(0, dev(q), dev(k), T)
    f = ws.view(torch.float32).cpu().numpy().reshape(2, batch, hq, T)
    s_gpu = p.pool.scores(0).cpu().numpy()
    n = c.n_windows
    worst_w = worst_s = 0.0
    for b in range(batch):
        w_o = token_weights(bf16_to_f64(q[b]), bf16_to_f64(k[b]))
        s_o = window_scores(w_o, w)
        ew = np.abs(f[1][b] - w_o)
        assert (ew <= 1e-5 * w_o + 1e-6 * T).all(), (name, b, ew.max())
        es = np.abs(s_gpu[b][:n] - s_o)
        assert (es <= 1e-5 * s_o + 1e-6 * T * hq).all(), (name, b, es.max())
        np.testing.assert_allclose(f[1][b].astype(np.float64).sum(axis=1), T, rtol=1e-5)
        worst_w, worst_s = max(worst_w, ew.max()), max(worst_s, (es / s_o).max())
        p.oracle[(0, b)].S[:n] = s_o
    log("%s: token-weight error %.2e, window-score relative error %.2e" % (name, worst_w, worst_s))
    # routing on the library's own scores: bit-exact tiers and transitions
    p.route(0, c.budget_frac, c.hi_frac)
    p.check_state(0)


@pytest.mark.timeout(600)
def test_prefill_scores_llama_32k():
    """The size the benchmark times: the Llama-3.1-8B head layout (32 query /
    8 kv heads, head_dim 128) over a 32768-token prefill.  Query heads 0 and
    31 (kv heads 0 and 7) against the oracle in float64, computed over blocks
    of query rows; every head's weights sum to T; the window scores are the
    window sums of the kernel's own token weights over all heads."""
    c = dataclasses.replace(CONFIGS["llama8b_32k"], name="prefill_32k", seed=42)
    T, n = c.context, c.n_windows
    p = Pair(c, seqs=[])
    k = kv_history(c, 0, 0)[0]
    p.pool.prefill(0, dev(k[None]), dev(kv_history(c, 0, 0)[1][None]), T)
    q = prefill_queries(c, 0, 0)
    ws = p.pool.prefill_scores(0, dev(q[None]), dev(k[None]), T)
    f = ws.view(torch.float32).cpu().numpy().reshape(2, 1, c.q_heads, T)
    w_gpu = f[1][0].astype(np.float64)
    np.testing.assert_allclose(w_gpu.sum(axis=1), T, rtol=1e-5)
    s_gpu = p.pool.scores(0).cpu().numpy()[0][:n].astype(np.float64)
    np.testing.assert_allclose(s_gpu, window_scores(w_gpu, c.window), rtol=1e-5)
    for h in (0, c.q_heads - 1):
        w_o = head_token_weights(bf16_to_f64(q[h]), bf16_to_f64(k[h // c.group]))
        ew = np.abs(w_gpu[h] - w_o)
        log("32K prefill, head %d: max token-weight error %.2e (relative %.2e), weights %.3g..%.3g"
            % (h, ew.max(), (ew / w_o).max(), w_o.min(), w_o.max()))
        assert (ew <= 1e-5 * w_o + 1e-6 * T).all(), (h, ew.max())
    assert p.pool.check() == 0


def test_prefill_scores_reject_bad_arguments():
    from tiered_int2_fp16_amd.binding import KvError
    c = CONFIGS["tiny"]
    p = Pair(c)
    p.load(0)
    q = torch.zeros(c.batch, c.q_heads, 64, c.head_dim, dtype=torch.int16, device="cuda")
    k = torch.zeros(c.batch, c.kv_heads, 64, c.head_dim, dtype=torch.int16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(KvError):
        p.pool.prefill_scores(0, q, k, 64, workspace=small)
