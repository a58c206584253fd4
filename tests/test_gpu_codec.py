"""Demote codes and promoted bf16 at the codec's edge cases, bit for bit
against the oracle.

The demote kernel decides each code without dividing: it compares x - m with
the half-way points (k + 1/2) s.  The windows here are built from groups that
such a decision (or any approximate quotient) could get wrong:

  * values exactly on the half-way points of every level, so that both an odd
    and an even k meet a tie (round half to even decides);
  * the nearest bf16 values on either side of those points;
  * s = 0 (every code 0), also with values beyond the fp16 range, where the
    stored min overflows to +-inf;
  * a min below -65504 with a small range (m = -inf: every code L) and one
    above +65504 (m = +inf: every code 0);
  * an fp16-infinite scale with a finite min (every code 0);
  * fp16-subnormal scales, signed zeros, and ordinary normal groups.

K groups run over the 32 tokens of a channel, V groups over 32 channels of a
token, so each group is placed once as a K column and once as a V row block.
"""
import numpy as np
import pytest

from oracle import codec

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.codec_cases import edge_groups  # noqa: E402
from tests.gpu_harness import dev, log  # noqa: E402


def _windows(bits, W, D, rng):
    """K, V bf16 bits [n][W][D] whose K columns and V row blocks are the edge
    groups (cycled), each group also reversed in half the placements."""
    groups = [g for _, g, _ in edge_groups(bits, rng)]
    per_win_k = (W // 32) * D
    n = max(2, -(-len(groups) // per_win_k) + 1)
    K = np.zeros((n, W, D), np.uint16)
    V = np.zeros((n, W, D), np.uint16)
    i = 0
    for w in range(n):
        for tile in range(W // 32):
            for d in range(D):
                g = groups[i % len(groups)]
                K[w, 32 * tile: 32 * tile + 32, d] = g if (i // len(groups)) % 2 == 0 else g[::-1]
                i += 1
    j = 0
    for w in range(n):
        for t in range(W):
            for blk in range(D // 32):
                g = groups[(j * 7) % len(groups)]
                V[w, t, 32 * blk: 32 * blk + 32] = np.roll(g, j % 32)
                j += 1
    return K, V


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("D,W", [(128, 32), (128, 64), (64, 32)])
def test_demote_codes_at_edge_cases(bits, D, W):
    from tiered_int2_fp16_amd import binding as B
    rng = np.random.default_rng(100 * bits + D + W)
    Kw, Vw = _windows(bits, W, D, rng)
    n = Kw.shape[0]
    cfg = B.make_config(1, 1, 1, 1, D, W, n, 1, n, n, bits)
    pool = B.Pool(cfg)
    T = n * W
    K = dev(Kw.reshape(1, 1, T, D))
    V = dev(Vw.reshape(1, 1, T, D))
    pool.prefill(0, K, V, T, dev(np.ones((1, n), np.float32)))
    pool.demote(0, dev(np.arange(n, dtype=np.int32)[None]), dev(np.array([n], np.int32)))
    assert pool.check() == 0
    entries = []
    for w in range(n):
        got = pool.read_ledger(0, 0, w).cpu().numpy()[0]
        e = codec.quantize_window(Kw[w], Vw[w], bits)
        entries.append(e)
        assert got.tobytes() == codec.entry_bytes(e, bits), (bits, D, W, w)
    # promote every window back: bf16_rne(c s + m), bit for bit; where the
    # group's scale overflowed fp16 (s = inf) a code 0 gives 0 * inf, NaN on
    # both sides, whose sign and payload the definition leaves open
    pool.promote(0, dev(np.arange(n, dtype=np.int32)[None]), dev(np.array([n], np.int32)))
    assert pool.check() == 0
    for w in range(n):
        got = pool.read_window(0, 0, w).cpu().numpy().view(np.uint16)[0]
        with np.errstate(invalid="ignore", over="ignore"):
            wk, wv = codec.promote_bits(entries[w])
        for part, want in ((got[0], wk), (got[1], wv)):
            nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
            assert np.array_equal(part[~nan], want[~nan]), (bits, D, W, w)
            pn = part[nan]
            assert np.all(((pn & 0x7F80) == 0x7F80) & ((pn & 0x7F) != 0)), (bits, D, W, w)
    log(f"{bits}-bit, head_dim {D}, window {W}: {n} windows of edge-case groups bit-exact, "
        "demoted and promoted")
