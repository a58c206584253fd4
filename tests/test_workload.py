"""Seeded generators: deterministic, right shapes, bf16-valued (CPU)."""
import numpy as np

from workload import CONFIGS, kv_history, new_kv, query, score_prior
from workload.synth import outlier_channels


def test_shapes_and_determinism():
    c = CONFIGS["tiny"]
    k, v = kv_history(c, 0, 0)
    assert k.shape == v.shape == (1, 2048, 64) and k.dtype == np.uint16
    k2, _ = kv_history(c, 0, 0)
    assert np.array_equal(k, k2)
    assert query(c, 0, 0).shape == (1, 4, 64)
    assert score_prior(c, 0, 0).shape == (32,)
    kn, vn = new_kv(c, 0, 3)
    assert kn.shape == (1, 1, 64)
    assert not np.array_equal(query(c, 0, 0), query(c, 0, 1))


def test_outlier_channels_are_scaled():
    c = CONFIGS["qwen7b_32k"]
    k, _ = kv_history(c, 0, 0, tokens=4096)
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    for h in range(c.kv_heads):
        ch = outlier_channels(c, 0, h)
        assert len(ch) == 4
        rms = np.sqrt((kf[h] ** 2).mean(0))
        others = np.setdiff1d(np.arange(c.head_dim), ch)
        assert rms[ch].min() > 5 * rms[others].max()


def test_config_shapes():
    assert CONFIGS["llama8b_32k"].n_windows == 256
    assert CONFIGS["qwen7b_32k"].group == 7
    assert CONFIGS["llama8b_128k_loop"].max_windows() == 1025
