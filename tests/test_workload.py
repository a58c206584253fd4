"""Seeded generators: deterministic, right shapes, bf16-valued (CPU)."""
import pytest
import numpy as np

from workload import CONFIGS, kv_history, new_kv, query, score_prior
from workload.synth import outlier_channels, small


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


def test_device_generator_is_seeded_and_shaped():
    torch = pytest.importorskip("torch")
    from workload import kv_history_device
    c = small(CONFIGS["qwen7b_32k"], context=256)
    k1, v1 = kv_history_device(c, 0, 1, "cpu")
    k2, v2 = kv_history_device(c, 0, 1, "cpu")
    assert k1.dtype == torch.int16 and tuple(k1.shape) == (c.kv_heads, 256, c.head_dim)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    k3, _ = kv_history_device(c, 0, 2, "cpu")
    assert not torch.equal(k1, k3)
    # bf16 bits of normal draws, outlier K channels scaled
    kf = (k1.to(torch.int32) << 16).view(torch.float32)
    vf = (v1.to(torch.int32) << 16).view(torch.float32)
    assert 0.9 < float(vf.std()) < 1.1
    ch = outlier_channels(c, 0, 0)
    mask = torch.zeros(c.head_dim, dtype=torch.bool)
    mask[torch.from_numpy(ch)] = True
    assert float(kf[0][:, mask].abs().mean()) > 5 * float(kf[0][:, ~mask].abs().mean())
