"""Workload shapes and seeded generators.

The shapes follow the model families and context lengths that the QEvict
summary evaluates (Llama-3.1-8B, Mistral-7B, Qwen2.5-7B; 5 % to 20 % budgets;
32K retrieval contexts, "Kernbijdragen" and "Resultaten" sections of
"Technische Samenvatting: QEvict").  No dataset or trained weight is used:
every tensor is drawn from a counter-seeded PCG64 stream, so any slice can be
regenerated independently of the others.

Values are bf16 bit patterns (``uint16``).  A normal draw in float32 is turned
into bf16 by dropping the low 16 bits (round toward zero): a way of drawing
bf16-valued numbers, not a rounding rule of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

# stream ids inside one config seed
_T_SCORES, _T_Q, _T_K, _T_V, _T_OUTLIER, _T_STEP_Q, _T_STEP_K, _T_STEP_V, _T_DEVICE_KV, _T_PREFILL_Q = range(10)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    context: int            # tokens already cached before the first decode step
    n_recent: int = 4       # always-bf16 tail windows
    budget_frac: float = 0.2
    hi_frac: float = 0.1
    k_outliers: int = 0     # outlier K channels per (layer, kv head)
    k_outlier_scale: float = 1.0
    steps: int = 1          # decode steps in the workload
    route_every: int = 0    # route after every `route_every` steps (0: never)
    append: bool = False    # decode steps append a new token
    # pre-state routing fractions when the workload starts from a state other
    # than the steady one (the full-step Mistral shape); None = use the above
    pre_budget_frac: float | None = None
    pre_hi_frac: float | None = None
    demote_per_seg: int = 0
    promote_per_seg: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def n_windows(self) -> int:
        return -(-self.context // self.window)

    @property
    def segments(self) -> int:
        return self.batch * self.layers

    def max_windows(self) -> int:
        extra = self.steps if self.append else 0
        return -(-(self.context + extra) // self.window)


CONFIGS: Dict[str, Config] = {
    # 1 seq, 1 layer, 4 q / 1 kv head, D 64, 2048 tokens in 32 windows of 64;
    # 2 K outlier channels x8; last 4 + top-4 bf16, next 12 INT2, rest evicted
    # (hi 0.25 -> 8 bf16 windows, budget 0.325 -> 12 INT2 windows).
    "tiny": Config("tiny", 1, 1, 1, 4, 1, 64, 64, 2048,
                   budget_frac=0.325, hi_frac=0.25,
                   k_outliers=2, k_outlier_scale=8.0),
    # Llama-3.1-8B attention shape at 32K context, 20 % budget, 10 % bf16.
    "llama8b_32k": Config("llama8b_32k", 2, 1, 1, 32, 8, 128, 128, 32768,
                          budget_frac=0.2, hi_frac=0.1),
    # Qwen2.5-7B shape (GQA group 7), batch 8, 5 % budget, 2 % bf16,
    # 4 K outlier channels x10.
    "qwen7b_32k": Config("qwen7b_32k", 3, 8, 1, 28, 4, 128, 128, 32768,
                         budget_frac=0.05, hi_frac=0.02,
                         k_outliers=4, k_outlier_scale=10.0),
    # Mistral-7B shape, full step over 32 layers, batch 32, 16K context,
    # 10 % budget: start from 12 bf16 / 21 INT2 windows, demote 8 and promote
    # 4 per (layer, sequence) before attention.
    "mistral7b_step": Config("mistral7b_step", 4, 32, 32, 32, 8, 128, 128, 16384,
                             budget_frac=0.1, hi_frac=1.0 / 16,
                             pre_budget_frac=0.125, pre_hi_frac=0.09375,
                             demote_per_seg=8, promote_per_seg=4),
    # Llama-3.1-8B shape, batch 4, 128K context, 64 decode steps that append
    # a token each; route after every 16 steps.
    "llama8b_128k_loop": Config("llama8b_128k_loop", 5, 4, 1, 32, 8, 128, 128, 131072,
                                budget_frac=0.2, hi_frac=0.1,
                                steps=64, route_every=16, append=True),
}


def _rng(cfg: Config, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, *ids])))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def outlier_channels(cfg: Config, layer: int, kvh: int) -> np.ndarray:
    if cfg.k_outliers == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg, _T_OUTLIER, layer, kvh).choice(
        cfg.head_dim, cfg.k_outliers, replace=False))


def kv_history(cfg: Config, layer: int, b: int,
               tokens: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of the cached context of sequence ``b`` in ``layer``.

    Returns two uint16 (bf16 bits) arrays of shape [kv_heads][tokens][head_dim].
    """
    t = cfg.context if tokens is None else tokens
    shape = (cfg.kv_heads, t, cfg.head_dim)
    k = _rng(cfg, _T_K, layer, b).standard_normal(shape, dtype=np.float32)
    for h in range(cfg.kv_heads):
        ch = outlier_channels(cfg, layer, h)
        if ch.size:
            k[h][:, ch] *= np.float32(cfg.k_outlier_scale)
    v = _rng(cfg, _T_V, layer, b).standard_normal(shape, dtype=np.float32)
    return _to_bf16_bits(k), _to_bf16_bits(v)


def kv_history_device(cfg: Config, layer: int, b: int, device):
    """K and V of the cached context of sequence ``b`` in ``layer``, drawn on
    ``device`` by torch's counter-based Philox generator (seeded from the
    config seed, layer and sequence): for full-size workloads whose contexts
    are too large to draw on the host.  Same distributions as
    :func:`kv_history` (normal, K outlier channels scaled, bf16 by dropping the
    low 16 bits), different streams.  Returns two int16 tensors holding bf16
    bits, [kv_heads][context][head_dim].
    """
    import torch
    seed = int(np.random.SeedSequence([cfg.seed, _T_DEVICE_KV, layer, b]).generate_state(1, np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (cfg.kv_heads, cfg.context, cfg.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    for h in range(cfg.kv_heads):
        ch = outlier_channels(cfg, layer, h)
        if ch.size:
            k[h][:, torch.from_numpy(ch).to(device)] *= cfg.k_outlier_scale
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return ((k.view(torch.int32) >> 16).to(torch.int16), (v.view(torch.int32) >> 16).to(torch.int16))


def score_prior(cfg: Config, layer: int, b: int) -> np.ndarray:
    """Seeded log-normal prior window scores, float32 [n_windows]."""
    return _rng(cfg, _T_SCORES, layer, b).lognormal(0.0, 1.0, cfg.n_windows).astype(np.float32)


def query(cfg: Config, layer: int, step: int = 0) -> np.ndarray:
    """Decode query of one step: uint16 (bf16 bits) [batch][q_heads][head_dim]."""
    g = _rng(cfg, _T_STEP_Q, layer, step)
    return _to_bf16_bits(g.standard_normal((cfg.batch, cfg.q_heads, cfg.head_dim), dtype=np.float32))


def prefill_queries(cfg: Config, layer: int, b: int) -> np.ndarray:
    """Queries of the prefill of sequence ``b`` (one per cached token): uint16
    (bf16 bits) [q_heads][context][head_dim], standard normal."""
    g = _rng(cfg, _T_PREFILL_Q, layer, b)
    return _to_bf16_bits(g.standard_normal((cfg.q_heads, cfg.context, cfg.head_dim), dtype=np.float32))


def new_kv(cfg: Config, layer: int, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """Key and value of the token a decode step appends: uint16 [batch][kv_heads][head_dim]."""
    shape = (cfg.batch, cfg.kv_heads, cfg.head_dim)
    k = _rng(cfg, _T_STEP_K, layer, step).standard_normal(shape, dtype=np.float32)
    for h in range(cfg.kv_heads):
        ch = outlier_channels(cfg, layer, h)
        if ch.size:
            k[:, h][:, ch] *= np.float32(cfg.k_outlier_scale)
    v = _rng(cfg, _T_STEP_V, layer, step).standard_normal(shape, dtype=np.float32)
    return _to_bf16_bits(k), _to_bf16_bits(v)


def small(cfg: Config, **overrides) -> Config:
    """A reduced copy of ``cfg`` (for parity runs the oracle finishes quickly)."""
    return dataclasses.replace(cfg, **overrides)
