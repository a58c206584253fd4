"""ctypes binding of libkvtier.so: argument marshalling only.

Functions carry the C ABI's names and take torch tensors (device memory) and
the current torch stream; every step of the path runs in the HIP library.  If
the library is missing the import of this module fails loudly: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libkvtier.so")

KV_OK, KV_EINVAL, KV_ENOMEM, KV_EBUDGET, KV_ESTATE, KV_EDEVICE = range(6)
KV_TIER_E, KV_TIER_Q, KV_TIER_F = 0, 1, 2
(KV_REGION_BF16, KV_REGION_LEDGER, KV_REGION_PAGES, KV_REGION_SCORES,
 KV_REGION_TOKENS, KV_REGION_WORK, KV_REGION_ERR) = range(7)
ERR_BITS = {1: "DEMOTE_STATE", 2: "PROMOTE_STATE", 4: "NO_BF16_SLOT", 8: "NO_LEDGER_SLOT",
            16: "APPEND_STATE", 32: "ITEM_RANGE", 64: "READ_MISSING", 128: "CAPACITY"}

EXPORTS = [
    "kv_pool_arena_bytes", "kv_ledger_entry_bytes", "kv_pool_create", "kv_pool_destroy",
    "kv_pool_region", "kv_prefill", "kv_demote_quantize", "kv_promote_dequantize",
    "kv_attn_workspace_bytes", "kv_tiered_decode_attn", "kv_score_route", "kv_read_ledger",
    "kv_read_window", "kv_tier_counts", "kv_pool_check", "kv_last_error",
    "kv_attn_profile", "kv_attn_timings", "kv_decode_step", "kv_route_diagnostics",
    "kv_prefill_scores_workspace_bytes", "kv_prefill_scores", "kv_decode_step_noalloc",
    "kv_apply_transitions", "kv_plan_transitions", "kv_move_planned",
    "kv_stream_probe",
]


class kv_pool_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "layers", "q_heads", "kv_heads", "head_dim", "window",
        "max_windows", "n_recent", "bf16_slots", "ledger_slots", "ledger_bits")]


_BF16 = (torch.int16, torch.bfloat16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16, torch.bfloat16)


class KvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvtier status {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tiered_int2_fp16_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    cfgp = ctypes.POINTER(kv_pool_config)
    sig = {
        "kv_pool_arena_bytes": (SZ, [cfgp]),
        "kv_ledger_entry_bytes": (SZ, [I32, I32, I32]),
        "kv_pool_create": (I32, [cfgp, P, SZ, P, ctypes.POINTER(P)]),
        "kv_pool_destroy": (I32, [P]),
        "kv_pool_region": (I32, [P, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "kv_prefill": (I32, [P, I32, P, P, I32, P, P]),
        "kv_demote_quantize": (I32, [P, I32, P, I32, P, P]),
        "kv_promote_dequantize": (I32, [P, I32, P, I32, P, P]),
        "kv_apply_transitions": (I32, [P, I32, P, I32, P, P, I32, P, P]),
        "kv_plan_transitions": (I32, [P, I32, P, I32, P, P, I32, P, P]),
        "kv_move_planned": (I32, [P, I32, P]),
        "kv_attn_workspace_bytes": (SZ, [P]),
        "kv_tiered_decode_attn": (I32, [P, I32, P, P, P, P, P, P, SZ, P]),
        "kv_decode_step": (I32, [P, I32, P, P, P, P, P, P, SZ, P]),
        "kv_decode_step_noalloc": (I32, [P, I32, P, P, P, P, P, P]),
        "kv_stream_probe": (I32, [P, SZ, SZ, I32, I32, P, P, ctypes.POINTER(ctypes.c_float)]),
        "kv_score_route": (I32, [P, I32, P, I32, D, D, P, P, P]),
        "kv_route_diagnostics": (I32, [P, I32, P, P, P, P]),
        "kv_prefill_scores_workspace_bytes": (SZ, [P, I32]),
        "kv_prefill_scores": (I32, [P, I32, P, P, I32, P, SZ, P]),
        "kv_read_ledger": (I32, [P, I32, I32, I32, P, P]),
        "kv_read_window": (I32, [P, I32, I32, I32, P, P]),
        "kv_tier_counts": (I32, [I32, I32, D, D, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "kv_pool_check": (I32, [P, P, ctypes.POINTER(I32)]),
        "kv_last_error": (ctypes.c_char_p, []),
        "kv_attn_profile": (I32, [P, I32]),
        "kv_attn_timings": (I32, [P, ctypes.POINTER(ctypes.c_float), I32, ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def _ck(status: int):
    if status != KV_OK:
        raise KvError(status, LIB.kv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_config(batch, layers, q_heads, kv_heads, head_dim, window, max_windows,
                n_recent=4, bf16_slots=None, ledger_slots=None, ledger_bits=2) -> kv_pool_config:
    return kv_pool_config(batch, layers, q_heads, kv_heads, head_dim, window, max_windows, n_recent,
                          max_windows if bf16_slots is None else bf16_slots,
                          max_windows if ledger_slots is None else ledger_slots, ledger_bits)


# ------------------------------------------------------------ C ABI names ---
def kv_pool_arena_bytes(cfg: kv_pool_config) -> int:
    n = LIB.kv_pool_arena_bytes(ctypes.byref(cfg))
    if n == 0:
        raise KvError(KV_EINVAL, LIB.kv_last_error().decode())
    return n


def kv_ledger_entry_bytes(window: int, head_dim: int, ledger_bits: int = 2) -> int:
    return LIB.kv_ledger_entry_bytes(window, head_dim, ledger_bits)


def kv_tier_counts(n, n_recent, budget_frac, hi_frac, ledger_bits=2):
    hi, lo = ctypes.c_int32(), ctypes.c_int32()
    _ck(LIB.kv_tier_counts(n, n_recent, budget_frac, hi_frac, ledger_bits, ctypes.byref(hi),
                           ctypes.byref(lo)))
    return hi.value, lo.value


def kv_pool_create(cfg: kv_pool_config, arena: torch.Tensor, stream=None):
    h = ctypes.c_void_p()
    _ck(LIB.kv_pool_create(ctypes.byref(cfg), _ptr(arena), arena.numel() * arena.element_size(),
                           _stream(stream), ctypes.byref(h)))
    return h


def kv_pool_destroy(h):
    _ck(LIB.kv_pool_destroy(h))


def kv_pool_region(h, which: int):
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    _ck(LIB.kv_pool_region(h, which, ctypes.byref(off), ctypes.byref(nb)))
    return off.value, nb.value


def kv_prefill(h, layer, k, v, tokens, prior=None, stream=None):
    _ck(LIB.kv_prefill(h, layer, _ptr(k), _ptr(v), tokens, _ptr(prior), _stream(stream)))


def kv_demote_quantize(h, layer, items, counts, stream=None):
    _ck(LIB.kv_demote_quantize(h, layer, _ptr(items), items.shape[-1], _ptr(counts), _stream(stream)))


def kv_promote_dequantize(h, layer, items, counts, stream=None):
    _ck(LIB.kv_promote_dequantize(h, layer, _ptr(items), items.shape[-1], _ptr(counts), _stream(stream)))


def kv_apply_transitions(h, layer, d_items, d_counts, p_items, p_counts, stream=None):
    _ck(LIB.kv_apply_transitions(h, layer, _ptr(d_items), d_items.shape[-1], _ptr(d_counts),
                                 _ptr(p_items), p_items.shape[-1], _ptr(p_counts), _stream(stream)))


def kv_plan_transitions(h, layer, d_items, d_counts, p_items, p_counts, stream=None):
    _ck(LIB.kv_plan_transitions(h, layer, _ptr(d_items), d_items.shape[-1], _ptr(d_counts),
                                _ptr(p_items), p_items.shape[-1], _ptr(p_counts), _stream(stream)))


def kv_move_planned(h, layer, stream=None):
    _ck(LIB.kv_move_planned(h, layer, _stream(stream)))


def kv_attn_workspace_bytes(h) -> int:
    return LIB.kv_attn_workspace_bytes(h)


def kv_tiered_decode_attn(h, layer, q, out, mass, workspace, k_new=None, v_new=None, stream=None):
    _ck(LIB.kv_tiered_decode_attn(h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(mass),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))


def kv_decode_step(h, layer, q, out, mass, workspace, k_new=None, v_new=None, stream=None):
    _ck(LIB.kv_decode_step(h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(mass),
                           _ptr(workspace), workspace.numel(), _stream(stream)))


def kv_decode_step_noalloc(h, layer, q, out, mass, k_new=None, v_new=None, stream=None):
    _ck(LIB.kv_decode_step_noalloc(h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(mass),
                                   _stream(stream)))


KV_NOALLOC_SCRATCH_BYTES = 16 << 20


def kv_score_route(h, layer, mass, do_route, budget_frac, hi_frac, transitions=None, counts=None,
                   stream=None):
    _ck(LIB.kv_score_route(h, layer, _ptr(mass), int(do_route), float(budget_frac), float(hi_frac),
                           _ptr(transitions), _ptr(counts), _stream(stream)))


def kv_route_diagnostics(h, layer, counts, shadow_mass, diag, stream=None):
    _ck(LIB.kv_route_diagnostics(h, layer, _ptr(counts), _ptr(shadow_mass), _ptr(diag), _stream(stream)))


def kv_prefill_scores(h, layer, q, k, tokens, workspace, stream=None):
    _ck(LIB.kv_prefill_scores(h, layer, _ptr(q), _ptr(k), int(tokens), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)))


def kv_read_ledger(h, layer, b, window, dst, stream=None):
    _ck(LIB.kv_read_ledger(h, layer, b, window, _ptr(dst), _stream(stream)))


def kv_read_window(h, layer, b, window, dst, stream=None):
    _ck(LIB.kv_read_window(h, layer, b, window, _ptr(dst), _stream(stream)))


def kv_stream_probe(src: torch.Tensor, nbytes: int, stride: int, count: int, workgroups: int,
                    sink: torch.Tensor, timed: bool = True, stream=None):
    """`count` back-to-back streaming reads of `nbytes` at src + i * stride;
    returns each launch's duration in milliseconds when `timed`."""
    if (count - 1) * stride + nbytes > src.numel() * src.element_size():
        raise ValueError("probe reads past the source tensor")
    if sink.numel() * sink.element_size() < 16 * workgroups:
        raise ValueError("sink needs 4 words per workgroup")
    ms = (ctypes.c_float * count)() if timed else None
    _ck(LIB.kv_stream_probe(_ptr(src), nbytes, stride, count, workgroups, _ptr(sink), _stream(stream), ms))
    return [ms[i] for i in range(count)] if timed else None


def kv_pool_check(h, stream=None) -> int:
    bits = ctypes.c_int32()
    st = LIB.kv_pool_check(h, _stream(stream), ctypes.byref(bits))
    if st not in (KV_OK, KV_ESTATE):
        _ck(st)
    return bits.value


def kv_attn_profile(h, capacity: int):
    _ck(LIB.kv_attn_profile(h, capacity))


def kv_attn_timings(h, cap: int = 1 << 16):
    buf = (ctypes.c_float * cap)()
    n = ctypes.c_int32()
    _ck(LIB.kv_attn_timings(h, buf, cap, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


# ------------------------------------------------------- tensor ownership ---
class Pool:
    """A pool over a torch-allocated arena, with its attention workspace."""

    def __init__(self, cfg: kv_pool_config, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        nbytes = kv_pool_arena_bytes(cfg)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.h = kv_pool_create(cfg, self.arena)
        self.workspace = torch.empty(max(kv_attn_workspace_bytes(self.h), 256), dtype=torch.uint8,
                                     device=self.device)
        self.bits = cfg.ledger_bits or 2
        self.entry_bytes = kv_ledger_entry_bytes(cfg.window, cfg.head_dim, self.bits)

    def close(self):
        if self.h is not None:
            kv_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def region(self, which: int, dtype=torch.uint8) -> torch.Tensor:
        off, nb = kv_pool_region(self.h, which)
        return self.arena[off:off + nb].view(dtype)

    def pages(self, layer: int) -> torch.Tensor:
        c = self.cfg
        return self.region(KV_REGION_PAGES, torch.int32).view(c.layers, c.batch, c.max_windows)[layer]

    def scores(self, layer: int) -> torch.Tensor:
        c = self.cfg
        return self.region(KV_REGION_SCORES, torch.float32).view(c.layers, c.batch, c.max_windows)[layer]

    def tokens(self, layer: int) -> torch.Tensor:
        c = self.cfg
        return self.region(KV_REGION_TOKENS, torch.int32).view(c.layers, c.batch)[layer]

    def _need(self, t, shape, dtypes, name):
        if t is None:
            return
        if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or t.device != self.device:
            raise ValueError(f"{name}: expected {tuple(shape)} {dtypes} on {self.device}, "
                             f"got {tuple(t.shape)} {t.dtype} on {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def prefill(self, layer, k, v, tokens, prior=None):
        c = self.cfg
        shape = (c.batch, c.kv_heads, tokens, c.head_dim)
        self._need(k, shape, _BF16, "k")
        self._need(v, shape, _BF16, "v")
        self._need(prior, (c.batch, -(-tokens // c.window)), (torch.float32,), "prior")
        kv_prefill(self.h, layer, k, v, tokens, prior)

    def _items(self, items, counts):
        c = self.cfg
        if items.dim() != 2 or items.shape[0] != c.batch:
            raise ValueError("items must be [batch][stride]")
        self._need(items, tuple(items.shape), (torch.int32,), "items")
        self._need(counts, (c.batch,), (torch.int32,), "counts")

    def demote(self, layer, items, counts):
        self._items(items, counts)
        kv_demote_quantize(self.h, layer, items, counts)

    def promote(self, layer, items, counts):
        self._items(items, counts)
        kv_promote_dequantize(self.h, layer, items, counts)

    def transitions(self, layer, d_items, d_counts, p_items, p_counts):
        """kv_apply_transitions: the demotions, then the promotions, one plan launch."""
        self._items(d_items, d_counts)
        self._items(p_items, p_counts)
        kv_apply_transitions(self.h, layer, d_items, d_counts, p_items, p_counts)

    def plan_transitions(self, layer, d_items, d_counts, p_items, p_counts, stream=None):
        """kv_plan_transitions on `stream` (default: the current stream)."""
        self._items(d_items, d_counts)
        self._items(p_items, p_counts)
        kv_plan_transitions(self.h, layer, d_items, d_counts, p_items, p_counts, stream)

    def move_planned(self, layer, stream=None):
        """kv_move_planned on `stream` (default: the current stream)."""
        kv_move_planned(self.h, layer, stream)

    def attn(self, layer, q, k_new=None, v_new=None, out=None, mass=None, want_mass=True, scores=False):
        """kv_tiered_decode_attn, or kv_decode_step when `scores` (fused score update)."""
        c = self.cfg
        if out is None:
            out = torch.empty(c.batch, c.q_heads, c.head_dim, dtype=torch.float32, device=self.device)
        if mass is None and want_mass:
            mass = torch.zeros(c.batch, c.q_heads, c.max_windows, dtype=torch.float32, device=self.device)
        self._need(q, (c.batch, c.q_heads, c.head_dim), _BF16, "q")
        self._need(k_new, (c.batch, c.kv_heads, c.head_dim), _BF16, "k_new")
        self._need(v_new, (c.batch, c.kv_heads, c.head_dim), _BF16, "v_new")
        self._need(out, (c.batch, c.q_heads, c.head_dim), (torch.float32,), "out")
        self._need(mass, (c.batch, c.q_heads, c.max_windows), (torch.float32,), "mass")
        fn = kv_decode_step if scores else kv_tiered_decode_attn
        fn(self.h, layer, q, out, mass, self.workspace, k_new, v_new)
        return out, mass

    def score_route(self, layer, mass, do_route, budget_frac=0.0, hi_frac=0.0, transitions=None,
                    counts=None):
        c = self.cfg
        if do_route and transitions is None:
            transitions = torch.zeros(3, c.batch, c.max_windows, dtype=torch.int32, device=self.device)
            counts = torch.zeros(4, c.batch, dtype=torch.int32, device=self.device)
        self._need(mass, (c.batch, c.q_heads, c.max_windows), (torch.float32,), "mass")
        if do_route:
            self._need(transitions, (3, c.batch, c.max_windows), (torch.int32,), "transitions")
            self._need(counts, (4, c.batch), (torch.int32,), "counts")
        kv_score_route(self.h, layer, mass, do_route, budget_frac, hi_frac, transitions, counts)
        return transitions, counts

    def apply_route(self, layer, transitions, counts):
        """Demotions then promotions of a routing event, straight from device lists."""
        self.transitions(layer, transitions[0], counts[0], transitions[1], counts[1])

    def diagnostics(self, layer, diag, counts=None, shadow_mass=None):
        """kv_route_diagnostics into diag float [batch][5] (churn, promotions,
        demotions, Global LIR, future missed mass)."""
        c = self.cfg
        self._need(diag, (c.batch, 5), (torch.float32,), "diag")
        self._need(counts, (4, c.batch), (torch.int32,), "counts")
        self._need(shadow_mass, (c.batch, c.q_heads, c.max_windows), (torch.float32,), "shadow_mass")
        kv_route_diagnostics(self.h, layer, counts, shadow_mass, diag)
        return diag

    def prefill_scores(self, layer, q, k, tokens, workspace=None):
        """kv_prefill_scores: scores from the prefill attention; returns the
        workspace (uint8) holding lse then the token weights."""
        c = self.cfg
        self._need(q, (c.batch, c.q_heads, tokens, c.head_dim), _BF16, "q")
        self._need(k, (c.batch, c.kv_heads, tokens, c.head_dim), _BF16, "k")
        if workspace is None:
            workspace = torch.empty(LIB.kv_prefill_scores_workspace_bytes(self.h, int(tokens)),
                                    dtype=torch.uint8, device=self.device)
        kv_prefill_scores(self.h, layer, q, k, tokens, workspace)
        return workspace

    def read_ledger(self, layer, b, w) -> torch.Tensor:
        dst = torch.empty(self.cfg.kv_heads, self.entry_bytes, dtype=torch.uint8, device=self.device)
        kv_read_ledger(self.h, layer, b, w, dst)
        return dst

    def read_window(self, layer, b, w) -> torch.Tensor:
        c = self.cfg
        dst = torch.empty(c.kv_heads, 2, c.window, c.head_dim, dtype=torch.int16, device=self.device)
        kv_read_window(self.h, layer, b, w, dst)
        return dst

    def check(self) -> int:
        return kv_pool_check(self.h)
