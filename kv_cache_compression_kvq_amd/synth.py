"""Seeded synthetic workloads for compressed-KV decode attention.

This module only describes shapes and draws random numbers. It holds none
of the method's arithmetic (no quantization, no attention, no selection), so
that the CPU oracle and the HIP path can both be fed from it without sharing
any computation.

Workload shapes follow the Llama-3-8B attention layer that the pages use for
their cache-size arithmetic (32 query heads, 8 KV heads, head_dim 128:
"KV cache quantization and eviction: FP8, INT4, H2O and attention sinks",
section "The bottleneck in numbers"). No dataset content is used anywhere;
these tensors stand in for the caches the pages evaluate on LongBench,
GSM8K, RULER and similar suites.

Every tensor is drawn from ``numpy.random.default_rng`` with a seed tuple
``[seed, cfg_id, stream, ...]`` so that any (batch, kv-head) unit can be
regenerated on its own, which lets the oracle check sampled units of the
large workloads without rebuilding the whole cache.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# Seed-stream identifiers (third element of the seed tuple).
_S_KEYS, _S_VALUES, _S_QUERY, _S_CHANNELS, _S_INJECT, _S_STEP, _S_PROTO, _S_SCORES = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tokens: int            # cached tokens T after the bulk append
    bits: int              # b
    group: int             # G (keys: G tokens per channel; values: G channels per token)
    residual: int          # R
    pool: int = 0          # N, outlier-pool capacity
    evict_cap: int = 32    # E, extra pool for displaced pool members
    sinks: int = 0         # S, attention sinks kept in fp16
    fp8_scale_k: float = 1.0  # b = 8: key / value scale of every KV head
    fp8_scale_v: float = 1.0
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    key_dist: str = "normal"     # "normal" or "zipf"
    inject_frac: float = 0.0     # fraction of tokens per unit with low-norm keys
    inject_scale: float = 0.01
    h2o: bool = False
    topk_frac: float = 0.0       # heavy-hitter budget as a fraction of T
    recent: int = 0              # recent window kept by the top-k
    seed: int = 0

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def topk_k(self) -> int:
        return int(self.topk_frac * self.tokens)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads. cfg_id only feeds the seed tuple.
WORKLOADS = {
    "tiny": Workload("tiny", 0, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=128,
                     tokens=1024, bits=2, group=32, residual=32,
                     outlier_channels=4, outlier_scale=20.0),
    "llama8b": Workload("llama8b", 1, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        tokens=8192, bits=2, group=32, residual=128,
                        outlier_channels=6, outlier_scale=15.0),
    # MiniKV's own group size (16 values share a scale and zero point) on the
    # same layer shape; not one of the five headline workloads
    "llama8b_g16": Workload("llama8b_g16", 8, batch=8, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, tokens=8192, bits=2, group=16, residual=128,
                            outlier_channels=6, outlier_scale=15.0),
    # prefill of a 4096-token prompt through the same layer (MiniKV's prompt
    # length), with the heavy-hitter column sums
    "prefill_llama8b": Workload("prefill_llama8b", 11, batch=1, n_q_heads=32, n_kv_heads=8,
                                head_dim=128, tokens=4096, bits=2, group=32, residual=128,
                                outlier_channels=6, outlier_scale=15.0, h2o=True,
                                topk_frac=0.2, recent=256),
    # the same layer with the FP8 E4M3 codec (scales 1.0, the default)
    "llama8b_fp8": Workload("llama8b_fp8", 10, batch=8, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, tokens=8192, bits=8, group=32, residual=128,
                            outlier_channels=6, outlier_scale=15.0),
    # the same layer with four attention sinks kept in fp16
    "llama8b_sinks": Workload("llama8b_sinks", 9, batch=8, n_q_heads=32, n_kv_heads=8,
                              head_dim=128, tokens=8192, bits=2, group=32, residual=128,
                              outlier_channels=6, outlier_scale=15.0, sinks=4),
    "long_b2g32": Workload("long_b2g32", 2, batch=1, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, tokens=131072, bits=2, group=32, residual=128,
                           outlier_channels=6, outlier_scale=15.0),
    "long_b2g128": Workload("long_b2g128", 3, batch=1, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, tokens=131072, bits=2, group=128, residual=128,
                            outlier_channels=6, outlier_scale=15.0),
    "long_b4g32": Workload("long_b4g32", 4, batch=1, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, tokens=131072, bits=4, group=32, residual=128,
                           outlier_channels=6, outlier_scale=15.0),
    "long_b4g128": Workload("long_b4g128", 5, batch=1, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, tokens=131072, bits=4, group=128, residual=128,
                            outlier_channels=6, outlier_scale=15.0),
    "ott": Workload("ott", 6, batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
                    tokens=4096, bits=2, group=32, residual=32, pool=3, evict_cap=32,
                    outlier_channels=6, outlier_scale=15.0, inject_frac=0.005),
    "ott_nopool": Workload("ott_nopool", 6, batch=32, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, tokens=4096, bits=2, group=32, residual=32,
                           pool=0, evict_cap=32, outlier_channels=6, outlier_scale=15.0,
                           inject_frac=0.005),
    "minikv": Workload("minikv", 7, batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       tokens=32768, bits=2, group=32, residual=128,
                       outlier_channels=6, outlier_scale=15.0, key_dist="zipf",
                       h2o=True, topk_frac=0.2, recent=256),
}


def outlier_channel_ids(w: Workload) -> np.ndarray:
    """The fixed key channels that carry the large magnitudes (shared by all units)."""
    rng = np.random.default_rng([w.seed, w.cfg_id, _S_CHANNELS])
    return np.sort(rng.permutation(w.head_dim)[: w.outlier_channels])


def _zipf_prototype_keys(w: Workload, b: int, h: int, n: int, start: int) -> np.ndarray:
    # 256 prototype key vectors per unit; token j picks prototype r with
    # probability proportional to r^-1.1, then adds 0.25-scaled noise.
    prng = np.random.default_rng([w.seed, w.cfg_id, _S_PROTO, b, h])
    protos = prng.standard_normal((256, w.head_dim), dtype=np.float32)
    weights = np.arange(1, 257, dtype=np.float64) ** -1.1
    weights /= weights.sum()
    rng = np.random.default_rng([w.seed, w.cfg_id, _S_KEYS, b, h, start])
    pick = rng.choice(256, size=n, p=weights)
    noise = rng.standard_normal((n, w.head_dim), dtype=np.float32)
    return protos[pick] + np.float32(0.25) * noise


def unit_kv(w: Workload, b: int, h: int, n: int | None = None, start: int = 0):
    """fp16 keys and values [n][head_dim] of unit (b, h) for tokens start .. start+n-1.

    Values are N(0,1). Keys are N(0,1) (or the Zipf prototype mixture) with
    ``outlier_channels`` channels scaled by ``outlier_scale``; with
    ``inject_frac`` > 0 a seeded set of tokens gets those channels scaled by
    ``inject_scale`` instead, which gives them a low key L1 norm.
    Calls with different ``start`` draw independent blocks (used for
    decode-step tokens appended after the bulk prefix).
    """
    n = w.tokens if n is None else n
    d = w.head_dim
    if w.key_dist == "zipf":
        k = _zipf_prototype_keys(w, b, h, n, start)
    else:
        rng = np.random.default_rng([w.seed, w.cfg_id, _S_KEYS, b, h, start])
        k = rng.standard_normal((n, d), dtype=np.float32)
    ch = outlier_channel_ids(w)
    if len(ch):
        base = k[:, ch].copy()
        k[:, ch] = base * np.float32(w.outlier_scale)
        if w.inject_frac > 0 and start == 0:
            irng = np.random.default_rng([w.seed, w.cfg_id, _S_INJECT, b, h])
            n_inj = int(w.inject_frac * n)
            pos = irng.choice(n, size=n_inj, replace=False)
            k[np.ix_(pos, ch)] = base[pos] * np.float32(w.inject_scale)
    vrng = np.random.default_rng([w.seed, w.cfg_id, _S_VALUES, b, h, start])
    v = vrng.standard_normal((n, d), dtype=np.float32)
    return k.astype(np.float16), v.astype(np.float16)


def injected_positions(w: Workload, b: int, h: int) -> np.ndarray:
    """Token positions that received low-norm keys in unit (b, h) (empty if none)."""
    if w.inject_frac <= 0 or w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    irng = np.random.default_rng([w.seed, w.cfg_id, _S_INJECT, b, h])
    n_inj = int(w.inject_frac * w.tokens)
    return np.sort(irng.choice(w.tokens, size=n_inj, replace=False))


def all_kv(w: Workload, n: int | None = None, start: int = 0):
    """fp16 K, V of every unit: arrays [batch][n_kv_heads][n][head_dim]."""
    n = w.tokens if n is None else n
    K = np.empty((w.batch, w.n_kv_heads, n, w.head_dim), dtype=np.float16)
    V = np.empty_like(K)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            K[b, h], V[b, h] = unit_kv(w, b, h, n, start)
    return K, V


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """fp16 decode queries [batch][n_q_heads][head_dim], N(0,1)."""
    rng = np.random.default_rng([w.seed, w.cfg_id, _S_QUERY, step])
    q = rng.standard_normal((w.batch, w.n_q_heads, w.head_dim), dtype=np.float32)
    return q.astype(np.float16)


def step_kv(w: Workload, step: int):
    """fp16 K, V [batch][n_kv_heads][1][head_dim] for one appended decode token."""
    return all_kv(w, n=1, start=w.tokens + 1 + step)


def score_rows(rows: int, T: int, seed: int = 0, ties: bool = False) -> np.ndarray:
    """Non-negative fp32 score rows [rows][T] for exercising heavy-hitter selection.

    With ``ties`` the values come from a small set so that many exact ties occur.
    """
    rng = np.random.default_rng([seed, 0, _S_SCORES, rows, T])
    if ties:
        return (rng.integers(0, 8, size=(rows, T)).astype(np.float32) * np.float32(0.125))
    x = rng.standard_exponential((rows, T), dtype=np.float32)
    return x / np.float32(T)
