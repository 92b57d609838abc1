"""Byte model of the compressed KV cache and of one decode step.

Host-side arithmetic only (sizes, not data):

* bits per stored element with metadata, b_bar = b + 32/g for one fp16 scale
  and one fp16 zero per group of g elements ("KV cache quantization and
  eviction: FP8, INT4, H2O and attention sinks", section "The bottleneck in
  numbers");
* cache bytes per token, kappa = 2 * L * n_kv * d_h * bytes_per_element (same
  section);
* the algorithmic bytes a decode step over the compressed cache must move,
  which is what throughput is quoted against.
"""
from __future__ import annotations

from dataclasses import dataclass


def bits_per_element(bits: int, group: int, meta_bits: int = 32) -> float:
    """b_bar = b + meta_bits / g (fp16 scale + fp16 zero = 32 bits per group)."""
    return bits + meta_bits / group


def group_bytes(bits: int, group: int) -> int:
    """Bytes held by one quantization group: packed codes plus fp16 scale and zero."""
    return group * bits // 8 + 4


def kv_bytes_per_token(layers: int, n_kv: int, head_dim: int, bytes_per_elem: float) -> float:
    """kappa = 2 * L * n_kv * d_h * b (keys and values)."""
    return 2 * layers * n_kv * head_dim * bytes_per_elem


def n_quantized(T: int, R: int, G: int) -> int:
    return max(0, (T - R) // G * G)


@dataclass(frozen=True)
class StepBytes:
    quantized: int     # packed K/V codes + fp16 scale/zero of the n_q quantized tokens
    residual: int      # fp16 K/V rows of the residual window
    pools: int         # fp16 K/V rows + int32 index of pool / extra-pool tokens
    query_out: int     # fp16 queries in, fp32 outputs out
    h2o: int           # fp32 accumulated scores read + written
    total: int


def decode_step_bytes(*, units: int, gqa: int, head_dim: int, tokens: int, bits: int,
                      group: int, residual: int, pool_tokens: int = 0,
                      h2o: bool = False, sinks: int = 0) -> StepBytes:
    """Algorithmic bytes of one decode-attention step over all units.

    Per unit: n_q*(d*b/4 + 4d/G + 4d/Gv) + n_res*4d + pool_tokens*(4d + 4)
    + r*d*2 (query) + r*d*4 (output) + [H2O] 8*T, with n_q counted after the
    S attention sinks and n_res = T - n_q (sinks and residual window, fp16).
    Scratch (split partials, logits) is implementation traffic and is not
    counted. ``pool_tokens`` is the total over all units.
    """
    d, G = head_dim, group
    gv = min(G, d)
    nq = n_quantized(max(0, tokens - sinks), residual, G)
    nres = tokens - nq
    meta = 0 if bits == 8 else 4 * d // G + 4 * d // gv  # FP8: no scale / zero words
    quant = units * nq * (d * bits // 4 + meta)
    resid = units * nres * 4 * d
    pools = pool_tokens * (4 * d + 4)
    qo = units * gqa * d * (2 + 4)
    h2o_b = units * tokens * 8 if h2o else 0
    return StepBytes(quant, resid, pools, qo, h2o_b, quant + resid + pools + qo + h2o_b)


def append_bytes(*, units: int, head_dim: int, n_new: int, bits: int, group: int,
                 groups_packed: int) -> int:
    """Algorithmic bytes of appending n_new tokens that complete ``groups_packed`` groups.

    fp16 K/V of the new tokens are read once and written to the residual ring;
    each packed group re-reads its G fp16 rows of K and V and writes codes and
    scale/zero for both.
    """
    d, G = head_dim, group
    gv = min(G, d)
    ring = units * n_new * 4 * d * 2
    per_group = G * 4 * d + G * (d * bits // 4) + 4 * d + G * 4 * d // gv
    return ring + units * groups_packed * per_group


def bulk_append_bytes(*, units: int, head_dim: int, tokens: int, n_quant: int, bits: int,
                      group: int) -> int:
    """Algorithmic bytes of appending a whole prefix of ``tokens`` to an empty cache.

    fp16 K/V of every token are read once; the ``n_quant`` quantized tokens
    write codes and scale/zero for keys and values, the rest are written to
    the fp16 residual ring.
    """
    d, G = head_dim, group
    gv = min(G, d)
    per_q = d * bits // 4 + (0 if bits == 8 else 4 * d // G + 4 * d // gv)
    return units * (tokens * 4 * d + n_quant * per_q + (tokens - n_quant) * 4 * d)


def evict_step_bytes(*, rows: int, tokens: int, sinks: int = 0) -> int:
    """One H2O eviction step: every unit's fp32 scores and eviction bitmap read
    once (the single word written per unit is not counted)."""
    n = tokens - sinks
    return rows * (tokens * 4 + (n + 31) // 32 * 4)


def prefill_flops(*, batch: int, n_q_heads: int, head_dim: int, tokens: int) -> int:
    """Causal attention of an n-token prompt: the two products Q K^T and P V,
    2 flops per multiply-add, over the n (n + 1) / 2 unmasked query-key pairs
    of every query head. Recomputing Q K^T for the column sums is
    implementation work and is not counted."""
    pairs = tokens * (tokens + 1) // 2
    return batch * n_q_heads * pairs * head_dim * 2 * 2


def topk_bytes(*, rows: int, tokens: int, k: int, w: int) -> int:
    """fp32 scores read once, int32 kept indices written."""
    return rows * tokens * 4 + rows * (k + w) * 4
