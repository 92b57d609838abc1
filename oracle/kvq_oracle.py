"""CPU oracle for low-bit KV-cache compression and decode attention.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. The product path
(kv_cache_compression_kvq_amd and its HIP library) never imports, calls or
links it, and this module imports nothing from the product path.

A plain, slow, readable numpy implementation of what the compressed-cache
decode path computes:

* quantization parameters in IEEE fp32 (numpy float32 arithmetic, round to
  nearest even), codes rounded half-to-even and clamped to [0, 2^b - 1];
* scale and zero-point stored in fp16;
* OTT outlier-token tracing with the pool replaced by the group mean;
* attention in fp64 on values dequantized from the stored fp16 scale/zero;
* H2O accumulated-attention increments and heavy-hitter selection.

Page citations name the page title and the section they come from:

[MiniKV]  "MiniKV: Pushing the Limits of LLM Inference via 2-Bit
          Layer-Discriminative KV Cache" (arXiv 2411.18077)
[OTT]     "Accurate KV Cache Quantization with Outlier Tokens Tracing"
          (papercache.org summary of the ACL 2025 paper)
[H2O]     "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of
          Large Language Models"
[POFE]    "KV cache quantization and eviction: FP8, INT4, H2O and attention
          sinks" (pofe.ai)
[KVTC]    "KV Cache Transform Coding for Compact Storage in LLM Inference"
          (arXiv 2511.01815)

Readings taken where the pages leave a step open:

R1  Codes use round-half-to-even. [OTT] "Background" prints a floor, while
    [POFE] "Minimal implementation" rounds; rounding is what gives the
    |x - x_hat| <= q/2 bound.
R2  The range is clamped below at 1e-8 before dividing ([POFE] "Minimal
    implementation"); codes are computed from the fp32 step q, dequantization
    uses the stored fp16 scale ([MiniKV] section 4.4: zero-point and scale are
    kept in FP16).
R3  One group size G for both axes: keys per channel over G tokens, values per
    token over G channels ([POFE] "FP8, KIVI and KVQuant": groups of 32 on both
    axes; [MiniKV] section 5.1: one group size for token- and channel-wise).
R4  Residual rule: after T tokens, n_q = floor((T - R)/G)*G tokens are
    quantized, the rest stay fp16 ([POFE] "Minimal implementation"); keys and
    values are compressed together ([OTT] "Experimental setup").
R5  Outlier score S_i is the exact L1 norm of the token's fp16 key ([OTT]
    "Method details" and appendix E); ties in the pool competition go to the
    older (smaller index) token.
R6  A token admitted to the pool has its K and V rows replaced, inside the
    group being quantized, by the per-channel mean of all G rows of that group
    (outliers included), computed exactly and rounded once to fp16 ([OTT]
    "Method details": replaced by the mean of all tokens).
R7  Pool members displaced by better candidates move to an extra pool of
    capacity E (32 on the page); when an admission needs a displacement and
    the extra pool is full, tracing stops for good and the rest of that group
    is quantized as is ([OTT] "Method details" and "Experimental setup").
R8  Every cached token counts exactly once in attention: pool and extra-pool
    tokens use their original fp16 K/V and their quantized slots are
    skipped; tokens at index >= n_q use the fp16 residual rows ([OTT]
    "Method details", decoding stage; [MiniKV] Algorithm 1, decoding).
R9  Softmax scale 1/sqrt(d), d = head_dim ([MiniKV] section 2, Eq. 1).
R10 The H2O score increment is the normalized softmax probability summed over
    the query heads that share one KV head ([POFE] "Heavy hitters" and
    "Minimal implementation"; [H2O] accumulated attention).
R11 Heavy-hitter selection keeps the k highest scores in [0, T - w) ordered by
    (score descending, index descending) plus the w most recent tokens, and
    returns ascending indices. Index-descending tie order is what repeated
    first-occurrence argmin eviction leaves behind ([POFE] "Minimal
    implementation"; [MiniKV] Algorithm 1, heavy-hitter selection).
R12 Attention sinks: the first S tokens of every unit stay in fp16 for good.
    They are never quantized, never traced by OTT and never evicted; the
    residual rule and the quantization groups apply to the tokens after them
    ([POFE] "Attention sinks and StreamingLLM": the key-value states of the
    first few tokens, four in StreamingLLM, are kept; "Failure modes": keep
    sinks pinned; [KVTC] section 2, Preliminaries: s = 4 sink tokens are
    left uncompressed).
R13 H2O eviction during decoding: after a step, while the cache holds more
    than B live tokens, the live token with the lowest accumulated score
    outside the w most recent ones (and not a sink) is evicted, one per step
    and per KV head ([H2O] greedy eviction; [POFE] "Heavy hitters" and
    h2o_evict in "Minimal implementation"). Ties go to the older token (a
    first-occurrence argmin); a NaN score ranks below every number (R11b).
    An evicted token drops out of attention and gets no further score; in the
    compressed cache its codes stay in place (its group's scale is shared).
R14 Pyramid budgets ([MiniKV] section 4.2): with average budget x and depth
    d over L layers the budgets fall linearly from 2x - x/d at the lowest
    layer to x/d at the highest (the page calls the layer with x/d
    "bottom-most" but also allocates more cache to lower layers, as the
    pyramid policy it follows does; the latter is taken), rounded down.
R15 FP8 codec (b = 8): every element is stored as FP8 E4M3 (OCP: bias 7,
    largest finite 448, S.1111.111 is NaN, no infinity) of x / s, with one fp32
    scale s per KV head for keys and one for values (1.0 unless set); the fp32
    quotient is rounded to the nearest E4M3 value, ties to even, and saturates
    at +-448 ([POFE] "FP8, KIVI and KVQuant": E4M3, largest finite value 448,
    a scale per tensor or per head, 1.0 by default; "Failure modes": FP8 casts
    must saturate instead of producing NaN). Dequantization is code value * s.
    The residual window and the 32-token granularity of n_q stay as for the
    integer codecs; there are no groups, zero points or outlier pools.
R16 Prefill scores ([MiniKV] section 4.3, selective flash-attention, and
    Algorithm 1, prefill): causal attention of the n prompt tokens gives the
    outputs X_O and, per KV head, A_cumul[j] = sum over the query heads of the
    head and over the query rows i >= j of the normalized probability P[i][j]
    (the page's buffer shape names "headDim" where the number of heads is
    meant). The heavy hitters of A_cumul plus a recent window are the tokens
    kept and quantized ([MiniKV] section 4.1, persistent context selection).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

RANGE_FLOOR = np.float32(1e-8)


# --------------------------------------------------------------------------
# Quantizer ([OTT] "Background": uniform / group quantization, step
# q = (X_max - X_min)/(2^b - 1); [POFE] "The quantiser and why the grouping
# axis matters" and "Minimal implementation").
# --------------------------------------------------------------------------

def minmax_quantize(x16: np.ndarray, axis: int, bits: int):
    """Asymmetric min-max quantization of fp16 data along ``axis``.

    Returns (codes uint8, scale fp16, zero fp16, q fp32). ``scale``, ``zero``
    and ``q`` keep ``axis`` as a length-1 dimension.

    The step is q = fl32(fl32(max(fl32(mx - mn), 1e-8)) / (2^b - 1)); the code
    is clamp(rint(fl32(fl32(x - mn) / q)), 0, 2^b - 1) with rint rounding half
    to even (R1, R2). The zero-point is the group minimum, exact in fp16.
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    levels = np.float32(2 ** bits - 1)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    rng = np.maximum(mx - mn, RANGE_FLOOR)
    q = rng / levels
    t = (x - mn) / q
    codes = np.clip(np.rint(t), np.float32(0), levels).astype(np.uint8)
    return codes, q.astype(np.float16), mn.astype(np.float16), q


def quantize_key_group(k16: np.ndarray, bits: int):
    """Keys of one group [G][d]: one (scale, zero) per channel over the G tokens.

    Returns codes [G][d], scale [d], zero [d] (fp16).
    """
    codes, s, z, _ = minmax_quantize(k16, axis=0, bits=bits)
    return codes, s[0], z[0]


def quantize_value_rows(v16: np.ndarray, bits: int, gv: int):
    """Values [n][d]: one (scale, zero) per token for each run of gv channels.

    Returns codes [n][d], scale [n][d/gv], zero [n][d/gv] (fp16).
    """
    n, d = v16.shape
    g = np.asarray(v16).reshape(n, d // gv, gv)
    codes, s, z, _ = minmax_quantize(g, axis=2, bits=bits)
    return codes.reshape(n, d), s[:, :, 0], z[:, :, 0]


def dequantize(codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """x_hat = code * scale + zero in fp64 from the stored fp16 parameters (R2)."""
    return codes.astype(np.float64) * scale16.astype(np.float64) + zero16.astype(np.float64)


# --------------------------------------------------------------------------
# FP8 E4M3 codec (R15).
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 byte: (-1)^s 2^(e-7) (1 + m/8) for e > 0,
    (-1)^s 2^-6 (m/8) for e = 0; S.1111.111 is NaN."""
    sgn, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = math.ldexp(1 + m / 8, e - 7) if e else math.ldexp(m / 8, -6)
    return -v if sgn else v


# the 127 finite non-negative magnitudes, ascending (codes 0x00 .. 0x7E)
_E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)])


def e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even of fp32 values to E4M3 codes (R15).

    Each |x| goes to the nearest finite magnitude; on a tie the even code
    (even mantissa) wins; |x| above the largest finite value (inf included)
    gives 448. The sign bit is the sign of x (so -0 -> 0x80)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat, res = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        a = abs(v)
        if math.isnan(a):
            c = 0x7F
        elif a >= _E4M3_POS[-1]:
            c = 0x7E
        else:
            hi = int(np.searchsorted(_E4M3_POS, a))      # first magnitude >= a
            if _E4M3_POS[hi] == a:
                c = hi
            else:
                lo = hi - 1
                dl, dh = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
                c = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        res[i] = c | (0x80 if math.copysign(1.0, v) < 0 else 0)
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of E4M3 codes."""
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.uint8)]


def fp8_quantize(x16: np.ndarray, scale: float) -> np.ndarray:
    """Codes of fp16 data with an fp32 scale: E4M3(fl32(x / s)) (R15)."""
    q = np.asarray(x16, dtype=np.float16).astype(np.float32) / np.float32(scale)
    return e4m3_encode(q)


# --------------------------------------------------------------------------
# Packing ([MiniKV] section 4.4: bit shifting packs 16 INT2 values into one
# INT32). Canonical order: within a token row, channel c goes to word
# c // (32/b) at bit offset b * (c % (32/b)), least significant first.
# --------------------------------------------------------------------------

def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    n, d = codes.shape
    per = 32 // bits
    words = np.zeros((n, d // per), dtype=np.uint64)
    for i in range(per):
        words |= codes[:, i::per].astype(np.uint64) << np.uint64(bits * i)
    return words.astype(np.uint32)


def unpack_rows(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    n = words.shape[0]
    per = 32 // bits
    out = np.zeros((n, d), dtype=np.uint8)
    mask = (1 << bits) - 1
    w = words.astype(np.uint64)
    for i in range(per):
        out[:, i::per] = ((w >> np.uint64(bits * i)) & np.uint64(mask)).astype(np.uint8)
    return out


# --------------------------------------------------------------------------
# Residual window (R4).
# --------------------------------------------------------------------------

def n_quantized(T: int, R: int, G: int) -> int:
    """Tokens held quantized after T appends: max(0, floor((T - R)/G) * G)."""
    return max(0, (T - R) // G * G)


# --------------------------------------------------------------------------
# OTT outlier-token tracing ([OTT] "Method details", appendix E).
# --------------------------------------------------------------------------

def key_l1_score(k16: np.ndarray) -> np.ndarray:
    """S_i = sum_c |K_{i,c}|, exact.

    fp16 magnitudes are integer multiples of 2^-24 below 2^16, so every
    partial sum of at most 128 of them is a multiple of 2^-24 below 2^23 and
    fits the 53-bit fp64 significand: the fp64 sum has no rounding.
    """
    return np.abs(np.asarray(k16, dtype=np.float16).astype(np.float64)).sum(axis=-1)


def group_mean_fp16(x16: np.ndarray) -> np.ndarray:
    """Per-channel mean of the G rows of a group, rounded once to fp16 (R6).

    The fp64 sum is exact (see key_l1_score), division by G (a power of two)
    is exact, and numpy's float64 -> float16 conversion rounds to nearest
    even directly from the double.
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    return (x.sum(axis=0) / x.shape[0]).astype(np.float16)


@dataclass
class PoolMember:
    score: float
    idx: int
    k: np.ndarray  # original fp16 key row
    v: np.ndarray  # original fp16 value row


@dataclass
class OutlierTracer:
    """Outlier pool of capacity N plus the extra pool of capacity E (R5-R7)."""
    N: int
    E: int
    pool: list = field(default_factory=list)
    evicted: list = field(default_factory=list)
    frozen: bool = False

    def compete(self, idx: np.ndarray, scores: np.ndarray, k16: np.ndarray, v16: np.ndarray):
        """One quantization step for the G tokens of a group.

        The group's tokens and the current pool are ranked together by
        (score, index) ascending; the N best form the new pool
        ([OTT] appendix E). Winners from the group are admitted in that order;
        each admission into a full pool moves the pool's current worst member
        to the extra pool. Returns the group positions admitted.
        """
        if self.N == 0 or self.frozen:
            return []
        cands = [(m.score, m.idx, -1) for m in self.pool]
        cands += [(float(scores[i]), int(idx[i]), i) for i in range(len(idx))]
        cands.sort(key=lambda c: (c[0], c[1]))
        winners = [c[2] for c in cands[: self.N] if c[2] >= 0]
        admitted = []
        for i in winners:
            if len(self.pool) == self.N:
                worst = max(self.pool, key=lambda m: (m.score, m.idx))
                if len(self.evicted) == self.E:
                    self.frozen = True
                    break
                self.pool.remove(worst)
                self.evicted.append(worst)
            self.pool.append(PoolMember(float(scores[i]), int(idx[i]),
                                        k16[i].copy(), v16[i].copy()))
            admitted.append(i)
        return admitted


# --------------------------------------------------------------------------
# One (batch, KV head) unit of the compressed cache.
# --------------------------------------------------------------------------

@dataclass
class CacheParams:
    bits: int
    group: int
    residual: int
    pool: int = 0
    evict_cap: int = 32
    head_dim: int = 128
    sinks: int = 0  # S: the first S tokens stay fp16 (R12)
    fp8_scale_k: float = 1.0  # b = 8: per-KV-head scales (R15)
    fp8_scale_v: float = 1.0

    @property
    def gv(self) -> int:
        return min(self.group, self.head_dim)


class UnitCache:
    """Keys/values of one unit: fp16 sinks, quantized groups, fp16 residual
    window, pools. Tokens S .. S + n_q - 1 are the quantized ones (R12)."""

    def __init__(self, p: CacheParams):
        self.p = p
        d = p.head_dim
        self._k16 = [np.zeros((0, d), dtype=np.float16)]  # every appended row, original
        self._v16 = [np.zeros((0, d), dtype=np.float16)]
        self.n_q = 0
        # one entry per quantized group; read through the concatenating properties below
        self._kcodes, self._kscale, self._kzero = [], [], []
        self._vcodes, self._vscale, self._vzero, self._replaced = [], [], [], []
        self.tracer = OutlierTracer(p.pool, p.evict_cap)

    @staticmethod
    def _cat(parts, shape, dtype):
        return np.concatenate(parts) if parts else np.zeros(shape, dtype=dtype)

    @property
    def k16(self) -> np.ndarray:
        if len(self._k16) > 1:
            self._k16 = [np.concatenate(self._k16)]
        return self._k16[0]

    @property
    def v16(self) -> np.ndarray:
        if len(self._v16) > 1:
            self._v16 = [np.concatenate(self._v16)]
        return self._v16[0]

    @property
    def kcodes(self):
        return self._cat(self._kcodes, (0, self.p.head_dim), np.uint8)

    @property
    def kscale(self):  # per group [n_q/G][d]
        return self._cat(self._kscale, (0, self.p.head_dim), np.float16)

    @property
    def kzero(self):
        return self._cat(self._kzero, (0, self.p.head_dim), np.float16)

    @property
    def vcodes(self):
        return self._cat(self._vcodes, (0, self.p.head_dim), np.uint8)

    @property
    def vscale(self):  # per token [n_q][d/gv]
        return self._cat(self._vscale, (0, self.p.head_dim // self.p.gv), np.float16)

    @property
    def vzero(self):
        return self._cat(self._vzero, (0, self.p.head_dim // self.p.gv), np.float16)

    @property
    def replaced(self):  # token was admitted to the pool
        return self._cat(self._replaced, (0,), bool)

    @property
    def T(self) -> int:
        return sum(x.shape[0] for x in self._k16)

    def append(self, k16: np.ndarray, v16: np.ndarray) -> None:
        """Append fp16 rows; quantize every group that leaves the residual window
        (the residual rule counts the tokens after the S sinks, R12)."""
        self._k16.append(np.asarray(k16, dtype=np.float16))
        self._v16.append(np.asarray(v16, dtype=np.float16))
        G, S = self.p.group, self.p.sinks
        T = self.T
        while self.n_q < n_quantized(max(0, T - S), self.p.residual, G):
            self._quantize_group(S + self.n_q)
            self.n_q += G

    def _quantize_group(self, t0: int) -> None:
        G = self.p.group
        kg = self.k16[t0:t0 + G].copy()
        vg = self.v16[t0:t0 + G].copy()
        if self.p.bits == 8:  # FP8 codec: per element, no groups or pools (R15)
            self._kcodes.append(fp8_quantize(kg, self.p.fp8_scale_k))
            self._vcodes.append(fp8_quantize(vg, self.p.fp8_scale_v))
            self._replaced.append(np.zeros(G, dtype=bool))
            return
        idx = np.arange(t0, t0 + G)
        admitted = self.tracer.compete(idx, key_l1_score(kg), kg, vg)
        replaced = np.zeros(G, dtype=bool)
        if admitted:
            mk, mv = group_mean_fp16(kg), group_mean_fp16(vg)
            for i in admitted:
                kg[i], vg[i] = mk, mv
                replaced[i] = True
        kc, ks, kz = quantize_key_group(kg, self.p.bits)
        vc, vs, vz = quantize_value_rows(vg, self.p.bits, self.p.gv)
        self._kcodes.append(kc)
        self._kscale.append(ks[None])
        self._kzero.append(kz[None])
        self._vcodes.append(vc)
        self._vscale.append(vs)
        self._vzero.append(vz)
        self._replaced.append(replaced)

    def dequantized_kv(self):
        """K_hat, V_hat [T][d] in fp64, each cached token exactly once (R8)."""
        G, gv, d, S = self.p.group, self.p.gv, self.p.head_dim, self.p.sinks
        n_q = self.n_q
        K = self.k16.astype(np.float64)  # sink and residual rows stay as stored (fp16)
        V = self.v16.astype(np.float64)
        if n_q and self.p.bits == 8:
            K[S:S + n_q] = e4m3_decode(self.kcodes) * float(np.float32(self.p.fp8_scale_k))
            V[S:S + n_q] = e4m3_decode(self.vcodes) * float(np.float32(self.p.fp8_scale_v))
        elif n_q:
            ks = np.repeat(self.kscale, G, axis=0)
            kz = np.repeat(self.kzero, G, axis=0)
            K[S:S + n_q] = dequantize(self.kcodes, ks, kz)
            vs = np.repeat(self.vscale, gv, axis=1)
            vz = np.repeat(self.vzero, gv, axis=1)
            V[S:S + n_q] = dequantize(self.vcodes, vs, vz)
        for m in self.tracer.pool + self.tracer.evicted:
            K[m.idx] = m.k.astype(np.float64)
            V[m.idx] = m.v.astype(np.float64)
        return K, V

    def pool_indices(self):
        return sorted(m.idx for m in self.tracer.pool)

    def evicted_indices(self):
        return [m.idx for m in self.tracer.evicted]


# --------------------------------------------------------------------------
# Decode attention ([MiniKV] section 2, Eq. 1 and Algorithm 1 decoding;
# [OTT] "Method details", decoding stage) and H2O scores.
# --------------------------------------------------------------------------

def unit_attention(K: np.ndarray, V: np.ndarray, q16: np.ndarray, live=None):
    """Attention of the r query heads q16 [r][d] over one unit's K, V [T][d] (fp64).

    Returns out [r][d] and the normalized probabilities p [r][T]:
    s = K q / sqrt(d); p = exp(s - max s) / sum; out = p V. With ``live`` (bool
    [T]) only those tokens are attended; the others get p = 0 (R13).
    """
    d = K.shape[1]
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    s = (q @ K.T) / math.sqrt(d)
    if live is not None:
        s[:, ~np.asarray(live, dtype=bool)] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V, p


def h2o_increment(p: np.ndarray) -> np.ndarray:
    """Score increment for one KV head: sum over its query heads of p [r][T] (R10)."""
    return p.sum(axis=0)


def prefill_attention(q16: np.ndarray, k16: np.ndarray, v16: np.ndarray):
    """Causal attention of one KV head's r query heads over n prompt tokens (R16).

    q16 [r][n][d], k16 / v16 [n][d] fp16. Returns the outputs [r][n][d] and
    A_cumul [n] = sum_h sum_i P_h[i][j], in fp64: S = Q K^T / sqrt(d) with
    keys after the query masked, P = softmax over each row."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    k = np.asarray(k16, dtype=np.float16).astype(np.float64)
    v = np.asarray(v16, dtype=np.float16).astype(np.float64)
    r, n, d = q.shape
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    out = np.empty((r, n, d))
    acum = np.zeros(n)
    for h in range(r):
        s = (q[h] @ k.T) / math.sqrt(d)
        s[future] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        out[h] = p @ v
        acum += p.sum(axis=0)
    return out, acum


def gather_rows(x16: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Rows idx of x16 [n][d] (the tokens kept after prefill selection)."""
    return np.asarray(x16)[np.asarray(idx, dtype=np.int64)]


def h2o_evict_one(scores: np.ndarray, live: np.ndarray, budget: int, recent: int, sinks: int):
    """One H2O eviction step for one KV head (R13).

    ``scores`` fp32 [T] accumulated attention, ``live`` bool [T] (updated in
    place). If more than ``budget`` tokens are live, the live token in
    [sinks, T - recent) with the lowest score is evicted; ties go to the lower
    index and NaN ranks lowest. Returns the evicted index or -1.
    """
    T = len(scores)
    if int(live.sum()) <= budget:
        return -1
    best, best_i = None, -1
    for t in range(sinks, T - recent):
        if not live[t]:
            continue
        v = float(scores[t])
        key = (0, 0.0) if math.isnan(v) else (1, v)   # NaN first, then by value
        if best is None or key < best:
            best, best_i = key, t
    if best_i >= 0:
        live[best_i] = False
    return best_i


def pyramid_budgets(n_layers: int, avg: int, depth: int):
    """Per-layer heavy-hitter budgets, lowest layer first (R14):
    b_l = (2x - x/d) - l (2x - 2x/d) / (L - 1), rounded down (exact rationals)."""
    from fractions import Fraction
    x, d = Fraction(avg), Fraction(depth)
    top, low = 2 * x - x / d, x / d
    if n_layers == 1:
        return [int(x)]
    return [math.floor(top - (top - low) * l / (n_layers - 1)) for l in range(n_layers)]


class CacheOracle:
    """All units of a [batch][n_kv_heads] cache, or a chosen subset of them."""

    def __init__(self, p: CacheParams, batch: int, n_kv_heads: int, units=None):
        self.p = p
        self.batch, self.n_kv_heads = batch, n_kv_heads
        self.unit_ids = list(units) if units is not None else [
            (b, h) for b in range(batch) for h in range(n_kv_heads)]
        self.units = {u: UnitCache(p) for u in self.unit_ids}

    def append_unit(self, u, k16: np.ndarray, v16: np.ndarray) -> None:
        self.units[u].append(k16, v16)

    def decode_unit(self, u, q16_group: np.ndarray):
        """out [r][d] and H2O increment [T] for unit u given its r query heads."""
        K, V = self.units[u].dequantized_kv()
        out, p = unit_attention(K, V, q16_group)
        return out, h2o_increment(p), p


# --------------------------------------------------------------------------
# Heavy-hitter selection ([H2O] accumulated attention; [POFE] "Heavy hitters"
# and "Minimal implementation"; [MiniKV] Algorithm 1) (R11).
# --------------------------------------------------------------------------

def topk_keep(scores: np.ndarray, k: int, w: int) -> np.ndarray:
    """Indices kept per row: top-k of [0, T-w) by (score desc, index desc) + [T-w, T).

    ``scores`` is fp32 [rows][T]; returns int32 [rows][k+w], ascending.
    +0 and -0 compare equal; numpy's sort puts NaN after every number in the
    descending order, so a NaN score ranks lowest and NaNs tie.
    """
    scores = np.asarray(scores, dtype=np.float32)
    rows, T = scores.shape
    out = np.empty((rows, k + w), dtype=np.int32)
    n = T - w
    idx = np.arange(n)
    for r in range(rows):
        s = scores[r, :n].astype(np.float64)
        order = np.lexsort((-idx, -s))  # primary: score desc, then index desc
        keep = np.sort(order[:k])
        out[r] = np.concatenate([keep, np.arange(n, T)]).astype(np.int32)
    return out
