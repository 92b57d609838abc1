"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against a value printed on the pages, a closed
form, an invariant, a special case that reduces to a textbook result, or a
brute force on tiny inputs written independently here (Python Fractions and
plain loops). Citations name the page title and section.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq_oracle as O
from tests.fp16ref import half_to_fraction, round_to_half, round_to_half_bits

F32 = np.float32


def fr32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---------------------------------------------------------------------------
# Quantizer ("Accurate KV Cache Quantization with Outlier Tokens Tracing",
# Background: uniform quantization with step q = (X_max - X_min)/(2^b - 1);
# "KV cache quantization and eviction", Minimal implementation).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,mn,q", [(2, -1.5, 0.5), (4, -2.0, 0.25), (2, 3.0, 2.0)])
def test_on_grid_values_are_exact(bits, mn, q):
    """Values mn + c*q with exactly representable q map to code c, zero error."""
    L = 2 ** bits - 1
    codes = np.arange(L + 1)
    x = (mn + codes * q).astype(np.float16)
    x = np.concatenate([x, x[::-1]])[:, None]
    c, s, z, qq = O.minmax_quantize(x, axis=0, bits=bits)
    assert float(qq[0, 0]) == q and float(s[0, 0]) == q and float(z[0, 0]) == mn
    assert np.array_equal(c[:, 0], np.concatenate([codes, codes[::-1]]))
    assert np.array_equal(O.dequantize(c, s, z), x.astype(np.float64))


def test_half_points_round_half_to_even():
    """b=2, range 3 -> q = 1; x = 0.5, 1.5, 2.5 give codes 0, 2, 2.

    Floor would give 0, 1, 2 and round-half-up 1, 2, 3.
    """
    x = np.array([0, 3, 0.5, 1.5, 2.5], dtype=np.float16)[:, None]
    c, _, _, q = O.minmax_quantize(x, axis=0, bits=2)
    assert float(q[0, 0]) == 1.0
    assert c[:, 0].tolist() == [0, 3, 0, 2, 2]


@pytest.mark.parametrize("bits", [2, 4])
def test_group_min_is_exact_and_max_is_top_code(bits):
    rng = np.random.default_rng(1)
    for _ in range(50):
        x = (rng.standard_normal((32, 16)) * rng.uniform(0.01, 30)).astype(np.float16)
        c, s, z, _ = O.minmax_quantize(x, axis=0, bits=bits)
        imin, imax = x.argmin(axis=0), x.argmax(axis=0)
        cols = np.arange(16)
        assert np.all(c[imin, cols] == 0)
        assert np.all(c[imax, cols] == 2 ** bits - 1)
        xh = O.dequantize(c, s, z)
        assert np.array_equal(xh[imin, cols], x[imin, cols].astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound_half_step(bits):
    """|x - (c*q + mn)| <= q/2 in exact arithmetic, up to the fp32 rounding of (x-mn)/q.

    Checked with Fractions on every element; q is the fp32 step as a rational.
    The stored fp16 scale adds at most c*|s16 - q|.
    """
    rng = np.random.default_rng(2)
    L = 2 ** bits - 1
    for trial in range(40):
        x = rng.standard_normal(32) * rng.uniform(0.001, 50)
        if trial % 4 == 0:
            x[rng.integers(32)] *= 40  # one far outlier
        x16 = x.astype(np.float16)[:, None]
        c, s, z, q = O.minmax_quantize(x16, axis=0, bits=bits)
        Q = fr32(q[0, 0])
        S = half_to_fraction(s[0, 0])
        mn = half_to_fraction(z[0, 0])
        for i in range(32):
            xi = half_to_fraction(x16[i, 0])
            ci = int(c[i, 0])
            assert 0 <= ci <= L
            slack = Fraction(1, 2 ** 22) * (abs(xi - mn) + Q)
            assert abs(xi - (ci * Q + mn)) <= Q / 2 + slack
            assert abs(xi - (ci * S + mn)) <= Q / 2 + slack + ci * abs(S - Q)


def test_constant_group_reconstructs_exactly():
    """mx == mn: the range is clamped to 1e-8, every code is 0 and x_hat == x."""
    for v in [0.0, -3.25, 1e-4, 65504.0]:
        x = np.full((32, 4), v, dtype=np.float16)
        c, s, z, q = O.minmax_quantize(x, axis=0, bits=2)
        assert np.all(c == 0)
        assert float(q[0, 0]) == float(np.float32(1e-8) / np.float32(3))
        assert np.array_equal(O.dequantize(c, s, z), x.astype(np.float64))


def test_quantizer_follows_fp32_steps_exactly():
    """Each code equals the hand-derived fp32 step computation done with Fractions.

    rint(fl32(fl32(x - mn)/q)) with q = fl32(fl32(mx - mn)/3); fl32 is an
    independent round-to-nearest-even to binary32 here.
    """
    def fl32(fr: Fraction) -> Fraction:
        if fr == 0:
            return fr
        a = abs(fr)
        e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        ulp = Fraction(2) ** (e - 23)
        n, r = divmod(a, ulp)
        if r * 2 > ulp or (r * 2 == ulp and n % 2 == 1):
            n += 1
        return (n * ulp) * (1 if fr > 0 else -1)

    def rint(fr: Fraction) -> int:
        n = math.floor(fr)
        r = fr - n
        if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
            n += 1
        return n

    rng = np.random.default_rng(3)
    for _ in range(30):
        x16 = (rng.standard_normal(16) * rng.uniform(0.01, 100)).astype(np.float16)
        c, s, z, q = O.minmax_quantize(x16[:, None], axis=0, bits=2)
        xs = [half_to_fraction(v) for v in x16]
        mn, mx = min(xs), max(xs)
        Q = fl32(fl32(mx - mn) / 3)
        assert fr32(q[0, 0]) == Q
        want = [min(3, max(0, rint(fl32(fl32(xi - mn) / Q)))) for xi in xs]
        assert c[:, 0].tolist() == want
        assert int(np.asarray(s[0, 0]).view(np.uint16)) == round_to_half_bits(Q)


def test_key_and_value_grouping_axes():
    """Keys: one (scale, zero) per channel over G tokens; values: per token per run of G channels."""
    rng = np.random.default_rng(4)
    k = (rng.standard_normal((32, 128)) * 3).astype(np.float16)
    kc, ks, kz = O.quantize_key_group(k, 2)
    assert ks.shape == (128,) and kz.shape == (128,)
    assert np.array_equal(kz, k.min(axis=0))
    v = rng.standard_normal((5, 128)).astype(np.float16)
    vc, vs, vz = O.quantize_value_rows(v, 2, 32)
    assert vs.shape == (5, 4)
    assert np.array_equal(vz, v.reshape(5, 4, 32).min(axis=2))
    # a channel-group's codes depend only on that group's 32 values
    v2 = v.copy()
    v2[:, 32:] = 7
    vc2, _, _ = O.quantize_value_rows(v2, 2, 32)
    assert np.array_equal(vc[:, :32], vc2[:, :32])


# ---------------------------------------------------------------------------
# Packing (MiniKV, section 4.4: 16 INT2 values shifted into one INT32).
# ---------------------------------------------------------------------------

def test_pack_bit_positions():
    c2 = np.array([[i % 4 for i in range(16)] * 8], dtype=np.uint8)   # 00,01,10,11 from the LSB
    assert O.pack_rows(c2, 2).tolist() == [[0xE4E4E4E4] * 8]
    c4 = np.array([list(range(8)) * 16], dtype=np.uint8)
    assert O.pack_rows(c4, 4).tolist() == [[0x76543210] * 16]
    one = np.zeros((1, 128), dtype=np.uint8)
    one[0, 17] = 3                        # channel 17 -> word 1, bits 2..3
    w = O.pack_rows(one, 2)
    assert w[0, 1] == 0b1100 and w.sum() == 0b1100


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** bits, size=(37, 128)).astype(np.uint8)
    w = O.pack_rows(c, bits)
    assert w.shape == (37, 128 * bits // 32)
    assert np.array_equal(O.unpack_rows(w, bits, 128), c)


# ---------------------------------------------------------------------------
# Byte model and stored layout (page worked values).
# ---------------------------------------------------------------------------

def test_bits_per_element_matches_pages(golden):
    from kv_cache_compression_kvq_amd import bytes_model as BM
    for case in golden["bits_per_element"]["cases"]:
        assert BM.bits_per_element(case["bits"], case["group"]) == case["bits_per_element"]
    g = golden["group_bytes"]
    assert BM.group_bytes(g["bits"], g["group"]) == g["bytes"]


def test_llama3_cache_sizes_match_pages(golden):
    from kv_cache_compression_kvq_amd import bytes_model as BM
    c = golden["llama3_8b_cache"]
    per_tok = {k: BM.kv_bytes_per_token(c["layers"], c["n_kv_heads"], c["head_dim"], b)
               for k, b in [("bf16", 2), ("fp8", 1),
                            ("int4_g32", BM.bits_per_element(4, 32) / 8),
                            ("int2_g32", BM.bits_per_element(2, 32) / 8)]}
    for k, gb in c["GB_128k"].items():
        assert round(per_tok[k] * c["tokens_128k"] / 1e9, 1) == gb
    full = per_tok["bf16"] * c["tokens_32k"]
    assert round(full / 1e9, 1) == c["GB_32k_full"]
    assert round(full * c["keep_fraction"] / 1e9, 2) == c["GB_32k_kept"]
    assert round(per_tok["bf16"] * c["fixed_entries"] / 1e6) == c["MB_fixed_entries"]
    t = golden["kvtc_table1"]
    assert BM.kv_bytes_per_token(t["layers"], t["n_kv_heads"], t["head_dim"], 2) * t["tokens"] \
        == t["MiB"] * 2 ** 20


def test_minikv_compression_numbers(golden):
    from kv_cache_compression_kvq_amd import bytes_model as BM
    m = golden["minikv_compression"]
    per_tok16 = 2 * m["layers"] * m["hidden"] * 2
    full = per_tok16 * (m["prompt"] + m["gen"])
    kept = m["prompt"] * m["budget"] + m["gen"]
    mini = 2 * m["layers"] * m["hidden"] * kept * BM.bits_per_element(m["bits"], m["group"]) / 8
    assert round(full / 1e9, 1) == m["GB_full"]
    # the page prints 0.33 GB (335.5 MB truncated) and an 86 % reduction
    assert abs(mini / 1e9 - m["GB_minikv"]) < 0.01
    assert round(100 * (1 - mini / full)) == 86


@pytest.mark.parametrize("bits,G", [(2, 32), (4, 32), (2, 128), (4, 16)])
def test_oracle_storage_is_b_plus_32_over_g_bits(bits, G):
    """Packed codes + fp16 scale/zero held by the oracle cost b + 32/G bits per element."""
    rng = np.random.default_rng(6)
    u = O.UnitCache(O.CacheParams(bits=bits, group=G, residual=0))
    k = rng.standard_normal((4 * G, 128)).astype(np.float16)
    u.append(k, k)
    n = u.n_q * 128
    kbytes = O.pack_rows(u.kcodes, bits).nbytes + u.kscale.nbytes + u.kzero.nbytes
    vbytes = O.pack_rows(u.vcodes, bits).nbytes + u.vscale.nbytes + u.vzero.nbytes
    assert 8 * kbytes / n == bits + 32 / G
    assert 8 * vbytes / n == bits + 32 / G


# ---------------------------------------------------------------------------
# Residual window ("KV cache quantization and eviction", Minimal implementation,
# kivi_compress split; MiniKV Algorithm 1 streaming buffer).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,G", [(0, 16), (32, 32), (128, 32), (5, 16), (128, 128)])
def test_residual_rule(R, G):
    for T in range(0, 3 * (R + G) + 7):
        nq = O.n_quantized(T, R, G)
        assert nq % G == 0 and nq >= 0
        if T >= R:
            assert R <= T - nq < R + G
        else:
            assert nq == 0
    # incremental simulation: quantize the oldest G whenever R+G rows are fp16
    fp16, nq = 0, 0
    for T in range(1, 400):
        fp16 += 1
        while fp16 >= R + G:
            fp16 -= G
            nq += G
        assert nq == O.n_quantized(T, R, G)


def test_incremental_and_bulk_appends_agree():
    rng = np.random.default_rng(7)
    p = O.CacheParams(bits=2, group=16, residual=8, pool=2, evict_cap=4)
    k = rng.standard_normal((200, 128)).astype(np.float16)
    v = rng.standard_normal((200, 128)).astype(np.float16)
    a, b = O.UnitCache(p), O.UnitCache(p)
    a.append(k, v)
    for i in range(0, 200, 7):
        b.append(k[i:i + 7], v[i:i + 7])
    for f in ["kcodes", "kscale", "kzero", "vcodes", "vscale", "vzero", "replaced"]:
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.pool_indices() == b.pool_indices() and a.evicted_indices() == b.evicted_indices()


# ---------------------------------------------------------------------------
# The dequantized cache every attention check reads ("MiniKV", section 4.4:
# one fp16 zero point and scale per group; "KV cache quantization and
# eviction", Minimal implementation: x_hat = code * scale + zero).
# ---------------------------------------------------------------------------

def _mixed_unit(bits, G, N, E, T=300, R=40, seed=31):
    """A unit with outlier key channels, low-norm tokens (pool admissions when
    N > 0) and two appends; returns the oracle unit and the raw fp16 rows."""
    rng = np.random.default_rng([seed, bits, G, N])
    k = rng.standard_normal((T, 128)).astype(np.float32)
    k[:, [3, 40, 77]] *= 15.0
    low = rng.choice(T, size=T // 12, replace=False)
    k[low] *= 0.02
    v = rng.standard_normal((T, 128)).astype(np.float32) * rng.uniform(0.2, 3.0, size=(T, 1))
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    u = O.UnitCache(O.CacheParams(bits=bits, group=G, residual=R, pool=N, evict_cap=E))
    u.append(k16[:137], v16[:137])
    u.append(k16[137:], v16[137:])
    return u, k16, v16


@pytest.mark.parametrize("bits,G,N,E", [(2, 32, 0, 0), (4, 64, 3, 4), (2, 128, 3, 1),
                                        (4, 16, 2, 8), (2, 16, 3, 32)])
def test_dequantized_rows_rebuilt_token_by_token(bits, G, N, E):
    """dequantized_kv() against a plain per-token loop: a quantized token takes,
    channel by channel, the (scale, zero) of its own key group and channel and of
    its own value channel group; pool and extra-pool tokens their original fp16
    rows; tokens at n_q and later the fp16 rows. Then, from the raw rows alone
    (pool members replaced by the exact group mean, rounded once to fp16), every
    zero point is the group minimum and every dequantized element is within half
    a step of the data: |x_hat - x| <= q/2 + L*|s16 - q| (+ fp32 slack), with q
    the exact (max - min) / L of the group."""
    u, k16, v16 = _mixed_unit(bits, G, N, E)
    T, d, L, gv = u.T, 128, 2 ** bits - 1, min(G, 128)
    n_q = u.n_q
    assert n_q >= 2 * G
    Kd, Vd = u.dequantized_kv()
    members = {m.idx for m in u.tracer.pool + u.tracer.evicted}
    if N:
        assert members, "construction should admit pool members"
    assert set(np.nonzero(u.replaced)[0].tolist()) == members
    kc, ks, kz = u.kcodes, u.kscale, u.kzero
    vc, vs, vz = u.vcodes, u.vscale, u.vzero
    for t in range(T):
        if t in members or t >= n_q:
            assert np.array_equal(Kd[t], k16[t].astype(np.float64)), t
            assert np.array_equal(Vd[t], v16[t].astype(np.float64)), t
            continue
        g = t // G
        for c in range(d):
            kw = float(kc[t, c]) * float(ks[g, c]) + float(kz[g, c])
            vw = float(vc[t, c]) * float(vs[t, c // gv]) + float(vz[t, c // gv])
            assert Kd[t, c] == kw and Vd[t, c] == vw, (t, c)

    def bound_ok(x, xh, lo, hi, s16):
        Q = max(hi - lo, Fraction(1, 10 ** 8)) / L
        S = half_to_fraction(s16)
        slack = Fraction(1, 2 ** 20) * (abs(x - lo) + Q)
        return abs(Fraction(float(xh)) - x) <= Q / 2 + L * abs(S - Q) + slack

    for g in range(n_q // G):
        rows = list(range(g * G, (g + 1) * G))
        krows = [[half_to_fraction(k16[t, c]) for c in range(d)] for t in rows]
        vrows = [[half_to_fraction(v16[t, c]) for c in range(d)] for t in rows]
        rep = [i for i, t in enumerate(rows) if t in members]
        if rep:
            mk = [half_to_fraction(round_to_half(sum(r[c] for r in krows) / G)) for c in range(d)]
            mv = [half_to_fraction(round_to_half(sum(r[c] for r in vrows) / G)) for c in range(d)]
            for i in rep:
                krows[i], vrows[i] = list(mk), list(mv)
        for c in range(d):
            col = [r[c] for r in krows]
            lo, hi = min(col), max(col)
            assert half_to_fraction(kz[g, c]) == lo, (g, c)
            for i, t in enumerate(rows):
                if t not in members:
                    assert bound_ok(col[i], Kd[t, c], lo, hi, ks[g, c]), (t, c)
        for i, t in enumerate(rows):
            if t in members:
                continue
            for j in range(d // gv):
                seg = vrows[i][j * gv:(j + 1) * gv]
                lo, hi = min(seg), max(seg)
                assert half_to_fraction(vz[t, j]) == lo, (t, j)
                for cc in range(gv):
                    assert bound_ok(seg[cc], Vd[t, j * gv + cc], lo, hi, vs[t, j]), (t, j, cc)


# ---------------------------------------------------------------------------
# Attention sinks ("KV cache quantization and eviction", Attention sinks and
# StreamingLLM; "KV Cache Transform Coding", section 2): the first S tokens
# stay fp16 and everything else behaves as a cache of the remaining tokens.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,G,N", [(4, 32, 0), (4, 16, 3), (1, 64, 2), (37, 32, 3)])
def test_sinks_are_fp16_and_the_rest_is_a_cache_of_the_later_tokens(S, G, N):
    rng = np.random.default_rng([41, S, G, N])
    T, R = 400, 40
    k = rng.standard_normal((T, 128)).astype(np.float32)
    k[:, [5, 60]] *= 15
    k[rng.choice(T, 30, replace=False)] *= 0.02
    k16 = k.astype(np.float16)
    v16 = rng.standard_normal((T, 128)).astype(np.float16)
    a = O.UnitCache(O.CacheParams(bits=2, group=G, residual=R, pool=N, evict_cap=5, sinks=S))
    for i0 in range(0, T, 53):  # ragged appends that cross the sink boundary
        a.append(k16[i0:i0 + 53], v16[i0:i0 + 53])
    b = O.UnitCache(O.CacheParams(bits=2, group=G, residual=R, pool=N, evict_cap=5))
    b.append(k16[S:], v16[S:])
    # the residual rule counts the tokens after the sinks
    assert a.n_q == b.n_q == max(0, (T - S - R) // G * G)
    assert R <= T - S - a.n_q < R + G
    for f in ["kcodes", "kscale", "kzero", "vcodes", "vscale", "vzero", "replaced"]:
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.pool_indices() == [i + S for i in b.pool_indices()]
    assert a.evicted_indices() == [i + S for i in b.evicted_indices()]
    Ka, Va = a.dequantized_kv()
    Kb, Vb = b.dequantized_kv()
    assert np.array_equal(Ka[:S], k16[:S].astype(np.float64))
    assert np.array_equal(Va[:S], v16[:S].astype(np.float64))
    assert np.array_equal(Ka[S:], Kb) and np.array_equal(Va[S:], Vb)
    # no sink is ever a pool member
    assert all(m.idx >= S for m in a.tracer.pool + a.tracer.evicted)


def test_sinks_covering_everything_is_plain_fp16_attention():
    rng = np.random.default_rng(43)
    k = rng.standard_normal((20, 128)).astype(np.float16)
    v = rng.standard_normal((20, 128)).astype(np.float16)
    u = O.UnitCache(O.CacheParams(bits=2, group=16, residual=0, sinks=32))
    u.append(k, v)
    assert u.n_q == 0
    K, V = u.dequantized_kv()
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))


# ---------------------------------------------------------------------------
# OTT: score, mean replacement, pool competition ("Accurate KV Cache
# Quantization with Outlier Tokens Tracing", Method details and appendix E).
# ---------------------------------------------------------------------------

def test_l1_score_is_exact():
    rng = np.random.default_rng(8)
    specials = np.array([65504, -65504, 6e-8, -6e-8, 1e-5, 2 ** -14, 0.0], dtype=np.float16)
    for _ in range(20):
        x = (rng.standard_normal(128) * rng.choice([1e-6, 1e-3, 1, 300, 20000])).astype(np.float16)
        x[:7] = specials
        want = sum(abs(half_to_fraction(v)) for v in x)
        assert Fraction(float(O.key_l1_score(x))) == want


def test_group_mean_rounds_once_to_fp16():
    """Mean of G rows: exact value rounded to nearest-even fp16, checked against Fractions.

    Includes means that sit just off an fp16 half-way point by less than an
    fp32 ulp, where rounding through fp32 first would give a different half.
    """
    rng = np.random.default_rng(9)
    for G in [16, 32, 128]:
        x = (rng.standard_normal((G, 64)) * rng.uniform(0.001, 500)).astype(np.float16)
        m = O.group_mean_fp16(x)
        for c in range(64):
            exact = sum(half_to_fraction(v) for v in x[:, c]) / G
            assert m[c].view(np.uint16) == round_to_half_bits(exact)
    G = 32
    col = np.full(G, 1.0, dtype=np.float16)
    col[0] = np.float16(1.0 + 2 ** -10)     # contributes 2^-10 / 32
    col[1] = np.float16(1.0 + 2 ** -10)
    # mean = 1 + 2^-10 * 2/32 = 1 + 2^-14: far below half an fp16 ulp (2^-11)
    assert O.group_mean_fp16(col[:, None])[0] == np.float16(1.0)
    # Constructed so that one rounding and two roundings disagree: 30 ones,
    # 2 + 2^-6 and the subnormal 2^-24 have the exact mean 1 + 2^-11 + 2^-29,
    # just above the fp16 half-way point 1 + 2^-11 by less than half an fp32 ulp
    # (2^-24). Rounded once it goes up to 1 + 2^-10; rounded to fp32 first it
    # lands on the half-way point and then ties to even, down to 1.0.
    col = np.full(G, 1.0, dtype=np.float16)
    col[7] = np.float16(2.0 + 2 ** -6)
    col[19] = np.float16(2.0 ** -24)
    exact = sum(half_to_fraction(v) for v in col) / G
    assert exact == 1 + Fraction(1, 2 ** 11) + Fraction(1, 2 ** 29)
    assert np.float32(float(exact)) == np.float32(1 + 2 ** -11)        # fp32 hits the tie
    assert round_to_half_bits(Fraction(1 + 2 ** -11)) == 0x3C00        # which ties down
    assert round_to_half_bits(exact) == np.float16(1 + 2 ** -10).view(np.uint16)
    assert O.group_mean_fp16(col[:, None])[0] == np.float16(1.0 + 2 ** -10)


def _brute_pool(history, N):
    """The N smallest (S, idx) among all tokens seen (appendix E, prefix form)."""
    return sorted(sorted(history)[:N], key=lambda t: t[1])


@pytest.mark.parametrize("N,G", [(1, 4), (3, 4), (3, 16), (5, 8)])
def test_ott_pool_is_prefix_topN_while_not_frozen(N, G):
    rng = np.random.default_rng(10 + N + G)
    tr = O.OutlierTracer(N, E=10 ** 6)
    history, admitted_total = [], 0
    for g in range(30):
        idx = np.arange(g * G, (g + 1) * G)
        s = rng.integers(0, 40, size=G).astype(np.float64)  # many exact ties
        k = np.zeros((G, 4), dtype=np.float16)
        adm = tr.compete(idx, s, k, k)
        admitted_total += len(adm)
        history += [(float(s[i]), int(idx[i])) for i in range(G)]
        want = _brute_pool(history, N)
        got = sorted(((m.score, m.idx) for m in tr.pool), key=lambda t: t[1])
        assert got == want
        # admitted tokens are exactly this group's members of the new pool
        assert sorted(int(idx[i]) for i in adm) == sorted(i for _, i in want if i >= g * G)
        # everything ever admitted is in the pool or the extra pool
        assert len(tr.evicted) == max(0, admitted_total - N)
        ever = {m.idx for m in tr.pool} | {m.idx for m in tr.evicted}
        assert len(ever) == admitted_total


def test_ott_freeze_when_extra_pool_full():
    """Descending norms: every group beats the pool, so the extra pool fills and tracing stops."""
    N, E, G = 3, 5, 4
    u = O.UnitCache(O.CacheParams(bits=2, group=G, residual=0, pool=N, evict_cap=E))
    T = 12 * G
    scale = np.linspace(10, 0.1, T).astype(np.float32)
    rng = np.random.default_rng(11)
    base = np.abs(rng.standard_normal(128)).astype(np.float32) + np.float32(0.5)
    k = (base[None, :] * scale[:, None]).astype(np.float16)
    S = O.key_l1_score(k)
    assert np.all(np.diff(S) < 0)
    u.append(k, k)
    tr = u.tracer
    assert tr.frozen and len(tr.evicted) == E and len(tr.pool) == N
    # admissions: group 0 fills the pool (3), then each later admission evicts one;
    # the (E+1)-th needed eviction freezes: total admitted = N + E.
    assert int(u.replaced.sum()) == N + E
    first_frozen_group = (N + E) // 3  # 3 admissions per group (top-3 of each group)
    assert not u.replaced[(first_frozen_group + 1) * G:].any()
    # the freezing group keeps the admissions made before the freeze
    kept = u.replaced[first_frozen_group * G:(first_frozen_group + 1) * G]
    assert kept.sum() == (N + E) - 3 * first_frozen_group


def test_ott_mean_replacement_removes_outlier_from_range():
    """A low-norm token is admitted; its quantized row is the group mean; the key step shrinks.

    Appendix D: one token at eps in a channel otherwise in [mu - sigma, mu + sigma]
    inflates q to ((mu + sigma) - eps)/(2^b - 1); with the token replaced by the
    mean, q <= (max - min(min_others, mean))/(2^b - 1).
    """
    G, mu, sigma, eps = 32, 20.0, 2.0, 0.5
    rng = np.random.default_rng(12)
    k = rng.standard_normal((G, 128)).astype(np.float32)
    k[:, 7] = rng.uniform(mu - sigma, mu + sigma, G)
    k[5, :] *= 0.01
    k[5, 7] = eps
    k16 = k.astype(np.float16)
    v16 = rng.standard_normal((G, 128)).astype(np.float16)
    S = O.key_l1_score(k16)
    assert S.argmin() == 5
    # without tracing
    u0 = O.UnitCache(O.CacheParams(bits=2, group=G, residual=0, pool=0))
    u0.append(k16, v16)
    q_no = fr32(np.float32(k16[:, 7].max()) - np.float32(k16[5, 7])) / 3
    assert abs(half_to_fraction(u0.kscale[0, 7]) - q_no) <= q_no * Fraction(1, 1024)
    # with tracing (N = 1)
    u1 = O.UnitCache(O.CacheParams(bits=2, group=G, residual=0, pool=1, evict_cap=4))
    u1.append(k16, v16)
    assert u1.pool_indices() == [5] and u1.replaced.tolist() == [i == 5 for i in range(G)]
    mean_k = O.group_mean_fp16(k16)
    others = np.delete(k16[:, 7], 5).astype(np.float64)
    lo = min(others.min(), float(mean_k[7]))
    assert float(u1.kscale[0, 7]) <= (others.max() - lo) / 3 * (1 + 2 ** -10)
    assert float(u1.kscale[0, 7]) < float(u0.kscale[0, 7]) / 4
    # the quantized slot reconstructs the mean row within half a step per channel
    kh, vh = u1.dequantized_kv()
    assert np.array_equal(kh[5], k16[5].astype(np.float64))  # pool row used in attention
    deq5 = O.dequantize(u1.kcodes[5], u1.kscale[0], u1.kzero[0])
    assert np.all(np.abs(deq5 - mean_k.astype(np.float64)) <= u1.kscale[0].astype(np.float64) / 2 + 1e-3)
    assert np.array_equal(u1.tracer.pool[0].v, v16[5])
    # exact construction: row 5 of K and V replaced by the mean of all G original
    # rows (outlier included), rounded once to fp16, then quantized as usual
    def exact_mean(x16):
        return np.array([round_to_half(sum(half_to_fraction(v) for v in x16[:, c]) / G)
                         for c in range(x16.shape[1])], dtype=np.float16)
    kr, vr = k16.copy(), v16.copy()
    kr[5], vr[5] = exact_mean(k16), exact_mean(v16)
    kc, ks, kz = O.quantize_key_group(kr, 2)
    vc, vs, vz = O.quantize_value_rows(vr, 2, G)
    assert np.array_equal(u1.kcodes, kc) and np.array_equal(u1.kscale[0], ks)
    assert np.array_equal(u1.kzero[0], kz)
    assert np.array_equal(u1.vcodes, vc) and np.array_equal(u1.vscale, vs)
    assert np.array_equal(u1.vzero, vz)


def test_ott_score_ties_prefer_older_token():
    tr = O.OutlierTracer(1, 4)
    k = np.zeros((4, 2), dtype=np.float16)
    adm = tr.compete(np.arange(4), np.array([3.0, 1.0, 1.0, 2.0]), k, k)
    assert adm == [1]
    adm = tr.compete(np.arange(4, 8), np.array([1.0, 5.0, 5.0, 5.0]), k, k)
    assert adm == [] and tr.pool[0].idx == 1


# ---------------------------------------------------------------------------
# Attention (MiniKV section 2, Eq. 1 and Algorithm 1, decoding; OTT decoding
# stage) and H2O scores ("KV cache quantization and eviction", Heavy hitters).
# ---------------------------------------------------------------------------

def _brute_attention(K, V, q):
    d = len(q)
    s = [sum(q[c] * K[j][c] for c in range(d)) / math.sqrt(d) for j in range(len(K))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = sum(e)
    return [sum(e[j] / l * V[j][c] for j in range(len(K))) for c in range(d)], [x / l for x in e]


def test_attention_matches_brute_force():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((9, 16)) * 2
    V = rng.standard_normal((9, 16))
    q = rng.standard_normal((3, 16)).astype(np.float16)
    out, p = O.unit_attention(K, V, q)
    for h in range(3):
        bo, bp = _brute_attention(K.tolist(), V.tolist(), q[h].astype(np.float64).tolist())
        assert np.allclose(out[h], bo, rtol=1e-12, atol=1e-14)
        assert np.allclose(p[h], bp, rtol=1e-12, atol=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 128)).astype(np.float16)
    V = rng.standard_normal((1, 128))
    out, p = O.unit_attention(rng.standard_normal((1, 128)), V, q)
    assert np.array_equal(out, np.repeat(V, 2, axis=0)) and np.all(p == 1)
    K = np.repeat(rng.standard_normal((1, 128)), 7, axis=0)
    V = rng.standard_normal((7, 128))
    out, _ = O.unit_attention(K, V, q)
    assert np.allclose(out, V.mean(axis=0)[None], rtol=1e-13, atol=1e-15)


def test_residual_covering_everything_is_plain_fp16_attention():
    rng = np.random.default_rng(15)
    p = O.CacheParams(bits=2, group=32, residual=64)
    u = O.UnitCache(p)
    k = rng.standard_normal((50, 128)).astype(np.float16)
    v = rng.standard_normal((50, 128)).astype(np.float16)
    u.append(k, v)
    assert u.n_q == 0
    K, V = u.dequantized_kv()
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))


def test_partitioned_softmax_equals_concatenated():
    """MiniKV Algorithm 1: softmax over [quantized ; residual] then
    A_quant deq(V_q) + A_unquant R_V equals per-partition (max, sum, out) merged."""
    rng = np.random.default_rng(16)
    p = O.CacheParams(bits=2, group=16, residual=20)
    u = O.UnitCache(p)
    k = rng.standard_normal((100, 128)).astype(np.float16)
    v = rng.standard_normal((100, 128)).astype(np.float16)
    u.append(k, v)
    K, V = u.dequantized_kv()
    q = rng.standard_normal((1, 128)).astype(np.float16)
    out, _ = O.unit_attention(K, V, q)
    parts = []
    for sl in [slice(0, u.n_q), slice(u.n_q, 100)]:
        s = (q.astype(np.float64) @ K[sl].T)[0] / math.sqrt(128)
        m = s.max()
        e = np.exp(s - m)
        parts.append((m, e.sum(), e @ V[sl]))
    M = max(m for m, _, _ in parts)
    Lsum = sum(l * math.exp(m - M) for m, l, _ in parts)
    merged = sum(o * math.exp(m - M) for m, _, o in parts) / Lsum
    assert np.allclose(out[0], merged, rtol=1e-12, atol=1e-14)


def test_each_token_counted_once_with_pools():
    rng = np.random.default_rng(17)
    p = O.CacheParams(bits=2, group=8, residual=8, pool=2, evict_cap=3)
    u = O.UnitCache(p)
    k = rng.standard_normal((120, 128)).astype(np.float16)
    k[::9] *= 0.05
    v = rng.standard_normal((120, 128)).astype(np.float16)
    u.append(k, v)
    assert u.tracer.evicted, "construction should displace pool members"
    K, V = u.dequantized_kv()
    for m in u.tracer.pool + u.tracer.evicted:
        assert np.array_equal(K[m.idx], k[m.idx].astype(np.float64))
        assert np.array_equal(V[m.idx], v[m.idx].astype(np.float64))
    assert K.shape[0] == 120


def test_h2o_increment_sums_to_gqa_ratio():
    rng = np.random.default_rng(18)
    c = O.CacheOracle(O.CacheParams(bits=2, group=16, residual=16), 1, 1)
    k = rng.standard_normal((300, 128)).astype(np.float16)
    c.append_unit((0, 0), k, k)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    _, inc, p = c.decode_unit((0, 0), q)
    assert abs(inc.sum() - 4) < 1e-12 and np.all(inc >= 0)
    assert np.allclose(inc, p.sum(axis=0))


# ---------------------------------------------------------------------------
# Heavy-hitter selection ("KV cache quantization and eviction", Minimal
# implementation h2o_evict: evict the lowest non-recent score, one per step).
# ---------------------------------------------------------------------------

def _argmin_eviction(scores, k, w):
    """Repeatedly evict the first-occurrence argmin outside the fixed recent window."""
    T = len(scores)
    alive = list(range(T - w))
    while len(alive) > k:
        vals = [scores[i] for i in alive]
        j = vals.index(min(vals))
        alive.pop(j)
    return alive + list(range(T - w, T))


@pytest.mark.parametrize("ties", [False, True])
def test_topk_equals_repeated_argmin_eviction(ties):
    rng = np.random.default_rng(19)
    for T, k, w in [(50, 10, 5), (64, 0, 8), (40, 40, 0), (33, 20, 13), (16, 0, 0), (20, 3, 17)]:
        if ties:
            s = (rng.integers(0, 3, size=(3, T)) * 0.5).astype(np.float32)
        else:
            s = rng.random((3, T)).astype(np.float32)
        got = O.topk_keep(s, k, w)
        for r in range(3):
            assert got[r].tolist() == _argmin_eviction(s[r].tolist(), k, w)


def test_topk_tie_order_prefers_newer():
    s = np.array([[1, 2, 2, 2, 0, 5]], dtype=np.float32)
    assert O.topk_keep(s, 2, 1).tolist() == [[2, 3, 5]]


def test_bulk_append_bytes_closed_form():
    """Bulk append moves every fp16 K/V row in once (2 * d * 2 bytes), writes
    the quantized tokens' codes and fp16 scale/zero (d*b/4 + 4d/G + 4d/Gv
    bytes) and the residual tokens' fp16 rows (4d bytes)."""
    from kv_cache_compression_kvq_amd import bytes_model as BM
    # 2-bit, G = 32, d = 128: 64 B of codes + 16 B key meta + 16 B value meta
    per_q = 128 * 2 // 4 + 4 * 128 // 32 + 4 * 128 // 32
    assert per_q == 96
    # B8 x 8 KV heads, T = 8192, R = 128: n_q = 8064
    got = BM.bulk_append_bytes(units=64, head_dim=128, tokens=8192, n_quant=8064, bits=2, group=32)
    assert got == 64 * (8192 * 512 + 8064 * 96 + 128 * 512) == 322174976
    # 4-bit, G = 128 (one value group per token): 128 + 4 + 4 bytes per quantized token
    got4 = BM.bulk_append_bytes(units=1, head_dim=128, tokens=300, n_quant=128, bits=4, group=128)
    assert got4 == 300 * 512 + 128 * 136 + 172 * 512


def test_topk_special_values_total_order():
    # NaN ranks below every number and NaNs tie; -0 == +0; ties keep the
    # larger index. Brute force over that total order on small rows.
    rng = np.random.default_rng(23)
    vals = np.array([np.nan, -np.inf, np.inf, 0.0, -0.0, 1.0, -1.0, 3e38, -3e38],
                    dtype=np.float32)
    for T, k, w in [(12, 5, 2), (9, 9, 0), (20, 7, 3), (15, 1, 0)]:
        s = vals[rng.integers(0, len(vals), size=(4, T))]
        got = O.topk_keep(s, k, w)
        n = T - w
        for r in range(4):
            def rank(i):
                x = float(s[r, i])
                return (0, 0.0, i) if x != x else (1, x, i)
            keep = sorted(sorted(range(n), key=rank, reverse=True)[:k])
            assert got[r].tolist() == keep + list(range(n, T))


# ---------------------------------------------------------------------------
# H2O eviction during decoding ("H2O: Heavy-Hitter Oracle", greedy eviction;
# "KV cache quantization and eviction", h2o_evict) and MiniKV's pyramid
# budgets (section 4.2).
# ---------------------------------------------------------------------------

def test_h2o_evict_one_is_a_first_occurrence_argmin():
    rng = np.random.default_rng(50)
    for trial in range(200):
        T = int(rng.integers(5, 60))
        sc = (rng.integers(0, 6, T) * 0.25).astype(np.float32)   # many exact ties
        if trial % 5 == 0:
            sc[rng.integers(T)] = np.nan
        live = rng.random(T) < 0.8
        S, w, B = int(rng.integers(0, 3)), int(rng.integers(0, 5)), int(rng.integers(1, T))
        want_live = live.copy()
        cand = [t for t in range(S, T - w) if live[t]]
        got = O.h2o_evict_one(sc, live, B, w, S)
        if int(want_live.sum()) <= B or not cand:
            assert got == -1 and np.array_equal(live, want_live)
            continue
        # numpy's argmin: the first NaN if any, else the first minimum
        sub = sc[cand].astype(np.float64)
        want = cand[int(np.argmin(sub))]
        assert got == want
        want_live[want] = False
        assert np.array_equal(live, want_live)


@pytest.mark.parametrize("S", [0, 4])
def test_repeated_eviction_on_static_scores_equals_one_shot_topk(S):
    """Evicting one token at a time down to the budget keeps the sinks, the
    recent window and the top-k of the rest: the one-shot selection."""
    rng = np.random.default_rng(51)
    T, w, B = 300, 20, 100
    sc = (rng.integers(0, 40, T) / 7).astype(np.float32)
    live = np.ones(T, dtype=bool)
    while O.h2o_evict_one(sc, live, B, w, S) >= 0:
        pass
    k = B - w - S
    keep_rest = O.topk_keep(sc[S:][None], k, w)[0] + S
    want = np.zeros(T, dtype=bool)
    want[:S] = True
    want[keep_rest] = True
    assert np.array_equal(live, want)


def test_attention_over_live_tokens_equals_attention_over_the_kept_rows():
    rng = np.random.default_rng(52)
    K = rng.standard_normal((50, 128))
    V = rng.standard_normal((50, 128))
    q = rng.standard_normal((4, 128)).astype(np.float16)
    live = rng.random(50) < 0.6
    out, p = O.unit_attention(K, V, q, live)
    out2, p2 = O.unit_attention(K[live], V[live], q)
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-13)
    assert np.all(p[:, ~live] == 0) and np.allclose(p[:, live], p2, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("L,x,d", [(32, 100, 7), (32, 1024, 2), (5, 13, 3), (2, 8, 4), (9, 50, 1)])
def test_pyramid_budgets(L, x, d):
    """MiniKV section 4.2: linear from 2x - x/d (lowest layer) to x/d (highest),
    average x. Checked against those endpoints, a constant step and the mean,
    in exact rationals."""
    b = O.pyramid_budgets(L, x, d)
    hi, lo = Fraction(2 * x) - Fraction(x, d), Fraction(x, d)
    assert b[0] == math.floor(hi) and b[-1] == math.floor(lo)
    step = (hi - lo) / (L - 1)
    exact = [hi - step * l for l in range(L)]
    assert sum(exact) == L * x                      # the average budget is x
    assert all(0 <= e - bl < 1 for e, bl in zip(exact, b))
    assert all(b[i] >= b[i + 1] for i in range(L - 1))
    if d == 1:
        assert b == [x] * L


# ---------------------------------------------------------------------------
# FP8 E4M3 codec ("KV cache quantization and eviction", FP8, KIVI and KVQuant:
# E4M3, largest finite value 448, a scale per head; Failure modes: casts must
# saturate).
# ---------------------------------------------------------------------------

def _e4m3_magnitudes_by_construction():
    """All finite non-negative E4M3 magnitudes as exact rationals, built binade
    by binade: the subnormal run k * 2^-9 (k = 0..7), then for each binade
    2^(e-7) with e = 1..15 its eight steps of 2^(e-10), the last binade
    stopping before the NaN pattern."""
    vals = [Fraction(k, 2 ** 9) for k in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                break
            vals.append(Fraction(2) ** (e - 7) + m * Fraction(2) ** (e - 10))
    return vals


def test_e4m3_table_matches_the_format(golden):
    g = golden["fp8_e4m3"]
    mags = _e4m3_magnitudes_by_construction()
    assert len(mags) == 127
    assert float(mags[-1]) == g["max_finite"] == O.e4m3_value(0x7E)
    for c in range(256):
        v = O.e4m3_value(c)
        if c & 0x7F == 0x7F:
            assert math.isnan(v)
            continue
        m = mags[c & 0x7F]
        assert Fraction(abs(v)) == m and (c < 0x80 or math.copysign(1, v) < 0)


def test_e4m3_encode_round_trips_rounds_to_even_and_saturates():
    mags = _e4m3_magnitudes_by_construction()
    codes = np.arange(256, dtype=np.uint8)
    finite = (codes & 0x7F) != 0x7F
    vals = O.e4m3_decode(codes[finite]).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes[finite])          # exact values stay
    # midpoints between neighbours go to the even code; just off them, to the nearer
    for i in range(126):
        mid = (mags[i] + mags[i + 1]) / 2
        x = np.float32(float(mid))
        assert Fraction(float(x)) == mid                                   # exact in fp32
        want = i if i % 2 == 0 else i + 1
        assert O.e4m3_encode(np.array([x]))[0] == want
        assert O.e4m3_encode(np.array([-x]))[0] == want | 0x80
        up, dn = np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))
        assert O.e4m3_encode(np.array([up]))[0] == i + 1
        assert O.e4m3_encode(np.array([dn]))[0] == i
    # saturation: the largest finite value and everything above it, infinity included
    big = np.array([448, 449, 463.9, 464, 480, 1e6, np.inf], dtype=np.float32)
    assert np.all(O.e4m3_encode(big) == 0x7E) and np.all(O.e4m3_encode(-big) == 0xFE)
    assert O.e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80


def test_e4m3_nearest_value_brute_force():
    rng = np.random.default_rng(60)
    x = (rng.standard_normal(3000) * np.exp(rng.uniform(-12, 7, 3000))).astype(np.float32)
    mags = np.array([float(m) for m in _e4m3_magnitudes_by_construction()])
    got = O.e4m3_decode(O.e4m3_encode(x))
    err = np.abs(np.abs(got) - np.abs(x.astype(np.float64)))
    best = np.min(np.abs(mags[None, :] - np.minimum(np.abs(x), 448)[:, None]), axis=1)
    assert np.all(err[np.abs(x) <= 448] == best[np.abs(x) <= 448])
    assert np.all(np.signbit(got) == np.signbit(x))  # values that round to zero keep their sign


def test_fp8_cache_rows_are_scaled_e4m3_values():
    """b = 8 units: quantized rows decode to E4M3 values times the head's scale,
    within half an E4M3 step of x / s (relative 2^-4 for normal values)."""
    rng = np.random.default_rng(61)
    k = (rng.standard_normal((300, 128)) * 3).astype(np.float16)
    v = rng.standard_normal((300, 128)).astype(np.float16)
    sk, sv = 0.0625, 1.5
    u = O.UnitCache(O.CacheParams(bits=8, group=32, residual=40, fp8_scale_k=sk, fp8_scale_v=sv))
    u.append(k[:77], v[:77])
    u.append(k[77:], v[77:])
    assert u.n_q == 256
    K, V = u.dequantized_kv()
    for X, x16, s in ((K, k, sk), (V, v, sv)):
        xs = x16[:256].astype(np.float64) / s
        xh = X[:256] / s
        assert np.all(np.abs(xh) <= 448)
        normal = np.abs(xs) >= 2 ** -6
        assert np.all(np.abs(xh - xs)[normal] <= np.abs(xs)[normal] * 2.0 ** -4)
        assert np.all(np.abs(xh - xs)[~normal] <= 2.0 ** -10)
        assert np.array_equal(X[256:], x16[256:].astype(np.float64))


# ---------------------------------------------------------------------------
# Prefill scores (MiniKV, section 4.3 selective flash-attention; Algorithm 1).
# ---------------------------------------------------------------------------

def test_prefill_attention_brute_force_loops():
    rng = np.random.default_rng(70)
    r, n, d = 2, 9, 128
    q = rng.standard_normal((r, n, d)).astype(np.float16)
    k = rng.standard_normal((n, d)).astype(np.float16)
    v = rng.standard_normal((n, d)).astype(np.float16)
    out, acum = O.prefill_attention(q, k, v)
    want_acum = [0.0] * n
    for h in range(r):
        for i in range(n):
            logits = [sum(float(q[h, i, c]) * float(k[j, c]) for c in range(d)) / math.sqrt(d)
                      for j in range(i + 1)]
            mx = max(logits)
            e = [math.exp(x - mx) for x in logits]
            tot = sum(e)
            for c in range(0, d, 17):
                o = sum(e[j] / tot * float(v[j, c]) for j in range(i + 1))
                assert abs(out[h, i, c] - o) <= 1e-12 * (1 + abs(o))
            for j in range(i + 1):
                want_acum[j] += e[j] / tot
    assert np.allclose(acum, want_acum, rtol=1e-12, atol=0)


def test_prefill_column_sums_closed_forms():
    """Equal keys: row i spreads 1/(i+1) over its i+1 keys, so A_cumul[j] is
    r * (H_n - H_j) (harmonic numbers) and the outputs are running means of V;
    in general the column sums add up to r * n (every row sums to 1)."""
    rng = np.random.default_rng(71)
    r, n, d = 3, 40, 128
    q = rng.standard_normal((r, n, d)).astype(np.float16)
    k = np.tile(rng.standard_normal((1, d)).astype(np.float16), (n, 1))
    v = rng.standard_normal((n, d)).astype(np.float16)
    out, acum = O.prefill_attention(q, k, v)
    H = [sum(Fraction(1, m) for m in range(1, t + 1)) for t in range(n + 1)]
    for j in range(n):
        assert abs(acum[j] - float(r * (H[n] - H[j]))) <= 1e-12 * r * n
    run = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(out, run[None], rtol=1e-12, atol=1e-13)
    q2 = rng.standard_normal((r, n, d)).astype(np.float16)
    k2 = rng.standard_normal((n, d)).astype(np.float16)
    _, a2 = O.prefill_attention(q2, k2, v)
    assert abs(a2.sum() - r * n) <= 1e-9 and np.all(a2 > 0)
    # the first token takes all of row 0 in every head; the last token appears
    # in the last row only
    assert a2[0] >= r - 1e-12 and a2[-1] <= r + 1e-12
    _, a1 = O.prefill_attention(q2[:, :1], k2[:1], v[:1])
    assert np.allclose(a1, [r])
