"""Host-side checks of the C ABI: the library loads, exports what include/kvq.h
declares, and rejects bad arguments before launching anything (no GPU needed:
every call below returns from validation)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT


def _header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text))


def test_library_exports_every_header_function(kvq):
    declared = _header_functions()
    assert declared == set(kvq.EXPORTS)
    for name in declared:
        assert getattr(kvq.lib(), name) is not None


def test_status_strings(kvq):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert kvq.status_string(code) and "unknown" not in kvq.status_string(code)
    assert "unknown" in kvq.status_string(7)


def _cfg(kvq, **kw):
    base = dict(bits=2, group=32, residual=128, pool=0, evict_cap=32, head_dim=128,
                n_q_heads=32, n_kv_heads=8, batch=8, max_tokens=8192)
    base.update(kw)
    return kvq.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), -2), (dict(bits=8, group=16), -2), (dict(bits=8, pool=3), -2),
    (dict(bits=16), -2), (dict(group=8), -2), (dict(group=48), -2),
    (dict(head_dim=64), -2), (dict(n_q_heads=64), -2), (dict(n_q_heads=12), -1),
    (dict(pool=65), -2), (dict(evict_cap=2000), -2), (dict(residual=-1), -1),
    (dict(batch=0), -1), (dict(max_tokens=0), -1), (dict(residual=1900, pool=64, evict_cap=64), -2),
    (dict(batch=8192), -2),  # B * Hkv above 65535
])
def test_bad_configs_rejected(kvq, kw, code):
    with pytest.raises(kvq.KvqError) as e:
        kvq.cache_bytes(_cfg(kvq, **kw))
    assert e.value.status == code


def test_cache_bytes_hold_the_documented_regions(kvq):
    """The arena covers every region include/kvq.h lists, each 256-byte aligned."""
    for kw in [dict(), dict(bits=4), dict(group=128, bits=4), dict(pool=3, residual=32),
               dict(n_q_heads=8, batch=1, max_tokens=100), dict(max_tokens=1)]:
        cfg = _cfg(kvq, **kw)
        n = kvq.cache_bytes(cfg)
        U = cfg.batch * cfg.n_kv_heads
        qcap = max(0, (cfg.max_tokens - cfg.residual) // cfg.group * cfg.group)
        codes = 2 * U * qcap * 128 * cfg.bits // 8
        meta = U * qcap // cfg.group * 128 * 4 + U * qcap * (128 // cfg.group) * 4
        ring = 2 * U * (cfg.residual + cfg.group) * 128 * 2
        pools = U * (cfg.pool + cfg.evict_cap) * (4 + 512) + U * cfg.pool * 8
        assert n >= codes + meta + ring + pools and n % 256 == 0


def _fake_handle(kvq, cfg, tokens):
    h = kvq.Cache()
    h.cfg = cfg
    h.tokens = tokens
    h.n_quant = max(0, (tokens - cfg.residual) // cfg.group * cfg.group)
    h.arena = 1 << 40
    h.arena_bytes = kvq.cache_bytes(cfg)
    h.q_cap = max(0, (cfg.max_tokens - cfg.residual) // cfg.group * cfg.group)
    h.ring_slots = cfg.residual + cfg.group
    return h


def test_validation_paths_launch_nothing(kvq):
    L = kvq.lib()
    cfg = _cfg(kvq)
    h = _fake_handle(kvq, cfg, 0)
    P = ctypes.c_void_p
    # appending nothing is a no-op; beyond capacity is refused
    assert L.kvq_quantize_append(ctypes.byref(h), None, None, 0, None) == 0
    assert L.kvq_quantize_append(ctypes.byref(h), P(1 << 40), P(1 << 40), 8193, None) == -3
    assert L.kvq_quantize_append(ctypes.byref(h), None, None, 5, None) == -1
    assert L.kvq_quantize_append(ctypes.byref(h), P(1 << 40), P(1 << 40), -1, None) == -1
    # decode over an empty cache, and with too small a workspace
    assert L.kvq_decode_attention(ctypes.byref(h), P(1), P(1), None, P(1), 1 << 30, None) == -1
    h2 = _fake_handle(kvq, cfg, 4096)
    need = kvq.decode_workspace(h2, True)
    assert need > kvq.decode_workspace(h2, False) > 0
    assert L.kvq_decode_attention(ctypes.byref(h2), P(1), P(1), P(1), P(1), need - 1, None) == -4
    assert L.kvq_decode_attention(ctypes.byref(h2), None, P(1), None, P(1), need, None) == -1
    # an inconsistent handle is refused
    h2.n_quant += 32
    assert L.kvq_decode_attention(ctypes.byref(h2), P(1), P(1), None, P(1), need, None) == -1
    # init: misaligned or short arenas
    hh = kvq.Cache()
    assert L.kvq_cache_init(ctypes.byref(cfg), P((1 << 40) + 8), 1 << 40, ctypes.byref(hh), None) == -1
    assert L.kvq_cache_init(ctypes.byref(cfg), P(1 << 40), 1024, ctypes.byref(hh), None) == -4
    # top-k argument checks; nothing to do for zero rows
    assert L.kvq_topk_evict(P(1), 4, 100, 90, 20, P(1), None, 0, None) == -1
    assert L.kvq_topk_evict(P(1), -1, 100, 10, 20, P(1), None, 0, None) == -1
    assert L.kvq_topk_evict(None, 0, 100, 10, 20, None, None, 0, None) == 0
    assert L.kvq_topk_evict(None, 3, 100, 10, 20, P(1), None, 0, None) == -1
    n = ctypes.c_size_t(7)
    assert L.kvq_topk_workspace(3, 100, 10, 20, ctypes.byref(n)) == 0 and n.value == 0
    assert L.kvq_topk_workspace(3, 100, 90, 20, ctypes.byref(n)) == -1
    # prefill and gather: query heads and units index the second grid dimension
    assert L.kvq_prefill_attention(P(1), P(1), P(1), 2048, 32, 8, 128, 64, P(1), None, P(1),
                                   1 << 40, None) == -2
    assert L.kvq_prefill_attention(P(1), P(1), P(1), 2047, 32, 8, 128, 0, P(1), None, P(1),
                                   1 << 40, None) == 0
    assert L.kvq_gather_kv(P(1), P(1), 8192, 8, 128, 64, P(1), 16, P(1), P(1), None) == -2
    assert L.kvq_gather_kv(P(1), P(1), 8191, 8, 128, 64, P(1), 0, P(1), P(1), None) == 0


def test_decode_step_validation_launches_nothing(kvq):
    """kvq_decode_step checks every argument before enqueuing anything and then
    leaves the handle as it was; its workspace is that of the cache after the
    append (T + 1 tokens)."""
    L = kvq.lib()
    P = ctypes.c_void_p
    cfg = _cfg(kvq, max_tokens=4097)
    h = _fake_handle(kvq, cfg, 4096)
    nxt = _fake_handle(kvq, cfg, 4097)
    need = kvq.decode_workspace(nxt, False)
    before = bytes(h)
    args = [P(1), P(1), P(1), P(1), None, P(1)]
    for i in (0, 1, 2, 3, 5):  # k, v, q, out, ws
        bad = list(args)
        bad[i] = None
        assert L.kvq_decode_step(ctypes.byref(h), *bad, need, None) == -1
    assert L.kvq_decode_step(ctypes.byref(h), *args, need - 1, None) == -4
    full = _fake_handle(kvq, cfg, 4097)
    assert L.kvq_decode_step(ctypes.byref(full), *args, need, None) == -3
    assert L.kvq_decode_step_timed(ctypes.byref(h), *args, need - 1, None, None, None) == -4
    assert bytes(h) == before
    # a group boundary: T = R + G - 1 -> T + 1 quantizes one group first
    cfg2 = _cfg(kvq, max_tokens=1000)
    h3 = _fake_handle(kvq, cfg2, 128 + 32 - 1)
    assert h3.n_quant == 0 and _fake_handle(kvq, cfg2, 160).n_quant == 32
    assert L.kvq_decode_step(ctypes.byref(h3), *args, 0, None) == -4


def test_decode_plan_covers_partials_and_logits(kvq):
    """Workspace grows by exactly U * r * T floats when scores are wanted."""
    cfg = _cfg(kvq, batch=2, n_kv_heads=8, n_q_heads=32, max_tokens=40000)
    for T in (1, 100, 160, 8192, 40000):
        h = _fake_handle(kvq, cfg, T)
        a, b = kvq.decode_workspace(h, False), kvq.decode_workspace(h, True)
        assert b - a == 16 * 4 * T * 4


@pytest.mark.parametrize("L,x,d", [(32, 100, 7), (32, 6553, 2), (5, 13, 3), (2, 8, 4), (1, 9, 5),
                                   (40, 0, 3), (4096, 1 << 24, 4096)])
def test_pyramid_budgets_match_the_oracle(kvq, L, x, d):
    """kvq_pyramid_budgets (host C, integer arithmetic) against the oracle's
    exact-rational budgets (MiniKV section 4.2)."""
    from oracle import kvq_oracle as O
    assert kvq.pyramid_budgets(L, x, d) == O.pyramid_budgets(L, x, d)
