"""Prefill attention with heavy-hitter scores (MiniKV, section 4.3, selective
flash-attention; Algorithm 1, prefill; section 4.1, persistent context
selection) through the C ABI, against the CPU oracle.

Outputs are checked to the decode bar (max-abs 2e-3, per-row L2 1e-3); the
column sums A_cumul to relative 1e-4 per token. The pipeline test feeds
A_cumul to kvq_topk_evict, gathers the kept rows with kvq_gather_kv, quantizes
them with kvq_quantize_append and decodes: the kept indices must equal the
oracle's selection on the same fp32 scores, the gathered rows must equal the
prompt rows bit for bit, and the cache and its attention must match an oracle
cache fed the same rows.
"""
import numpy as np
import pytest
import torch

from kv_cache_compression_kvq_amd import abi, synth
from oracle import kvq_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(kvq):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _prompt(batch, hkv, r, n, seed):
    rng = np.random.default_rng([seed, batch, hkv, r, n])
    q = rng.standard_normal((batch, hkv * r, n, 128)).astype(np.float16)
    k = rng.standard_normal((batch, hkv, n, 128)).astype(np.float32)
    k[..., [7, 77]] *= 8.0  # a few large channels, as in the decode workloads
    v = rng.standard_normal((batch, hkv, n, 128)).astype(np.float16)
    return q, k.astype(np.float16), v


def _run(q, k, v, with_acc=True):
    batch, hq, n, _ = q.shape
    hkv = k.shape[1]
    dev = "cuda"
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    out = torch.full((batch, hq, n, 128), float("nan"), device=dev)
    acc = torch.full((batch, hkv, n), float("nan"), device=dev) if with_acc else None
    ws = torch.empty(abi.prefill_workspace(batch, hq, n), dtype=torch.uint8, device=dev)
    abi.prefill_attention(qt, kt, vt, batch, hq, hkv, n, out, acc, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (acc.cpu().numpy() if with_acc else None), (kt, vt)


@pytest.mark.parametrize("r,n", [(4, 1), (4, 17), (4, 64), (4, 100), (2, 300), (1, 129),
                                 (4, 513)])
def test_prefill_outputs_and_column_sums(r, n):
    batch, hkv = 2, 2
    q, k, v = _prompt(batch, hkv, r, n, seed=1)
    out, acc, _ = _run(q, k, v)
    for b in range(batch):
        for h in range(hkv):
            ref, acum = O.prefill_attention(q[b, h * r:(h + 1) * r], k[b, h], v[b, h])
            H.check_outputs(out[b, h * r:(h + 1) * r], ref, f"prefill_r{r} unit {(b, h)}")
            H.check_h2o(acc[b, h], 0.0, acum, f"prefill_r{r} unit {(b, h)}")


def test_prefill_without_scores_leaves_nothing_undefined():
    q, k, v = _prompt(1, 2, 4, 200, seed=2)
    out, _, _ = _run(q, k, v, with_acc=False)
    assert np.all(np.isfinite(out))
    ref, _ = O.prefill_attention(q[0, 4:8], k[0, 1], v[0, 1])
    H.check_outputs(out[0, 4:8], ref, "prefill_noacc unit (0, 1)")


def test_prefill_llama8b_layer_sampled_heads():
    """One Llama-3-8B layer at a 2048-token prompt (32 / 8 heads), two KV heads
    checked in full."""
    batch, hkv, r, n = 1, 8, 4, 2048
    q, k, v = _prompt(batch, hkv, r, n, seed=3)
    out, acc, _ = _run(q, k, v)
    for h in (0, 5):
        ref, acum = O.prefill_attention(q[0, h * r:(h + 1) * r], k[0, h], v[0, h])
        H.check_outputs(out[0, h * r:(h + 1) * r], ref, f"prefill_8b unit {(0, h)}")
        H.check_h2o(acc[0, h], 0.0, acum, f"prefill_8b unit {(0, h)}")


@pytest.mark.parametrize("bits,group", [(2, 16), (2, 32), (8, 32)])
def test_prefill_selection_feeds_the_quantized_cache(bits, group):
    """MiniKV Algorithm 1, prefill: A_cumul -> heavy hitters + recent window ->
    kept rows -> 2-bit (or FP8) cache -> first decode step."""
    batch, hkv, r, n = 2, 2, 4, 700
    keep_k, recent = 200, 64
    q, k, v = _prompt(batch, hkv, r, n, seed=4)
    _, acc, (kd, vd) = _run(q, k, v)
    rows = batch * hkv
    idx = torch.empty((rows, keep_k + recent), dtype=torch.int32, device="cuda")
    accd = torch.from_numpy(acc).cuda()
    abi.topk_evict(accd, rows, n, keep_k, recent, idx)
    torch.cuda.synchronize()
    want_idx = O.topk_keep(acc.reshape(rows, n), keep_k, recent)
    np.testing.assert_array_equal(idx.cpu().numpy(), want_idx)
    nk = keep_k + recent
    ko = torch.empty((batch, hkv, nk, 128), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    abi.gather_kv(kd, vd, batch, hkv, n, idx, nk, ko, vo)
    torch.cuda.synchronize()
    kg, vg = ko.cpu().numpy(), vo.cpu().numpy()
    for u in range(rows):
        b, h = divmod(u, hkv)
        assert np.array_equal(kg[b, h].view(np.uint16), O.gather_rows(k[b, h], want_idx[u]).view(np.uint16))
        assert np.array_equal(vg[b, h].view(np.uint16), O.gather_rows(v[b, h], want_idx[u]).view(np.uint16))
    w = synth.WORKLOADS["llama8b"].with_(name=f"selected_b{bits}g{group}", batch=batch,
                                          n_kv_heads=hkv, n_q_heads=hkv * r, tokens=nk,
                                          bits=bits, group=group, residual=32)
    gc = H.GpuCache(w)
    gc.append(kg, vg)
    orc = H.oracle_units(w, [(b, h) for b in range(batch) for h in range(hkv)], kg, vg)
    st = gc.state()
    for u, key in enumerate(sorted(orc)):
        H.check_unit_state(st, u, orc[key])
    qd = synth.queries(w)
    out = gc.decode(qd).cpu().numpy()
    for (b, h), uc in orc.items():
        Kd, Vd = uc.dequantized_kv()
        ref, _ = O.unit_attention(Kd, Vd, qd[b, h * r:(h + 1) * r])
        H.check_outputs(out[b, h * r:(h + 1) * r], ref, f"{w.name} unit {(b, h)}")
