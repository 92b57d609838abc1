"""kvq_decode_attention_noalloc (static device scratch, no allocation) against
kvq_decode_attention (caller workspace) through the C ABI: the same kernels,
so outputs and H2O scores must agree bit for bit. Two calls in a row, the
second on a smaller cache, then a call that would need more scratch than the
library holds is refused before anything is launched."""
import numpy as np
import pytest
import torch

from kv_cache_compression_kvq_amd import abi, synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(kvq):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _cache(w, splits):
    K, V = synth.all_kv(w)
    gc = H.GpuCache(w)
    s0 = 0
    for n in splits:
        gc.append(K[:, :, s0:s0 + n], V[:, :, s0:s0 + n])
        s0 += n
    return gc


def _both(gc, q, with_acc):
    w = gc.w
    qt = torch.from_numpy(q).cuda()
    out_ws = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    acc0 = torch.rand((w.batch, w.n_kv_heads, w.tokens), device="cuda") if with_acc else None
    acc_ws = acc0.clone() if with_acc else None
    acc_na = acc0.clone() if with_acc else None
    ws = torch.empty(abi.decode_workspace(gc.h, with_acc), dtype=torch.uint8, device="cuda")
    abi.decode_attention(gc.h, qt, out_ws, acc_ws, ws)
    abi.decode_attention_noalloc(gc.h, qt, out_na, acc_na)
    torch.cuda.synchronize()
    assert torch.isfinite(out_na).all()
    assert torch.equal(out_ws, out_na)
    if with_acc:
        assert torch.equal(acc_ws, acc_na)
    return out_na


def test_noalloc_matches_workspace_entry_point_twice_shrinking():
    big = synth.WORKLOADS["llama8b"].with_(name="noalloc_big", batch=4, tokens=5000, pool=3,
                                           evict_cap=8, inject_frac=0.01)
    small = big.with_(name="noalloc_small", batch=1, n_kv_heads=2, n_q_heads=8, tokens=700,
                    residual=40, pool=0)
    g1 = _cache(big, [4000, 1000])
    g2 = _cache(small, [700])
    for gc in (g1, g2):
        ws = abi.decode_workspace(gc.h, True)
        assert ws <= abi.NOALLOC_SCRATCH_BYTES, ws
    _both(g1, synth.queries(big), with_acc=True)
    _both(g2, synth.queries(small), with_acc=True)
    # and once more without H2O scores, large then small again
    _both(g1, synth.queries(big, 1), with_acc=False)
    _both(g2, synth.queries(small, 1), with_acc=False)


def test_noalloc_refuses_more_than_its_scratch():
    # one sequence of 300000 tokens, 8 KV heads: the H2O logits alone need
    # 8 * 4 * 300000 * 4 bytes (38 MB) of scratch, more than the library holds
    w = synth.WORKLOADS["llama8b"].with_(name="noalloc_long", batch=1, tokens=300000)
    gc = H.GpuCache(w)
    zeros = torch.zeros((w.batch, w.n_kv_heads, w.tokens, w.head_dim), dtype=torch.float16,
                        device="cuda")
    abi.quantize_append(gc.h, zeros, zeros, w.tokens)
    torch.cuda.synchronize()
    del zeros
    need = abi.decode_workspace(gc.h, True)
    assert need > abi.NOALLOC_SCRATCH_BYTES
    q = torch.from_numpy(synth.queries(w)).cuda()
    out = torch.zeros((w.batch, w.n_q_heads, w.head_dim), device="cuda")
    acc = torch.zeros((w.batch, w.n_kv_heads, w.tokens), device="cuda")
    with pytest.raises(abi.KvqError) as e:
        abi.decode_attention_noalloc(gc.h, q, out, acc)
    assert e.value.status == abi.KVQ_ESCRATCH
    torch.cuda.synchronize()
    assert not acc.any() and not out.any()  # nothing was launched
    # without scores the same cache fits; all keys are zero, so every output
    # row is the mean of the (zero) values
    _both(gc, synth.queries(w), with_acc=False)
