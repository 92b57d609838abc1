#!/usr/bin/env python3
"""Benchmark: decode steps over a 2/4-bit compressed KV cache on one MI355X.

A step is one decode step of one attention layer at the chosen workload, every
row of the hot path it touches included:
  * append the step's new token to every (batch, KV head) unit (residual ring;
    when a group leaves the window: OTT scoring / pool scan if the workload has
    a pool, quantize + pack);
  * attention over the compressed cache (fused dequant + split-K kernel, merge);
  * for workloads with H2O scores (minikv): accumulate the scores instead of
    appending, then select heavy hitters (top-k + recent window).

Inputs are seeded synthetic tensors of the workload's shapes, resident in HBM
before timing. The cache is replicated past the 256 MB Infinity Cache and the
steps rotate over the replicas, as the layers of a model would, so that no step
reads data left cached by the previous one. The timed steps are captured once
in a HIP graph and replayed (the loop is launch-bound otherwise).

value = algorithmic bytes of all timed steps / their time (GB/s). The roofline
entry times the fused attention kernel alone through HIP events attached to its
dispatch. The CPU baseline times the oracle on a bounded sample of units.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attention GB/s and % of MI355X HBM peak; tokens·heads/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0  # dense fp16 matrix-core peak of MI355X
REPLICA_BYTES = 600e6  # total cache bytes the rotation spans (> 256 MB Infinity Cache)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama8b")
    p.add_argument("--no-graph", action="store_true", help="launch the timed steps eagerly")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="timed CPU work for the oracle baseline (0 disables it)")
    p.add_argument("--kernel-reps", type=int, default=4,
                   help="event-timed attention launches per replica for the roofline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (counter calibration runs)")
    p.add_argument("--rows", nargs="*", default=None, metavar="ROW",
                   help="instead of the step line: time each row of the hot path on the "
                        f"workload it is measured at, one JSON line per row ({', '.join(ROWS)}; "
                        "no names = all)")
    p.add_argument("--reps", type=int, default=20, help="timed calls per row (--rows)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t helpers on the HIP runtime torch has loaded (same soname)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        f = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)


def source_sha() -> str:
    h = hashlib.sha256()
    for f in ("kvq_decode.hip", "kvq_internal.h"):
        with open(os.path.join(ROOT, "kv_cache_compression_kvq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_entry(workload: str, kernel_alg_bytes: float):
    """HBM traffic of the attention kernel from the committed rocprofv3 counter
    summary, when it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha():
        return None
    return {"fetch_bytes": t["fetch_bytes"], "write_bytes": t["write_bytes"],
            "total_bytes": t["fetch_bytes"] + t["write_bytes"],
            "vs_algorithmic": (t["fetch_bytes"] + t["write_bytes"]) / kernel_alg_bytes,
            "copy_scale": t["copy_scale"], "source": os.path.relpath(path, ROOT)}


def cpu_baseline(w, seconds: float, picks=None):
    """The oracle (numpy, fp64 attention, one thread) on a bounded sample of
    units: per sampled unit, repeated decode steps of the same kind the GPU
    times. Setup (quantizing the prefix) is not timed. ``picks`` selects
    units by position in a fixed seeded permutation (default: the first 4)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from kv_cache_compression_kvq_amd import bytes_model as BM, synth
    from oracle import kvq_oracle as O

    p = O.CacheParams(bits=w.bits, group=w.group, residual=w.residual, pool=w.pool,
                      evict_cap=w.evict_cap, head_dim=w.head_dim)
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    rng = np.random.default_rng(1)
    perm = rng.permutation(len(units))
    pick = [units[perm[i % len(units)]] for i in (picks if picks is not None
                                                  else range(min(4, len(units))))]
    r = w.gqa
    total_t, total_bytes, steps, used = 0.0, 0, 0, set()
    with threadpool_limits(limits=1):
        caches = {}
        for (b, h) in pick:
            k, v = synth.unit_kv(w, b, h)
            uc = O.UnitCache(p)
            uc.append(k, v)
            caches[(b, h)] = uc
        q = synth.queries(w)
        n_max = 4000
        new_tok = {} if w.h2o else {
            u: synth.unit_kv(w, u[0], u[1], n=n_max, start=w.tokens + 1) for u in pick}
        i = 0
        while total_t < seconds and steps < n_max:
            b, h = pick[i % len(pick)]
            uc = caches[(b, h)]
            t0 = time.perf_counter()
            if not w.h2o:
                j = i // len(pick)
                uc.append(new_tok[(b, h)][0][j:j + 1], new_tok[(b, h)][1][j:j + 1])
            K, V = uc.dequantized_kv()
            _, pr = O.unit_attention(K, V, q[b, h * r:(h + 1) * r])
            if w.h2o:
                acc = O.h2o_increment(pr).astype(np.float32)[None]
                O.topk_keep(acc, w.topk_k, w.recent)
            total_t += time.perf_counter() - t0
            pools = len(uc.tracer.pool) + len(uc.tracer.evicted)
            total_bytes += BM.decode_step_bytes(
                units=1, gqa=r, head_dim=w.head_dim, tokens=uc.T, bits=w.bits, group=w.group,
                residual=w.residual, pool_tokens=pools, h2o=w.h2o).total
            steps += 1
            used.add((b, h))
            i += 1
    return {"value": total_bytes / total_t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} single-unit decode steps over {len(used)} of {len(units)} "
                      f"(batch, KV head) units of the same workload, "
                      f"{'H2O scores + top-k' if w.h2o else 'append one token + attention'}, "
                      f"numpy fp64, BLAS limited to 1 thread, {total_t:.1f} s",
            "bytes": total_bytes, "seconds": total_t, "steps": steps}


def _cpu_model() -> str:
    """The host CPU's model string (/proc/cpuinfo), or '' when unavailable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _cpu_worker(job):
    name, i, seconds = job
    from kv_cache_compression_kvq_amd import synth
    return cpu_baseline(synth.WORKLOADS[name], seconds, picks=[i])


def cpu_baselines(w, seconds: float):
    """The oracle on one core, then on every core of this process's CPU set
    (at most 16, the share of one GPU) at once, one unit per worker process.
    Runs before anything touches the GPU: the workers are forked."""
    import multiprocessing

    single = cpu_baseline(w, seconds)
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    with multiprocessing.get_context("fork").Pool(n) as pool:
        res = pool.map(_cpu_worker, [(w.name, i, seconds) for i in range(n)])
    value = sum(r["bytes"] / r["seconds"] for r in res) / 1e9
    steps = sum(r["steps"] for r in res)
    out = {"value": value, "unit": "GB/s", "cores": n, "kind": "oracle", "cpu_model": _cpu_model(),
           "host_cpus": os.cpu_count(),
           "sample": f"{n} worker processes, one (batch, KV head) unit each, running at once: "
                     f"{steps} single-unit decode steps of the same workload, numpy fp64, "
                     f"one BLAS thread per worker, about {seconds:.0f} s each; value = sum of "
                     f"the workers' rates",
           "single_thread": {k: single[k] for k in ("value", "unit", "cores", "sample")}}
    return out


# Rows of the hot path timed by --rows: name -> (workload, what the timed call runs).
ROWS = {
    "append_llama8b": ("llama8b", "a4-a7: bulk quantize + pack of the whole prefix, ring store"),
    "append_ott": ("ott", "a1-a7: OTT scores + pool scan, mean replacement, quantize + pack, ring"),
    "decode_h2o_minikv": ("minikv", "a8-a10: fused decode + merge with H2O accumulation"),
    "topk_minikv": ("minikv", "a11: heavy-hitter top-k + recent window"),
    "evict_minikv": ("minikv", "f2: one H2O eviction per KV head (budget 20% + 256 recent)"),
    "topk_long": ("long_b2g32", "a11: heavy-hitter top-k (20% + 256 recent) over 131072-token rows"),
    "decode_llama8b_g16": ("llama8b_g16", "a8-a10: fused decode + merge at group size 16"),
    "decode_llama8b_sinks": ("llama8b_sinks", "a8-a10 with 4 attention sinks in the fp16 partition"),
    "prefill_llama8b": ("prefill_llama8b", "f1: causal prefill attention + A_cumul column sums "
                                          "(selective flash-attention)"),
    "append_llama8b_fp8": ("llama8b_fp8", "f4: bulk FP8 E4M3 encode of the whole prefix, ring store"),
    "decode_llama8b_fp8": ("llama8b_fp8", "f4: fused FP8 E4M3 decode + merge"),
    "decode_long_b2g32": ("long_b2g32", "a8-a10: fused decode + merge, split-K over context"),
    "decode_long_b2g128": ("long_b2g128", "a8-a10: fused decode + merge, split-K over context"),
    "decode_long_b4g32": ("long_b4g32", "a8-a10: fused decode + merge, split-K over context"),
    "decode_long_b4g128": ("long_b4g128", "a8-a10: fused decode + merge, split-K over context"),
    "append_long_b2g32": ("long_b2g32", "a4-a7: bulk quantize + pack of the whole prefix, ring store"),
    "append_long_b2g128": ("long_b2g128", "a4-a7: bulk quantize + pack of the whole prefix, ring store"),
    "append_long_b4g32": ("long_b4g32", "a4-a7: bulk quantize + pack of the whole prefix, ring store"),
    "append_long_b4g128": ("long_b4g128", "a4-a7: bulk quantize + pack of the whole prefix, ring store"),
}


def rows_main(args):
    """Time each row's ABI call with events on the stream it launches on.

    Inputs are resident in HBM; caches and sources rotate over replicas that
    together exceed the 256 MB Infinity Cache. One JSON line per row:
    algorithmic bytes of one call (the byte model), mean call time, GB/s and
    the fraction of the 8 TB/s HBM peak.
    """
    import torch

    from kv_cache_compression_kvq_amd import abi, bytes_model as BM, synth

    if not os.path.exists(abi.LIB_PATH):
        from kv_cache_compression_kvq_amd import build as B
        B.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    names = args.rows or list(ROWS)
    for n in names:
        if n not in ROWS:
            print(f"unknown row {n}; rows: {', '.join(ROWS)}", file=sys.stderr)
            sys.exit(2)

    def cfg_of(w):
        return abi.make_config(bits=w.bits, group=w.group, residual=w.residual, pool=w.pool,
                               evict_cap=w.evict_cap, head_dim=w.head_dim, n_q_heads=w.n_q_heads,
                               n_kv_heads=w.n_kv_heads, batch=w.batch, max_tokens=w.tokens,
                               sinks=w.sinks)

    def timed(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            fn(i, a, b)
        torch.cuda.synchronize()
        return 1e3 * sum(a.elapsed_time(b) for a, b in evs) / reps  # us

    def emit(name, w, us, nbytes, extra):
        gbs = nbytes / (us * 1e-6) / 1e9
        line = {"row": name, "workload": w.name, "what": ROWS[name][1], "us_per_call": round(us, 3),
                "alg_bytes": int(nbytes), "GB/s": round(gbs, 2),
                "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        line.update(extra)
        print(json.dumps(line), flush=True)

    loaded = {}

    def source(w):
        # fp16 K/V of the whole prefix, replicated past the Infinity Cache
        if w.name not in loaded:
            loaded.clear()
            K, V = synth.all_kv(w)
            src_bytes = 2 * K.nbytes
            n_src = max(2, math.ceil(REPLICA_BYTES / src_bytes))
            Kd = torch.from_numpy(K).to(dev)
            Vd = torch.from_numpy(V).to(dev)
            loaded[w.name] = [(Kd, Vd)] + [(Kd.clone(), Vd.clone()) for _ in range(n_src - 1)]
        return loaded[w.name]

    def caches(w, n_min=2):
        cfg = cfg_of(w)
        nb = abi.cache_bytes(cfg)
        n_rep = max(n_min, math.ceil(REPLICA_BYTES / nb))
        out = []
        for _ in range(n_rep):
            arena = torch.empty(nb, dtype=torch.uint8, device=dev)
            out.append({"arena": arena, "h": abi.cache_init(cfg, arena)})
        return cfg, out

    for name in names:
        w = synth.WORKLOADS[ROWS[name][0]]
        U, d = w.units, w.head_dim
        if name.startswith("prefill"):
            # q, k, v of the prompt resident in HBM; replicas past the Infinity Cache
            n, Hq, Hkv = w.tokens, w.n_q_heads, w.n_kv_heads
            g = torch.Generator(device=dev).manual_seed(0)
            per = (Hq + 2 * Hkv) * n * d * 2
            n_rep = max(2, math.ceil(REPLICA_BYTES / per))
            bufs = [(torch.randn((w.batch, Hq, n, d), generator=g, device=dev).half(),
                     torch.randn((w.batch, Hkv, n, d), generator=g, device=dev).half(),
                     torch.randn((w.batch, Hkv, n, d), generator=g, device=dev).half())
                    for _ in range(n_rep)]
            out = torch.empty((w.batch, Hq, n, d), device=dev)
            acc = torch.empty((w.batch, Hkv, n), device=dev)
            ws = torch.empty(abi.prefill_workspace(w.batch, Hq, n), dtype=torch.uint8, device=dev)

            def call(i, a, b):
                qq, kk, vv = bufs[i % n_rep]
                a.record()
                abi.prefill_attention(qq, kk, vv, w.batch, Hq, Hkv, n, out, acc, ws)
                b.record()

            timed(call, 2)
            us = timed(call, args.reps)
            fl = BM.prefill_flops(batch=w.batch, n_q_heads=Hq, head_dim=d, tokens=n)
            tfs = fl / (us * 1e-6) / 1e12
            line = {"row": name, "workload": w.name, "what": ROWS[name][1],
                    "us_per_call": round(us, 3), "alg_flops": int(fl), "TFLOP/s": round(tfs, 2),
                    "roofline": {"bound": "mfma", "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                                 "frac": round(tfs / MFMA_F16_PEAK_TFS, 4)},
                    "kernels": ["prefill_fwd_kernel", "prefill_colsum_kernel"],
                    "prompt": n}
            print(json.dumps(line), flush=True)
            del bufs, out, acc, ws
            torch.cuda.empty_cache()
            continue
        if name == "topk_long":
            # seeded exponential scores of every KV head's row, replicas past
            # the Infinity Cache; the split (workspace) path, with the
            # one-workgroup-per-row time beside it
            T, k, wr = w.tokens, int(0.2 * w.tokens), 256
            s0 = torch.from_numpy(synth.score_rows(U, T, seed=5)).to(dev)
            n_rep = max(2, math.ceil(REPLICA_BYTES / s0.numel() / 4))
            srows = [s0] + [s0.clone() for _ in range(n_rep - 1)]
            idx = torch.empty((U, k + wr), dtype=torch.int32, device=dev)
            nws = abi.topk_workspace(U, T, k, wr)
            tws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
            times = {}
            for with_ws in (False, True):
                def call(i, a, b):
                    a.record()
                    abi.topk_evict(srows[i % n_rep], U, T, k, wr, idx, tws if with_ws else None,
                                   nws if with_ws else 0)
                    b.record()

                timed(call, 2)
                times[with_ws] = timed(call, args.reps)
            emit(name, w, times[True], BM.topk_bytes(rows=U, tokens=T, k=k, w=wr),
                 {"kernels": ["topk_slice_hist_kernel", "topk_slice_select_kernel"], "k": k,
                  "recent": wr, "rows": U, "workspace_bytes": nws,
                  "us_one_workgroup_per_row": round(times[False], 3)})
            del srows, s0, tws, idx
            torch.cuda.empty_cache()
            continue
        if name.startswith("append"):
            srcs = source(w)
            cfg, reps = caches(w)

            def call(i, a, b):
                rep = reps[i % len(reps)]
                kd, vd = srcs[i % len(srcs)]
                h = abi.cache_init(cfg, rep["arena"])
                a.record()
                abi.quantize_append(h, kd, vd, w.tokens)
                b.record()
                rep["h"] = h

            timed(call, 2)  # warm-up
            us = timed(call, args.reps)
            nq = BM.n_quantized(w.tokens, w.residual, w.group)
            nbytes = BM.bulk_append_bytes(units=U, head_dim=d, tokens=w.tokens, n_quant=nq,
                                          bits=w.bits, group=w.group)
            emit(name, w, us, nbytes, {"kernels": ["pack_kernel (scores)", "ott_scan_kernel",
                                                   "pack_kernel (repair)", "ring_store_kernel"]
                                       if w.pool else ["pack8_kernel" if w.bits == 8
                                                       else "pack_kernel", "ring_store_kernel"]})
            continue
        srcs = source(w)
        cfg, reps = caches(w)
        for i, rep in enumerate(reps):
            kd, vd = srcs[i % len(srcs)]
            abi.quantize_append(rep["h"], kd, vd, w.tokens)
            rep["acc"] = torch.zeros((w.batch, w.n_kv_heads, w.tokens), device=dev) \
                if w.h2o else None
        loaded.clear()
        q = torch.from_numpy(synth.queries(w)).to(dev)
        out = torch.empty((w.batch, w.n_q_heads, d), device=dev)
        ws = torch.empty(abi.decode_workspace(reps[0]["h"], w.h2o), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        if name.startswith("decode"):
            def call(i, a, b):
                rep = reps[i % len(reps)]
                a.record()
                abi.decode_attention(rep["h"], q, out, rep["acc"], ws)
                b.record()

            timed(call, 2)
            us = timed(call, args.reps)
            nbytes = BM.decode_step_bytes(units=U, gqa=w.gqa, head_dim=d, tokens=w.tokens,
                                          bits=w.bits, group=w.group, residual=w.residual,
                                          h2o=w.h2o, sinks=w.sinks).total
            emit(name, w, us, nbytes, {"kernels": ["decode8_kernel" if w.bits == 8 else "decode_kernel",
                                                   "merge_kernel"]})
        elif name.startswith("evict"):  # one eviction step on accumulated scores
            for rep in reps:
                abi.decode_attention(rep["h"], q, out, rep["acc"], ws)
            budget = w.topk_k + w.recent

            def call(i, a, b):
                rep = reps[i % len(reps)]
                a.record()
                abi.evict_step(rep["h"], rep["acc"], budget, w.recent)
                b.record()

            timed(call, 2)
            us = timed(call, args.reps)
            emit(name, w, us, BM.evict_step_bytes(rows=U, tokens=w.tokens, sinks=w.sinks),
                 {"kernels": ["evict_step_kernel"], "budget": budget, "recent": w.recent})
        else:  # top-k over the accumulated scores of a decode call
            for rep in reps:
                abi.decode_attention(rep["h"], q, out, rep["acc"], ws)
            k, wr = w.topk_k, w.recent
            idx = torch.empty((U, k + wr), dtype=torch.int32, device=dev)
            nws = abi.topk_workspace(U, w.tokens, k, wr)
            tws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

            def call(i, a, b):
                rep = reps[i % len(reps)]
                a.record()
                abi.topk_evict(rep["acc"], U, w.tokens, k, wr, idx, tws, nws)
                b.record()

            timed(call, 2)
            us = timed(call, args.reps)
            kernels = (["topk_slice_hist_kernel", "topk_slice_select_kernel"] if nws
                       else ["topk_reg_kernel"])
            emit(name, w, us, BM.topk_bytes(rows=U, tokens=w.tokens, k=k, w=wr),
                 {"kernels": kernels, "k": k, "recent": wr, "workspace_bytes": nws})
        del reps, ws, out
        torch.cuda.empty_cache()
    if args.copy_calibration:
        # a plain 256 MiB device copy: the counter scale for the runs above
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def main():
    args = parse_args()
    # CPU oracle baseline first, while no process has touched the GPU
    cpu_line = None
    if args.rows is None and args.cpu_seconds > 0 and args.gpus == 1:
        from kv_cache_compression_kvq_amd import synth as _synth
        cpu_line = cpu_baselines(_synth.WORKLOADS[args.workload], args.cpu_seconds)
    if args.rows is not None:
        if args.gpus != 1:
            print("bench.py: kvq runs on one GPU; --rows takes no --gpus above 1", file=sys.stderr)
            sys.exit(2)
        rows_main(args)
        return
    if args.gpus != 1:
        print(f"bench.py: kvq runs on one GPU; --gpus {args.gpus} is not supported "
              "(the (batch, KV head) units would shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_compression_kvq_amd import abi, bytes_model as BM, synth

    if not os.path.exists(abi.LIB_PATH):
        from kv_cache_compression_kvq_amd import build as B
        B.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    U, r, d = w.units, w.gqa, w.head_dim
    hip = HipEvents()

    # ---- inputs, resident in HBM before timing -----------------------------
    K, V = synth.all_kv(w)
    Kd = torch.from_numpy(K).to(dev)
    Vd = torch.from_numpy(V).to(dev)
    del K, V
    append_mode = not w.h2o
    n_total = args.warmup + args.steps
    cfg0 = abi.make_config(bits=w.bits, group=w.group, residual=w.residual, pool=w.pool,
                           evict_cap=w.evict_cap, head_dim=d, n_q_heads=w.n_q_heads,
                           n_kv_heads=w.n_kv_heads, batch=w.batch, max_tokens=w.tokens)
    cache_bytes0 = abi.cache_bytes(cfg0)
    n_rep = max(2, math.ceil(REPLICA_BYTES / cache_bytes0))
    per_rep = math.ceil(n_total / n_rep) if append_mode else 0
    # Replica i starts (i * G / n_rep) tokens into its residual window, so that
    # the steps reach the end of the window (and quantize a group) at evenly
    # spread times: about 1 step in G packs a group, as in a long decode.
    phases = [(i * w.group) // n_rep if append_mode else 0 for i in range(n_rep)]
    max_tokens = w.tokens + max(phases) + per_rep
    reps = []
    for i in range(n_rep):
        cfg = abi.make_config(bits=w.bits, group=w.group, residual=w.residual, pool=w.pool,
                              evict_cap=w.evict_cap, head_dim=d, n_q_heads=w.n_q_heads,
                              n_kv_heads=w.n_kv_heads, batch=w.batch, max_tokens=max_tokens,
                              sinks=w.sinks)
        arena = torch.empty(abi.cache_bytes(cfg), dtype=torch.uint8, device=dev)
        h = abi.cache_init(cfg, arena)
        abi.quantize_append(h, Kd, Vd, w.tokens)
        if phases[i]:
            abi.quantize_append(h, Kd[:, :, :phases[i]].contiguous(), Vd[:, :, :phases[i]].contiguous(),
                                phases[i])
        acc = torch.zeros((w.batch, w.n_kv_heads, w.tokens), device=dev) if w.h2o else None
        reps.append({"arena": arena, "h": h, "acc": acc})
    del Kd, Vd
    if append_mode:
        ks = torch.empty((n_total, w.batch, w.n_kv_heads, 1, d), dtype=torch.float16)
        vs = torch.empty_like(ks)
        for i in range(n_total):
            a, b = synth.step_kv(w, i)
            ks[i], vs[i] = torch.from_numpy(a), torch.from_numpy(b)
        ks, vs = ks.to(dev), vs.to(dev)
    n_q_rot = 8
    qs = torch.stack([torch.from_numpy(synth.queries(w, i)) for i in range(n_q_rot)]).to(dev)
    out = torch.empty((w.batch, w.n_q_heads, d), device=dev)
    # workspace for every T a replica reaches (the plan depends on T)
    hmax = abi.Cache()
    ctypes.memmove(ctypes.byref(hmax), ctypes.byref(reps[0]["h"]), ctypes.sizeof(hmax))
    ws_bytes = 0
    for T in range(w.tokens, max_tokens + 1):
        hmax.tokens = T
        hmax.n_quant = max(0, (T - w.sinks - w.residual) // w.group * w.group)
        ws_bytes = max(ws_bytes, abi.decode_workspace(hmax, w.h2o))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    k_hh = w.topk_k
    idx = torch.empty((U, k_hh + w.recent), dtype=torch.int32, device=dev) if w.h2o else None
    tk_nws = abi.topk_workspace(U, w.tokens, k_hh, w.recent) if w.h2o else 0
    tk_ws = torch.empty(max(tk_nws, 1), dtype=torch.uint8, device=dev) if w.h2o else None
    torch.cuda.synchronize()

    step_bytes = []   # algorithmic bytes of each executed step (host bookkeeping)
    step_tokens = []  # cached token x KV-head entries read by each step
    step_packs = []   # groups quantized by each step (per unit)

    def pool_tokens(rep):
        if w.pool == 0:
            return 0
        cnt = rep["arena"][rep["h"].off_counters:rep["h"].off_counters + 16 * U]
        c = cnt.view(torch.int32).view(U, 4).cpu()
        return int(c[:, 0].sum() + c[:, 1].sum())

    pools_now = [pool_tokens(rp) for rp in reps]

    def decode_bytes(h, pools):
        return BM.decode_step_bytes(units=U, gqa=r, head_dim=d, tokens=h.tokens, bits=w.bits,
                                    group=w.group, residual=w.residual, pool_tokens=pools,
                                    h2o=w.h2o).total

    def step(i, ev=(None, None)):
        rep = reps[i % n_rep]
        h = rep["h"]
        nb = 0
        q = qs[i % n_q_rot]
        if append_mode:
            # one decode step: append the token, then attend (the attention
            # kernel stores the token into the fp16 ring)
            nq0 = h.n_quant
            if ev[0] is not None:
                abi.decode_step_timed(h, ks[i], vs[i], q, out, rep["acc"], ws, ev[0], ev[1])
            else:
                abi.decode_step(h, ks[i], vs[i], q, out, rep["acc"], ws)
            nb += BM.append_bytes(units=U, head_dim=d, n_new=1, bits=w.bits, group=w.group,
                                  groups_packed=(h.n_quant - nq0) // w.group)
            step_packs.append((h.n_quant - nq0) // w.group)
        elif ev[0] is not None:
            abi.decode_attention_timed(rep["h"], q, out, rep["acc"], ws, ev[0], ev[1])
        else:
            abi.decode_attention(rep["h"], q, out, rep["acc"], ws)
        nb += decode_bytes(h, pools_now[i % n_rep])
        if w.h2o:
            abi.topk_evict(rep["acc"], U, w.tokens, k_hh, w.recent, idx, tk_ws, tk_nws)
            nb += BM.topk_bytes(rows=U, tokens=w.tokens, k=k_hh, w=w.recent)
        step_bytes.append(nb)
        step_tokens.append(U * h.tokens)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_bytes.clear()
    step_tokens.clear()
    step_packs.clear()

    use_graph = not args.no_graph
    if use_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=cap):
            for j in range(args.steps):
                step(args.warmup + j)
        torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    if use_graph:
        g.replay()
    else:
        for j in range(args.steps):
            step(args.warmup + j)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    if use_graph:
        # the replayed steps must give what an eager launch gives on the same state
        last = reps[(args.warmup + args.steps - 1) % n_rep]
        ref = torch.empty_like(out)
        got = out.clone()
        acc_copy = last["acc"].clone() if w.h2o else None
        abi.decode_attention(last["h"], qs[(args.warmup + args.steps - 1) % n_q_rot], ref,
                             acc_copy, ws)
        torch.cuda.synchronize()
        if not torch.equal(got, ref):
            raise RuntimeError("graph replay result differs from an eager launch")

    # ---- the fused attention kernel alone, timed by events on its dispatch ----
    evs = [(hip.create(), hip.create()) for _ in range(args.kernel_reps * n_rep)]
    kbytes = []
    for i, ev in enumerate(evs):
        rep = reps[i % n_rep]
        abi.decode_attention_timed(rep["h"], qs[i % n_q_rot], out, rep["acc"], ws, ev[0], ev[1])
        kbytes.append(decode_bytes(rep["h"], pools_now[i % n_rep]))
    torch.cuda.synchronize()
    kms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    kernel_us = 1e3 * sum(kms) / len(kms)
    kernel_bytes = sum(kbytes) / len(kbytes)
    achieved = kernel_bytes / (kernel_us * 1e-6) / 1e9

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # Same-run streaming ceiling: one read-only pass over 1 GiB (kvq_stream_read,
    # every 16-byte word loaded once), event-timed, median of 5 runs: what
    # this machine's HBM delivers to a plain stream of reads, next to the 8 TB/s peak.
    big = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    abi.stream_read(big, sink)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        abi.stream_read(big, sink)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    stream_gbs = big.numel() / (sorted(times)[2] * 1e-3) / 1e9
    del big, sink

    value = sum(step_bytes) / (total_ms * 1e-3) / 1e9
    tok_heads = sum(step_tokens) / (total_ms * 1e-3)
    h0 = reps[0]["h"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": d, "tokens": w.tokens,
                   "bits": w.bits, "group": w.group, "residual": w.residual, "pool": w.pool,
                   "h2o": w.h2o, "replicas": n_rep, "hip_graph": use_graph,
                   "step": "append 1 token + attention; replicas at spread window phases, so "
                           "about 1 step in G also quantizes a group (every unit)"
                   if append_mode else "attention with H2O scores + top-k",
                   "groups_quantized_in_timed_steps": int(sum(step_packs))},
        "stream_read_GBps": round(stream_gbs, 1),
        "pct_of_stream_read": round(100 * value / stream_gbs, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_heads_per_s": round(tok_heads, 1),
        "query_head_scores_per_s": round(tok_heads * r, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "frac_of_stream_read": round(achieved / stream_gbs, 4),
                     "traffic": None,
                     "kernel": "decode_kernel", "kernel_us": round(kernel_us, 3),
                     "kernel_alg_bytes": int(kernel_bytes), "source_sha": source_sha()},
        "cpu_baseline": None,
    }
    tr = traffic_entry(w.name, kernel_bytes)
    if tr is not None:
        # HBM bytes per launch from the rocprofv3 counter runs, calibrated by a copy
        line["roofline"]["traffic"] = int(tr["total_bytes"])
        line["roofline"]["traffic_detail"] = tr
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_line
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
