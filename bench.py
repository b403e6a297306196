"""Benchmark of the LSA hot path on one MI355X.

One step = one pass of the whole prefill path over one synthetic layer:
build_bucket_cache over all T keys, lsa_index_prefill for all Tq queries,
lsa_sparse_attention over the resulting lists.  Default workload: T = Tq =
131,072, bf16 K/V, 32 query / 4 KV heads, head_dim 128, 1,024-component latent
mixture, flat search, k = 2,048, 4 sinks, 512-key window.

Prints one JSON line (metric: prefill query tok/s per layer).  The roofline
object describes the dominant kernel, timed with HIP events on the stream the
kernels run on; the cpu_baseline object times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cfg", type=int, default=2, help="workload (2 = 128K prefill, flat)")
    ap.add_argument("--mode", default="flat", choices=["flat", "tree"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def cpu_baseline(w, X, Y, budget_s: float):
    """Time the CPU oracle (one thread) on a bounded sample of the step: the
    bucket-cache build over every block, then index + attention for evenly
    spaced queries until the time budget is spent; scale to all Tq queries."""
    from threadpoolctl import threadpool_limits

    import lsa_synth as S
    from oracle import lsa_oracle as O
    with threadpool_limits(limits=1):
        prm = O.Params(k=w.k, n_sink=w.n_sink, window=w.window, index_dtype=w.dtype)
        nb_total = w.T // 512
        t0 = time.perf_counter()
        cache = O.build_cache(X, prm)
        t_build = time.perf_counter() - t0
        positions = np.linspace(w.q_start, w.T - 1, 256).astype(np.int64)
        rng = np.random.default_rng(0)
        rng.shuffle(positions)
        n_q, t_q = 0, 0.0
        t_start = time.perf_counter()
        for p in positions:
            q, _ = S.normal_rows(w, "q", np.array([p]), w.Hq * w.D)       # input, not timed
            t1 = time.perf_counter()
            r = O.index_query(Y[p - w.q_start], int(p), cache)
            t2 = time.perf_counter()
            sel = r.idx[:r.count]
            k, _ = S.normal_rows(w, "k", sel, w.Hkv * w.D)                 # input, not timed
            v, _ = S.normal_rows(w, "v", sel, w.Hkv * w.D)
            t3 = time.perf_counter()
            O.attention_query(q.reshape(w.Hq, w.D), k.reshape(-1, w.Hkv, w.D),
                              v.reshape(-1, w.Hkv, w.D), np.arange(len(sel)), len(sel))
            t4 = time.perf_counter()
            t_q += (t2 - t1) + (t4 - t3)
            n_q += 1
            if time.perf_counter() - t_start > budget_s:
                break
        t_query = t_q / n_q
    t_step = t_build + t_query * w.Tq
    return dict(value=w.Tq / t_step, unit="query tok/s", cores=1, kind="oracle",
                sample=f"bucket-cache build over all {nb_total} blocks ({t_build:.1f} s) timed in "
                       f"full; index + attention timed for {n_q} evenly spaced queries "
                       f"({t_query * 1e3:.1f} ms each, input generation excluded) and scaled to "
                       f"{w.Tq} queries; one thread")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa

    w = S.WORKLOADS[args.cfg]
    if w.batch != 1:
        raise SystemExit("bench.py times prefill workloads (cfg 1, 2, 4, 5)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    X, Y, _ = S.latent_inputs(w)
    Xd = torch.from_numpy(X).to(dev)
    Yd = torch.from_numpy(Y).to(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Q = torch.empty((w.Tq, w.Hq, w.D), dtype=tdt, device=dev)
    K = torch.empty((w.T, w.Hkv, w.D), dtype=tdt, device=dev)
    V = torch.empty((w.T, w.Hkv, w.D), dtype=tdt, device=dev)
    for t, name, off in ((Q, "q", w.q_start * w.Hq * w.D), (K, "k", 0), (V, "v", 0)):
        S.device_fill_normal(t.data_ptr(), t.numel(), S.philox_key(w.cfg, name), off, w.dtype == "bf16",
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f}s")

    mode = lsa.LSA_TREE if args.mode == "tree" else lsa.LSA_FLAT
    p = lsa.Params(k=w.k, n_sink=w.n_sink, window=w.window, mode=mode, beam=w.beam,
                   index_dtype=lsa.LSA_BF16 if w.dtype == "bf16" else lsa.LSA_F32)
    L = lsa.list_len(p)
    nbytes = lsa.lib().lsa_cache_bytes(__import__("ctypes").byref(p.c()), w.T)
    cache_mem = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    idx = torch.empty((w.Tq, L), dtype=torch.int32, device=dev)
    cnt = torch.empty((w.Tq,), dtype=torch.int32, device=dev)
    ws = torch.empty(lsa.index_workspace_bytes(p, w.Tq), dtype=torch.uint8, device=dev)
    out = torch.empty_like(Q)

    class _Cache(lsa.BucketCache):
        def __init__(self):  # reuse the same device memory every step
            import ctypes
            self.params = p
            self.mem = cache_mem
            h = ctypes.c_void_p()
            lsa._check("lsa_cache_init", lsa.lib().lsa_cache_init(
                ctypes.byref(p.c()), w.T, lsa._ptr(cache_mem), nbytes, ctypes.byref(h)))
            self.handle = h

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(times=None):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        c = _Cache()
        e0.record()
        c.build(Xd)
        e1.record()
        lsa.index_prefill(c, Yd, w.q_start, p, workspace=ws, out=(idx, cnt))
        e2.record()
        lsa.sparse_attention(Q, K, V, idx, cnt, out=out)
        e3.record()
        if times is not None:
            times.append((e0, e1, e2, e3))
        return c

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(times)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    stage = np.array([[a.elapsed_time(b), b.elapsed_time(c), c.elapsed_time(d)]
                      for a, b, c, d in times])
    t_build, t_index, t_attn = stage.mean(axis=0)
    log(f"per step: build {t_build:.3f} ms, index {t_index:.3f} ms, attention {t_attn:.3f} ms; "
        f"wall {ms_step:.3f} ms")

    # algorithmic bytes of the attention launch: gathered K and V rows for every
    # KV head, plus Q, O and the index lists
    total_rows = int(cnt.to(torch.int64).sum().item())
    esz = 2 if w.dtype == "bf16" else 4
    attn_bytes = (total_rows * w.Hkv * w.D * esz * 2 + 2 * w.Tq * w.Hq * w.D * esz
                  + w.Tq * L * 4)
    achieved = attn_bytes / (t_attn * 1e-3) / 1e9
    # algorithmic FLOPs of flat scoring: 2 * 64 per eligible (query, bucket) pair
    pos = np.arange(w.q_start, w.T, dtype=np.int64)
    pairs = int((64 * (pos // 512)).sum())
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None,
                    kernel="k_attn_bf16" if w.dtype == "bf16" else "k_attn_f32",
                    algorithmic_bytes=attn_bytes, kernel_ms=round(float(t_attn), 4))
    value = w.Tq / (ms_step * 1e-3)
    res = {
        "metric": "prefill query tok/s per layer", "value": round(value, 1),
        "unit": "query tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "Tq": w.Tq, "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.D, "k": w.k, "mode": args.mode, "n_sink": w.n_sink,
                   "window": w.window, "latent_components": w.n_comp, "parallelism": "none"},
        "stages_ms": {"build": round(float(t_build), 4), "index": round(float(t_index), 4),
                      "attention": round(float(t_attn), 4)},
        "scoring": {"pairs": pairs, "algorithmic_tflop": round(pairs * 128 / 1e12, 4)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        cb = cpu_baseline(w, X, Y, args.cpu_seconds)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
