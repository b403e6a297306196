"""Benchmark of the LSA hot path on one MI355X.

One step = one pass of the whole prefill path over one synthetic layer:
build_bucket_cache over all T keys, lsa_index_prefill for all Tq queries,
lsa_sparse_attention over the resulting lists (which the library runs as
back-to-back launches of 1,024 query rows).  Default workload: T = Tq =
131,072, bf16 K/V, 32 query / 4 KV heads, head_dim 128, 1,024-component latent
mixture, flat search, k = 2,048, 4 sinks, 512-key window.

Prints one JSON line (metric: prefill query tok/s per layer).  The roofline
object describes the dominant kernel (the attention), timed with HIP events on
the stream its launches run on and reported per launch; the cpu_baseline object times the CPU oracle on a bounded
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


def workload_name(name: str, mode: str) -> str:
    """The workload's name with its indexing-mode suffix set to the mode actually run."""
    for suffix in ("_flat", "_tree"):
        if name.endswith(suffix):
            return name[: -len(suffix)] + "_" + mode
    return name


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
    ap.add_argument("--decode", action="store_true",
                    help="time decode steps (cfg 3: 16 sequences at 1M; cfg 5: one at 10M)")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode attention splits (0: the library's lsa_attention_default_splits)")
    ap.add_argument("--tree-sweep", action="store_true",
                    help="last chunk (cfg 4, 5): index time and far-key recall against flat "
                         "search for tree beam widths and leaf levels")
    ap.add_argument("--whole-context", action="store_true",
                    help="prefill the whole context in chunks of the workload's query count "
                         "(cfg 4, 5): append a chunk of keys, index its queries, attend")
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


def attention_kernel_name(lsa, w, B: int, Tmax: int) -> str:
    """The attention kernel (template instance) that lsa_sparse_attention runs."""
    if w.dtype != "bf16":
        return "k_attn_f32"
    if w.Hkv != 4:
        return "k_attn_bf16<1, 0>"
    nw = 1 if lsa.attention_head_major(B, Tmax, w.Hkv, w.D, lsa.LSA_BF16) else 4
    return f"k_attn_bf16<{nw}, 4>"


def measured_traffic(kernel: str, workload: str, rows_per_launch: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none, it was taken on another kernel, the kernel source
    changed since, or its launches covered another number of query rows."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    stem = kernel.split("<")[0]
    path = os.path.join(root, "profiles", f"{stem}.{workload}.traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        if fields["kernel"] != kernel:
            return None
        src = open(os.path.join(root, fields["kernel_source"]), "rb").read()
        if hashlib.sha256(src).hexdigest()[:16] != fields["kernel_source_sha256_16"]:
            return None
        if int(fields["rows_per_launch"]) != rows_per_launch:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def bench_decode(args, w, dev):
    """Batched decode: every sequence holds T cached tokens; each step appends one
    key per sequence (clustering a block when it fills), builds the index lists
    and runs split attention.  512 consecutive steps: 511 steady steps and one
    block-completing step."""
    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa
    B = w.batch if args.cfg == 3 else 1
    T, n_steps = w.T, 512
    Tmax = T + n_steps
    mode = lsa.LSA_TREE if args.mode == "tree" else lsa.LSA_FLAT
    p = lsa.Params(k=w.k, n_sink=w.n_sink, window=w.window, mode=mode, beam=w.beam)
    L = lsa.list_len(p)
    if args.splits <= 0:
        args.splits = lsa.attention_default_splits(B, L)
    caches, keys_new, queries = [], [], []
    t_gen = time.perf_counter()
    for b in range(B):
        X, Y, _ = S.latent_inputs(w, seq=b, T=Tmax, query_rows=(T, Tmax))
        c = lsa.BucketCache(p, Tmax)
        c.build(torch.from_numpy(X[:T]).to(dev))
        caches.append(c)
        keys_new.append(X[T:Tmax])
        queries.append(Y)
        del X
    torch.cuda.synchronize()
    log(f"{B} caches of {T} tokens built ({time.perf_counter() - t_gen:.1f}s with input generation)")
    kn = torch.from_numpy(np.stack(keys_new, axis=1).copy()).to(dev)      # [steps, B, 64]
    qn = torch.from_numpy(np.stack(queries, axis=1).copy()).to(dev)
    tdt = torch.bfloat16
    Kc = torch.empty((B, Tmax, w.Hkv, w.D), dtype=tdt, device=dev)
    Vc = torch.empty_like(Kc)
    Qd = torch.empty((n_steps, B, 1, w.Hq, w.D), dtype=tdt, device=dev)
    cs = torch.cuda.current_stream().cuda_stream
    for b in range(B):
        S.device_fill_normal(Kc[b].data_ptr(), Kc[b].numel(), S.philox_key(w.cfg, "k", b), 0, True, cs)
        S.device_fill_normal(Vc[b].data_ptr(), Vc[b].numel(), S.philox_key(w.cfg, "v", b), 0, True, cs)
    qsrc = torch.empty((n_steps, w.Hq * w.D), dtype=tdt, device=dev)
    for b in range(B):
        S.device_fill_normal(qsrc.data_ptr(), qsrc.numel(), S.philox_key(w.cfg, "q", b),
                             T * w.Hq * w.D, True, cs)
        Qd[:, b, 0] = qsrc.view(n_steps, w.Hq, w.D)
    idx = torch.empty((B, L), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(lsa.index_workspace_bytes(p, B), dtype=torch.uint8, device=dev)
    wsa = torch.empty(max(lsa.lib().lsa_attention_workspace_bytes(B, 1, w.Hq, w.D, args.splits), 1),
                      dtype=torch.uint8, device=dev)
    out = torch.empty((B, 1, w.Hq, w.D), dtype=tdt, device=dev)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []
    for s_ in range(n_steps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        lsa.index_decode(caches, qn[s_], kn[s_], p, workspace=ws, out=(idx, cnt))
        e1.record()
        lsa.sparse_attention(Qd[s_], Kc, Vc, idx.view(B, 1, L), cnt.view(B, 1), splits=args.splits,
                             out=out, workspace=wsa)
        e2.record()
        marks.append((e0, e1, e2))
    torch.cuda.synchronize()
    tim = np.array([[a.elapsed_time(b_), b_.elapsed_time(c_)] for a, b_, c_ in marks]) * 1e3
    fire = [i for i in range(n_steps) if (T + i + 1) % 512 == 0]
    steady = [i for i in range(8, n_steps) if i not in fire]
    st = tim[steady]
    tot_steady = float(np.median(st.sum(axis=1)))
    res = {
        "metric": f"decode us/token ({args.mode})", "value": round(tot_steady, 2), "unit": "us/token",
        "n_gpus": 1, "steps": len(steady), "warmup": 8, "ms_per_step": round(tot_steady / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_name(w.name if args.cfg == 3 else "decode_t10m_b1_bf16",
                                             args.mode), "T": T,
                   "batch": B, "k": w.k, "mode": args.mode, "attention_splits": args.splits,
                   "parallelism": "none"},
        "stages_us": {"index_decode": round(float(np.median(st[:, 0])), 2),
                      "attention": round(float(np.median(st[:, 1])), 2)},
        "firing_step_us": {"index_decode": round(float(tim[fire[0], 0]), 2),
                           "attention": round(float(tim[fire[0], 1]), 2)} if fire else None,
        "per_sequence_step_us": round(tot_steady / B, 3),
    }
    print(json.dumps(res), flush=True)


def bench_tree_sweep(args, w, dev):
    """Tree beam search against flat search on the workload's last chunk.  For
    beam widths 8..64 and leaf levels from the default (the smallest level
    where beam * 2^level reaches the B buckets to keep) upward -- stopping the
    beam higher up and ranking every bucket under it flat, the two-stage search
    -- the chunk's index time (HIP events, best of three) and each query's
    far-key recall: the share of its exact flat list's far keys (outside the
    sinks and the window) that the tree list also holds."""
    import ctypes

    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa

    if w.batch != 1 or w.q_start == 0:
        raise SystemExit("--tree-sweep needs a last-chunk workload (cfg 4, 5)")
    X, Y, _ = S.latent_inputs(w)
    Xd, Yd = torch.from_numpy(X).to(dev), torch.from_numpy(Y).to(dev)
    del X, Y
    base = dict(k=w.k, n_sink=w.n_sink, window=w.window, index_dtype=lsa.LSA_BF16)
    c = lsa.BucketCache(lsa.Params(mode=lsa.LSA_TREE, **base), w.T)
    c.build(Xd)
    torch.cuda.synchronize()
    ws = torch.empty(lsa.index_workspace_bytes(lsa.Params(**base), w.Tq), dtype=torch.uint8,
                     device=dev)

    def run(p):
        best, out = None, None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = lsa.index_prefill(c, Yd, w.q_start, p, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
        return best, out

    pos = torch.arange(w.q_start, w.T, device=dev, dtype=torch.int64)[:, None]

    def far_keys(idx):
        i64 = idx.to(torch.int64)
        m = (i64 >= w.n_sink) & (i64 <= pos - w.window)   # neither a sink nor a window key
        rows = torch.arange(w.Tq, device=dev, dtype=torch.int64)[:, None].expand_as(i64)
        return rows[m], rows[m] * w.T + i64[m], m.sum(dim=1)

    flat_ms, (fidx, _) = run(lsa.Params(mode=lsa.LSA_FLAT, **base))
    _, fkey, fcount = far_keys(fidx)
    points = []
    for beam in (8, 16, 32, 64):
        p0 = lsa.Params(mode=lsa.LSA_TREE, beam=beam, **base)
        l0 = 0
        while beam << l0 < lsa.top_buckets(p0):
            l0 += 1
        for leaf in range(l0, l0 + 4):
            p = lsa.Params(mode=lsa.LSA_TREE, beam=beam, leaf_level=leaf, **base)
            if lsa.lib().lsa_check_params(ctypes.byref(p.c())) != 0:
                break
            ms, (tidx, _) = run(p)
            trow, tkey, _ = far_keys(tidx)
            hit = torch.isin(tkey, fkey)
            hits = torch.bincount(trow[hit], minlength=w.Tq).to(torch.float64)
            rec = hits / fcount.clamp(min=1).to(torch.float64)
            rec = rec[fcount > 0]
            points.append(dict(beam=beam, leaf_level=leaf, scored_under_beam=beam << leaf,
                               index_ms=round(ms, 4), recall_mean=round(rec.mean().item(), 4),
                               recall_p10=round(torch.quantile(rec, 0.1).item(), 4),
                               recall_min=round(rec.min().item(), 4)))
            log(f"beam {beam:3d} leaf {leaf:2d}: index {ms:7.3f} ms, recall {points[-1]['recall_mean']:.3f}")
    default = next(q for q in points if q["beam"] == 64)
    res = {
        "metric": "tree/flat far-key recall (beam 64, default leaf level)",
        "value": default["recall_mean"], "unit": "fraction", "n_gpus": 1, "steps": 3, "warmup": 0,
        "ms_per_step": default["index_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name.replace("_tree", "") + "_tree_sweep", "T": w.T, "Tq": w.Tq,
                   "k": w.k, "parallelism": "none"},
        "flat_index_ms": round(flat_ms, 4),
        "points": points,
    }
    print(json.dumps(res), flush=True)


def bench_whole_context(args, w, dev):
    """The whole context prefilled in chunks of w.Tq queries, aligned so that the
    last chunk is the workload's measured final chunk (the first one is shorter).
    Per chunk: build_bucket_cache appends the chunk's latent keys (clustering the
    blocks that fill up, rebuilding the tree's right edge in tree mode), then
    lsa_index_prefill indexes the chunk's queries and lsa_sparse_attention
    attends over their lists.  K and V hold all T tokens; Q and the output are
    one chunk's buffers, reused (their values do not change the work; the
    per-position latent queries decide the lists).  One step = the whole
    context; no warm-up beyond one small chunk on a scratch cache."""
    import ctypes

    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa

    if w.batch != 1 or w.q_start == 0:
        raise SystemExit("--whole-context needs a last-chunk workload (cfg 4, 5)")
    t_gen = time.perf_counter()
    X, Y, _ = S.latent_inputs(w, query_rows=(0, w.T))
    Xd = torch.from_numpy(X).to(dev)
    Yd = torch.from_numpy(Y).to(dev)
    del X, Y
    C = w.Tq
    Q = torch.empty((C, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    K = torch.empty((w.T, w.Hkv, w.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for t, name, off in ((Q, "q", w.q_start * w.Hq * w.D), (K, "k", 0), (V, "v", 0)):
        S.device_fill_normal(t.data_ptr(), t.numel(), S.philox_key(w.cfg, name), off, True,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f}s")
    mode = lsa.LSA_TREE if args.mode == "tree" else lsa.LSA_FLAT
    p = lsa.Params(k=w.k, n_sink=w.n_sink, window=w.window, mode=mode, beam=w.beam,
                   index_dtype=lsa.LSA_BF16)
    L = lsa.list_len(p)
    nbytes = lsa.lib().lsa_cache_bytes(ctypes.byref(p.c()), w.T)
    cache_mem = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    idx = torch.empty((C, L), dtype=torch.int32, device=dev)
    cnt = torch.empty((C,), dtype=torch.int32, device=dev)
    ws = torch.empty(lsa.index_workspace_bytes(p, C), dtype=torch.uint8, device=dev)
    out = torch.empty_like(Q)
    rows_total = torch.zeros((), dtype=torch.int64, device=dev)

    def fresh_cache():
        c = lsa.BucketCache.__new__(lsa.BucketCache)
        c.params, c.mem = p, cache_mem
        h = ctypes.c_void_p()
        lsa._check("lsa_cache_init", lsa.lib().lsa_cache_init(
            ctypes.byref(p.c()), w.T, lsa._ptr(cache_mem), nbytes, ctypes.byref(h)))
        c.handle = h
        return c

    first = w.T - (w.T - 1) // C * C if w.T % C else C
    bounds = [(0, first)] + [(s0, s0 + C) for s0 in range(first, w.T, C)]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # warm-up: the first chunk on a scratch cache
    c = fresh_cache()
    c.build(Xd[:first])
    lsa.index_prefill(c, Yd[:first], 0, p, workspace=ws, out=(idx[:first], cnt[:first]))
    lsa.sparse_attention(Q[:first], K, V, idx[:first], cnt[:first], out=out[:first])
    torch.cuda.synchronize()
    c = fresh_cache()
    marks = []
    t0 = time.perf_counter()
    for i, (s0, s1) in enumerate(bounds):
        n = s1 - s0
        e = [ev() for _ in range(4)]
        e[0].record()
        c.build(Xd[s0:s1])
        e[1].record()
        lsa.index_prefill(c, Yd[s0:s1], s0, p, workspace=ws, out=(idx[:n], cnt[:n]))
        e[2].record()
        lsa.sparse_attention(Q[:n], K, V, idx[:n], cnt[:n], out=out[:n])
        e[3].record()
        rows_total += cnt[:n].to(torch.int64).sum()
        marks.append(e)
        if (i + 1) % 50 == 0:
            log(f"chunk {i + 1}/{len(bounds)} queued, {time.perf_counter() - t0:.1f}s")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = np.array([[a.elapsed_time(b), b.elapsed_time(c_), c_.elapsed_time(d)] for a, b, c_, d in marks])
    t_build, t_index, t_attn = st.sum(axis=0)
    total_ms = marks[0][0].elapsed_time(marks[-1][3])
    log(f"whole context: {total_ms:.1f} ms on the GPU ({wall:.1f} s wall): build {t_build:.1f}, "
        f"index {t_index:.1f}, attention {t_attn:.1f} ms over {len(bounds)} chunks")
    launches = sum(-(-(s1 - s0) // lsa.attention_launch_rows()) for s0, s1 in bounds)
    whole_name = workload_name(w.name, args.mode).replace("_q32k", "_whole").replace("_q8k", "_whole")
    if not whole_name.endswith("_" + args.mode):
        whole_name += "_" + args.mode
    attn_bytes = (int(rows_total.item()) * w.Hkv * w.D * 2 * 2 + 2 * w.T * w.Hq * w.D * 2
                  + w.T * L * 4)
    achieved = attn_bytes / (t_attn * 1e-3) / 1e9
    res = {
        "metric": f"whole-context prefill query tok/s per layer ({args.mode})",
        "value": round(w.T / (total_ms * 1e-3), 1), "unit": "query tok/s", "n_gpus": 1,
        "steps": 1, "warmup": 1, "ms_per_step": round(total_ms, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": whole_name, "T": w.T, "chunk": C, "chunks": len(bounds),
                   "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D, "k": w.k, "mode": args.mode,
                   "parallelism": "none"},
        "stages_ms": {"build": round(float(t_build), 2), "index": round(float(t_index), 2),
                      "attention": round(float(t_attn), 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": attention_kernel_name(lsa, w, 1, w.T),
                     "launches_per_step": launches,
                     "algorithmic_bytes": round(attn_bytes / launches),
                     "kernel_ms": round(float(t_attn) / launches, 4)},
        "wall_s": round(wall, 2),
    }
    print(json.dumps(res), flush=True)


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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode:
        return bench_decode(args, w, dev)
    if args.whole_context:
        return bench_whole_context(args, w, dev)
    if args.tree_sweep:
        return bench_tree_sweep(args, w, dev)
    if w.batch != 1:
        raise SystemExit("prefill timing needs a single-sequence workload (cfg 1, 2, 4, 5)")
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

    full_prefill = w.q_start == 0
    prebuilt = None
    build_once_ms = None
    if not full_prefill:
        # last prefill chunk of a long context: the cache of every full block
        # exists before the chunk; building it is timed once, separately
        prebuilt = _Cache()
        b0, b1 = ev(), ev()
        b0.record()
        prebuilt.build(Xd)
        b1.record()
        torch.cuda.synchronize()
        build_once_ms = b0.elapsed_time(b1)
        log(f"cache for {w.T // 512} blocks built in {build_once_ms:.2f} ms")

    def step(times=None):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        if full_prefill:
            c = _Cache()
            e0.record()
            c.build(Xd)
        else:
            c = prebuilt
            e0.record()
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
    kname = attention_kernel_name(lsa, w, 1, w.T)
    # the bf16 attention runs as back-to-back launches of up to launch_rows query
    # rows; bytes and time are reported per launch, averaged over the step's launches
    launch_rows = min(lsa.attention_launch_rows(), w.Tq) if w.dtype == "bf16" else w.Tq
    launches = -(-w.Tq // launch_rows)
    t_launch = t_attn / launches
    traffic = measured_traffic(kname, workload_name(w.name, args.mode), launch_rows)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=None if traffic is None else round(traffic),
                    kernel=kname, launches_per_step=launches,
                    algorithmic_bytes=round(attn_bytes / launches),
                    kernel_ms=round(float(t_launch), 4))
    if traffic is not None:
        roofline["traffic_gbs"] = round(traffic / (t_launch * 1e-3) / 1e9, 1)
        roofline["traffic_frac"] = round(traffic / (t_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    value = w.Tq / (ms_step * 1e-3)
    res = {
        "metric": f"prefill query tok/s per layer ({args.mode})", "value": round(value, 1),
        "unit": "query tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": workload_name(w.name, args.mode), "T": w.T, "Tq": w.Tq,
                   "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.D, "k": w.k, "mode": args.mode, "n_sink": w.n_sink,
                   "window": w.window, "latent_components": w.n_comp, "parallelism": "none"},
        "stages_ms": {"build": round(float(t_build), 4), "index": round(float(t_index), 4),
                      "attention": round(float(t_attn), 4)},
        "step": ("build + index + attention" if full_prefill else
                 "index + attention for the last chunk (cache built before timing)"),
        "scoring": {"pairs": pairs, "algorithmic_tflop": round(pairs * 128 / 1e12, 4)},
        "roofline": roofline,
    }
    if build_once_ms is not None:
        res["cache_build_ms"] = round(build_once_ms, 3)
    if not args.no_cpu_baseline and w.T <= 1 << 17:
        log("timing the CPU oracle on a sample ...")
        cb = cpu_baseline(w, X, Y, args.cpu_seconds)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
