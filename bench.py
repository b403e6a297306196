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
import gc
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector


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
    ap.add_argument("--scan", type=int, default=0, choices=[0, 1, 4, 8],
                    help="index with a scan baseline instead of LSA buckets: a token scan (1) "
                         "or a block scan over runs of 4 or 8 keys")
    ap.add_argument("--baselines", action="store_true",
                    help="LSA flat search and the token / block-4 / block-8 scans on the same "
                         "workload, one after the other, with their step times side by side")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline workload only (skip the 10M last-chunk and 16 x 1M decode "
                         "lines folded into the default run)")
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


_CPU = {}   # oracle state handed to the forked CPU-baseline workers


def _cpu_build(blocks):
    """Worker: the oracle's clustering of some blocks, timed."""
    from threadpoolctl import threadpool_limits

    from oracle import lsa_oracle as O
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.build_cache(_CPU["X"], _CPU["prm"], blocks=blocks)
        return time.perf_counter() - t0


def _cpu_queries(positions):
    """Worker: index + attention of the oracle for queries at `positions` until
    its time budget is spent.  Input generation (the Q/K/V rows a query reads)
    is not timed.  Returns (queries done, seconds in the oracle)."""
    from threadpoolctl import threadpool_limits

    import lsa_synth as S
    from oracle import lsa_oracle as O
    w, cache, Y = _CPU["w"], _CPU["cache"], _CPU["Y"]
    n, busy, t_start = 0, 0.0, time.perf_counter()
    with threadpool_limits(limits=1):
        for p in positions:
            q, _ = S.normal_rows(w, "q", np.array([p]), w.Hq * w.D)
            t1 = time.perf_counter()
            r = O.index_query(Y[p - w.q_start], int(p), cache)
            t2 = time.perf_counter()
            sel = r.idx[:r.count]
            k, _ = S.normal_rows(w, "k", sel, w.Hkv * w.D)
            v, _ = S.normal_rows(w, "v", sel, w.Hkv * w.D)
            t3 = time.perf_counter()
            O.attention_query(q.reshape(w.Hq, w.D), k.reshape(-1, w.Hkv, w.D),
                              v.reshape(-1, w.Hkv, w.D), np.arange(len(sel)), len(sel))
            busy += (t2 - t1) + (time.perf_counter() - t3)
            n += 1
            if time.perf_counter() - t_start > _CPU["budget"]:
                break
    return n, busy


def cpu_baseline(w, X, Y, budget_s: float):
    """The CPU oracle (plain fp64 NumPy, not tuned) on the host's cores: one
    forked worker process per core, one BLAS thread each.  The bucket-cache
    build over every block is split across the workers (wall time of the
    slowest); index + attention runs on evenly spaced queries, each worker
    stopping when its time budget is spent; the query rate is the sum of the
    workers' rates.  The step is extrapolated to all Tq queries."""
    import multiprocessing as mp

    from oracle import lsa_oracle as O
    cores = len(os.sched_getaffinity(0))
    prm = O.Params(k=w.k, n_sink=w.n_sink, window=w.window, index_dtype=w.dtype)
    nb_total = w.T // 512
    _CPU.update(X=X, prm=prm)
    ctx = mp.get_context("fork")
    chunks = [c for c in np.array_split(np.arange(nb_total), cores) if len(c)]
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pool.map(_cpu_build, [c.tolist() for c in chunks])
    t_build = time.perf_counter() - t0
    cache = O.build_cache(X, prm)          # the same cache, for the query workers (not timed)
    positions = np.unique(np.linspace(w.q_start, w.T - 1, min(w.Tq, 2048 * cores)).astype(np.int64))
    np.random.default_rng(0).shuffle(positions)
    _CPU.update(w=w, cache=cache, Y=Y, budget=budget_s)
    with ctx.Pool(cores) as pool:
        parts = pool.map(_cpu_queries, [positions[i::cores] for i in range(cores)])
    _CPU.clear()
    n_q = sum(n for n, _ in parts)
    rate = sum(n / b for n, b in parts if b > 0)       # queries per second, all workers
    t_step = t_build + w.Tq / rate
    return dict(value=w.Tq / t_step, unit="query tok/s", cores=cores, kind="oracle",
                sample=f"bucket-cache build over all {nb_total} blocks timed in full "
                       f"({t_build:.2f} s on {cores} worker processes); index + attention "
                       f"timed for {n_q} evenly spaced queries ({rate:.1f} queries/s over all "
                       f"workers, input generation excluded) and scaled to {w.Tq} queries; "
                       f"{cores} processes x 1 BLAS thread")


def attention_kernel_name(lsa, w, B: int, Tmax: int, prefill: bool = False) -> str:
    """The attention kernel (template instance) that lsa_sparse_attention runs;
    with prefill, the two kernels that lsa_sparse_attention_prefill runs per
    launch of up to lsa_attention_launch_rows() rows (the near set's dense
    tiles, then the far entries' gather; in the one-workgroup-per-row layout
    the gather takes the near keys too, and runs alone)."""
    if w.dtype != "bf16":
        return "k_attn_f32"
    nw = 1
    if w.Hkv != 4:
        far = "k_attn_bf16<1, 0" + (", true>" if prefill else ">")
    else:
        nw = 1 if lsa.attention_head_major(B, Tmax, w.Hkv, w.D, lsa.LSA_BF16) else 4
        far = f"k_attn_bf16<{nw}, 4" + (", true>" if prefill else ">")
    return f"k_near_attn<{w.Hq // w.Hkv}> + {far}" if prefill and nw == 1 else far


def measured_traffic(kernel: str, workload: str, rows_per_launch: int, root: str | None = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none, it was taken on another kernel, the kernel source
    changed since, or its launches covered another number of query rows.
    A summary of several kernels (a launch of the prefill attention runs the
    near-set kernel and the gather) lists their sources, comma separated,
    and hashes them concatenated."""
    import hashlib
    root = root or os.path.dirname(os.path.abspath(__file__))
    stem = kernel.split("<")[0] if "+" not in kernel else "attention_prefill"
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
        src = b"".join(open(os.path.join(root, f.strip()), "rb").read()
                       for f in fields["kernel_source"].split(","))
        if hashlib.sha256(src).hexdigest()[:16] != fields["kernel_source_sha256_16"]:
            return None
        if int(fields["rows_per_launch"]) != rows_per_launch:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def attention_roofline(lsa, torch, w, idx, cnt, L: int, t_attn_ms: float, kname: str,
                       workload: str) -> dict:
    """Roofline of the attention kernel, per launch (averaged over the step's
    launches of up to lsa_attention_launch_rows() query rows).

    Algorithmic work of a launch: 4 * head_dim FLOP per (query head, listed
    key) -- q.k and p.v, a multiply-add counted as 2 -- and its compulsory
    bytes: the K and V rows (all KV heads) of the distinct keys that its rows
    list, plus Q, O, the lists and counts.  Its intensity (FLOP per compulsory
    byte) against the ridge of the two peaks decides which roof binds: above
    it the MFMA roof (achieved = FLOP / time), below it the HBM roof
    (achieved = compulsory bytes / time).  The logical gather (every listed
    row's bytes, cache hits included) is reported beside it; where the caches
    serve the gather, its rate can exceed HBM peak and is not a roofline
    fraction.  `traffic` is the counter-measured bytes that cross the L2 per
    launch when the committed counter summary matches this kernel.

    The roof that binds: the gather's rows reach the CUs from L2, the
    Infinity Cache or HBM, and only the bytes that leave the L2 load the
    memory side.  When the counters match this kernel, `achieved` is those
    bytes per launch over the launch time against HBM peak (basis
    "traffic"); otherwise the compulsory bytes are used (basis
    "compulsory").  Both rates, and the MFMA share, are reported beside it."""
    esz = 2 if w.dtype == "bf16" else 4
    Tq = idx.shape[0]
    launch_rows = min(lsa.attention_launch_rows(), Tq) if w.dtype == "bf16" else Tq
    launches = -(-Tq // launch_rows)
    t_launch = t_attn_ms / launches
    cnt64 = cnt.to(torch.int64).clamp(min=0, max=L)
    total_rows = int(cnt64.sum().item())
    flop = total_rows * w.Hq * 4 * w.D
    row_bytes = w.Hkv * w.D * esz * 2
    col = torch.arange(L, device=idx.device)[None, :]
    uniq = 0
    for r0 in range(0, Tq, launch_rows):
        r1 = min(Tq, r0 + launch_rows)
        sub = idx[r0:r1]
        uniq += int(torch.unique(sub[col < cnt64[r0:r1, None]]).numel())
    fixed = 2 * Tq * w.Hq * w.D * esz + Tq * L * 4 + Tq * 4
    compulsory = uniq * row_bytes + fixed
    logical = total_rows * row_bytes + fixed
    intensity = flop / compulsory
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    sec = t_launch * 1e-3
    traffic = measured_traffic(kname, workload, launch_rows)
    mfma_tflops = flop / launches / sec / 1e12
    compulsory_gbs = compulsory / launches / sec / 1e9
    if traffic is not None:
        achieved, peak, unit, bound, basis = traffic / sec / 1e9, HBM_PEAK_GBS, "GB/s", "hbm", "traffic"
    elif intensity >= ridge:
        achieved, peak, unit, bound, basis = mfma_tflops, mfma_peak, "TFLOP/s", "mfma", "flop"
    else:
        achieved, peak, unit, bound, basis = compulsory_gbs, HBM_PEAK_GBS, "GB/s", "hbm", "compulsory"
    roof = dict(bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit,
                frac=round(achieved / peak, 4), traffic=None if traffic is None else round(traffic),
                basis=basis, kernel=kname, launches_per_step=launches,
                kernel_ms=round(float(t_launch), 4),
                algorithmic_flop=round(flop / launches),
                mfma_tflops=round(mfma_tflops, 1), mfma_frac=round(mfma_tflops / mfma_peak, 4),
                compulsory_bytes=round(compulsory / launches),
                compulsory_gbs=round(compulsory_gbs, 1),
                compulsory_frac=round(compulsory_gbs / HBM_PEAK_GBS, 4),
                intensity_flop_per_byte=round(intensity, 1), ridge_flop_per_byte=round(ridge, 1),
                logical_bytes=round(logical / launches),
                logical_gbs=round(logical / launches / sec / 1e9, 1))
    return roof


def run_decode(w, dev, mode_name: str, splits: int = 0, batch: int | None = None) -> dict:
    """Batched decode: every sequence holds T cached tokens; each step appends one
    key per sequence (clustering a block when it fills), builds the index lists
    and runs split attention.  512 consecutive steps: 511 steady steps and one
    block-completing step; the first 8 are warm-up."""
    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa
    B = batch or w.batch
    T, n_steps = w.T, 512
    Tmax = T + n_steps
    mode = lsa.LSA_TREE if mode_name == "tree" else lsa.LSA_FLAT
    p = lsa.Params(k=w.k, n_sink=w.n_sink, window=w.window, mode=mode, beam=w.beam)
    L = lsa.list_len(p)
    if splits <= 0:
        splits = lsa.attention_default_splits(B, L)
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
    wsa = torch.empty(max(lsa.lib().lsa_attention_workspace_bytes(B, 1, w.Hq, w.D, splits), 1),
                      dtype=torch.uint8, device=dev)
    out = torch.empty((B, 1, w.Hq, w.D), dtype=tdt, device=dev)
    status_off = lsa.lib().lsa_index_status_offset(__import__("ctypes").byref(p.c()), B)
    status = ws[status_off:status_off + 4 * B].view(torch.int32)
    fallbacks = torch.zeros((), dtype=torch.int64, device=dev)
    rows_listed = torch.zeros((), dtype=torch.int64, device=dev)
    # the bookkeeping reductions run once here, so that loading their kernels
    # (done on first use) falls before the first timed step, not inside it
    fallbacks += status.sum()
    rows_listed += cnt.sum()
    fallbacks.zero_()
    rows_listed.zero_()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []
    # a full collection of Python's garbage collector takes tens of ms with
    # torch loaded; host-bound steps of ~100 us would time it as GPU work
    gc.collect()
    gc.disable()
    for s_ in range(n_steps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        lsa.index_decode(caches, qn[s_], kn[s_], p, workspace=ws, out=(idx, cnt))
        e1.record()
        lsa.sparse_attention(Qd[s_], Kc, Vc, idx.view(B, 1, L), cnt.view(B, 1), splits=splits,
                             out=out, workspace=wsa)
        e2.record()
        marks.append((e0, e1, e2))
        if s_ >= 8:      # outside the timed interval of the steps
            fallbacks += status.sum()
            rows_listed += cnt.sum()
    torch.cuda.synchronize()
    gc.enable()
    tim = np.array([[a.elapsed_time(b_), b_.elapsed_time(c_)] for a, b_, c_ in marks]) * 1e3
    fire = [i for i in range(n_steps) if (T + i + 1) % 512 == 0]
    steady = [i for i in range(8, n_steps) if i not in fire]
    st = tim[steady]
    tot = st.sum(axis=1)
    tot_steady = float(np.median(tot))
    idx_us = float(np.median(st[:, 0]))
    # roofline of the indexing stage (the dominant one): its algorithmic bytes
    # are the eligible buckets' centroids (the HBM stream every query scores;
    # 128 B each in bf16, a member word of 4 B for each kept bucket aside)
    elig = T // 512 * 64          # eligible buckets of a steady step's query
    cent_bytes = B * elig * 64 * 2
    kv_bytes = float(rows_listed.item()) / len(steady) * w.Hkv * w.D * 2 * 2
    achieved = cent_bytes / (idx_us * 1e-6) / 1e9
    name = w.name if w.cfg == 3 else "decode_t10m_b1_bf16_flat"
    res = {
        "metric": f"decode us/token ({mode_name})", "value": round(tot_steady, 2), "unit": "us/token",
        "n_gpus": 1, "steps": len(steady), "warmup": 8, "ms_per_step": round(tot_steady / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_name(name, mode_name), "T": T,
                   "batch": B, "k": w.k, "mode": mode_name, "attention_splits": splits,
                   "parallelism": "none"},
        "step_us": {"median": round(tot_steady, 2), "p99": round(float(np.percentile(tot, 99)), 2),
                    "max": round(float(tot.max()), 2), "max_at_step": int(steady[int(tot.argmax())]),
                    "completing_steps": fire},
        "stages_us": {"index_decode": round(idx_us, 2),
                      "attention": round(float(np.median(st[:, 1])), 2)},
        "firing_step_us": {"index_decode": round(float(tim[fire[0], 0]), 2),
                           "attention": round(float(tim[fire[0], 1]), 2)} if fire else None,
        "per_sequence_step_us": round(tot_steady / B, 3),
        "exact_fallbacks": {"queries": int(fallbacks.item()), "of": B * (n_steps - 8)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "lsa_index_decode (all launches of the indexing stage)",
                     "algorithmic_bytes": cent_bytes, "kernel_ms": round(idx_us / 1e3, 5),
                     "attention_gather_bytes": round(kv_bytes),
                     "attention_gather_gbs": round(kv_bytes / (float(np.median(st[:, 1])) * 1e-6)
                                                   / 1e9, 1)},
    }
    return res


def bench_decode(args, w, dev):
    res = run_decode(w, dev, args.mode, args.splits, w.batch if args.cfg == 3 else 1)
    print(json.dumps(res), flush=True)


def bench_tree_sweep(args, w, dev):
    """Tree beam search against flat search on the workload's last chunk.  For
    beam widths 8..64 and leaf levels from the default (the smallest level
    where beam * 2^level reaches the B buckets to keep) upward -- stopping the
    beam higher up and ranking every bucket under it flat, the two-stage search
    -- the chunk's index time (HIP events, best of three) and each query's
    far-key recall: the share of its exact flat list's far keys (outside the
    sinks and the window) that the tree list also holds.  Then beams of 128,
    256 and 512, and beam 64 with a fixed-level first stage (start level =
    the leaf level, +2, +4), each at its default leaf level."""
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
    # wider beams (one workgroup per query) at their default leaf level, and
    # beam 64 with a fixed-level first stage: every node of level `start`
    # scored, the best 64 kept, then the descent (start = leaf level: the
    # two-stage search)
    wide = []
    for beam, start in ((128, -1), (256, -1), (512, -1), (64, 0), (64, 2), (64, 4)):
        p0 = lsa.Params(mode=lsa.LSA_TREE, beam=beam, **base)
        l0 = 0
        while beam << l0 < lsa.top_buckets(p0):
            l0 += 1
        st = -1 if start < 0 else l0 + start
        p = lsa.Params(mode=lsa.LSA_TREE, beam=beam, start_level=st, **base)
        if lsa.lib().lsa_check_params(ctypes.byref(p.c())) != 0:
            continue
        ms, (tidx, _) = run(p)
        trow, tkey, _ = far_keys(tidx)
        hit = torch.isin(tkey, fkey)
        hits = torch.bincount(trow[hit], minlength=w.Tq).to(torch.float64)
        rec = (hits / fcount.clamp(min=1).to(torch.float64))[fcount > 0]
        wide.append(dict(beam=beam, leaf_level=l0, start_level=st, index_ms=round(ms, 4),
                         recall_mean=round(rec.mean().item(), 4),
                         recall_p10=round(torch.quantile(rec, 0.1).item(), 4)))
        log(f"beam {beam:3d} start {st:2d}: index {ms:7.3f} ms, recall {wide[-1]['recall_mean']:.3f}")
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
        "wide_and_fixed_level": wide,
    }
    print(json.dumps(res), flush=True)


def bench_whole_context(args, w, dev):
    """The whole context prefilled in chunks of w.Tq queries, aligned so that the
    last chunk is the workload's measured final chunk (the first one is shorter).
    Per chunk: build_bucket_cache appends the chunk's latent keys (clustering the
    blocks that fill up, rebuilding the tree's right edge in tree mode), then
    lsa_index_prefill indexes the chunk's queries and
    lsa_sparse_attention_prefill attends over their lists (the near set dense
    per tile of rows, the far entries gathered).  K and V hold all T tokens; Q and the output are
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
    ws_attn = torch.empty(lsa.lib().lsa_prefill_attention_workspace_bytes(1, C, w.Hq, w.D),
                          dtype=torch.uint8, device=dev)

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
    lsa.sparse_attention_prefill(Q[:first], K, V, idx[:first], cnt[:first], 0, p, out=out[:first],
                                 workspace=ws_attn)
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
        lsa.sparse_attention_prefill(Q[:n], K, V, idx[:n], cnt[:n], s0, p, out=out[:n],
                                     workspace=ws_attn)
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


SCAN_NAMES = {1: "token_scan", 4: "block4_scan", 8: "block8_scan"}


def run_prefill(w, dev, mode_name: str, steps: int, warmup: int, calib_copy: bool = False,
                cpu_seconds: float = 0.0, scan_keys: int = 0) -> dict:
    """One prefill step = build_bucket_cache over all T keys (full-context
    workloads) + lsa_index_prefill for all Tq queries + lsa_sparse_attention
    over their lists; last-chunk workloads build the cache of every full
    block once before timing and time index + attention.  Inputs are resident
    in HBM before the timed region; stage times come from HIP events on the
    stream the launches run on."""
    import ctypes

    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa

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
    log(f"{w.name}: inputs ready in {time.perf_counter() - t_gen:.1f}s")

    mode = lsa.LSA_TREE if mode_name == "tree" else lsa.LSA_FLAT
    p = lsa.Params(k=w.k, n_sink=w.n_sink, window=w.window, mode=mode, beam=w.beam,
                   index_dtype=lsa.LSA_BF16 if w.dtype == "bf16" else lsa.LSA_F32,
                   scan_keys=scan_keys)
    if scan_keys:
        mode_name = SCAN_NAMES[scan_keys]
    L = lsa.list_len(p)
    nbytes = lsa.lib().lsa_cache_bytes(ctypes.byref(p.c()), w.T)
    cache_mem = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    idx = torch.empty((w.Tq, L), dtype=torch.int32, device=dev)
    cnt = torch.empty((w.Tq,), dtype=torch.int32, device=dev)
    ws = torch.empty(lsa.index_workspace_bytes(p, w.Tq), dtype=torch.uint8, device=dev)
    out = torch.empty_like(Q)
    # bf16 lists of the method (and of the scans) hold the sinks and the
    # window: the prefill attention takes that near set dense per tile of rows
    prefill_attn = w.dtype == "bf16"
    ws_attn = torch.empty(max(lsa.lib().lsa_prefill_attention_workspace_bytes(1, w.Tq, w.Hq, w.D), 1),
                          dtype=torch.uint8, device=dev) if prefill_attn else None

    def fresh_cache():   # a cache over the same device memory, every step
        c = lsa.BucketCache.__new__(lsa.BucketCache)
        c.params, c.mem = p, cache_mem
        h = ctypes.c_void_p()
        lsa._check("lsa_cache_init", lsa.lib().lsa_cache_init(
            ctypes.byref(p.c()), w.T, lsa._ptr(cache_mem), nbytes, ctypes.byref(h)))
        c.handle = h
        return c

    ev = lambda: torch.cuda.Event(enable_timing=True)
    full_prefill = w.q_start == 0
    prebuilt = None
    build_once_ms = None
    if not full_prefill:
        # last prefill chunk of a long context: the cache of every full block
        # exists before the chunk; building it is timed once, separately
        prebuilt = fresh_cache()
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
            c = fresh_cache()
            e0.record()
            c.build(Xd)
        else:
            c = prebuilt
            e0.record()
        e1.record()
        lsa.index_prefill(c, Yd, w.q_start, p, workspace=ws, out=(idx, cnt))
        e2.record()
        if prefill_attn:
            lsa.sparse_attention_prefill(Q, K, V, idx, cnt, w.q_start, p, out=out, workspace=ws_attn)
        else:
            lsa.sparse_attention(Q, K, V, idx, cnt, out=out)
        e3.record()
        if times is not None:
            times.append((e0, e1, e2, e3))
        return c

    if calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(times)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    stage = np.array([[a.elapsed_time(b), b.elapsed_time(c), c.elapsed_time(d)]
                      for a, b, c, d in times])
    t_build, t_index, t_attn = stage.mean(axis=0)
    log(f"per step: build {t_build:.3f} ms, index {t_index:.3f} ms, attention {t_attn:.3f} ms; "
        f"wall {ms_step:.3f} ms")
    fallbacks = lsa.exact_fallbacks(p, w.Tq, ws)
    # flat scoring: 2 * 64 FLOP per eligible (query, bucket) pair; a scan
    # scores the runs of b keys that end before the window
    pos = np.arange(w.q_start, w.T, dtype=np.int64)
    if scan_keys:
        pairs = int((np.maximum(pos - w.window + 1, 0) // scan_keys).sum())
    else:
        pairs = int((64 * (pos // 512)).sum())
    kname = attention_kernel_name(lsa, w, 1, w.T, prefill_attn)
    wname = workload_name(w.name, mode_name)
    if not wname.endswith("_" + mode_name):
        wname += "_" + mode_name
    roofline = attention_roofline(lsa, torch, w, idx, cnt, L, float(t_attn), kname, wname)
    res = {
        "metric": f"prefill query tok/s per layer ({mode_name.replace('_', ' ')})",
        "value": round(w.Tq / (ms_step * 1e-3), 1),
        "unit": "query tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": wname, "T": w.T, "Tq": w.Tq, "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.D, "k": w.k, "mode": mode_name, "n_sink": w.n_sink,
                   "window": w.window, "latent_components": w.n_comp, "parallelism": "none"},
        "stages_ms": {"build": round(float(t_build), 4), "index": round(float(t_index), 4),
                      "attention": round(float(t_attn), 4)},
        "step": ("build + index + attention" if full_prefill else
                 "index + attention for the last chunk (cache built before timing)"),
        "exact_fallbacks": {"queries": fallbacks, "of": w.Tq},
        "scoring": {"pairs": pairs, "algorithmic_tflop": round(pairs * 128 / 1e12, 4)},
        "roofline": roofline,
    }
    if build_once_ms is not None:
        res["cache_build_ms"] = round(build_once_ms, 3)
    del Q, K, V, Xd, Yd, cache_mem, idx, cnt, ws, out, prebuilt, ws_attn
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        log("timing the CPU oracle on a sample ...")
        cb = cpu_baseline(w, X, Y, cpu_seconds)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    return res


def bench_baselines(args, w, dev):
    """LSA's flat search next to the in-repo baselines on the same workload:
    the token scan and the block scans over runs of 4 and 8 keys (same
    expansion, sinks, window and attention).  Prints one JSON line: LSA's
    step, and each baseline's step, index and attention times with its ratio
    to LSA's."""
    runs = {"lsa_flat": run_prefill(w, dev, "flat", args.steps, args.warmup)}
    for b in (1, 4, 8):
        runs[SCAN_NAMES[b]] = run_prefill(w, dev, "flat", args.steps, args.warmup, scan_keys=b)
    lsa_r = runs["lsa_flat"]
    res = {k: v for k, v in lsa_r.items() if k not in ("cpu_baseline",)}
    res["baselines"] = {}
    for name, r in runs.items():
        st = r["stages_ms"]
        res["baselines"][name] = {
            "ms_per_step": r["ms_per_step"], "stages_ms": st,
            "index_vs_lsa": round(st["index"] / lsa_r["stages_ms"]["index"], 3),
            "step_vs_lsa": round(r["ms_per_step"] / lsa_r["ms_per_step"], 3),
            "scores_per_step": r["scoring"]["pairs"],
            "exact_fallbacks": r["exact_fallbacks"]}
    d = run_dense(w, dev)
    d["step_vs_lsa"] = round(d["ms_per_step"] / lsa_r["ms_per_step"], 3)
    res["baselines"]["dense_causal_attention"] = d
    print(json.dumps(res), flush=True)


def run_dense(w, dev) -> dict:
    """Dense causal attention (every query attends to every key up to its
    position) over the workload's query rows: all of them up to 8,192 rows,
    else the last 2,048 rows of the chunk, scaled by the rows' share of the
    chunk's key count (each row's work is proportional to its position)."""
    import torch

    import lsa_synth as S
    import sparse_attention_indexing_amd as lsa
    rows = w.Tq if w.Tq <= 8192 else 2048
    r0 = w.Tq - rows
    Q = torch.empty((rows, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    K = torch.empty((w.T, w.Hkv, w.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    cs = torch.cuda.current_stream().cuda_stream
    for t, name, off in ((Q, "q", (w.q_start + r0) * w.Hq * w.D), (K, "k", 0), (V, "v", 0)):
        S.device_fill_normal(t.data_ptr(), t.numel(), S.philox_key(w.cfg, name), off, True, cs)
    out = torch.empty_like(Q)
    lsa.dense_attention(Q[: min(rows, 64)], K, V, w.q_start + r0, out=out[: min(rows, 64)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    lsa.dense_attention(Q, K, V, w.q_start + r0, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    pos = np.arange(w.q_start, w.T, dtype=np.float64)
    keys_all = float((pos + 1).sum())
    keys_run = float((pos[r0:] + 1).sum())
    flop = keys_run * w.Hq * 4 * w.D
    ms_all = ms * keys_all / keys_run
    del Q, K, V, out
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms_all, 3), "measured_rows": rows, "measured_ms": round(ms, 3),
            "scaled": rows != w.Tq,
            "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def _extra_summary(r: dict) -> dict:
    keep = ("metric", "value", "unit", "ms_per_step", "step_us", "stages_ms", "stages_us",
            "firing_step_us", "cache_build_ms", "exact_fallbacks", "roofline", "config",
            "per_sequence_step_us", "step")
    return {k: r[k] for k in keep if k in r}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    import lsa_synth as S

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
    if args.baselines:
        return bench_baselines(args, w, dev)
    headline = args.cfg == 2 and args.mode == "flat" and not args.no_extra and not args.scan
    res = run_prefill(w, dev, args.mode, args.steps, args.warmup, args.calib_copy,
                      0.0 if args.no_cpu_baseline or w.T > 1 << 17 or args.scan
                      else args.cpu_seconds, scan_keys=args.scan)
    if headline:
        # the metric's other ends, on the same GPU in the same run: the 10M
        # last prefill chunk (flat), one step of the 16 x 1M decode batch and
        # one step of a single 10M-token sequence's decode
        res["extra"] = {}
        r10 = run_prefill(S.WORKLOADS[5], dev, "flat", min(args.steps, 3), 1)
        res["extra"][r10["config"]["workload"]] = _extra_summary(r10)
        torch.cuda.empty_cache()
        rdec = run_decode(S.WORKLOADS[3], dev, "flat")
        res["extra"][rdec["config"]["workload"]] = _extra_summary(rdec)
        torch.cuda.empty_cache()
        rdec10 = run_decode(S.WORKLOADS[5], dev, "flat", batch=1)
        res["extra"][rdec10["config"]["workload"]] = _extra_summary(rdec10)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
