"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle builds every block (in forked worker processes)
and recomputes sampled queries one by one; Q/K/V rows it needs come from the
host generator while the GPU gets the same tensors from the device generator."""
import sys
import time

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from parity_util import (FB, attention_from_rows, cache_to_host, compare_cache, compare_lists,
                         compare_tree, device_normal, gpu_cache, host_rows,
                         oracle_cache_parallel, oracle_params, oracle_tree_parallel)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()


def _attn_check(w, q_dev_rows, out, idx, cnt, rows, seq=0, label=""):
    err = 0.0
    for i, r in enumerate(rows):
        ref = attention_from_rows(w, q_dev_rows[i], idx[r], int(cnt[r]), seq)
        err = max(err, float(np.abs(out[r].astype(np.float64) - ref).max()))
    say(f"{label} attention max abs err {err:.3g} over {len(rows)} queries")
    assert err <= 2e-2


def test_prefill_128k_full_size():
    say("case: prefill T=131072 flat (benchmark workload)")
    w = S.WORKLOADS[2]
    X, Y, _ = S.latent_inputs(w)
    p = lsa.Params(k=w.k)
    c = gpu_cache(X, p)
    Yd = torch.from_numpy(Y).cuda()
    idx, cnt = lsa.index_prefill(c, Yd, w.q_start, p, stats=FB)
    Q = device_normal(w, "q", (w.Tq, w.Hq, w.D))
    K = device_normal(w, "k", (w.T, w.Hkv, w.D))
    V = device_normal(w, "v", (w.T, w.Hkv, w.D))
    # the benchmark's layout at this size: one workgroup per (row, KV head)
    assert lsa.attention_head_major(1, w.T, w.Hkv, w.D, lsa.LSA_BF16)
    out = lsa.sparse_attention(Q, K, V, idx, cnt)
    # the benchmark's attention: the near set dense per tile of 16 rows, the
    # far entries gathered per row
    out_p = lsa.sparse_attention_prefill(Q, K, V, idx, cnt, w.q_start, p)
    torch.cuda.synchronize()
    d = float((out_p.float() - out.float()).abs().max().item())
    say(f"prefill attention vs lsa_sparse_attention over all {w.Tq} rows: max abs diff {d:.3g}")
    assert d <= 1e-2
    oc = oracle_cache_parallel(X, oracle_params(p))
    say("build", compare_cache(cache_to_host(c), oc, X))
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    rows = np.unique(np.concatenate([np.linspace(0, w.Tq - 1, 96).astype(int), np.arange(w.Tq - 16, w.Tq)]))
    say("index", compare_lists(idx_h[rows], cnt_h[rows], rows, Y[rows], oc))
    arows = rows[::8]
    q_rows = host_rows(w, "q", arows, w.Hq * w.D)
    _attn_check(w, q_rows, out.float().cpu().numpy(), idx_h, cnt_h, arows, label="prefill 128K")
    # every list holds its near set once, so near_union reorders it: the
    # oracle attention over the list is the prefill attention's reference
    for r in arows:
        assert sorted(O.near_union(idx_h[r], int(cnt_h[r]), w.q_start + int(r), oracle_params(p),
                                   w.T).tolist()) == sorted(idx_h[r, :cnt_h[r]].tolist())
    _attn_check(w, q_rows, out_p.float().cpu().numpy(), idx_h, cnt_h, arows,
                label="prefill 128K (near + far)")


def test_prefill_1m_tree_and_flat():
    say("case: T=1M last 8192 queries, tree (beam 64) and flat")
    w = S.WORKLOADS[4]
    X, Y, _ = S.latent_inputs(w)
    pt = lsa.Params(k=w.k, mode=lsa.LSA_TREE, beam=w.beam)
    pf = lsa.Params(k=w.k, mode=lsa.LSA_FLAT)
    c = gpu_cache(X, pt)
    Yd = torch.from_numpy(Y).cuda()
    it, ct = lsa.index_prefill(c, Yd, w.q_start, pt, stats=FB)
    i_f, c_f = lsa.index_prefill(c, Yd, w.q_start, pf, stats=FB)
    torch.cuda.synchronize()
    t0 = time.time()
    oc = oracle_cache_parallel(X, oracle_params(pt))
    g = cache_to_host(c)
    say("build", compare_cache(g, oc, X), f"{time.time() - t0:.1f}s")
    ot = O.build_tree(oc)
    assert len(g["levels"]) == ot.height == 17
    # the seeded inputs have no near-tie pairing: every level is compared
    assert compare_tree(g, ot, 1e-12, "T=1M") == ot.height
    rows = np.linspace(0, w.Tq - 1, 24).astype(int)
    it_h, ct_h, if_h, cf_h = it.cpu().numpy(), ct.cpu().numpy(), i_f.cpu().numpy(), c_f.cpu().numpy()
    say("tree index", compare_lists(it_h[rows], ct_h[rows], w.q_start + rows, Y[rows], oc, "tree", ot))
    say("flat index", compare_lists(if_h[rows], cf_h[rows], w.q_start + rows, Y[rows], oc))
    # tree vs flat: share of the flat far keys the tree also finds (all queries)
    near = 4 + 512
    rec = []
    for r in range(0, w.Tq, 64):
        a = set(if_h[r, :cf_h[r]].tolist())
        b = set(it_h[r, :ct_h[r]].tolist())
        rec.append((len(a & b) - near) / max(1, len(a) - near))
    say(f"tree/flat far-key recall: mean {np.mean(rec):.3f} min {np.min(rec):.3f}")
    # wider beams and the fixed-level search (a flat first stage over a
    # coarse level): lists against the oracle, recall against flat search
    for beam, start in ((256, -1), (64, 6), (64, 4)):
        pv = lsa.Params(k=w.k, mode=lsa.LSA_TREE, beam=beam, start_level=start)
        iv, cv = lsa.index_prefill(c, Yd, w.q_start, pv, stats=FB)
        torch.cuda.synchronize()
        iv_h, cv_h = iv.cpu().numpy(), cv.cpu().numpy()
        oc_v = O.BucketCache(oracle_params(pv), oc.n_blocks, oc.centroids, oc.members, oc.pooled,
                             oc.block_min_gap, oc.block_ess)
        say(f"beam {beam} start level {start}",
            compare_lists(iv_h[rows], cv_h[rows], w.q_start + rows, Y[rows], oc_v, "tree", ot))
        rec = []
        for r in range(0, w.Tq, 64):
            a = set(if_h[r, :cf_h[r]].tolist())
            b = set(iv_h[r, :cv_h[r]].tolist())
            rec.append((len(a & b) - near) / max(1, len(a) - near))
        say(f"beam {beam} start level {start}: far-key recall vs flat {np.mean(rec):.3f}")


def _completed_block(gpu_cache_obj, X, b, p):
    """The block `b` that a decode step completed matches the oracle's clustering."""
    g = cache_to_host(gpu_cache_obj)
    assert g["n_blocks"] == b + 1
    sub = O.build_cache(X[b * 512:(b + 1) * 512], oracle_params(p))
    gl = dict(n_blocks=1, cent=g["cent"][b * 64:(b + 1) * 64], pooled=g["pooled"][b * 64:(b + 1) * 64])
    compare_cache(gl, sub, X[b * 512:(b + 1) * 512])
    return g


def test_decode_1m_16_sequences():
    """One step of the 16-sequence decode workload (its launch shapes): 16
    caches of 1,048,576 tokens, sequences 0 and 9 one key short of a full block
    (their new key completes it and the block is clustered in the step), the
    others steady.  Every sequence's list against the oracle over its own
    cache, every sequence's split attention against the oracle."""
    say("case: decode T=1M x 16 sequences, two block-completing")
    w = S.WORKLOADS[3]
    B = w.batch
    lens = [w.T - 1 if b in (0, 9) else w.T for b in range(B)]
    p = lsa.Params(k=w.k)
    caches, keys, qs, Xs = [], [], [], []
    for b, n in enumerate(lens):
        X, Y, _ = S.latent_inputs(w, seq=b, T=n + 1, query_rows=(n, n + 1))
        caches.append(gpu_cache(X[:n], p, max_tokens=n + 1))
        keys.append(X[n])
        qs.append(Y[0])
        Xs.append(X)
    st = {}
    idx, cnt = lsa.index_decode(caches, torch.from_numpy(np.stack(qs)).cuda(),
                                torch.from_numpy(np.stack(keys)).cuda(), p, stats=st)
    say(f"exact fallbacks: {st['exact_fallbacks']} of {B}")
    Tmax = w.T + 1
    K = torch.stack([device_normal(w, "k", (Tmax, w.Hkv, w.D), seq=b) for b in range(B)])
    V = torch.stack([device_normal(w, "v", (Tmax, w.Hkv, w.D), seq=b) for b in range(B)])
    Q = torch.stack([device_normal(w, "q", (1, w.Hq, w.D), seq=b, row0=n) for b, n in enumerate(lens)])
    splits = lsa.attention_default_splits(B, idx.shape[1])
    out = lsa.sparse_attention(Q, K, V, idx.view(B, 1, -1), cnt.view(B, 1), splits=splits)
    torch.cuda.synchronize()
    del K, V
    idx_h, cnt_h, out_h = idx.cpu().numpy(), cnt.cpu().numpy(), out.float().cpu().numpy()
    err = 0.0
    for b, n in enumerate(lens):
        oc = oracle_cache_parallel(Xs[b][:n + 1], oracle_params(p))
        say(f"seq {b} (p={n})", compare_lists(idx_h[b:b + 1], cnt_h[b:b + 1], [n], qs[b][None], oc))
        if n % 512 == 511:
            _completed_block(caches[b], Xs[b], n // 512, p)
        qrow = host_rows(w, "q", [n], w.Hq * w.D, seq=b)[0]
        ref = attention_from_rows(w, qrow, idx_h[b], int(cnt_h[b]), seq=b)
        err = max(err, float(np.abs(out_h[b, 0] - ref).max()))
        Xs[b] = None
    say(f"decode attention ({splits} splits) max abs err {err:.3g} over {B} sequences")
    assert err <= 2e-2


# ---------------------------------------------------------------- 10M tokens

T_FIRE = 19530 * 512 + 511     # a 10M-scale decode position whose key completes block 19,530


@pytest.fixture(scope="module")
def ctx10m():
    """The 10,000,000-token workload: latent keys up to position 10M (the
    decode step's key included), the prefill chunk's queries and the decode
    queries; a tree-mode GPU cache over the first 10M keys; the oracle's
    cache and tree over the 19,531 full blocks (which every step below sees)."""
    w = S.WORKLOADS[5]
    t0 = time.time()
    X, Y, _ = S.latent_inputs(w, T=w.T + 1, query_rows=(w.q_start, w.T + 1))
    yf = S.latent_inputs(w, T=T_FIRE + 1, query_rows=(T_FIRE, T_FIRE + 1))[1][0]
    say(f"10M inputs {time.time() - t0:.1f}s")
    pt = lsa.Params(k=w.k, mode=lsa.LSA_TREE, beam=w.beam)
    c = gpu_cache(X[:w.T], pt)
    t0 = time.time()
    oc = oracle_cache_parallel(X[:w.T + 1], oracle_params(pt))
    assert oc.n_blocks == 19531
    say(f"oracle cache {time.time() - t0:.1f}s")
    t0 = time.time()
    ot = oracle_tree_parallel(oc)
    say(f"oracle tree {time.time() - t0:.1f}s ({ot.height} levels)")
    return dict(w=w, X=X, Y=Y, yf=yf, c=c, oc=oc, ot=ot, pt=pt)


def test_prefill_10m_flat_and_tree_last_chunk(ctx10m):
    """The last 32,768-query chunk at 10M tokens, flat and tree (beam 64, 21
    levels): every block and every tree level of the cache against the oracle,
    64 sampled queries' lists in each mode, and 16 sampled queries' attention
    in each mode, in the launch configuration the benchmark times."""
    say("case: T=10M, last 32768 queries, flat and tree")
    w, X, Y, c = ctx10m["w"], ctx10m["X"], ctx10m["Y"], ctx10m["c"]
    oc, ot = ctx10m["oc"], ctx10m["ot"]
    g = cache_to_host(c)
    say("build", compare_cache(g, oc, X[:w.T]))
    assert len(g["levels"]) == ot.height == 21
    compare_tree(g, ot, 1e-12, "T=10M")
    Yd = torch.from_numpy(np.ascontiguousarray(Y[:w.Tq])).cuda()
    pf = lsa.Params(k=w.k)
    i_f, c_f = lsa.index_prefill(c, Yd, w.q_start, pf, stats=FB)
    i_t, c_t = lsa.index_prefill(c, Yd, w.q_start, ctx10m["pt"], stats=FB)
    Q = device_normal(w, "q", (w.Tq, w.Hq, w.D), row0=w.q_start)
    K = device_normal(w, "k", (w.T, w.Hkv, w.D))
    V = device_normal(w, "v", (w.T, w.Hkv, w.D))
    # the benchmark's layout at this size: one workgroup per query row
    assert not lsa.attention_head_major(1, w.T, w.Hkv, w.D, lsa.LSA_BF16)
    o_f = lsa.sparse_attention(Q, K, V, i_f, c_f)
    o_t = lsa.sparse_attention(Q, K, V, i_t, c_t)
    # the benchmark's attention (near set dense per tile, far entries gathered)
    op_f = lsa.sparse_attention_prefill(Q, K, V, i_f, c_f, w.q_start, pf)
    op_t = lsa.sparse_attention_prefill(Q, K, V, i_t, c_t, w.q_start, ctx10m["pt"])
    torch.cuda.synchronize()
    for a_, b_, m_ in ((op_f, o_f, "flat"), (op_t, o_t, "tree")):
        d = float((a_.float() - b_.float()).abs().max().item())
        say(f"10M {m_}: prefill attention vs lsa_sparse_attention, all rows: max abs diff {d:.3g}")
        assert d <= 1e-2
    # the device generator fills all 5.12e9 elements like the host rows (this
    # needs a grid-stride launch: a dispatch holds fewer than 2^32 work-items)
    for r in [0, 2097152, 8388608, w.T - 1]:
        assert np.array_equal(K[r].float().cpu().numpy().reshape(-1).astype(np.float64),
                              host_rows(w, "k", [r], w.Hkv * w.D)[0]), f"K row {r}"
    del K, V
    rows = np.unique(np.concatenate([np.linspace(0, w.Tq - 1, 60).astype(int),
                                     [w.Tq - 1, w.Tq - 2, w.Tq - 129, w.Tq - 130]]))
    arows = rows[:: max(1, len(rows) // 16)][:16]
    q_rows = host_rows(w, "q", w.q_start + arows, w.Hq * w.D)
    for mode, idx, cnt, out, out_p in (("flat", i_f, c_f, o_f, op_f), ("tree", i_t, c_t, o_t, op_t)):
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        say(f"{mode} index", compare_lists(idx_h[rows], cnt_h[rows], w.q_start + rows, Y[rows], oc,
                                          mode, ot if mode == "tree" else None, parallel=True))
        _attn_check(w, q_rows, out.float().cpu().numpy(), idx_h, cnt_h, arows,
                    label=f"prefill 10M {mode}")
        _attn_check(w, q_rows, out_p.float().cpu().numpy(), idx_h, cnt_h, arows,
                    label=f"prefill 10M {mode} (near + far)")


def test_decode_10m_flat_and_tree_steady_and_completing(ctx10m):
    """Batch-1 decode at 10M tokens in both modes: a steady step at position
    10,000,000 and a step whose key completes block 19,530 (position
    9,999,871; the block is clustered and, in tree mode, the tree's right
    edge rebuilt in the step).  Lists against the oracle; the completed block
    and, in tree mode, every tree level against the oracle's; split attention
    against the oracle."""
    say("case: decode T=10M batch 1, flat and tree, steady and block-completing")
    w, X, Y, oc, ot = ctx10m["w"], ctx10m["X"], ctx10m["Y"], ctx10m["oc"], ctx10m["ot"]
    Tmax = w.T + 1
    K = device_normal(w, "k", (Tmax, w.Hkv, w.D))
    V = device_normal(w, "v", (Tmax, w.Hkv, w.D))
    err = 0.0
    for mode in (lsa.LSA_FLAT, lsa.LSA_TREE):
        p = lsa.Params(k=w.k, mode=mode, beam=w.beam)
        for n, y in ((w.T, Y[-1]), (T_FIRE, ctx10m["yf"])):
            say(f"decode mode={mode} p={n}")
            c = gpu_cache(X[:n], p, max_tokens=n + 1)
            st = {}
            idx, cnt = lsa.index_decode([c], torch.from_numpy(y[None].copy()).cuda(),
                                        torch.from_numpy(X[n][None].copy()).cuda(), p, stats=st)
            Q = device_normal(w, "q", (1, 1, w.Hq, w.D), row0=n)
            splits = lsa.attention_default_splits(1, idx.shape[1])
            out = lsa.sparse_attention(Q, K[None], V[None], idx.view(1, 1, -1), cnt.view(1, 1),
                                       splits=splits)
            torch.cuda.synchronize()
            say(f"exact fallbacks: {st['exact_fallbacks']}; attention splits {splits}")
            idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
            say("index", compare_lists(idx_h, cnt_h, [n], y[None], oc,
                                       "tree" if mode == lsa.LSA_TREE else "flat",
                                       ot if mode == lsa.LSA_TREE else None))
            if n == T_FIRE:
                g = _completed_block(c, X, n // 512, p)
                if mode == lsa.LSA_TREE:
                    compare_tree(g, ot, 1e-12, "T=10M after the completing decode step")
            ref = attention_from_rows(w, host_rows(w, "q", [n], w.Hq * w.D)[0], idx_h[0],
                                      int(cnt_h[0]))
            err = max(err, float(np.abs(out.float().cpu().numpy()[0, 0] - ref).max()))
            del c
    say(f"decode attention max abs err {err:.3g}")
    assert err <= 2e-2
