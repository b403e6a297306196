"""GPU parity of lsa_sparse_attention_prefill (near set dense per tile of rows,
the list's other entries gathered on top) against the oracle: attention over
near_union of each row's list.  Oracle lists, random lists that break the
method's layout (missing window keys, duplicates, invalid and non-causal
entries), every GQA group size, both gather layouts, several sequences with
launch and tile boundaries inside them, negative and zero scales."""
import sys

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from parity_util import bf16_tensor, oracle_index_parallel, oracle_params

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()


def _workload(Hq, Hkv):
    return S.Workload(**{**S.WORKLOADS[2].__dict__, "Hq": Hq, "Hkv": Hkv})


def _qkv(w, B, T, q_rows):
    """Host fp64 copies and device bf16 tensors: q [B, len(q_rows), Hq, D],
    k / v [B, T, Hkv, D] (sequence b draws from generator stream b)."""
    qs, ks, vs, Qd, Kd, Vd = [], [], [], [], [], []
    for b in range(B):
        q, qb = S.normal_rows(w, "q", q_rows, w.Hq * w.D, b)
        k, kb = S.normal_rows(w, "k", np.arange(T), w.Hkv * w.D, b)
        v, vb = S.normal_rows(w, "v", np.arange(T), w.Hkv * w.D, b)
        qs.append(q.reshape(-1, w.Hq, w.D)); ks.append(k.reshape(T, w.Hkv, w.D))
        vs.append(v.reshape(T, w.Hkv, w.D))
        Qd.append(bf16_tensor(qb).view(-1, w.Hq, w.D)); Kd.append(bf16_tensor(kb).view(T, w.Hkv, w.D))
        Vd.append(bf16_tensor(vb).view(T, w.Hkv, w.D))
    return qs, ks, vs, torch.stack(Qd).cuda(), torch.stack(Kd).cuda(), torch.stack(Vd).cuda()


def _check(out, qs, ks, vs, idx, cnt, q_start, prm, rows, label, scale=None, tol=2e-2):
    """out [B, Tq, Hq, D] against the oracle over near_union of each listed row."""
    B = len(qs)
    err = 0.0
    for b in range(B):
        T = ks[b].shape[0]
        for r in rows:
            lst = O.near_union(idx[b, r], int(cnt[b, r]), q_start + int(r), prm, T)
            ref = O.attention_query(qs[b][r], ks[b], vs[b], lst, len(lst), scale)
            err = max(err, float(np.abs(out[b, r].astype(np.float64) - ref).max()))
    say(f"{label}: max abs err {err:.3g} over {B * len(rows)} rows")
    assert err <= tol


def _run(Q, K, V, idx, cnt, q_start, p, scale=None):
    out = lsa.sparse_attention_prefill(Q, K, V, torch.from_numpy(idx).cuda(),
                                       torch.from_numpy(cnt).cuda(), q_start, p, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def test_prefill_attention_on_oracle_lists_all_rows():
    """T = 8,192, every query: the oracle's own lists; the result also equals
    lsa_sparse_attention over the same lists within two bf16 roundings."""
    say("case: prefill attention, oracle lists, T=8192, all rows")
    w = S.WORKLOADS[2]
    T = 8192
    X, Y, _ = S.latent_inputs(w, T=T, query_rows=(0, T))
    p = lsa.Params(k=2048)
    prm = oracle_params(p)
    oc = O.build_cache(X, prm)
    res = oracle_index_parallel(np.arange(T), Y, oc)
    L = lsa.list_len(p)
    idx = np.full((1, T, L), -1, np.int32)
    cnt = np.zeros((1, T), np.int32)
    for r, x in enumerate(res):
        idx[0, r, :x.count] = x.idx[:x.count]
        cnt[0, r] = x.count
    qs, ks, vs, Q, K, V = _qkv(w, 1, T, np.arange(T))
    out = _run(Q, K, V, idx, cnt, 0, p)
    plain = lsa.sparse_attention(Q, K, V, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    d = float(np.abs(out - plain.float().cpu().numpy()).max())
    say(f"prefill vs plain attention over all {T} rows: max abs diff {d:.3g}")
    assert d <= 1e-2
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(500, 530), np.arange(1000, T, 173),
                                     np.arange(T - 20, T)]))
    _check(out, qs, ks, vs, idx, cnt, 0, prm, rows, "oracle lists")


def _odd_lists(rng, T, q_start, Tq, L, prm):
    """Lists that break the method's layout: random sorted far keys, part of
    the window missing, some entries repeated, entries at or past T, -1, keys
    after the query, empty and full rows."""
    idx = np.full((Tq, L), -1, np.int32)
    cnt = np.zeros(Tq, np.int32)
    for r in range(Tq):
        p = q_start + r
        kind = r % 7
        near = O.near_set(p, prm)
        if kind == 0:
            lst = []
        elif kind == 1:      # the method's layout
            far = np.setdiff1d(np.arange(p + 1), near)
            nf = min(len(far), 300, L - len(near))
            lst = list(near[near < prm.n_sink]) + sorted(rng.choice(far, size=nf, replace=False).tolist()) \
                + list(near[near >= prm.n_sink])
        else:
            n = int(rng.integers(1, L))
            lst = rng.integers(0, p + 1, size=n).tolist()
            if kind == 2:
                lst += [T, T + 5, -1, -7]
            if kind == 3:
                lst += rng.integers(p + 1, T, size=min(20, T - p - 1)).tolist() if p + 1 < T else []
            if kind == 4:
                lst = sorted(lst) + [p, p, p - 1]
            if kind == 5:
                lst = sorted(set(lst))
            lst = lst[:L]
        idx[r, :len(lst)] = lst
        cnt[r] = len(lst)
    return idx, cnt


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (64, 4), (24, 3), (16, 1)])
def test_prefill_attention_odd_lists_every_group_size(Hq, Hkv):
    say(f"case: prefill attention, odd lists, Hq={Hq} Hkv={Hkv}")
    w = _workload(Hq, Hkv)
    T, q_start, Tq = 2600, 2200, 300
    p = lsa.Params(k=256, n_sink=4, window=512)
    prm = oracle_params(p)
    rng = np.random.default_rng(Hq * 10 + Hkv)
    idx, cnt = _odd_lists(rng, T, q_start, Tq, 900, prm)
    qs, ks, vs, Q, K, V = _qkv(w, 1, T, np.arange(q_start, q_start + Tq))
    out = _run(Q, K, V, idx[None], cnt[None], q_start, p)
    _check(out, qs, ks, vs, idx[None], cnt[None], q_start, prm, np.arange(Tq), "odd lists")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_prefill_attention_negative_and_zero_scale(scale):
    say(f"case: prefill attention, scale={scale}")
    w = S.WORKLOADS[2]
    T, q_start, Tq = 1500, 1200, 200
    p = lsa.Params(k=256, n_sink=3, window=100)
    prm = oracle_params(p)
    idx, cnt = _odd_lists(np.random.default_rng(5), T, q_start, Tq, 400, prm)
    qs, ks, vs, Q, K, V = _qkv(w, 1, T, np.arange(q_start, q_start + Tq))
    out = _run(Q, K, V, idx[None], cnt[None], q_start, p, scale=scale)
    _check(out, qs, ks, vs, idx[None], cnt[None], q_start, prm, np.arange(Tq), f"scale {scale}",
           scale=scale)


def test_prefill_attention_sequences_launch_and_tile_boundaries():
    """Three sequences of 1,000 rows (launches of 1,024 rows cut sequences and
    16-row tiles), 64 sinks and a 2,048-key window: the method's layout with
    random far keys; sampled rows around every boundary against the oracle,
    every row against lsa_sparse_attention."""
    say("case: prefill attention, 3 sequences x 1000 rows, window 2048, 64 sinks")
    w = S.WORKLOADS[2]
    B, T, q_start, Tq = 3, 4000, 2900, 1000
    p = lsa.Params(k=512, n_sink=64, window=2048)
    prm = oracle_params(p)
    L = lsa.list_len(p)
    rng = np.random.default_rng(11)
    idx = np.full((B, Tq, L), -1, np.int32)
    cnt = np.zeros((B, Tq), np.int32)
    for b in range(B):
        for r in range(Tq):
            pos = q_start + r
            near = O.near_set(pos, prm)
            far = np.setdiff1d(np.arange(pos + 1), near)
            f = np.sort(rng.choice(far, size=min(len(far), int(rng.integers(0, p.k + 1))), replace=False))
            lst = np.concatenate([near[near < p.n_sink], f, near[near >= p.n_sink]])
            idx[b, r, :len(lst)] = lst
            cnt[b, r] = len(lst)
    qs, ks, vs, Q, K, V = _qkv(w, B, T, np.arange(q_start, q_start + Tq))
    out = _run(Q, K, V, idx, cnt, q_start, p)
    plain = lsa.sparse_attention(Q, K, V, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    d = float(np.abs(out - plain.float().cpu().numpy()).max())
    say(f"prefill vs plain attention over all {B * Tq} rows: max abs diff {d:.3g}")
    assert d <= 1e-2
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 17], np.arange(20, 30), [47, 48],
                                     np.arange(Tq - 12, Tq)]))
    _check(out, qs, ks, vs, idx, cnt, q_start, prm, rows, "3 sequences")


def test_prefill_attention_row_layout():
    """K/V caches above 256 MiB: the gather takes one workgroup per row (four
    waves, one per KV head) on top of the near state."""
    say("case: prefill attention, one workgroup per row")
    w = S.WORKLOADS[2]
    T, q_start, Tq = 3000, 2500, 100
    p = lsa.Params(k=256)
    prm = oracle_params(p)
    idx, cnt = _odd_lists(np.random.default_rng(3), T, q_start, Tq, 800, prm)
    # entries at or past T would name the larger cache's zero rows, which
    # count in the softmax: keep the lists inside [0, T) or invalid (< 0)
    idx[idx >= T] = -1
    qs, ks, vs, Q, K, V = _qkv(w, 1, T, np.arange(q_start, q_start + Tq))
    Tmax = (256 << 20) // (w.Hkv * w.D * 2) + 1
    assert not lsa.attention_head_major(1, Tmax, w.Hkv, w.D, lsa.LSA_BF16)
    Kr = torch.zeros((1, Tmax, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
    Vr = torch.zeros_like(Kr)
    Kr[:, :T] = K
    Vr[:, :T] = V
    del K, V
    out = _run(Q, Kr, Vr, idx[None], cnt[None], q_start, p)
    _check(out, qs, ks, vs, idx[None], cnt[None], q_start, prm, np.arange(Tq), "row layout")


@pytest.mark.parametrize("n_sink,window", [(4, 512), (3, 100)])
def test_prefill_attention_row_layout_early_rows(n_sink, window):
    """One workgroup per row, where the gather appends the row's near keys
    itself: rows from position 0 on, so that for the first rows the sinks and
    the window overlap and the near set is every key up to the row, with odd
    lists; two sequences."""
    say(f"case: prefill attention, one workgroup per row, rows from 0, n_sink={n_sink} window={window}")
    w = S.WORKLOADS[2]
    B, T, q_start, Tq = 2, 900, 0, 700
    p = lsa.Params(k=256, n_sink=n_sink, window=window)
    prm = oracle_params(p)
    idx = np.full((B, Tq, 800), -1, np.int32)
    cnt = np.zeros((B, Tq), np.int32)
    for b in range(B):
        idx[b], cnt[b] = _odd_lists(np.random.default_rng(100 * b + window), T, q_start, Tq, 800, prm)
    idx[idx >= T] = -1            # past T the larger cache's zero rows would count
    qs, ks, vs, Q, K, V = _qkv(w, B, T, np.arange(q_start, q_start + Tq))
    Tmax = (256 << 20) // (w.Hkv * w.D * 2) + 1
    assert not lsa.attention_head_major(B, Tmax, w.Hkv, w.D, lsa.LSA_BF16)
    Kr = torch.zeros((B, Tmax, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
    Vr = torch.zeros_like(Kr)
    Kr[:, :T] = K
    Vr[:, :T] = V
    del K, V
    out = _run(Q, Kr, Vr, idx, cnt, q_start, p)
    rows = np.unique(np.concatenate([np.arange(0, 12), np.arange(95, 110), np.arange(500, 530),
                                     np.arange(Tq - 8, Tq)]))
    _check(out, qs, ks, vs, idx, cnt, q_start, prm, rows, "row layout, early rows")
