"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test compares the oracle with a brute-force computation, a library
routine, a closed form, an invariant, or a number the pages print.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import lsa_synth as S
from oracle import lsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _c1_cache(nblocks=8, dtype="f32", k=256):
    w = S.WORKLOADS[1]
    X, Y, _ = S.latent_inputs(w, T=nblocks * 512, query_rows=(0, nblocks * 512))
    prm = O.Params(k=k, index_dtype=dtype)
    return X, Y, prm, O.build_cache(X, prm)


# ---------------------------------------------------------------- Ward cost

def _ess(pts):
    pts = np.asarray(pts, np.float64)
    c = pts.mean(axis=0)
    return float(((pts - c) ** 2).sum())


def test_ward_cost_equals_brute_force_ess_increase():
    """Ward's merge cost is the increase of the total within-cluster sum of squares."""
    rng = np.random.default_rng(1)
    for trial in range(200):
        na, nb = rng.integers(1, 5, size=2)
        A = rng.standard_normal((na, 64)) * rng.uniform(0.1, 3)
        B = rng.standard_normal((nb, 64)) + rng.standard_normal(64)
        brute = _ess(np.vstack([A, B])) - _ess(A) - _ess(B)
        closed = O.ward_cost(na, A.mean(0), nb, B.mean(0))
        assert closed == pytest.approx(brute, rel=1e-10, abs=1e-12)


def test_ward_total_cost_telescopes_to_final_ess():
    """Singletons have zero ESS and every merge adds exactly its cost."""
    X, _, prm, _ = _c1_cache(nblocks=2)
    for b in range(2):
        res, P = O.cluster_block(X[b * 512:(b + 1) * 512], prm)
        final = sum(_ess(P[c]) for c in res.clusters)
        assert sum(res.merge_costs) == pytest.approx(final, rel=1e-10)


def _brute_greedy(points, cap, target):
    """Greedy merging evaluated by brute force: every candidate merge is scored by
    recomputing ESS(union) - ESS(a) - ESS(b) from the member points, pairs are
    enumerated in lexicographic id order and the first strict minimum wins."""
    clusters = {i: [i] for i in range(len(points))}
    while len(clusters) > target:
        best = None
        ids = sorted(clusters)
        for a, b in itertools.combinations(ids, 2):
            ca, cb = clusters[a], clusters[b]
            if len(ca) + len(cb) > cap:
                continue
            d = _ess(points[ca + cb]) - _ess(points[ca]) - _ess(points[cb])
            if best is None or d < best[0]:
                best = (d, a, b)
        d, a, b = best
        clusters[a] = sorted(clusters[a] + clusters.pop(b))
    return [clusters[i] for i in sorted(clusters)]


@pytest.mark.parametrize("n,cap,target", [(8, 2, 4), (10, 4, 4), (12, 3, 5), (12, 4, 6)])
def test_ward_greedy_matches_exhaustive_replay(n, cap, target):
    rng = np.random.default_rng(n * 100 + cap)
    for trial in range(20):
        pts = rng.standard_normal((n, 64))
        res = O.ward_merge(pts, cap, target)
        if res.min_gap < 1e-9:
            continue
        assert res.clusters == _brute_greedy(pts, cap, target)


def test_ward_without_cap_equals_scipy_ward_linkage():
    """With the cap lifted, greedy Ward reproduces SciPy's Ward dendrogram cut at 64."""
    from scipy.cluster.hierarchy import fcluster, linkage
    X, _, prm, _ = _c1_cache(nblocks=4)
    checked = 0
    for b in range(4):
        P = O.pool_keys(O.normalize_keys(X[b * 512:(b + 1) * 512]))
        res = O.ward_merge(P, cap=128, target=64)
        if res.min_gap < 1e-9:
            continue
        lab = fcluster(linkage(P, method="ward"), t=64, criterion="maxclust")
        ours = sorted(tuple(c) for c in res.clusters)
        theirs = sorted(tuple(np.flatnonzero(lab == v)) for v in np.unique(lab))
        assert ours == theirs
        checked += 1
    assert checked >= 2


def test_ward_respects_cap_and_tie_rule():
    # four identical points: every pair ties, so pairs go lowest-id first
    pts = np.zeros((4, 64))
    res = O.ward_merge(pts, cap=2, target=2)
    assert res.clusters == [[0, 1], [2, 3]]
    assert res.gaps[0] == 0.0
    # a far point can only join when the cap allows
    pts = np.vstack([np.zeros((3, 64)), np.full((1, 64), 5.0)])
    res = O.ward_merge(pts, cap=2, target=2)
    assert res.clusters == [[0, 1], [2, 3]]


# ---------------------------------------------------------------- pooling, buckets

def test_normalise_and_pool_are_sums_of_unit_keys():
    X, _, prm, _ = _c1_cache(nblocks=1)
    K = O.normalize_keys(X)
    assert np.allclose(np.linalg.norm(K, axis=1), 1.0, atol=1e-15)
    P = O.pool_keys(K)
    assert P.shape == (128, 64)
    assert np.all(np.linalg.norm(P, axis=1) <= 4 + 1e-12)
    e = np.eye(64)
    assert np.linalg.norm(O.pool_keys(np.vstack([e[3]] * 4))[0]) == pytest.approx(4.0)
    assert np.linalg.norm(O.pool_keys(e[:4])[0]) == pytest.approx(2.0)
    assert np.allclose(O.pool_keys(O.normalize_keys(X[:8] * 7.5)), P[:2])


def test_bucket_partition_invariants_and_counts():
    X, _, prm, c = _c1_cache(nblocks=8, dtype="bf16")
    st = _golden("structural_counts.json")
    assert c.n_buckets == 8 * 64
    assert 2 * prm.n_buckets == st["buckets_first_1024_tokens"]["value"]
    for b in range(8):
        seen = []
        for g in range(b * 64, (b + 1) * 64):
            m = c.members[g]
            assert 4 <= len(m) <= st["keys_per_bucket"]["max"]
            assert m == sorted(m) and all(b * 512 <= x < (b + 1) * 512 for x in m)
            assert all(m[i + 1] - m[i] == 1 for i in range(len(m) - 1) if (i + 1) % 4)
            seen += m
        assert sorted(seen) == list(range(b * 512, (b + 1) * 512))
        # canonical numbering: buckets in increasing order of smallest member
        firsts = [c.members[g][0] for g in range(b * 64, (b + 1) * 64)]
        assert firsts == sorted(firsts)
    assert np.mean([len(m) for m in c.members]) == st["keys_per_bucket"]["mean"]


def test_centroid_is_normalised_sum_of_member_unit_keys():
    X, _, prm, c = _c1_cache(nblocks=2, dtype="bf16")
    for g in range(0, 128, 7):
        keys = X[c.members[g]].astype(np.float64)
        v = (keys / np.linalg.norm(keys, axis=1, keepdims=True)).sum(0)
        v /= np.linalg.norm(v)
        assert np.array_equal(c.centroids[g], O.round_bf16(v))
        assert np.linalg.norm(c.centroids[g]) == pytest.approx(1.0, abs=8e-3)


def test_round_bf16_matches_torch_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.float32([1.00390625, 1.01171875, -1.00390625, 3e-39, 1e-41])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_normalize_query_by_hand():
    """A 3-4-5 query: unit length first (0.6, 0.8), then the index dtype's
    rounding (0.6 is not a bf16 value: 0.6015625 is its nearest, 0.8 rounds
    to 0.80078125); a zero query stays zero."""
    y = np.zeros(64)
    y[0], y[1] = 3.0, 4.0
    f = O.normalize_query(y, "f32")
    assert f[0] == np.float64(np.float32(0.6)) and f[1] == np.float64(np.float32(0.8))
    assert not f[2:].any()
    b = O.normalize_query(y, "bf16")
    assert b[0] == 0.6015625 and b[1] == 0.80078125
    assert not O.normalize_query(np.zeros(64), "bf16").any()


def test_decode_fires_when_a_block_fills():
    """Appending the key at position p completes block p // 512 exactly when p
    is the block's last position (511, 1023, ...); [visual] "How the hierarchy
    is built": a block is clustered once its 512 keys are present."""
    prm = O.Params()
    assert [p for p in range(0, 2048) if O.decode_fires(p, prm)] == [511, 1023, 1535, 2047]


# ---------------------------------------------------------------- worked counts

def test_worked_query_counts_from_the_pages():
    g = _golden("worked_query_counts.json")
    prm = O.Params(n_sink=g["n_sink"], window=g["window"])
    p = g["position"]
    assert O.far_range_size(p, prm) == g["far_range"]
    assert O.eligible_buckets(p, prm) == g["eligible_buckets"]
    assert O.far_range_size(p, prm) // 8 == g["block_of_8_scores"]


def test_flat_score_count_is_about_T_over_8():
    st = _golden("structural_counts.json")
    prm = O.Params()
    n = O.eligible_buckets(10_000_000, prm)
    assert abs(n - st["flat_scores_10M"]["value"]) / st["flat_scores_10M"]["value"] < 1e-3


def test_tree_level_counts_match_pages():
    st = _golden("structural_counts.json")
    # three levels inside a block (key -> pooled is two binary levels, pooled -> bucket one)
    assert O.tree_height(1_048_576 // 8) + 3 == st["tree_levels"]["1M"]
    assert O.tree_height((10_000_000 // 512) * 64) + 3 == st["tree_levels"]["10M"]
    ex = st["worked_tree_example"]
    n = O.beam_score_count(ex["levels"], ex["beam"], ex["branching"])
    assert n == ex["scores"]
    assert ex["branching"] ** ex["levels"] >= ex["context"]
    assert abs(ex["context"] / n - ex["reduction"]) / ex["reduction"] < 0.01


# ---------------------------------------------------------------- ranking, expansion

def _toy_cache(centroids, members, prm):
    nb = len(centroids) // prm.n_buckets
    return O.BucketCache(prm, nb, np.asarray(centroids, np.float64), members,
                         [None] * len(members), np.full(nb, np.inf), np.zeros(nb))


def test_expansion_worked_example_by_hand():
    """Hand-worked: 3 blocks of 8 keys with 2 buckets of 4 each (n_pool=4,
    block=8, 2 buckets/block, cap 4 keys), query at p=20, k=5, 2 sinks, window 4."""
    prm = O.Params(n_pool=4, block=8, n_buckets=2, cap_keys=4, k=5, n_sink=2, window=4,
                   index_dtype="f32", d_latent=2)
    e0, e1 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    cent = [e0 * 0.2 + e1, e0, e1, e0 * 0.5 + e1 * 0.5, e0, e0]
    members = [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15],
               [16, 17, 18, 19], [20, 21, 22, 23]]
    c = _toy_cache(np.array([x / np.linalg.norm(x) for x in cent]), members, prm)
    p = 20                                       # qb = 2: buckets 0..3 eligible
    r = O.index_query(np.array([0.0, 1.0]), p, c)
    # scores: b2 = 1, b0 = .98, b3 = .707, b1 = 0 -> order 2, 0, 3, 1
    assert list(r.ranked) == [2, 0, 3, 1]
    # near = {0, 1} U {17..20}; far: 8,9,10,11 from b2, then 2 (0 and 1 skipped) -> k=5
    assert r.count == 2 + 5 + 4
    assert list(r.idx[:r.count]) == [0, 1, 2, 8, 9, 10, 11, 17, 18, 19, 20]
    assert r.last_rank == 1


def test_flat_rank_ties_go_to_lower_bucket():
    prm = O.Params(n_pool=4, block=8, n_buckets=2, cap_keys=4, k=4, n_sink=0, window=1,
                   index_dtype="f32", d_latent=2)
    cent = np.array([[0.0, 1.0], [1.0, 0.0], [1.0, 0.0], [0.6, 0.8]])
    c = _toy_cache(cent, [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15]], prm)
    r = O.index_query(np.array([1.0, 0.0]), 16, c)
    assert list(r.ranked) == [1, 2, 3, 0]
    assert list(r.idx[:r.count]) == [4, 5, 6, 7, 16]
    assert r.exempt          # buckets 1 and 2 tie exactly at the truncation boundary


@pytest.mark.parametrize("p", [0, 2, 3, 511, 512, 1023, 1500, 4095])
def test_index_list_invariants(p):
    X, Y, prm, c = _c1_cache(nblocks=8)
    r = O.index_query(Y[p], p, c)
    lst = r.idx[:r.count]
    assert np.all(r.idx[r.count:] == -1)
    assert np.all(np.diff(lst) > 0) and lst[0] >= 0 and lst[-1] <= p
    near = O.near_set(p, prm)
    assert set(near) <= set(lst)
    avail = p + 1 - len(near)
    assert r.count - len(near) == min(prm.k, O.eligible_buckets(p, prm) * 8 - len(
        set(near) & set(range(O.eligible_buckets(p, prm) * 8))))
    assert r.count - len(near) <= avail
    assert all(x // 512 < p // 512 for x in set(lst) - set(near))


def test_k_covering_every_key_gives_dense_causal_list():
    X, Y, prm, _ = _c1_cache(nblocks=8)
    prm2 = O.Params(k=5000, index_dtype="f32")
    c = O.build_cache(X, prm2)
    for p in [0, 700, 1535, 4095]:
        r = O.index_query(Y[p], p, c)
        elig_keys = O.eligible_buckets(p, prm2) * 8
        expect = np.union1d(O.near_set(p, prm2), np.arange(elig_keys))
        assert np.array_equal(r.idx[:r.count], expect)
        if p % 512 == 511 or p < 512:
            assert np.array_equal(expect, np.arange(p + 1))


# ---------------------------------------------------------------- attention

def test_attention_with_full_list_equals_dense_causal_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D = 64, 4, 2, 128
    q = rng.standard_normal((T, Hq, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    for p in [0, 1, 17, 63]:
        out = O.attention_query(q[p], K, V, np.arange(p + 1), p + 1)
        assert np.allclose(out, ref[p], atol=1e-12)


def test_attention_window_only_equals_sliding_window_softmax():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    T, H, D, W = 40, 2, 128, 8
    q = rng.standard_normal((T, H, D))
    K = rng.standard_normal((T, H, D))
    V = rng.standard_normal((T, H, D))
    i = np.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(K).permute(1, 0, 2),
        torch.from_numpy(V).permute(1, 0, 2), attn_mask=torch.from_numpy(mask))
    ref = ref.permute(1, 0, 2).numpy()
    prm = O.Params(n_sink=0, window=W, k=0)
    for p in [0, 5, 39]:
        near = O.near_set(p, prm)
        assert np.allclose(O.attention_query(q[p], K, V, near, len(near)), ref[p], atol=1e-12)


# ---------------------------------------------------------------- tree

def test_tree_structure_invariants():
    X, _, prm, c = _c1_cache(nblocks=8, dtype="bf16")
    t = O.build_tree(c)
    assert t.height == O.tree_height(c.n_buckets) == 9
    for l in range(1, t.height + 1):
        lv, below = t.levels[l], t.levels[l - 1]
        n_below = below["cent"].shape[0]
        assert lv["cent"].shape[0] == -(-n_below // 2)
        kids = lv["child"][lv["child"] >= 0]
        assert sorted(kids) == list(range(n_below))      # one parent per node
        for g0 in range(0, n_below - n_below % 128, 128):  # full groups pair perfectly
            par = lv["child"][g0 // 2:(g0 + 128) // 2]
            assert np.all(par >= 0)
        assert np.array_equal(lv["min_block"], [below["min_block"][ch[ch >= 0]].min()
                                                for ch in lv["child"]])
        assert np.allclose(np.linalg.norm(lv["cent"], axis=1), 1.0, atol=1e-2)


def test_tree_with_beam_wider_than_every_level_equals_flat():
    X, Y, prm, _ = _c1_cache(nblocks=8, dtype="bf16")
    prm_w = O.Params(k=256, index_dtype="bf16", beam=4096)
    c = O.build_cache(X, prm_w)
    t = O.build_tree(c)
    for p in [600, 2000, 4095]:
        a = O.index_query(Y[p], p, c, "flat")
        b = O.index_query(Y[p], p, c, "tree", t)
        assert np.array_equal(a.ranked, b.ranked)
        assert np.array_equal(a.idx, b.idx)


def test_leaf_level_reading():
    assert O.leaf_level(O.Params(k=2048, beam=64)) == 4
    assert O.leaf_level(O.Params(k=4096, beam=64)) == 5


# ---------------------------------------------------------------- max over heads

def test_max_over_heads_bucket_scores_hand_worked():
    """[catalog "Key points"], N-LSA: bucket selection uses the max score across
    heads.  Two query heads e0, e1 and three buckets: A = (0.9, 0.1), B = (0.5,
    0.8), C = (0.7, 0.7) (not normalised: the pin is about the rule).  Max over
    heads: A 0.9, B 0.8, C 0.7 -> A, B, C.  The mean would rank C first
    (0.7 > 0.65 = B > 0.5 = A), head 0 alone A, C, B, head 1 alone B, C, A."""
    cent = np.array([[0.9, 0.1], [0.5, 0.8], [0.7, 0.7]])
    yh = np.eye(2)
    s = O.bucket_scores(yh, cent)
    assert np.array_equal(s, [0.9, 0.8, 0.7])
    assert list(np.lexsort((np.arange(3), -s))) == [0, 1, 2]
    # one head is the plain dot product; identical heads change nothing
    assert np.array_equal(O.bucket_scores(yh[0], cent), cent[:, 0])
    assert np.array_equal(O.bucket_scores(np.stack([yh[1]] * 4), cent), cent[:, 1])


def test_max_over_heads_lists_by_hand():
    """The hand-worked three-block example with two query heads: head 0 = e0,
    head 1 = e1 (2-d).  Bucket scores (max): b0 = max(0.196, 0.98) = 0.98,
    b1 = 1, b2 = 1, b3 = 0.707 -> order b1, b2 (tie, lower first), b0, b3."""
    prm = O.Params(n_pool=4, block=8, n_buckets=2, cap_keys=4, k=5, n_sink=2, window=4,
                   index_dtype="f32", d_latent=2)
    e0, e1 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    cent = [e0 * 0.2 + e1, e0, e1, e0 * 0.5 + e1 * 0.5, e0, e0]
    members = [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15],
               [16, 17, 18, 19], [20, 21, 22, 23]]
    nb = 3
    c = O.BucketCache(prm, nb, np.array([x / np.linalg.norm(x) for x in cent]), members,
                      [None] * 6, np.full(nb, np.inf), np.zeros(nb))
    r = O.index_query(np.stack([e0, e1]), 20, c)
    assert list(r.ranked) == [1, 2, 0, 3]
    # far: 4,5,6,7 from b1, then 8 from b2 (k = 5); sinks 0, 1; window 17..20
    assert list(r.idx[:r.count]) == [0, 1, 4, 5, 6, 7, 8, 17, 18, 19, 20]
    assert r.exempt          # b1 and b2 tie at 1 and b2 is the cut bucket
