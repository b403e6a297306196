"""Hand-worked pins for the oracle's tree (build_tree, tree_rank) and for the
bucket bound top_b.

Every expected value here is worked out by hand from the reading of the pages
([catalog "Key points"]: a binary tree over the buckets searched by a beam per
level; [visual "How the hierarchy is built"]: the block process repeated on
the buckets; [visual "What one query actually does"]: the beam keeps only the
best nodes of each level), on trees small enough to check by eye.  Trees for
tree_rank are written out node by node, so a wrong build cannot hide a wrong
search.  tests/test_oracle_mutations.py checks that a plausible mistake in
either function fails at least one of these pins.
"""
import math

import numpy as np

from oracle import lsa_oracle as O

D = 64


def _unit_score(s: float, axis: int) -> np.ndarray:
    """A unit vector whose dot product with e0 is exactly s (rest on one other axis)."""
    v = np.zeros(D)
    v[0] = s
    v[axis] = math.sqrt(1.0 - s * s)
    return v


def _tiny_params(**kw) -> O.Params:
    """Blocks of 8 keys with 2 buckets of one pooled item (4 keys) each."""
    base = dict(block=8, n_buckets=2, n_pool=4, cap_keys=4, k=4, n_sink=0, window=1,
                index_dtype="f32", beam=1, leaf_level=0)
    base.update(kw)
    return O.Params(**base)


def _tiny_cache(prm: O.Params, cents: np.ndarray) -> O.BucketCache:
    n = cents.shape[0]
    nb = n // prm.n_buckets
    members = [[4 * g + i for i in range(4)] for g in range(n)]
    pooled = [[g % prm.n_buckets] for g in range(n)]
    return O.BucketCache(prm, nb, np.asarray(cents, np.float64), members, pooled,
                         np.full(nb, np.inf), np.zeros(nb))


def _level(cents, child, minb):
    return dict(cent=np.asarray(cents, np.float64), child=np.asarray(child, np.int64),
                min_block=np.asarray(minb, np.int64))


def _tree(cache: O.BucketCache, upper: list) -> O.Tree:
    n0 = cache.n_buckets
    lv0 = _level(cache.centroids, np.full((n0, 2), -1), np.arange(n0) // cache.params.n_buckets)
    return O.Tree([lv0] + upper, [math.inf] * len(upper))


E0 = np.eye(D)[0]


# ---------------------------------------------------------------- tree_rank

def _two_level_case(prm):
    """Buckets b0..b3 (blocks 0, 1) with scores 0, 0.6, -0.8, 0.9 against e0;
    level 1: A = (b0, b1) scoring 0.7 and B = (b2, b3) scoring 0.1; a root."""
    cents = np.stack([_unit_score(0.0, 1), _unit_score(0.6, 2), _unit_score(-0.8, 3),
                      _unit_score(0.9, 4)])
    c = _tiny_cache(prm, cents)
    t = _tree(c, [_level([_unit_score(0.7, 5), _unit_score(0.1, 6)], [[0, 1], [2, 3]], [0, 1]),
                  _level([_unit_score(0.5, 7)], [[0, 1]], [0])])
    return c, t


def test_tree_rank_beam1_follows_the_parent_not_the_best_bucket():
    """Beam 1: the descent keeps A (0.7 > 0.1) and then b1 (0.6 > 0), although
    b3 (0.9, under B) is the best bucket overall.  Scores: 2 children of the
    root, 2 children of A, then the 1 bucket under the beam."""
    c, t = _two_level_case(_tiny_params(beam=1, leaf_level=0))
    order, s_all, gap, n_scores = O.tree_rank(E0, c, t, 16)      # block 2: all 4 eligible
    assert order.tolist() == [1]
    assert n_scores == 2 + 2 + 1
    assert math.isclose(gap, 0.6)
    assert s_all[1] == 0.6 and np.isnan(s_all[3])
    # stopping the beam at level 1 ranks every bucket under A, best first
    c, t = _two_level_case(_tiny_params(beam=1, leaf_level=1))
    order, _, _, n_scores = O.tree_rank(E0, c, t, 16)
    assert order.tolist() == [1, 0] and n_scores == 2 + 2
    # flat search on the same buckets reaches b3 first
    assert O.flat_rank(E0, c, 16)[0].tolist() == [3, 1, 0, 2]


def _three_level_case(prm):
    """8 buckets (4 blocks).  Level 1: N0..N3 = (b0 b1), (b2 b3), (b4 b5), (b6 b7)
    scoring 0.3, 0.5, 0.8, 0.1; level 2: M0 = (N0 N1) 0.9, M1 = (N2 N3) 0.2.
    Buckets score 0.99, -0.5, 0.4, 0.95, 0.2, 0.6, 0.97, 0.0."""
    bs = [0.99, -0.5, 0.4, 0.95, 0.2, 0.6, 0.97, 0.0]
    c = _tiny_cache(prm, np.stack([_unit_score(s, 1 + i) for i, s in enumerate(bs)]))
    l1 = _level([_unit_score(s, 10 + i) for i, s in enumerate([0.3, 0.5, 0.8, 0.1])],
                [[0, 1], [2, 3], [4, 5], [6, 7]], [0, 1, 2, 3])
    l2 = _level([_unit_score(0.9, 20), _unit_score(0.2, 21)], [[0, 1], [2, 3]], [0, 2])
    l3 = _level([_unit_score(0.5, 30)], [[0, 1]], [0])
    return c, _tree(c, [l1, l2, l3])


def test_tree_rank_beam2_three_levels():
    """Beam 2: level 2 keeps both M0 and M1; level 1 keeps N2 (0.8) and N1
    (0.5) of N0..N3; level 0 keeps b3 (0.95) and b5 (0.6) of b2..b5.  b0 (0.99)
    and b6 (0.97) are never reached: their parents lost at level 1."""
    c, t = _three_level_case(_tiny_params(beam=2, leaf_level=0))
    order, _, _, n_scores = O.tree_rank(E0, c, t, 40)             # block 5: all eligible
    assert order.tolist() == [3, 5]
    assert n_scores == 2 + 4 + 4 + 2
    c, t = _three_level_case(_tiny_params(beam=2, leaf_level=1))
    order, _, _, _ = O.tree_rank(E0, c, t, 40)
    assert order.tolist() == [3, 5, 2, 4]                         # b2..b5 ranked flat


def test_fixed_level_search_scores_every_node_of_its_start_level():
    """The fixed-level (two-stage) search of [visual "A worked example"]'s table
    of search styles, on the three-level tree with beam 1: started at level 1
    (= the stopping level), every level-1 node is scored and N2 (0.8) wins, so
    b5 (0.6) and b4 (0.2) are ranked -- where the descent from the root keeps
    M0 (0.9 > 0.2) and then N1 (0.5 > 0.3) and ranks b3, b2.  Started at level
    2 with the beam running to the buckets, the first stage keeps M0 and the
    descent goes N1, then b3."""
    c, t = _three_level_case(_tiny_params(beam=1, leaf_level=1))
    assert O.tree_rank(E0, c, t, 40)[0].tolist() == [3, 2]
    c, t = _three_level_case(_tiny_params(beam=1, leaf_level=1, start_level=1))
    order, _, gap, n_scores = O.tree_rank(E0, c, t, 40)
    assert order.tolist() == [5, 4] and n_scores == 4 + 2
    assert math.isclose(gap, 0.8 - 0.5)
    c, t = _three_level_case(_tiny_params(beam=1, leaf_level=0, start_level=2))
    assert O.tree_rank(E0, c, t, 40)[0].tolist() == [3]
    # beam 2 from level 1: N2 and N1 -> b2..b5 ranked flat (the same as the
    # descent, whose level 2 keeps both nodes)
    c, t = _three_level_case(_tiny_params(beam=2, leaf_level=1, start_level=1))
    assert O.tree_rank(E0, c, t, 40)[0].tolist() == [3, 5, 2, 4]


def test_fixed_level_search_masks_ineligible_nodes():
    """The first stage of the fixed-level search skips nodes whose smallest block
    is not before the query's block: in the masking case (query in block 2)
    started at level 1 with beam 1, N2 (0.99, block 2 only) is skipped and N1
    (0.6) wins."""
    bs = [0.2, 0.1, 0.4, 0.5, 0.99, 0.98]
    prm = _tiny_params(beam=1, leaf_level=1, start_level=1)
    c = _tiny_cache(prm, np.stack([_unit_score(s, 1 + i) for i, s in enumerate(bs)]))
    l1 = _level([_unit_score(0.3, 10), _unit_score(0.6, 11), _unit_score(0.99, 12)],
                [[0, 1], [2, 3], [4, 5]], [0, 1, 2])
    l2 = _level([_unit_score(0.5, 20), _unit_score(0.99, 12)], [[0, 1], [2, -1]], [0, 2])
    l3 = _level([_unit_score(0.5, 30)], [[0, 1]], [0])
    t = _tree(c, [l1, l2, l3])
    order, _, _, n_scores = O.tree_rank(E0, c, t, 16)
    assert order.tolist() == [3, 2] and n_scores == 2 + 2


def test_tree_rank_tie_at_the_beam_boundary_keeps_the_lower_node():
    """Level 1 scores 0.5, 0.7, 0.5 with beam 2: N1 and the lower of the two tied
    nodes, N0, are kept (ranking ties go to the lower index), so the buckets
    under N0 and N1 (b0..b3), not those under N2, are ranked.  The reported
    beam-boundary gap is 0."""
    bs = [0.1, 0.2, 0.3, 0.4, 0.9, 0.8]
    prm = _tiny_params(beam=2, leaf_level=1)
    c = _tiny_cache(prm, np.stack([_unit_score(s, 1 + i) for i, s in enumerate(bs)]))
    l1 = _level([_unit_score(0.5, 10), _unit_score(0.7, 11), _unit_score(0.5, 12)],
                [[0, 1], [2, 3], [4, 5]], [0, 1, 2])
    l2 = _level([_unit_score(0.6, 20), _unit_score(0.5, 12)], [[0, 1], [2, -1]], [0, 2])
    l3 = _level([_unit_score(0.5, 30)], [[0, 1]], [0])
    t = _tree(c, [l1, l2, l3])
    order, _, gap, _ = O.tree_rank(E0, c, t, 24)                  # block 3: all eligible
    assert order.tolist() == [3, 2, 1, 0]
    assert gap == 0.0


def test_tree_rank_masks_subtrees_with_no_eligible_block():
    """Query in block 2: blocks 0 and 1 are eligible.  N2 = (b4, b5) lies wholly
    in block 2 and scores highest (0.99), as does its one-child parent M1; the
    descent must skip both (their smallest block is not below 2) and go
    through M0 to N1 (0.6 > 0.3), ranking b2, b3.  Without the mask the beam
    would end on N2, whose buckets the leaf phase drops, and no far key would
    be found."""
    bs = [0.2, 0.1, 0.4, 0.5, 0.99, 0.98]
    prm = _tiny_params(beam=1, leaf_level=1, k=8)
    c = _tiny_cache(prm, np.stack([_unit_score(s, 1 + i) for i, s in enumerate(bs)]))
    l1 = _level([_unit_score(0.3, 10), _unit_score(0.6, 11), _unit_score(0.99, 12)],
                [[0, 1], [2, 3], [4, 5]], [0, 1, 2])
    l2 = _level([_unit_score(0.5, 20), _unit_score(0.99, 12)], [[0, 1], [2, -1]], [0, 2])
    l3 = _level([_unit_score(0.5, 30)], [[0, 1]], [0])
    t = _tree(c, [l1, l2, l3])
    p = 16                                                        # block 2, qb = 2
    order, _, _, _ = O.tree_rank(E0, c, t, p)
    assert order.tolist() == [3, 2]
    # the list: far keys of b3 (12..15) then b2 (8..11), up to k = 8, plus the
    # query itself (window 1, no sinks)
    r = O.index_query(E0, p, c, "tree", t)
    assert r.idx[:r.count].tolist() == [8, 9, 10, 11, 12, 13, 14, 15, 16]


def test_tree_rank_leaf_phase_drops_ineligible_buckets():
    """A beam node may straddle the causal boundary: N1 = (b2, b4) has its
    smallest block 1 < 2, so it is eligible for a query in block 2, but its
    child b4 (block 2) is not; the leaf phase ranks b2 only, although b4
    scores higher."""
    bs = [0.1, 0.2, 0.3, 0.4, 0.9, 0.8]
    prm = _tiny_params(beam=1, leaf_level=1)
    c = _tiny_cache(prm, np.stack([_unit_score(s, 1 + i) for i, s in enumerate(bs)]))
    l1 = _level([_unit_score(0.2, 10), _unit_score(0.8, 11), _unit_score(0.5, 12)],
                [[0, 1], [2, 4], [3, 5]], [0, 1, 1])
    l2 = _level([_unit_score(0.6, 20), _unit_score(0.5, 12)], [[0, 1], [2, -1]], [0, 1])
    l3 = _level([_unit_score(0.5, 30)], [[0, 1]], [0])
    t = _tree(c, [l1, l2, l3])
    order, _, _, _ = O.tree_rank(E0, c, t, 16)                    # block 2, qb = 2
    assert order.tolist() == [2]


# ---------------------------------------------------------------- build_tree

def test_build_tree_parent_centroid_is_the_rounded_unit_sum():
    """Two buckets e0, e1 pair into a root with centroid round(unit(e0 + e1)):
    1/sqrt(2) = 0.70710678... rounds to the bfloat16 value 0.70703125
    (1.0110101b x 2^-1); not the children's mean (0.5, 0.5) nor the unrounded
    unit vector."""
    prm = _tiny_params(index_dtype="bf16")
    c = _tiny_cache(prm, np.eye(D)[:2])
    t = O.build_tree(c)
    assert t.height == 1
    root = t.levels[1]
    expect = np.zeros(D)
    expect[:2] = 0.70703125
    assert np.array_equal(root["cent"][0], expect)
    assert root["child"].tolist() == [[0, 1]] and root["min_block"].tolist() == [0]


def test_build_tree_one_child_parent_copies_its_child_bit_for_bit():
    """Three buckets (blocks 0, 1, 2) in one group: b0 = e0 and b1 (close to
    e0) pair; b2 = (0.5, 0.25) is left over and becomes a one-child parent
    whose centroid is b2's, not renormalised (norm 0.559).  Parents are
    ordered by their smaller child: (b0, b1), then (b2); their smallest blocks
    are 0 and 2."""
    prm = _tiny_params(index_dtype="bf16", n_buckets=1)
    cents = np.zeros((3, D))
    cents[0, 0] = 1.0
    cents[1, 0], cents[1, 1] = 0.96875, 0.25
    cents[2, 2], cents[2, 3] = 0.5, 0.25
    c = _tiny_cache(prm, cents)
    t = O.build_tree(c)
    l1 = t.levels[1]
    assert l1["child"].tolist() == [[0, 1], [2, -1]]
    assert np.array_equal(l1["cent"][1], cents[2])
    assert l1["min_block"].tolist() == [0, 2]
    # (1.96875, 0.25) / 1.98456 = (0.992034, 0.125973) -> bf16 254/256, 129/1024
    pair = np.zeros(D)
    pair[0], pair[1] = 0.9921875, 0.1259765625
    assert np.array_equal(l1["cent"][0], pair)
    assert t.height == 2


def test_build_tree_pairs_only_inside_groups_of_128():
    """130 buckets: level 1 pairs nodes 0..127 among themselves (64 parents)
    and 128, 129 together (parent 64), although bucket 128 is a copy of bucket
    0 (distance 0, the closest pair of the whole level).  Level 2 then pairs
    the 65 level-1 nodes inside one group, leaving one one-child parent."""
    prm = _tiny_params(index_dtype="bf16")
    rng = np.random.default_rng(5)
    cents = O.round_bf16(O.unit(rng.standard_normal((130, D))))
    cents[128] = cents[0]
    cents[129] = -cents[0]
    c = _tiny_cache(prm, cents)
    t = O.build_tree(c)
    l1 = t.levels[1]
    assert l1["cent"].shape[0] == 65
    assert l1["child"][64].tolist() == [128, 129]
    first = l1["child"][:64]
    assert sorted(first.ravel().tolist()) == list(range(128))
    # parents are ordered by their smaller child, which is listed first
    assert np.all(first[:, 0] < first[:, 1])
    assert first[:, 0].tolist() == sorted(first[:, 0].tolist()) and first[0, 0] == 0
    assert l1["min_block"][64] == 64
    l2 = t.levels[2]
    assert l2["cent"].shape[0] == 33 and int((l2["child"][:, 1] < 0).sum()) == 1


# ---------------------------------------------------------------- top_b

def test_top_b_reading_by_hand():
    """ceil(k/4) clean buckets give k far keys; on top, every bucket of the
    eligible blocks the window reaches, and one bucket per pooled sink item."""
    assert O.Params(k=2048).top_b == 512 + 64 + 1
    assert O.Params(k=256, window=2048).top_b == 64 + 4 * 64 + 1
    assert O.Params(k=256, window=2049).top_b == 64 + 4 * 64 + 1
    assert O.Params(k=256, window=2050).top_b == 64 + 5 * 64 + 1
    assert O.Params(k=256, n_sink=64).top_b == 64 + 64 + 16
    assert O.Params(k=256, n_sink=0, window=1).top_b == 64
    # the beam stops at the smallest level l with beam * 2^l >= top_b:
    # 64 * 2^3 = 512 >= 321 > 256 = 64 * 2^2
    assert O.leaf_level(O.Params(k=256, window=2048, beam=64)) == 3
    assert O.leaf_level(O.Params(k=2048, n_sink=64, beam=16)) == 6       # 16 * 64 >= 592


def test_top_b_buckets_always_hold_k_far_keys():
    """On seeded clustered latents with windows up to 2,048 and up to 64 sinks,
    the rank of the last bucket the oracle opens is below top_b for every
    query; with window 2,048 the former bound ceil(k/4) + 65 is too small for
    queries at the end of a block, whose window covers three whole eligible
    blocks of recent (and so similar) keys."""
    import lsa_synth as S
    w = S.WORKLOADS[1]
    X, Y, _ = S.latent_inputs(w, T=4096, query_rows=(0, 4096))
    worst_old = 0
    for window, n_sink in ((2048, 4), (512, 64), (1, 0), (1000, 9)):
        prm = O.Params(k=256, index_dtype="f32", window=window, n_sink=n_sink)
        c = O.build_cache(X, prm)
        for p in list(range(511, 4096, 512)) + list(range(600, 4096, 157)):
            r = O.index_query(Y[p], p, c)
            if r.last_rank is not None:
                assert r.last_rank < prm.top_b, (window, n_sink, p, r.last_rank)
                if window == 2048:
                    worst_old = max(worst_old, r.last_rank + 1)
    assert worst_old > -(-256 // 4) + 65
