"""CPU oracle for the Latent Sparse Attention (LSA) indexing + sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or constants) and imports
nothing from it; both sides are fed the same seeded inputs by ``lsa_synth``.

Everything is plain fp64 NumPy, step by step in the order the pages describe,
with no blocking or fusion.  Page citations use these short names:

  [summary]  "Latent Sparse Attention: Towards Subquadratic Ultra-Long Context
             Attention" (paper summary page)
  [catalog]  "Latent Sparse Attention (LSA): A Card-Catalog Approach to
             Subquadratic Ultra-Long Context Attention" (forum post)
  [72x]      "Latent Sparse Attention: 72x in One Layer, 9x for the Whole Model
             at 10M Tokens" (blog post with a partial re-implementation)
  [visual]   "Latent Sparse Attention at 10M tokens -- Hierarchical key
             clusters" (explainer)
  [Ward63]   J. H. Ward, "Hierarchical Grouping to Optimize an Objective
             Function", JASA 1963 (cited by [catalog], "References")

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * pooled key = SUM of 4 unit keys; Ward weights count pooled keys; the size
    cap of 16 keys is 4 pooled keys; exactly 64 buckets per 512-key block;
  * greedy global-minimum Ward among cap-feasible pairs, ties to the smallest
    (id_a, id_b), a cluster's id is its smallest pooled index;
  * buckets numbered 64*block + rank of id; members ascending;
  * bucket g is eligible for the query at position p iff g // 64 < p // 512;
  * window = the 512 positions [p-511, p] (query included); sinks clipped to p;
  * top_p unbounded; fewer far keys than k -> take them all;
  * attention scale 1/sqrt(D);
  * tree: pairing inside consecutive groups of 128 nodes of the level below,
    points = stored unit centroids with weight 1, leftover node copied up;
    beam on levels >= l*, then flat ranking of all eligible buckets under the
    final beam (l* = smallest l with beam * 2^l >= top_b, the bucket count
    that provably holds k far keys: ceil(k/4) + 65 for the default window
    and sinks).

Pins (tests marked "not gpu"): brute-force ESS for the Ward cost, SciPy's Ward
linkage when the cap is off, the telescoping ESS invariant, exhaustive greedy
replay on tiny blocks, partition/cap/causality invariants, the worked counts
of [72x] "One real query, start to finish", dense causal attention (NumPy and
torch SDPA) when k covers every key, tree == flat when the beam is wider than
every level, and the level counts of [catalog] "Key points".
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GAP_EXEMPT = 1e-5   # near-tie threshold: decisions closer than this may differ


@dataclass(frozen=True)
class Params:
    """Method hyper-parameters.  [catalog "Key points"], [72x "The same steps in general"]."""
    d_latent: int = 64
    n_pool: int = 4             # keys summed into one pooled key
    block: int = 512            # keys per cluster block
    n_buckets: int = 64         # buckets per full block
    cap_keys: int = 16          # max keys per bucket
    k: int = 2048               # far keys per query
    n_sink: int = 4
    window: int = 512
    index_dtype: str = "bf16"   # "bf16" | "f32": stored centroids and queries
    beam: int = 64              # tree beam width
    leaf_level: int = -1        # -1: automatic l*
    start_level: int = -1       # tree: level whose nodes are all scored first; -1: the root

    @property
    def items_per_block(self) -> int:
        return self.block // self.n_pool

    @property
    def cap_items(self) -> int:
        return self.cap_keys // self.n_pool

    @property
    def list_len(self) -> int:
        return self.n_sink + self.window + self.k

    @property
    def top_b(self) -> int:
        """Buckets that provably hold k far keys when ranked best-first.

        A bucket with no sink or window key gives at least n_pool far keys, so
        ceil(k / n_pool) such buckets suffice.  The buckets that can hold a
        sink or window key are counted on top: every bucket of each eligible
        block the window reaches back into (ceil((window - 1) / block) blocks)
        and one bucket per pooled item of the sinks (ceil(n_sink / n_pool)).
        With the default window of 512 and 4 sinks this is ceil(k / 4) + 65.
        """
        win_blocks = -(-(self.window - 1) // self.block)
        return (-(-self.k // self.n_pool) + self.n_buckets * win_blocks
                + -(-self.n_sink // self.n_pool))


# --------------------------------------------------------------------------
# rounding to the index dtype
# --------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest-even bfloat16 value (returned as fp64).

    bfloat16 keeps 8 significant bits; x = m * 2^e with 0.5 <= |m| < 1, so the
    quantum is 2^(e-8), floored at the subnormal quantum 2^-133.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def round_index(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    return round_bf16(x)


def unit(v: np.ndarray) -> np.ndarray:
    """v / ||v|| in fp64 (zero vector if the norm is below 1e-30)."""
    v = np.asarray(v, np.float64)
    n = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    return np.where(n < 1e-30, 0.0, v / np.where(n < 1e-30, 1.0, n))


# --------------------------------------------------------------------------
# (a1) normalise + pool   [catalog "Key points"], [visual "How the hierarchy is built"]
# --------------------------------------------------------------------------

def normalize_keys(X: np.ndarray) -> np.ndarray:
    """Latent keys are length-normalised so dot products are cosines."""
    return unit(np.asarray(X, np.float64))


def pool_keys(Khat: np.ndarray, n_pool: int = 4) -> np.ndarray:
    """Every n_pool consecutive unit keys are summed (not averaged) into one pooled key."""
    T = (Khat.shape[0] // n_pool) * n_pool
    return Khat[:T].reshape(-1, n_pool, Khat.shape[1]).sum(axis=1)


# --------------------------------------------------------------------------
# (a2) Ward merging inside one block   [Ward63], [catalog "Key points"],
#      [72x "The same steps in general"], [visual "How the hierarchy is built"]
# --------------------------------------------------------------------------

def ward_cost(n_a: float, m_a: np.ndarray, n_b: float, m_b: np.ndarray) -> float:
    """Increase of the within-cluster sum of squares when clusters a and b merge:
    n_a n_b / (n_a + n_b) * ||m_a - m_b||^2, with m the cluster means [Ward63]."""
    d = m_a - m_b
    return n_a * n_b / (n_a + n_b) * float(np.dot(d, d))


@dataclass
class WardResult:
    clusters: list          # list of sorted member-index lists, ordered by id (= min member)
    merge_costs: list       # cost of each merge, in merge order
    gaps: list              # per merge: second-smallest minus smallest feasible cost

    @property
    def min_gap(self) -> float:
        return min(self.gaps) if self.gaps else math.inf


def ward_merge(points: np.ndarray, cap: int, target: int) -> WardResult:
    """Greedy agglomerative Ward merging of ``points`` down to ``target`` clusters.

    Start from singletons (size 1, mean = the point, id = its index).  While
    more than ``target`` clusters remain, merge the pair (a, b), id_a < id_b,
    of smallest Ward cost among pairs with n_a + n_b <= cap; exact ties go to
    the lexicographically smallest (id_a, id_b).  The merged cluster has size
    n_a + n_b, mean (n_a m_a + n_b m_b) / (n_a + n_b) and id min(id_a, id_b).
    The cost matrix entries of the clusters that did not change are kept.
    """
    pts = np.asarray(points, np.float64)
    n_items = pts.shape[0]
    size = np.ones(n_items)
    mean = pts.copy()
    members = [[i] for i in range(n_items)]
    active = np.ones(n_items, bool)
    upper = np.triu(np.ones((n_items, n_items), bool), 1)      # pairs a < b
    diff = pts[:, None, :] - pts[None, :, :]
    cost = np.where(upper, 0.5 * np.sum(diff * diff, axis=2), np.inf)  # singletons: 1*1/2
    merge_costs, gaps = [], []
    n_active = n_items
    while n_active > target:
        # feasible pairs: both active, a < b, combined size within the cap
        feas = upper & active[:, None] & active[None, :] & (
            (size[:, None] + size[None, :]) <= cap)
        vals = np.where(feas, cost, np.inf).ravel()
        flat = int(np.argmin(vals))          # first minimum in row-major order = smallest (a, b)
        best = vals[flat]
        if not np.isfinite(best):
            raise RuntimeError("no feasible merge left")
        second = np.partition(vals, 1)[1] if vals.size > 1 else np.inf
        gaps.append(float(second - best))
        a, b = divmod(flat, n_items)
        merge_costs.append(float(best))
        n_new = size[a] + size[b]
        mean[a] = (size[a] * mean[a] + size[b] * mean[b]) / n_new
        size[a] = n_new
        members[a] = sorted(members[a] + members[b])
        active[b] = False
        cost[b, :] = np.inf
        cost[:, b] = np.inf
        # costs between the merged cluster and every other active cluster
        others = np.flatnonzero(active)
        others = others[others != a]
        d = mean[others] - mean[a]
        c = size[a] * size[others] / (size[a] + size[others]) * np.sum(d * d, axis=1)
        lo = others < a
        cost[others[lo], a] = c[lo]
        cost[a, others[~lo]] = c[~lo]
        n_active -= 1
    clusters = [members[i] for i in np.flatnonzero(active)]
    return WardResult(clusters=clusters, merge_costs=merge_costs, gaps=gaps)


# --------------------------------------------------------------------------
# bucket cache: centroids + member tables   [catalog "Summary", "Key points"],
# [visual "How the hierarchy is built"]
# --------------------------------------------------------------------------

@dataclass
class BucketCache:
    params: Params
    n_blocks: int
    centroids: np.ndarray        # [n_blocks*64, 64] fp64 holding index-dtype values
    members: list                # per bucket: ascending list of key positions
    pooled: list                 # per bucket: ascending list of block-local pooled indices
    block_min_gap: np.ndarray    # per block: smallest Ward decision gap
    block_ess: np.ndarray        # per block: total within-bucket sum of squares

    @property
    def n_buckets(self) -> int:
        return self.centroids.shape[0]

    def block_exempt(self, b: int) -> bool:
        return self.block_min_gap[b] < GAP_EXEMPT


def ess(points: np.ndarray) -> float:
    """Within-cluster sum of squared distances to the cluster mean."""
    p = np.asarray(points, np.float64)
    return float(np.sum((p - p.mean(axis=0)) ** 2))


def cluster_block(X_block: np.ndarray, prm: Params):
    """One full block of keys -> (clusters by id, WardResult, pooled keys)."""
    P = pool_keys(normalize_keys(X_block), prm.n_pool)
    res = ward_merge(P, prm.cap_items, prm.n_buckets)
    return res, P


def build_cache(X: np.ndarray, prm: Params, blocks=None) -> BucketCache:
    """Cluster every full block of the latent keys X [T, 64].

    A partial trailing block is not clustered (the recent window covers it).
    ``blocks`` restricts the work to a subset (other buckets are left as NaN).
    """
    T = X.shape[0]
    nb = T // prm.block
    M = prm.n_buckets
    cent = np.full((nb * M, prm.d_latent), np.nan)
    members = [None] * (nb * M)
    pooled = [None] * (nb * M)
    gaps = np.full(nb, np.inf)
    ess_tot = np.zeros(nb)
    todo = range(nb) if blocks is None else blocks
    for b in todo:
        res, P = cluster_block(X[b * prm.block:(b + 1) * prm.block], prm)
        gaps[b] = res.min_gap
        ess_tot[b] = sum(ess(P[c]) for c in res.clusters)
        for r, c in enumerate(res.clusters):
            g = b * M + r
            s = P[c].sum(axis=0)
            cent[g] = round_index(unit(s), prm.index_dtype)
            pooled[g] = list(c)
            members[g] = [b * prm.block + prm.n_pool * j + i
                          for j in c for i in range(prm.n_pool)]
    return BucketCache(prm, nb, cent, members, pooled, gaps, ess_tot)


# --------------------------------------------------------------------------
# (a3) tree over the buckets   [catalog "Summary", "Key points"],
#      [visual "How the hierarchy is built"]  -- reading: groups of 128
# --------------------------------------------------------------------------
TREE_GROUP = 128


@dataclass
class Tree:
    levels: list        # levels[l] = dict(cent [n_l,64], child [n_l,2] (-1 = none), min_block [n_l])
    group_min_gap: list  # per level >= 1: smallest pairing gap over its groups

    @property
    def height(self) -> int:
        return len(self.levels) - 1


def pair_group(points: np.ndarray) -> WardResult:
    """One group of a tree level: greedy Ward merging of its nodes with a size
    cap of 2, down to ceil(n / 2) nodes (pairs, and one leftover if n is odd)."""
    return ward_merge(points, cap=2, target=-(-len(points) // 2))


def build_tree(cache: BucketCache, dtype: str | None = None, mapper=map) -> Tree:
    """Repeat the merging on the buckets to form a binary tree.

    Level 0 is the buckets (points = stored centroids).  Each higher level
    splits the level below, in order, into groups of 128 nodes and pairs nodes
    greedily by smallest Ward cost for singletons (half the squared distance),
    ties to the smallest pair, until at most one node of the group is left;
    a leftover node becomes a one-child parent whose centroid is copied.
    Parents are ordered by their smaller child; a pair's centroid is the
    rounded unit vector of the sum of the two child centroids.  Stops when a
    level has one node.  The groups of a level are independent; ``mapper``
    (the builtin map, or a process pool's) applies pair_group to them.
    """
    dtype = dtype or cache.params.index_dtype
    n0 = cache.n_buckets
    lv0 = dict(cent=cache.centroids.copy(),
               child=np.full((n0, 2), -1, np.int64),
               min_block=np.arange(n0) // cache.params.n_buckets)
    levels, gaps = [lv0], []
    while levels[-1]["cent"].shape[0] > 1:
        below = levels[-1]
        n = below["cent"].shape[0]
        cent, child, minb, lvl_gap = [], [], [], math.inf
        groups = [np.arange(g0, min(n, g0 + TREE_GROUP)) for g0 in range(0, n, TREE_GROUP)]
        results = mapper(pair_group, [below["cent"][idx] for idx in groups])
        for idx, res in zip(groups, results):
            lvl_gap = min(lvl_gap, res.min_gap)
            for c in res.clusters:            # ordered by smaller child
                kids = idx[c]
                if len(kids) == 2:
                    cent.append(round_index(unit(below["cent"][kids].sum(axis=0)), dtype))
                    child.append([kids[0], kids[1]])
                else:
                    cent.append(below["cent"][kids[0]].copy())
                    child.append([kids[0], -1])
                minb.append(below["min_block"][kids].min())
        levels.append(dict(cent=np.array(cent), child=np.array(child, np.int64),
                           min_block=np.array(minb, np.int64)))
        gaps.append(lvl_gap)
    return Tree(levels, gaps)


def leaf_level(prm: Params) -> int:
    """Smallest l with beam * 2^l >= top_b (beam levels stop there)."""
    if prm.leaf_level >= 0:
        return prm.leaf_level
    l = 0
    while prm.beam * (1 << l) < prm.top_b:
        l += 1
    return l


# --------------------------------------------------------------------------
# (a4) query normalisation + flat scoring + causal mask + ranking
#      [visual "What one query actually does"], [72x "The same steps in general"]
# --------------------------------------------------------------------------

def normalize_query(y: np.ndarray, dtype: str) -> np.ndarray:
    """The query is length-normalised, then rounded to the index dtype."""
    return round_index(unit(np.asarray(y, np.float64)), dtype)


def eligible_buckets(p: int, prm: Params) -> int:
    """Buckets of complete blocks before the query's own block: g < 64 * (p // 512)."""
    return prm.n_buckets * (p // prm.block)


def bucket_scores(yhat: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Score of every bucket: yhat . c.  With several query heads (yhat [H, d];
    [catalog "Key points"], N-LSA: bucket selection uses the max score across
    heads) a bucket's score is the largest of its H dot products."""
    if yhat.ndim == 1:
        return cent @ yhat
    return (cent @ yhat.T).max(axis=1)


def flat_rank(yhat: np.ndarray, cache: BucketCache, p: int):
    """Score every eligible bucket centroid; order by (score desc, bucket asc)."""
    ne = eligible_buckets(p, cache.params)
    s = bucket_scores(yhat, cache.centroids[:ne])
    order = np.lexsort((np.arange(ne), -s))
    return order, s


def _keep_best(nodes: np.ndarray, sc: np.ndarray, width: int):
    """The `width` best nodes by (score desc, node asc), in node order, and the
    gap between the width-th and (width+1)-th scores (inf if all are kept)."""
    o = np.lexsort((nodes, -sc))
    gap = math.inf
    if len(o) > width:
        srt = sc[o]
        gap = srt[width - 1] - srt[width]
    return np.sort(nodes[o[:width]]), gap


def tree_rank(yhat: np.ndarray, cache: BucketCache, tree: Tree, p: int):
    """Beam descent, then flat ranking under the final beam.

    The descent starts at the root, or -- with prm.start_level = s below the
    root -- by scoring every eligible node of level s and keeping the best
    `beam` of them: the coarse first stage of the fixed-level search in
    [visual "A worked example"]'s table of search styles (score coarse groups,
    then refine inside the winners).  With s = l* that is the two-stage search;
    in between, a flat first stage and a beam below it.

    Returns (ranked buckets, bucket scores (NaN where not scored), smallest
    beam-boundary gap, number of node scores).
    """
    prm = cache.params
    qb = p // prm.block
    lstar = leaf_level(prm)
    H = tree.height
    n0 = cache.n_buckets
    s_all = np.full(n0, np.nan)
    n_scores = 0
    beam_gap = math.inf
    if lstar >= H:
        order, s = flat_rank(yhat, cache, p)
        s_all[:len(s)] = s
        return order, s_all, beam_gap, len(s)
    S = H if prm.start_level < 0 else min(max(prm.start_level, lstar), H)
    if S == H:
        beam = np.array([0])                  # the root, at level H
    else:
        lv = tree.levels[S]
        nodes = np.flatnonzero(lv["min_block"] < qb)
        sc = lv["cent"][nodes] @ yhat
        n_scores += len(nodes)
        beam, beam_gap = _keep_best(nodes, sc, prm.beam)
    for lvl in range(S - 1, lstar - 1, -1):
        above = tree.levels[lvl + 1]
        here = tree.levels[lvl]
        kids = above["child"][beam].ravel()
        kids = kids[kids >= 0]
        kids = kids[here["min_block"][kids] < qb]
        sc = here["cent"][kids] @ yhat
        n_scores += len(kids)
        o = np.lexsort((kids, -sc))
        if len(o) > prm.beam:
            srt = sc[o]
            beam_gap = min(beam_gap, srt[prm.beam - 1] - srt[prm.beam])
        beam = np.sort(kids[o[:prm.beam]])
    # collect the buckets under the final beam
    nodes = beam
    for lvl in range(lstar, 0, -1):
        ch = tree.levels[lvl]["child"][nodes].ravel()
        nodes = ch[ch >= 0]
    nodes = nodes[nodes < eligible_buckets(p, prm)]
    sc = cache.centroids[nodes] @ yhat
    n_scores += len(nodes)
    s_all[nodes] = sc
    o = np.lexsort((nodes, -sc))
    return nodes[o], s_all, beam_gap, n_scores


# --------------------------------------------------------------------------
# (a6) expansion + sinks + window   [72x "The same steps in general",
#      "One real query, start to finish"], [visual "What one query actually does"]
# --------------------------------------------------------------------------

def near_set(p: int, prm: Params) -> np.ndarray:
    """The first n_sink keys (clipped to p) and the window [p - W + 1, p]."""
    sinks = np.arange(min(prm.n_sink, p + 1))
    win = np.arange(max(0, p - prm.window + 1), p + 1)
    return np.union1d(sinks, win)


def near_union(idx: np.ndarray, count: int, p: int, prm: Params, T: int) -> np.ndarray:
    """The keys a query reads when its near set is taken whole: the list's
    valid entries (in [0, T)) outside the near set, in list order, then the
    near set (sinks and window) ascending.  Every list this method writes holds
    its near set once, so for such a list this is a reordering of the list
    itself; for other lists it is the list with its near entries replaced by
    the full near set."""
    near = near_set(p, prm)
    near_s = set(int(x) for x in near)
    far = [int(e) for e in np.asarray(idx[:count]).tolist() if 0 <= e < T and int(e) not in near_s]
    return np.asarray(far + [int(x) for x in near if x < T], np.int64)


def expand(order: np.ndarray, cache: BucketCache, p: int, near: np.ndarray):
    """Open buckets best-first, appending their keys (ascending) that are not
    in the near set, until exactly k far keys are collected.

    Returns (far keys in collection order, rank of the last opened bucket or
    None when every ranked bucket was opened without reaching k).
    """
    k = cache.params.k
    near_s = set(int(x) for x in near)
    far = []
    if k == 0:
        return far, None
    for r, g in enumerate(order):
        for key in cache.members[int(g)]:
            if key not in near_s:
                far.append(key)
                if len(far) == k:
                    return far, r
    return far, None


def rank_gap_exempt(order: np.ndarray, scores: np.ndarray, r) -> bool:
    """Near tie around the truncated bucket: only swaps across ranks r-1/r and
    r/r+1 can change which keys are taken."""
    if r is None:
        return False
    s = scores[order]
    if r >= 1 and s[r - 1] - s[r] < GAP_EXEMPT:
        return True
    if r + 1 < len(s) and s[r] - s[r + 1] < GAP_EXEMPT:
        return True
    return False


@dataclass
class IndexResult:
    idx: np.ndarray          # [L_max] ascending key positions, -1 padded
    count: int
    exempt: bool
    ranked: np.ndarray       # ranked buckets considered
    last_rank: object        # rank of the truncated bucket (or None)
    n_scores: int


def index_query(y: np.ndarray, p: int, cache: BucketCache, mode: str = "flat",
                tree: Tree | None = None) -> IndexResult:
    """Index list of the query at position p: sorted(near | far), one list shared
    by every head [visual "What one query actually does"].  y [d], or [H, d]
    for max-over-heads bucket scores (flat mode)."""
    prm = cache.params
    yhat = normalize_query(y, prm.index_dtype)
    beam_gap = math.inf
    if mode == "flat":
        order, s = flat_rank(yhat, cache, p)
        scores = s
        n_scores = len(s)
    else:
        order, s_all, beam_gap, n_scores = tree_rank(yhat, cache, tree, p)
        scores = s_all
    near = near_set(p, prm)
    far, r = expand(order, cache, p, near)
    lst = np.union1d(near, np.array(far, np.int64))
    out = np.full(prm.list_len, -1, np.int64)
    out[:len(lst)] = lst
    exempt = rank_gap_exempt(order, scores, r) or beam_gap < GAP_EXEMPT
    return IndexResult(out, len(lst), exempt, order, r, n_scores)


# --------------------------------------------------------------------------
# (a7) gather softmax attention over the list   [visual "Intro",
#      "What one query actually does"], [72x "The same steps in general"]
# --------------------------------------------------------------------------

def attention_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
                    count: int, scale: float | None = None) -> np.ndarray:
    """Ordinary softmax attention of every head over the listed keys.

    q [Hq, D], K/V [T, Hkv, D]; head h uses KV head h * Hkv // Hq.
    """
    q = np.asarray(q, np.float64)
    Hq, D = q.shape
    Hkv = K.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    sel = np.asarray(idx[:count], np.int64)
    out = np.zeros((Hq, D))
    for h in range(Hq):
        hk = h * Hkv // Hq
        Kh = np.asarray(K[sel, hk], np.float64)
        Vh = np.asarray(V[sel, hk], np.float64)
        logits = (Kh @ q[h]) * scale
        w = np.exp(logits - logits.max())
        w /= w.sum()
        out[h] = w @ Vh
    return out


# --------------------------------------------------------------------------
# (a8) decode step   [visual "How the hierarchy is built"]
# --------------------------------------------------------------------------

def decode_fires(p: int, prm: Params) -> bool:
    """Appending the key at position p completes block p // 512 iff (p+1) % 512 == 0."""
    return (p + 1) % prm.block == 0


# --------------------------------------------------------------------------
# analytic counts used as pins   [72x "Why choosing costs so much",
# "One real query, start to finish"], [catalog "Key points"],
# [visual "A worked example"]
# --------------------------------------------------------------------------

def far_range_size(p: int, prm: Params) -> int:
    """Keys that have to be chosen: every key up to p minus the near set."""
    return p + 1 - len(near_set(p, prm))


def tree_height(n_buckets: int) -> int:
    """Levels above the buckets when every level halves (rounding up)."""
    h, n = 0, n_buckets
    while n > 1:
        n = -(-n // 2)
        h += 1
    return h


def beam_score_count(levels: int, beam: int, branching: int) -> int:
    """Scores of a beam descent that expands ``beam`` nodes into ``branching``
    children on each of ``levels`` levels."""
    return levels * beam * branching
