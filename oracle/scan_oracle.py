"""CPU oracle for the indexers Latent Sparse Attention is compared with: the
token scan and the block scans.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  Like lsa_oracle it
shares no code with the HIP library and imports nothing from it.  Plain fp64
NumPy, one query at a time.

What the pages say ([72x] = "Latent Sparse Attention: 72x in One Layer, 9x
for the Whole Model at 10M Tokens"):
  * "Why choosing costs so much": a token scan scores every key (10M scores
    per query at 10M tokens), a block scan each run of 4 adjacent keys (2.5M),
    LSA each bucket of about 8 keys (about 1.25M); the figures are the context
    divided by the group size.
  * "One real query, start to finish": with the first 4 keys and the latest
    512 always read, the query at token 23,711 has 23,195 keys to choose; the
    token scan scores all of them, a block cut to runs of 8 makes 2,899
    scores; each method is allowed the same number of far keys.

Readings taken where the pages are silent (listed with their reasons in the
design notes of the repository):
  * S-1 a run is an aligned group of b consecutive keys, [b j, b j + b);
  * S-2 a run is summarised like a bucket: the unit vector of the sum of its
    unit keys, rounded to the index dtype (for b = 1, the unit key);
  * S-3 the scan scores every run that ends at or before the first window key
    (b j + b <= p - W + 1) and holds a key that is not a sink
    (b j + b > n_sink): 23,195 runs of 1 and 2,899 runs of 8 at the worked
    query, the pages' two counts;
  * S-4 runs are ranked by (score desc, run asc) and opened best first, their
    keys that are not sinks taken in ascending order, until k far keys are
    collected; the list is the sorted union with the sinks and the window,
    as for LSA.  The query is normalised and rounded as for LSA.
"""
from __future__ import annotations

import numpy as np

from .lsa_oracle import (IndexResult, Params, near_set, normalize_keys, normalize_query,
                         rank_gap_exempt, round_index, unit)


def run_directions(X: np.ndarray, b: int) -> np.ndarray:
    """Unit vector of the sum of the unit keys of every complete aligned run of
    b keys (reading S-1, S-2), fp64, not rounded."""
    X = np.asarray(X, np.float64)
    n = (X.shape[0] // b) * b
    return unit(normalize_keys(X[:n]).reshape(-1, b, X.shape[1]).sum(axis=1))


def run_summaries(X: np.ndarray, b: int, dtype: str) -> np.ndarray:
    """The stored run summaries: run_directions rounded to the index dtype."""
    return round_index(run_directions(X, b), dtype)


def scan_runs(p: int, b: int, prm: Params) -> tuple:
    """The runs [j_lo, j_hi) a scan scores for the query at p (reading S-3):
    runs that end at or before the window's first key and hold a key that is
    not a sink."""
    s_end = min(prm.n_sink, p + 1)
    w_start = max(0, p - prm.window + 1)
    j_hi = w_start // b                  # b j + b <= w_start
    j_lo = s_end // b                    # b j + b > s_end
    return j_lo, max(j_lo, j_hi)


def scan_rank(yhat: np.ndarray, summaries: np.ndarray, p: int, b: int, prm: Params):
    """Score every scanned run; order them by (score desc, run asc).
    Returns (ranked run ids, their scores in that order... as an array over the
    scanned runs, indexed like the ranked ids)."""
    j_lo, j_hi = scan_runs(p, b, prm)
    runs = np.arange(j_lo, j_hi)
    s = summaries[j_lo:j_hi] @ yhat
    order = np.lexsort((runs, -s))
    return runs[order], s[order]


def scan_expand(ranked: np.ndarray, b: int, p: int, prm: Params, near: np.ndarray):
    """Open runs best first, taking their keys (ascending) that are not in the
    near set, until k far keys are collected (reading S-4).  Returns (far keys,
    rank of the last opened run or None)."""
    near_s = set(int(x) for x in near)
    far = []
    if prm.k == 0:
        return far, None
    for r, j in enumerate(ranked):
        for key in range(b * int(j), b * int(j) + b):
            if key not in near_s:
                far.append(key)
                if len(far) == prm.k:
                    return far, r
    return far, None


def scan_index_query(y: np.ndarray, p: int, summaries: np.ndarray, b: int,
                     prm: Params) -> IndexResult:
    """Index list of the query at position p under a scan of runs of b keys."""
    yhat = normalize_query(y, prm.index_dtype)
    ranked, s_sorted = scan_rank(yhat, summaries, p, b, prm)
    near = near_set(p, prm)
    far, r = scan_expand(ranked, b, p, prm, near)
    lst = np.union1d(near, np.array(far, np.int64))
    out = np.full(prm.list_len, -1, np.int64)
    out[:len(lst)] = lst
    # near ties around the truncated run (scores indexed by rank)
    exempt = rank_gap_exempt(np.arange(len(ranked)), s_sorted, r)
    return IndexResult(out, len(lst), exempt, ranked, r, len(ranked))


def scan_top_b(prm: Params, b: int) -> int:
    """Runs that provably hold k far keys: every scanned run gives b far keys
    except those holding a sink."""
    return -(-prm.k // b) + -(-prm.n_sink // b)
