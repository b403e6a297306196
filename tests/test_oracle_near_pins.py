"""Pins of the oracle's near_union: the keys a prefill query reads when its near
set (sinks and recent window) is attended whole and only its list's other
entries are gathered ([72x "The same steps in general"]; [visual "What one
query actually does"]: every list holds the sinks and the window).  Hand-worked
cases, and the property that on a list the method itself writes, near_union is
a reordering of that list."""
import numpy as np
import pytest

from oracle import lsa_oracle as O

pytestmark = pytest.mark.filterwarnings("ignore")


def test_near_union_hand_worked():
    # p = 10, 2 sinks, window 3: near set {0, 1} U {8, 9, 10}.  The list holds
    # sink 0, far key 5 twice, window key 9, an entry past T = 11 and a -1:
    # kept are 5 and 5 (duplicates stay), then the whole near set.
    prm = O.Params(k=4, n_sink=2, window=3)
    got = O.near_union(np.array([0, 5, 5, 9, 12, -1]), 6, 10, prm, 11)
    assert got.tolist() == [5, 5, 0, 1, 8, 9, 10]


def test_near_union_clips_sinks_to_the_query():
    # p = 1 < 4 sinks: the near set is {0, 1}; a non-causal entry 3 is not near
    prm = O.Params(k=4, n_sink=4, window=3)
    assert O.near_union(np.array([3]), 1, 1, prm, 11).tolist() == [3, 0, 1]


def test_near_union_count_limits_the_list():
    # entries past the count are not read; an empty list gives the near set
    prm = O.Params(k=4, n_sink=1, window=2)
    assert O.near_union(np.array([4, 2, 7]), 2, 6, prm, 8).tolist() == [4, 2, 0, 5, 6]
    assert O.near_union(np.array([4, 2, 7]), 0, 6, prm, 8).tolist() == [0, 5, 6]


def test_near_union_window_only_query_near_start():
    # the window reaches back past 0 and overlaps the sinks: near = [0, p]
    prm = O.Params(k=4, n_sink=2, window=8)
    assert O.near_union(np.array([0, 1, 2, 3]), 4, 3, prm, 100).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("n_sink,window,k", [(4, 512, 64), (9, 700, 100), (0, 1, 32)])
def test_near_union_reorders_a_method_list(n_sink, window, k):
    rng = np.random.default_rng(7)
    T = 2048
    prm = O.Params(k=k, n_sink=n_sink, window=window)
    X = rng.standard_normal((T, prm.d_latent))
    cache = O.build_cache(X, prm)
    for p in (0, 3, 600, 1100, T - 1):
        y = rng.standard_normal(prm.d_latent)
        r = O.index_query(y, p, cache)
        got = O.near_union(r.idx, r.count, p, prm, T)
        assert sorted(got.tolist()) == sorted(r.idx[:r.count].tolist()), p
