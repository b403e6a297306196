"""The parallel forms of the oracle used by the full-size GPU tests give the
same results as the oracle's plain sequential calls (CPU only)."""
import numpy as np

import lsa_synth as S
from oracle import lsa_oracle as O
from parity_util import oracle_cache_parallel, oracle_index_parallel, oracle_tree_parallel


def test_parallel_oracle_equals_sequential_oracle():
    w = S.WORKLOADS[4]
    T = 80 * 512 + 100
    X, Y, _ = S.latent_inputs(w, T=T, query_rows=(T - 300, T))
    prm = O.Params(k=256)
    seq = O.build_cache(X, prm)
    par = oracle_cache_parallel(X, prm, procs=4)
    assert np.array_equal(seq.centroids, par.centroids) and seq.members == par.members
    t_seq = O.build_tree(seq)
    t_par = oracle_tree_parallel(par)
    assert t_seq.height == t_par.height and t_seq.group_min_gap == t_par.group_min_gap
    for a, b in zip(t_seq.levels, t_par.levels):
        for key in ("cent", "child", "min_block"):
            assert np.array_equal(a[key], b[key])
    pos = np.arange(T - 300, T, 7)
    for mode, tree in (("flat", None), ("tree", t_seq)):
        got = oracle_index_parallel(pos, Y[pos - (T - 300)], par, mode, tree)
        for p, r in zip(pos, got):
            e = O.index_query(Y[p - (T - 300)], int(p), seq, mode, tree)
            assert r.count == e.count and np.array_equal(r.idx, e.idx) and r.exempt == e.exempt
