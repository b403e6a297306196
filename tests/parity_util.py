"""Helpers for the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare them (the oracle never sees a GPU result)."""
from __future__ import annotations

import numpy as np
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O


def oracle_params(p: lsa.Params) -> O.Params:
    return O.Params(k=p.k, n_sink=p.n_sink, window=p.window,
                    index_dtype="bf16" if p.index_dtype == lsa.LSA_BF16 else "f32",
                    beam=p.beam, leaf_level=p.leaf_level)


def gpu_cache(X: np.ndarray, p: lsa.Params, max_tokens=None, chunks=None) -> lsa.BucketCache:
    c = lsa.BucketCache(p, max_tokens or X.shape[0])
    Xd = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    if chunks is None:
        c.build(Xd)
    else:
        o = 0
        for n in chunks:
            c.build(Xd[o:o + n].contiguous())
            o += n
    torch.cuda.synchronize()
    return c


def unpack_members(m: np.ndarray) -> list:
    out = []
    for w in m.astype(np.uint32):
        js = [(int(w) >> (8 * e)) & 0xFF for e in range(4)]
        out.append([j for j in js if j != 0xFF])
    return out


def cache_to_host(c: lsa.BucketCache) -> dict:
    v = c.view()
    cent = v["centroids"].float().cpu().numpy().astype(np.float64)
    mem = v["members"].cpu().numpy().view(np.uint32)
    levels = [dict(cent=l["centroids"].float().cpu().numpy().astype(np.float64),
                   child=l["child"].cpu().numpy(), min_block=l["min_block"].cpu().numpy())
              for l in v["levels"]]
    return dict(n_blocks=v["n_blocks"], cent=cent, pooled=unpack_members(mem), levels=levels)


def compare_cache(g: dict, oc: O.BucketCache, X: np.ndarray) -> dict:
    """Partitions and centroids bit-exact outside near-tie blocks; exempt
    blocks still satisfy the invariants and match the oracle's total ESS."""
    nb = oc.n_blocks
    assert g["n_blocks"] == nb
    exempt = mismatched = 0
    for b in range(nb):
        gp = g["pooled"][b * 64:(b + 1) * 64]
        op = oc.pooled[b * 64:(b + 1) * 64]
        # invariants hold for every block
        flat = sorted(j for m in gp for j in m)
        assert flat == list(range(128)), f"block {b}: not a partition"
        assert all(1 <= len(m) <= 4 for m in gp), f"block {b}: cap"
        assert all(m == sorted(m) for m in gp)
        assert [m[0] for m in gp] == sorted(m[0] for m in gp), f"block {b}: bucket order"
        if oc.block_exempt(b):
            exempt += 1
            P = O.pool_keys(O.normalize_keys(X[b * 512:(b + 1) * 512]))
            ess = sum(O.ess(P[m]) for m in gp)
            assert abs(ess - oc.block_ess[b]) <= 1e-6 * oc.block_ess[b], f"block {b}: ESS"
            if gp != op:
                mismatched += 1
            continue
        assert gp == op, f"block {b}: partition differs from the oracle"
        assert np.array_equal(g["cent"][b * 64:(b + 1) * 64], oc.centroids[b * 64:(b + 1) * 64]), \
            f"block {b}: centroids differ"
    return dict(blocks=nb, exempt=exempt, exempt_mismatched=mismatched)


def check_list_invariants(lst: np.ndarray, cnt: int, p: int, prm: O.Params):
    v = lst[:cnt]
    assert np.all(lst[cnt:] == -1)
    assert np.all(np.diff(v) > 0) and v[0] == 0 and v[-1] == p
    near = O.near_set(p, prm)
    assert np.isin(near, v).all()
    far = np.setdiff1d(v, near)
    assert len(far) <= prm.k
    assert np.all(far // 512 < p // 512)


def compare_lists(idx: np.ndarray, cnt: np.ndarray, positions, ys, oc: O.BucketCache,
                  mode="flat", tree=None) -> dict:
    """GPU lists vs oracle lists, query by query."""
    exempt = differ = 0
    for row, (p, y) in enumerate(zip(positions, ys)):
        r = O.index_query(y, int(p), oc, mode, tree)
        gl, gc = idx[row], int(cnt[row])
        check_list_invariants(gl, gc, int(p), oc.params)
        same = gc == r.count and np.array_equal(gl[:gc], r.idx[:r.count])
        if r.exempt:
            exempt += 1
            differ += not same
            continue
        assert same, f"query at position {p}: list differs from the oracle"
    return dict(queries=len(positions), exempt=exempt, exempt_differ=differ)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
