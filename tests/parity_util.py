"""Helpers for the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare them (the oracle never sees a GPU result)."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from oracle import scan_oracle as SO


class FallbackReport:
    """A `stats` sink for the binding's index calls: prints, for every call,
    how many queries took the exact top-B fallback (their candidate list from
    the sampled threshold was unusable), and keeps the running total."""

    def __init__(self):
        self.total = 0
        self.calls = 0

    def __setitem__(self, key, value):
        self.total += value
        self.calls += 1
        print(f"index call {self.calls}: {key} = {value} (running total {self.total})", flush=True)


FB = FallbackReport()


def oracle_params(p: lsa.Params) -> O.Params:
    return O.Params(k=p.k, n_sink=p.n_sink, window=p.window,
                    index_dtype="bf16" if p.index_dtype == lsa.LSA_BF16 else "f32",
                    beam=p.beam, leaf_level=p.leaf_level, start_level=p.start_level)


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


def compare_tree(g: dict, ot: O.Tree, gap: float, label: str = "") -> int:
    """Tree levels bit-exact (children, smallest block, centroids) from level 1
    up to the first level where some group's pairing decision has a gap below
    `gap` (a near tie, where both pairings are correct and everything above may
    differ); the levels above are checked for structure only.  Prints and
    returns the number of levels compared exactly."""
    assert len(g["levels"]) == ot.height
    exact = 0
    for l, lv in enumerate(g["levels"], start=1):
        n_below = ot.levels[l - 1]["cent"].shape[0]
        kids = lv["child"][lv["child"] >= 0]
        assert sorted(kids.tolist()) == list(range(n_below)), f"level {l}: not one parent per node"
        if exact == l - 1 and ot.group_min_gap[l - 1] >= gap:
            assert np.array_equal(lv["child"], ot.levels[l]["child"]), f"level {l} children"
            assert np.array_equal(lv["min_block"], ot.levels[l]["min_block"]), f"level {l} min_block"
            assert np.array_equal(lv["cent"], ot.levels[l]["cent"]), f"level {l} centroids"
            exact = l
    print(f"{label} tree levels compared bit for bit: {exact} of {ot.height}"
          + ("" if exact == ot.height else
             f" (level {exact + 1} has a pairing gap of {ot.group_min_gap[exact]:.3g})"), flush=True)
    return exact


def check_list_invariants(lst: np.ndarray, cnt: int, p: int, prm: O.Params):
    v = lst[:cnt]
    assert np.all(lst[cnt:] == -1)
    assert np.all(np.diff(v) > 0) and v[-1] == p and (v[0] == 0 or prm.n_sink == 0)
    near = O.near_set(p, prm)
    assert np.isin(near, v).all()
    far = np.setdiff1d(v, near)
    assert len(far) <= prm.k
    assert np.all(far // 512 < p // 512)


def n_procs() -> int:
    """Worker processes for the oracle: the CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_G = {}   # oracle state handed to forked workers


def _scan_rows(job):
    out = []
    for p, y in job:
        r = SO.scan_index_query(y, int(p), _G["summ"], _G["b"], _G["prm"])
        r.ranked = None
        out.append(r)
    return out


def compare_scan_lists(idx: np.ndarray, cnt: np.ndarray, positions, ys, summ: np.ndarray, b: int,
                       prm: O.Params, parallel: bool = False) -> dict:
    """GPU scan lists vs the scan oracle's, query by query (bit-exact outside
    near ties at the truncated run)."""
    pairs = list(zip([int(p) for p in positions], list(ys)))
    _G.update(summ=summ, b=b, prm=prm)
    procs = n_procs() if parallel else 1
    if procs > 1 and len(pairs) >= 8:
        jobs = [pairs[i::procs] for i in range(procs)]
        with mp.get_context("fork").Pool(procs) as pool:
            parts = pool.map(_scan_rows, jobs)
        ref = [None] * len(pairs)
        for i, part in enumerate(parts):
            ref[i::procs] = part
    else:
        ref = _scan_rows(pairs)
    _G.clear()
    exempt = differ = 0
    for row, (p, _) in enumerate(pairs):
        r = ref[row]
        gl, gc = idx[row], int(cnt[row])
        v = gl[:gc]
        assert np.all(gl[gc:] == -1) and np.all(np.diff(v) > 0) and v[-1] == p
        assert np.isin(O.near_set(p, prm), v).all()
        same = gc == r.count and np.array_equal(v, r.idx[:r.count])
        if r.exempt:
            exempt += 1
            differ += not same
            continue
        assert same, f"query at position {p}: scan list (b = {b}) differs from the oracle"
    return dict(queries=len(pairs), exempt=exempt, exempt_differ=differ)


def _index_rows(job):
    out = []
    for p, y in job:
        r = O.index_query(y, int(p), _G["oc"], _G["mode"], _G["tree"])
        r.ranked = None          # the full ranking is not compared; keep the transfer small
        out.append(r)
    return out


def oracle_index_parallel(positions, ys, oc: O.BucketCache, mode="flat", tree=None) -> list:
    """O.index_query for every (position, query), queries split across forked
    worker processes (numpy only; no GPU use in the workers)."""
    pairs = list(zip([int(p) for p in positions], list(ys)))
    procs = n_procs()
    if procs == 1 or len(pairs) < 8:
        _G.update(oc=oc, mode=mode, tree=tree)
        return _index_rows(pairs)
    _G.update(oc=oc, mode=mode, tree=tree)
    jobs = [pairs[i::procs] for i in range(procs)]
    with mp.get_context("fork").Pool(procs) as pool:
        parts = pool.map(_index_rows, jobs)
    _G.clear()
    out = [None] * len(pairs)
    for i, part in enumerate(parts):
        out[i::procs] = part
    return out


def oracle_tree_parallel(oc: O.BucketCache) -> O.Tree:
    """O.build_tree with the groups of each level paired in worker processes."""
    with mp.get_context("fork").Pool(n_procs()) as pool:
        return O.build_tree(oc, mapper=lambda f, xs: pool.map(f, xs, chunksize=32))


def compare_lists(idx: np.ndarray, cnt: np.ndarray, positions, ys, oc: O.BucketCache,
                  mode="flat", tree=None, parallel=False) -> dict:
    """GPU lists vs oracle lists, query by query."""
    exempt = differ = 0
    ref = oracle_index_parallel(positions, ys, oc, mode, tree) if parallel else None
    for row, (p, y) in enumerate(zip(positions, ys)):
        r = ref[row] if parallel else O.index_query(y, int(p), oc, mode, tree)
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


# ---------------------------------------------------------------- parallel oracle build
_PX = None
_PPRM = None


def _build_part(blocks):
    c = O.build_cache(_PX, _PPRM, blocks=blocks)
    M = _PPRM.n_buckets
    sel = np.concatenate([np.arange(b * M, (b + 1) * M) for b in blocks])
    return (blocks, c.centroids[sel], [c.members[g] for g in sel], [c.pooled[g] for g in sel],
            c.block_min_gap[blocks], c.block_ess[blocks])


def oracle_cache_parallel(X: np.ndarray, prm: O.Params, procs: int | None = None) -> O.BucketCache:
    """The oracle's build_cache over all full blocks, blocks split across forked
    worker processes (numpy only; no GPU use in the workers)."""
    global _PX, _PPRM
    procs = procs or n_procs()
    nb = X.shape[0] // prm.block
    if nb <= 64:
        return O.build_cache(X, prm)
    _PX, _PPRM = X, prm
    chunks = [c for c in np.array_split(np.arange(nb), procs * 8) if len(c)]
    with mp.get_context("fork").Pool(procs) as pool:
        parts = pool.map(_build_part, chunks)
    M = prm.n_buckets
    cent = np.full((nb * M, prm.d_latent), np.nan)
    members, pooled = [None] * (nb * M), [None] * (nb * M)
    gaps, ess = np.full(nb, np.inf), np.zeros(nb)
    for blocks, ce, me, po, ga, es in parts:
        sel = np.concatenate([np.arange(b * M, (b + 1) * M) for b in blocks])
        cent[sel] = ce
        for g, m, q in zip(sel, me, po):
            members[g], pooled[g] = m, q
        gaps[blocks], ess[blocks] = ga, es
    _PX = None
    return O.BucketCache(prm, nb, cent, members, pooled, gaps, ess)


def device_normal(w, tensor: str, shape, seq: int = 0, row0: int = 0):
    """A Q/K/V tensor generated on the GPU (same Philox definition as the host rows)."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = torch.empty(shape, dtype=dt, device="cuda")
    width = int(np.prod(shape[1:]))
    S.device_fill_normal(t.data_ptr(), t.numel(), S.philox_key(w.cfg, tensor, seq), row0 * width,
                         w.dtype == "bf16", torch.cuda.current_stream().cuda_stream)
    return t


def host_rows(w, tensor: str, rows, width: int, seq: int = 0):
    """Rows of a Q/K/V tensor from the host generator, as float64."""
    vals, _ = S.normal_rows(w, tensor, np.asarray(rows), width, seq)
    return vals.astype(np.float64)


def attention_from_rows(w, q_row: np.ndarray, idx: np.ndarray, count: int, seq: int = 0):
    """Oracle attention of one query whose K/V rows come from the host generator."""
    sel = np.asarray(idx[:count], np.int64)
    k = host_rows(w, "k", sel, w.Hkv * w.D, seq).reshape(-1, w.Hkv, w.D)
    v = host_rows(w, "v", sel, w.Hkv * w.D, seq).reshape(-1, w.Hkv, w.D)
    return O.attention_query(q_row.reshape(w.Hq, w.D), k, v, np.arange(len(sel)), len(sel))
