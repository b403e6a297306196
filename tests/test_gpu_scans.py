"""GPU parity of the scan baselines (a token scan over every key, block scans
over aligned runs of 4 and 8 keys) against the scan oracle, through the C ABI:
run summaries bit-exact, index lists bit-exact outside near ties at the
truncated run, at the 4K parity size (every query), 32K, and the 128K, 1M and
10M workload shapes the benchmark times (sampled queries)."""
import sys
import time

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from oracle import scan_oracle as SO
from parity_util import (FB, attention_from_rows, compare_scan_lists, device_normal, host_rows,
                         oracle_params)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()


def _scan_cache(X, p, T=None):
    c = lsa.BucketCache(p, T or X.shape[0])
    c.build(torch.from_numpy(np.ascontiguousarray(X)).cuda())
    torch.cuda.synchronize()
    return c


def _summaries_match(c, X, b, prm):
    got = c.view()["centroids"].float().cpu().numpy().astype(np.float64)
    ref = SO.run_summaries(X[:(X.shape[0] // 512) * 512], b, prm.index_dtype)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"b={b}: {int((got != ref).any(axis=1).sum())} run summaries differ"


@pytest.mark.parametrize("b", [1, 4, 8])
@pytest.mark.parametrize("dtype", [lsa.LSA_F32, lsa.LSA_BF16])
def test_scan_summaries_and_lists_4k_all_queries(b, dtype):
    say(f"case: scan b={b} T=4096 dtype={dtype} all queries")
    w = S.WORKLOADS[1]
    X, Y, _ = S.latent_inputs(w, T=4096, query_rows=(0, 4096))
    p = lsa.Params(k=256, index_dtype=dtype, scan_keys=b)
    c = _scan_cache(X, p)
    prm = oracle_params(p)
    _summaries_match(c, X, b, prm)
    idx, cnt = lsa.index_prefill(c, torch.from_numpy(Y).cuda(), 0, p, stats=FB)
    torch.cuda.synchronize()
    summ = SO.run_summaries(X, b, prm.index_dtype)
    say("scan index", compare_scan_lists(idx.cpu().numpy(), cnt.cpu().numpy(), range(4096), Y,
                                         summ, b, prm, parallel=True))


@pytest.mark.parametrize("b,k,n_sink", [(1, 256, 4), (1, 2048, 4), (4, 2048, 4), (8, 2048, 4),
                                        (8, 256, 5), (4, 1000, 9)])
def test_scan_lists_32k(b, k, n_sink):
    """The bf16 prefill kernels (sampled threshold, high- and low-pass
    scoring, selection) on scans at T=32,768, sinks that fill runs partly."""
    say(f"case: scan b={b} T=32768 bf16 k={k} n_sink={n_sink}")
    w = S.WORKLOADS[2]
    T = 32768
    X, Y, _ = S.latent_inputs(w, T=T, query_rows=(0, T))
    p = lsa.Params(k=k, n_sink=n_sink, scan_keys=b)
    c = _scan_cache(X, p)
    idx, cnt = lsa.index_prefill(c, torch.from_numpy(Y).cuda(), 0, p, stats=FB)
    torch.cuda.synchronize()
    prm = oracle_params(p)
    summ = SO.run_summaries(X, b, "bf16")
    pos = np.unique(np.concatenate([np.arange(0, T, 211), np.arange(511, T, 1024), np.arange(T - 8, T),
                                    [0, 1, 515, 516, 517, 520]]))
    say("scan index", compare_scan_lists(idx.cpu().numpy()[pos], cnt.cpu().numpy()[pos], pos, Y[pos],
                                         summ, b, prm, parallel=True))


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_scans_at_workload_sizes(cfg):
    """The token scan and the block scans of 4 and 8 on the 128K prefill, the
    1M last chunk and the 10M last chunk, as the benchmark runs them: run
    summaries bit-exact (all of them), sampled lists against the oracle, and
    the attention over a few of the token scan's lists."""
    w = S.WORKLOADS[cfg]
    say(f"case: scans at {w.name}")
    t0 = time.time()
    X, Y, _ = S.latent_inputs(w)
    say(f"inputs {time.time() - t0:.1f}s")
    Yd = torch.from_numpy(Y).cuda()
    rows = np.unique(np.concatenate([np.linspace(0, w.Tq - 1, 24 if cfg == 5 else 40).astype(int),
                                     [w.Tq - 1]]))
    for b in (1, 4, 8):
        p = lsa.Params(k=w.k, scan_keys=b)
        c = _scan_cache(X, p)
        idx, cnt = lsa.index_prefill(c, Yd, w.q_start, p, stats=FB)
        torch.cuda.synchronize()
        prm = oracle_params(p)
        t0 = time.time()
        got = c.view()["centroids"]
        summ = SO.run_summaries(X[:(w.T // 512) * 512], b, "bf16")
        assert np.array_equal(got.float().cpu().numpy().astype(np.float64), summ), f"b={b} summaries"
        del got, c
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        say(f"b={b}", compare_scan_lists(idx_h[rows], cnt_h[rows], w.q_start + rows, Y[rows], summ, b,
                                         prm, parallel=True), f"oracle {time.time() - t0:.1f}s")
        if b == 1:
            arows = rows[::6]
            Q = device_normal(w, "q", (w.Tq, w.Hq, w.D), row0=w.q_start)
            K = device_normal(w, "k", (w.T, w.Hkv, w.D))
            V = device_normal(w, "v", (w.T, w.Hkv, w.D))
            out = lsa.sparse_attention(Q, K, V, idx, cnt)
            torch.cuda.synchronize()
            del K, V, Q
            out_h = out.float().cpu().numpy()
            q_rows = host_rows(w, "q", w.q_start + arows, w.Hq * w.D)
            err = max(float(np.abs(out_h[r] - attention_from_rows(w, q_rows[i], idx_h[r],
                                                                  int(cnt_h[r]))).max())
                      for i, r in enumerate(arows))
            say(f"token-scan attention max abs err {err:.3g} over {len(arows)} queries")
            assert err <= 2e-2
        del idx, cnt, summ
