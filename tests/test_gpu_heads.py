"""GPU parity of the max-over-heads bucket score ([catalog "Key points"],
N-LSA: bucket selection uses the max score across heads): each query position
brings H latent query heads and a bucket scores the largest of its H dot
products; lists against the oracle's (bit-exact outside near ties), through
the C ABI, with the sampled threshold and with exact selection."""
import sys

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from parity_util import FB, compare_lists, gpu_cache, oracle_cache_parallel, oracle_params

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()


@pytest.mark.parametrize("H,k,exact", [(8, 256, 0), (8, 2048, 0), (4, 256, 0), (2, 1000, 0),
                                       (8, 256, 1)])
def test_max_over_heads_lists_32k(H, k, exact):
    say(f"case: max over {H} heads T=32768 k={k} exact={exact}")
    w = S.WORKLOADS[2]
    T = 32768
    X, _, _ = S.latent_inputs(w, T=T, query_rows=(0, 1))
    Yh = S.latent_query_heads(w, H, 0, T)
    p = lsa.Params(k=k, score_heads=H, exact_select=exact)
    c = gpu_cache(X, p)
    idx, cnt = lsa.index_prefill(c, torch.from_numpy(Yh).cuda(), 0, p, stats=FB)
    torch.cuda.synchronize()
    oc = O.build_cache(X, oracle_params(p))
    pos = np.unique(np.concatenate([np.arange(0, T, 173), np.arange(511, T, 2048),
                                    np.arange(T - 8, T), [0, 1, 512, 513]]))
    say("index", compare_lists(idx.cpu().numpy()[pos], cnt.cpu().numpy()[pos], pos, Yh[pos], oc,
                               parallel=True))


def test_max_over_heads_128k_full_size():
    """The 128K prefill shape with the GQA group's 8 query heads per position:
    sampled lists against the oracle."""
    say("case: max over 8 heads, T=131072")
    w = S.WORKLOADS[2]
    X, _, _ = S.latent_inputs(w, query_rows=(0, 1))
    Yh = S.latent_query_heads(w, 8, 0, w.T)
    p = lsa.Params(k=w.k, score_heads=8)
    c = gpu_cache(X, p)
    idx, cnt = lsa.index_prefill(c, torch.from_numpy(Yh).cuda(), 0, p, stats=FB)
    torch.cuda.synchronize()
    oc = oracle_cache_parallel(X, oracle_params(p))
    rows = np.unique(np.concatenate([np.linspace(0, w.T - 1, 80).astype(int), [w.T - 1]]))
    say("index", compare_lists(idx.cpu().numpy()[rows], cnt.cpu().numpy()[rows], rows, Yh[rows],
                               oc, parallel=True))
