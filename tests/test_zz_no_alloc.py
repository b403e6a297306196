"""The allocation-free attention entry point (lsa_sparse_attention_static)
against lsa_sparse_attention with a caller workspace, through the C ABI: two
calls in a row on the library's fixed array, the second one smaller, each
equal bit for bit to the workspace call (same kernels, same splits) and within
the attention tolerance of the oracle."""
import sys

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _lists(rng, positions, L):
    idx = np.full((len(positions), L), -1, np.int32)
    cnt = np.zeros(len(positions), np.int32)
    for i, pos in enumerate(positions):
        n = min(L - 17 * (i % 3), int(pos) + 1)
        idx[i, :n] = np.sort(rng.choice(int(pos) + 1, size=n, replace=False))
        cnt[i] = n
    return idx, cnt


def _case(dtype, B, T, L, splits, seed):
    w = S.WORKLOADS[2]
    D, Hq, Hkv = w.D, w.Hq, w.Hkv
    rng = np.random.default_rng(seed)
    pos = np.full(B, T - 1)
    q = rng.standard_normal((B, 1, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(x).to(tdt).cuda() for x in (q, k, v))
    qr, kr, vr = (t.float().cpu().numpy().astype(np.float64) for t in (Q, K, V))
    idx, cnt = _lists(rng, pos, L)
    I = torch.from_numpy(idx).cuda().view(B, 1, L)
    C = torch.from_numpy(cnt).cuda().view(B, 1)
    return Q, K, V, I, C, qr, kr, vr, idx, cnt


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_attention_matches_workspace_attention(dtype):
    tol = 2e-2 if dtype == "bf16" else 1e-4
    calls = [(16, 6000, 2564, 16, 1), (3, 3000, 900, 8, 2)]     # the second call is smaller
    for B, T, L, splits, seed in calls:
        say(f"case: static attention {dtype} B={B} T={T} L={L} splits={splits}")
        Q, K, V, I, C, qr, kr, vr, idx, cnt = _case(dtype, B, T, L, splits, seed)
        need = lsa.lib().lsa_attention_workspace_bytes(B, 1, Q.shape[2], Q.shape[3], splits)
        assert 0 < need <= (16 << 20)
        out = torch.empty_like(Q)
        got = lsa.sparse_attention_static(Q, K, V, I, C, splits=splits, out=out)
        ref = lsa.sparse_attention(Q, K, V, I, C, splits=splits)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"B={B}: differs from the workspace call"
        g = got.float().cpu().numpy()
        err = max(np.abs(g[b, 0] - O.attention_query(qr[b, 0], kr[b], vr[b], idx[b], cnt[b])).max()
                  for b in range(B))
        say(f"max abs err vs oracle {err:.3g}")
        assert err <= tol
